"""The rocprofv3 trace summariser (host logic): kernel-name to site mapping
and the even split of overlapping kernels' time."""
import pytest

from whisper_audio_encoder_amd import trace_summary as ts


def test_site_of_kernel_names():
    g = "void wk::(anonymous namespace)::gemm_kernel<256, 256, 128, 64, 8, {e}, {t}>(wk::(anonymous namespace)::GemmP)"
    assert ts.site_of(g.format(e=0, t=1)) == "fc1"
    assert ts.site_of(g.format(e=0, t=0)) == "conv1"
    assert ts.site_of(g.format(e=2, t=0)) == "oproj"
    assert ts.site_of(g.format(e=2, t=1)) == "fc2"
    assert ts.site_of(g.format(e=3, t=0)) == "qkv"
    g8 = "void wk::(anonymous namespace)::gemm_kernel<256, 256, 128, 64, 8, {e}, {t}, {pp}>(wk::(anonymous namespace)::GemmP)"
    assert ts.site_of(g8.format(e=0, t=1, pp=1)) == "fc1"
    assert ts.site_of(g8.format(e=2, t=1, pp=0)) == "fc2"
    assert ts.site_of(g8.format(e=4, t=0, pp=1)) == "xkv"
    assert ts.site_of("_ZN2wk12_GLOBAL__N_111attn_kernelEPKDF16_S2_S2_PDF16_iii") == "attn"
    assert ts.site_of("void wk::(anonymous namespace)::ln_kernel<5, false>(float const*)") == "ln"
    assert ts.site_of("void wk::(anonymous namespace)::ln_kernel<5, true>(float const*)") == "lnf"
    assert ts.site_of("__amd_rocclr_copyBuffer") is None


def test_fair_share_splits_overlaps_evenly():
    # a: [0, 10), b: [5, 15), c: [20, 30) -> a 5 + 2.5, b 2.5 + 5, c 10; busy 25
    share, busy = ts.fair_share_ns([(0, 10, "a"), (5, 15, "b"), (20, 30, "c")])
    assert busy == 25
    assert share["a"] == pytest.approx(7.5) and share["b"] == pytest.approx(7.5) and share["c"] == pytest.approx(10)
    # sequential kernels keep their own durations; the shares add up to the busy time
    share, busy = ts.fair_share_ns([(0, 4, "x"), (4, 9, "y"), (9, 10, "x")])
    assert (share["x"], share["y"], busy) == (5, 5, 10)
    share, busy = ts.fair_share_ns([(0, 12, "x"), (2, 4, "y"), (3, 8, "z")])
    assert sum(share.values()) == pytest.approx(busy) == 12


def test_util_by_grid_recovers_the_clock(tmp_path):
    """GEMM dispatches of two grid sizes: GRBM_GUI_ACTIVE (summed over 8
    XCDs) = 8 (2.0 GHz x duration + 5000 cycles); the slope over the longest
    third gives the clock, the intercept the cycles outside the dispatch."""
    import csv
    path = tmp_path / "c.csv"
    name = "void wk::(anonymous namespace)::gemm_kernel<256, 256, 128, 64, 8, 0, 0, 1>(wk::(anonymous namespace)::GemmP)"
    with open(path, "w", newline="") as fh:
        w = csv.writer(fh)
        w.writerow(["Dispatch_Id", "Grid_Size", "Workgroup_Size", "Kernel_Name", "Counter_Name", "Counter_Value",
                    "Start_Timestamp", "End_Timestamp"])
        did = 0
        for wgs, clk in ((1024, 2.0), (32, 2.4)):
            for dur in (10000, 20000, 40000, 80000, 160000, 320000):
                did += 1
                cyc = 8 * (clk * dur + 5000)
                busy = 1024 * 0.5 * clk * dur
                w.writerow([did, wgs * 512, 512, name, "GRBM_GUI_ACTIVE", cyc, 0, dur])
                w.writerow([did, wgs * 512, 512, name, "SQ_VALU_MFMA_BUSY_CYCLES", busy, 0, dur])
    table = ts.utilisation_by_grid(str(path))
    rows = [r.split("|")[1:-1] for r in table.splitlines()[2:]]
    got = {int(r[2]): (float(r[5]), r[6].strip(), r[7].strip()) for r in rows}
    assert got[1024][0] == pytest.approx(2.0, abs=0.005) and got[32][0] == pytest.approx(2.4, abs=0.005)
    assert got[1024][1] == "5.0 k" and got[1024][2] == "50.0%"


def test_stalls_per_wave_and_shares(tmp_path):
    """Two attention dispatches of 100 waves: instructions per wave and the
    waiting and VALU-active shares of the waves' resident cycles."""
    import csv
    path = tmp_path / "s.csv"
    name = "_ZN2wk12_GLOBAL__N_111attn_kernelEPKDF16_S2_S2_PDF16_iii"
    vals = {"SQ_WAVES": 100, "SQ_WAVE_CYCLES": 10000, "SQ_WAIT_INST_ANY": 4000, "SQ_ACTIVE_INST_VALU": 2000,
            "SQ_INSTS_VALU": 12400, "SQ_INSTS_MFMA": 1700, "SQ_INSTS_LDS": 1600}
    with open(path, "w", newline="") as fh:
        w = csv.writer(fh)
        w.writerow(["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value", "Start_Timestamp", "End_Timestamp"])
        for did in (1, 2):
            for k, v in vals.items():
                w.writerow([did, name, k, v, 0, 5000])
    row = ts.stalls(str(path)).splitlines()[2].split("|")[1:-1]
    assert [c.strip() for c in row] == ["attn", "2", "5.0", "100", "124", "17", "16", "40%", "20%"]
