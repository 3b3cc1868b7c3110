"""End-to-end parity on the GPU: wenc_forward through the C ABI against the
fp64 oracle on the five seeded workloads, plus stage taps, determinism,
batch invariance, the stream split, chunking, poisoned scratch, weight
reloads and the error paths.

Every workload runs at its full batch in the same launch configuration the
benchmark times, and the oracle checks EVERY window of every workload (one
test case per window, so each case stays short; the GPU forward of a
workload runs once and is shared).  The pages verify each stage against an
independent implementation (whisper README, "How it is verified"; CKE page,
"Why CKE Builds It This Way"): the stage taps below compare conv1, the stem
and the residual after every block with the oracle's values on every
workload.
"""
import functools

import numpy as np
import pytest
import torch

import oracle
from tests.gpu_util import DEV, check_encoder_tolerance, dev, host, row_cosine, say
from whisper_audio_encoder_amd import synth, wenc
from whisper_audio_encoder_amd.configs import CONFIGS

pytestmark = pytest.mark.gpu

NAMES = ["c0", "c1", "c2", "c3", "c4"]


@functools.lru_cache(maxsize=None)
def inputs(name):
    cfg = CONFIGS[name]
    mel, params = synth.make_inputs(cfg)
    return cfg, mel, params, synth.pack_blob(cfg, params)


@functools.lru_cache(maxsize=None)
def oracle_taps(name):
    """The oracle's stage values of window 0 (conv1, stem, every block, output)."""
    cfg, mel, params, _ = inputs(name)
    return oracle.encode(mel[0], params, cfg.n_layer, cfg.n_head, cfg.ln_eps, bool(cfg.final_ln), taps=True)


@functools.lru_cache(maxsize=None)
def oracle_window(name, item):
    """The oracle's output for one window (kept: other test files reuse it)."""
    if item == 0:
        return oracle_taps(name)["out"]
    cfg, mel, params, _ = inputs(name)
    return oracle.encode(mel[item], params, cfg.n_layer, cfg.n_head, cfg.ln_eps, bool(cfg.final_ln))


oracle_out = oracle_window


@functools.lru_cache(maxsize=None)
def encoder(name, max_batch=None):
    cfg, _, _, blob = inputs(name)
    return wenc.Encoder(cfg, blob, max_batch=max_batch)


@functools.lru_cache(maxsize=None)
def gpu_out(name):
    """The workload's whole batch through one wenc_forward (host copy)."""
    cfg, mel, _, _ = inputs(name)
    say(f"encoder {name} batch {cfg.batch}")
    out = host(encoder(name).forward(dev(mel)))
    assert out.shape == (cfg.batch, cfg.n_ctx, cfg.d_model)
    assert np.isfinite(out).all()
    return out


CASES = [(n, i) for n in NAMES for i in range(CONFIGS[n].batch)]


@pytest.mark.timeout(300)
@pytest.mark.parametrize("name,item", CASES, ids=[f"{n}-w{i}" for n, i in CASES])
def test_encoder_matches_oracle(name, item):
    out = gpu_out(name)
    check_encoder_tolerance(out[item], oracle_window(name, item), f"{name} window {item}")


@pytest.mark.timeout(300)
@pytest.mark.parametrize("name", NAMES)
def test_stage_taps(name):
    """conv1 (after its GELU), the stem (conv2 + GELU + positions) and the
    residual after every block of window 0, each against the oracle's value
    at that stage: relative error per tensor <= 1e-2 and per-row cosine
    >= 0.9999."""
    cfg, mel, _, _ = inputs(name)
    say(f"taps {name}: c1, stem, {cfg.n_layer} blocks")
    enc = encoder(name)
    m = dev(mel[:1])
    ref = oracle_taps(name)
    stages = [(wenc.WENC_TAP_C1, ref["c1"], "c1"), (wenc.WENC_TAP_STEM, ref["x0"], "stem")]
    stages += [(wenc.WENC_TAP_BLOCK + l, ref["blocks"][l], f"block{l}") for l in range(cfg.n_layer)]
    worst = 0.0
    for tap, want, what in stages:
        got = host(enc.tap(m, tap))[0].astype(np.float64)
        rel = np.linalg.norm(got - want) / np.linalg.norm(want)
        cos = row_cosine(got, want).min()
        worst = max(worst, rel)
        assert rel <= 1e-2, f"{name} {what}: relative error {rel}"
        assert cos >= 0.9999, f"{name} {what}: min row cosine {cos}"
    say(f"taps {name}: worst relative error {worst:.2e} over {len(stages)} stages")


@pytest.mark.timeout(300)
def test_sharpened_attention_matches_oracle():
    """With the workloads' N(0, 0.02) weights attention is nearly uniform, and
    an attention that returned mean(V) would still pass end to end.  Here wq
    and wk of every layer are scaled x5 (scores x25, spread of a few units),
    at the base-sized workload's shape, and every window must still match
    the oracle.  tests/test_oracle_mutations.py shows on the CPU that a
    mean(V) attention fails this comparison."""
    cfg, mel, params, _ = inputs("c2")
    sp = synth.sharpen_attention(params, cfg.n_layer, 5.0)
    say("sharpened attention c2 (wq, wk x5)")
    enc = wenc.Encoder(cfg, synth.pack_blob(cfg, sp))
    try:
        out = host(enc.forward(dev(mel)))
    finally:
        enc.close()
    for it in range(cfg.batch):
        ref = oracle.encode(mel[it], sp, cfg.n_layer, cfg.n_head, cfg.ln_eps, bool(cfg.final_ln))
        check_encoder_tolerance(out[it], ref, f"sharpened c2 window {it}")


def test_deterministic():
    name = "c2"
    cfg, mel, _, _ = inputs(name)
    say("determinism c2")
    a = host(encoder(name).forward(dev(mel)))
    assert np.array_equal(a, gpu_out(name))


@pytest.mark.timeout(300)
@pytest.mark.parametrize("name", ["c2", "c3", "c4"])
def test_batch_invariant_every_window(name):
    """Each window of the batched forward equals, bit for bit, a forward of
    that window alone (windows straddle tile boundaries and the tile-size
    split differently in the two launches)."""
    cfg, mel, _, _ = inputs(name)
    say(f"batch invariance {name}, {cfg.batch} single-window forwards")
    full = gpu_out(name)
    enc = encoder(name)
    for b in range(cfg.batch):
        single = host(enc.forward(dev(mel[b:b + 1])))
        assert np.array_equal(single[0], full[b]), f"{name} window {b}"


@pytest.mark.timeout(300)
@pytest.mark.parametrize("streams", [1, 3, 4])
def test_stream_split_changes_no_bit(monkeypatch, streams):
    """The forward splits a chunk's windows over several streams
    (WENC_SPLIT_STREAMS, default 2); any split gives the same bits,
    including uneven groups (c2's 8 windows in 3, a batch of 5 in 4)."""
    name = "c2"
    cfg, mel, _, blob = inputs(name)
    say(f"stream split {streams} c2")
    monkeypatch.setenv("WENC_SPLIT_STREAMS", str(streams))
    enc = wenc.Encoder(cfg, blob)
    try:
        out = host(enc.forward(dev(mel)))
        five = host(enc.forward(dev(mel[:5])))
    finally:
        enc.close()
    assert np.array_equal(out, gpu_out(name))
    assert np.array_equal(five, gpu_out(name)[:5])


def test_chunking_matches_full_batch():
    name = "c2"
    cfg, mel, _, blob = inputs(name)
    say("chunking c2 max_batch 3")
    small = wenc.Encoder(cfg, blob, max_batch=3)
    try:
        chunked = host(small.forward(dev(mel)))
    finally:
        small.close()
    assert np.array_equal(gpu_out(name), chunked)


def test_poisoned_scratch_gives_same_output(monkeypatch):
    """Scratch filled with NaN at creation: no kernel may read what it did not write."""
    name = "c1"
    cfg, mel, _, blob = inputs(name)
    say("poisoned scratch c1")
    monkeypatch.setenv("WENC_POISON_SCRATCH", "1")
    enc = wenc.Encoder(cfg, blob)
    try:
        out = host(enc.forward(dev(mel)))
    finally:
        enc.close()
    assert np.array_equal(out, gpu_out(name))


def test_non_finite_input_propagates_within_its_window():
    """A NaN or an infinity in one window's mel is not sanitised: that
    window's whole memory becomes NaN (every position attends to the
    poisoned keys), as in the oracle, and the other windows' outputs keep
    every bit."""
    name = "c2"
    cfg, mel, params, _ = inputs(name)
    say("non-finite mel c2")
    enc = encoder(name)
    clean = gpu_out(name)
    bad = mel.copy()
    bad[2, 1234, 17] = np.nan
    bad[5, 2999, 0] = np.inf
    out = host(enc.forward(dev(bad)))
    for b in (2, 5):
        assert np.isnan(out[b]).all(), b
    for b in (0, 1, 3, 4, 6, 7):
        assert np.array_equal(out[b], clean[b]), b
    small = CONFIGS["c0"]
    m0, p0 = synth.make_inputs(small)
    m0 = m0.copy()
    m0[0, 1234, 17] = np.nan
    ref = oracle.encode(m0[0], p0, small.n_layer, small.n_head)
    assert np.isnan(ref).all()


def test_debug_sync_mode_gives_same_output(monkeypatch):
    """WENC_DEBUG_SYNC=1 (a stream synchronise and error check after every
    launch) changes no result bit and reports success."""
    name = "c1"
    cfg, mel, _, blob = inputs(name)
    say("debug sync c1")
    monkeypatch.setenv("WENC_DEBUG_SYNC", "1")
    enc = wenc.Encoder(cfg, blob)
    try:
        out = host(enc.forward(dev(mel)))
    finally:
        enc.close()
    assert np.array_equal(out, gpu_out(name))


def test_no_final_ln_and_zero_layers():
    base = CONFIGS["c0"]
    rng_cfg = base.with_(n_layer=0, final_ln=0, name="c0-l0")
    mel, params = synth.make_inputs(rng_cfg)
    say("zero layers, no final LN")
    enc = wenc.Encoder(rng_cfg, synth.pack_blob(rng_cfg, params))
    try:
        out = host(enc.forward(dev(mel)))[0]
    finally:
        enc.close()
    ref = oracle.encode(mel[0], params, 0, rng_cfg.n_head, final_ln=False)
    check_encoder_tolerance(out, ref, "L=0 no final LN")


@pytest.mark.timeout(300)
def test_reload_waits_for_forwards_in_flight():
    """wenc_load on a loaded handle first lets every forward already queued
    (here on a torch side stream, which does not wait for the null stream)
    finish on the old weights; forwards after it use the new ones.  A blob of
    the wrong size changes nothing."""
    name = "c2"
    cfg, mel, params, blob = inputs(name)
    _, params2 = synth.make_inputs(cfg, seed=cfg.seed + 17)
    blob2 = synth.pack_blob(cfg, params2)
    say("reload while forwards are queued, c2")
    fresh = wenc.Encoder(cfg, blob2)
    try:
        want_new = host(fresh.forward(dev(mel)))
    finally:
        fresh.close()
    want_old = gpu_out(name)
    assert not np.array_equal(want_new, want_old)
    enc = wenc.Encoder(cfg, blob)
    try:
        m = dev(mel)
        outs = [torch.empty((cfg.batch, cfg.n_ctx, cfg.d_model), device=DEV) for _ in range(4)]
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            # ~0.1 s of GPU work, longer than the host repack of the new blob
            for i in range(96):
                enc.forward(m, outs[i % 4])
        wenc.wenc_load(enc.h, blob2)
        torch.cuda.synchronize()
        for o in outs:
            assert np.array_equal(host(o), want_old)
        assert np.array_equal(host(enc.forward(m)), want_new)
        with pytest.raises(wenc.WencError) as e:
            wenc.wenc_load(enc.h, blob[:-2])
        assert e.value.code == wenc.WENC_EINVAL
        assert np.array_equal(host(enc.forward(m)), want_new)
    finally:
        enc.close()


def _misaligned(shape, dtype, offset_bytes):
    """A device tensor whose data pointer sits offset_bytes past an aligned one."""
    n = int(np.prod(shape)) * torch.tensor([], dtype=dtype).element_size() + offset_bytes
    raw = torch.zeros(n + 64, dtype=torch.uint8, device=DEV)
    base = (-raw.data_ptr()) % 64
    return raw[base + offset_bytes: base + n]


def test_error_paths():
    cfg, mel, _, blob = inputs("c0")
    say("error paths")
    h = wenc.wenc_create(wenc.make_config(cfg))
    try:
        m = dev(mel)
        out = torch.empty((1, cfg.n_ctx, cfg.d_model), device=DEV)
        with pytest.raises(wenc.WencError) as e:
            wenc.wenc_forward(h, m, 1, out)
        assert e.value.code == wenc.WENC_ESTATE
        with pytest.raises(wenc.WencError) as e:
            wenc.wenc_load(h, blob[:-2])
        assert e.value.code == wenc.WENC_EINVAL and "exactly" in str(e.value)
        with pytest.raises(wenc.WencError) as e:
            wenc.wenc_forward(h, m, 1, out)
        assert e.value.code == wenc.WENC_ESTATE  # a rejected blob loads nothing
        wenc.wenc_load(h, blob)
        with pytest.raises(wenc.WencError) as e:
            wenc.wenc_forward(h, m, -1, out)
        assert e.value.code == wenc.WENC_EINVAL
        wenc.wenc_forward(h, m, 0, out)  # empty batch: a no-op
        with pytest.raises(wenc.WencError) as e:
            wenc.wenc_forward_tap(h, m, 1, wenc.WENC_TAP_BLOCK + cfg.n_layer, out)
        assert e.value.code == wenc.WENC_EINVAL
    finally:
        wenc.wenc_destroy(h)


def test_misaligned_pointers_are_rejected():
    """Every entry point whose kernels use 16-byte vector accesses on a
    caller's buffer rejects a pointer that is not 16-byte aligned (4-byte for
    the log-mel audio samples) with WENC_EINVAL, before any launch."""
    name = "c0"
    cfg, mel, _, _ = inputs(name)
    say("misaligned pointers")
    enc = encoder(name)
    h = enc.h
    m = dev(mel)
    out = torch.empty((1, cfg.n_ctx, cfg.d_model), device=DEV)
    bad_m = _misaligned(m.shape, torch.float32, 4)
    bad_m.copy_(m.view(torch.uint8).reshape(-1))
    bad_out = _misaligned(out.shape, torch.float32, 8)

    def expect_einval(fn, *args):
        with pytest.raises(wenc.WencError) as e:
            fn(*args)
        assert e.value.code == wenc.WENC_EINVAL and "aligned" in str(e.value), str(e.value)

    expect_einval(wenc.wenc_forward, h, bad_m, 1, out)
    expect_einval(wenc.wenc_forward, h, m, 1, bad_out)
    expect_einval(wenc.wenc_forward_ctx, h, bad_m[: 4 * 1000 * cfg.n_mels], 1, 500, out)
    expect_einval(wenc.wenc_forward_tap, h, bad_m, 1, wenc.WENC_TAP_STEM, out)
    audio = torch.zeros((1, 160 * cfg.n_frames), device=DEV)
    expect_einval(wenc.wenc_log_mel, h, _misaligned(audio.shape, torch.float32, 2), 1, m)
    expect_einval(wenc.wenc_log_mel, h, audio, 1, bad_m)
    xkv = torch.empty((1, 1, cfg.n_ctx, cfg.d_model), dtype=torch.float16, device=DEV)
    enc.load_cross(synth.pack_cross_blob(cfg, synth.make_cross_params(cfg, 1), 1), 1)
    expect_einval(wenc.wenc_prepare_cross, h, bad_out, 1, cfg.n_ctx, xkv, xkv)
    expect_einval(wenc.wenc_prepare_cross, h, out, 1, cfg.n_ctx, _misaligned(xkv.shape, torch.float16, 2), xkv)
    # the aligned calls still work afterwards
    assert np.array_equal(host(enc.forward(m, out)), gpu_out(name))


def test_enomem_reports_free_memory():
    # fc1 activations of 2000 windows at d_ff 65536: ~390 GB, beyond any one GPU
    cfg = CONFIGS["c4"].with_(n_layer=1, d_ff=65536)
    say("enomem")
    big = wenc.make_config(cfg, max_batch=2000)
    import ctypes
    h = ctypes.c_void_p()
    rc = wenc.lib().wenc_create(ctypes.byref(big), ctypes.byref(h))
    assert rc == wenc.WENC_ENOMEM and h.value is None
    msg = wenc.wenc_last_error()
    assert "cannot allocate" in msg and "free" in msg
