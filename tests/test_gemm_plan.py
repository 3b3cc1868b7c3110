"""The GEMM tile planner (host logic, no device): which tile kernels a launch
uses for M x N outputs on a given number of compute units.

Every plan sums each output over k in the same order, so a plan changes
timing only; the GPU tests check that all plans give the same bits.  Here:
the decisions on the encoder's own shapes (those measured fastest on the
MI355X's 256 CUs) and invariants over a sweep of shapes and CU counts.
"""
import math

import pytest

from whisper_audio_encoder_amd import wenc

SMALL, BIG, SPLIT = 0, 1, 2

# (M as the kernel sees it, N) -> plan on 256 CUs; QKV rows are padded to 1504 per window
ENCODER_PLANS = {
    "c4 fc1": ((24000, 5120), (SPLIT, 89 * 256)),
    "c4 fc2 / out_proj / conv2": ((24000, 1280), (BIG, 24000)),
    "c4 qkv": ((16 * 1504, 3840), (BIG, 16 * 1504)),
    "c4 conv1": ((48000, 1280), (BIG, 48000)),
    "c4 cross K/V": ((24000, 2560), (BIG, 24000)),
    "c3 fc1": ((24000, 3072), (SPLIT, 85 * 256)),
    "c3 qkv": ((16 * 1504, 2304), (SPLIT, 85 * 256)),
    "c3 fc2 / out_proj": ((24000, 768), (SMALL, 0)),
    "c3 conv1": ((48000, 768), (SPLIT, 170 * 256)),
    "c2 fc1": ((12000, 2048), (SMALL, 0)),
    "c0 fc1": ((1500, 1536), (SMALL, 0)),
}


@pytest.mark.parametrize("name", list(ENCODER_PLANS))
def test_plan_on_encoder_shapes(name):
    (M, N), want = ENCODER_PLANS[name]
    assert wenc.wenc_k_gemm_plan(M, N, 256) == want


# the same projections for one half of the batch when wenc_forward runs the
# two halves on two streams side by side (measured fastest that way)
SHARED_PLANS = {
    "c4 fc1": ((12000, 5120), (BIG, 12000)),
    "c4 out_proj / fc2": ((12000, 1280), (BIG, 12000)),
    "c3 out_proj / fc2": ((12000, 768), (BIG, 12000)),
    "c3 qkv": ((8 * 1504, 2304), (BIG, 8 * 1504)),
    "c2 out_proj / fc2 / conv2": ((6000, 512), (SMALL, 0)),
    "c2 conv1": ((12000, 512), (SMALL, 0)),
    "c2 qkv": ((4 * 1504, 1536), (BIG, 4 * 1504)),
    "c2 fc1": ((6000, 2048), (BIG, 6000)),
}


@pytest.mark.parametrize("name", list(SHARED_PLANS))
def test_plan_on_two_streams(name):
    (M, N), want = SHARED_PLANS[name]
    assert wenc.wenc_k_gemm_plan(M, N, 256, streams=2) == want


@pytest.mark.parametrize("streams", [2, 3, 4])
def test_shared_plan_invariants(streams):
    for cus in (80, 256, 304):
        for N in (64, 512, 768, 1280, 2304, 5120):
            for M in range(1, 40000, 1499):
                kind, rows = wenc.wenc_k_gemm_plan(M, N, cus, streams=streams)
                tm, tn = math.ceil(M / 256), math.ceil(N / 256)
                # whole launches on one tile size, big from 0.75 tiles per unit of the CU share on
                assert kind in (SMALL, BIG), (M, N, cus, kind)
                assert (kind == SMALL) == (4 * tm * tn < 3 * (cus // streams)), (M, N, cus, streams)
                assert rows == (M if kind == BIG else 0)


def test_forced_and_unsplit_plans():
    for M, N in ((24000, 5120), (1500, 384), (1, 64), (100000, 768)):
        assert wenc.wenc_k_gemm_plan(M, N, 256, tile=1) == (BIG, M)
        assert wenc.wenc_k_gemm_plan(M, N, 256, tile=0) == (SMALL, 0)
        assert wenc.wenc_k_gemm_plan(M, N, 256, split=0)[0] != SPLIT


@pytest.mark.parametrize("cus", [80, 256, 304])
def test_plan_invariants(cus):
    for N in (64, 384, 768, 1280, 2304, 3072, 3840, 5120, 6000):
        for M in range(1, 70000, 997):
            kind, rows = wenc.wenc_k_gemm_plan(M, N, cus)
            tm, tn = math.ceil(M / 256), math.ceil(N / 256)
            # big tiles only when they fill the CUs at least 1.75 times over
            assert (kind == SMALL) == (4 * tm * tn < 7 * cus), (M, N, cus, kind)
            if kind == BIG:
                assert rows == M
            if kind == SPLIT:
                # a whole number of 256-row tile rows, within the searched window,
                # and the big launch never needs more rounds than the unsplit one
                assert rows % 256 == 0 and 0 < rows < M and rows >= 256 * (tm - 64), (M, N, cus, rows)
                assert math.ceil(rows // 256 * tn / cus) <= math.ceil(tm * tn / cus)
                # the split only pays where the unsplit last round is partly idle
                assert (tm * tn) % cus != 0


def test_plan_rejects_bad_arguments():
    for args in ((0, 64, 256, -1, 1), (64, 0, 256, -1, 1), (64, 64, 0, -1, 1), (64, 64, 256, 2, 1),
                 (64, 64, 256, -2, 1), (64, 64, 256, -1, 2), (64, 64, 256, -1, 1, 0)):
        with pytest.raises(ValueError):
            wenc.wenc_k_gemm_plan(*args)
