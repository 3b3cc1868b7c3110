"""The five synthetic encoder workloads and their shapes.

Shapes follow the Whisper family table on "How Audio Becomes Words: Whisper's
Kernels Step By Step On A CPU" (section "Tiny, Base, Small, Large: What
Actually Changes": tiny 4 layers / 384 / 6 heads, base 6 / 512 / 8, small
12 / 768 / 12, large 32 / 1280 / 20 with 128 mel bins for v3) and the encoder
description on the whisper 0.9.0 API page (section model.nu: 3000 log-mel
frames in, 1500 positions out, fc1 widening d -> 4d per the circuit figure of
the CKE page).
"""
from __future__ import annotations

import dataclasses


@dataclasses.dataclass(frozen=True)
class EncoderConfig:
    name: str
    batch: int
    n_mels: int
    d_model: int
    n_head: int
    d_ff: int
    n_layer: int
    seed: int
    head_dim: int = 64
    n_frames: int = 3000
    n_ctx: int = 1500
    ln_eps: float = 1e-5
    final_ln: int = 1

    def flops_per_window(self) -> int:
        """Algorithmic FLOPs (2 per multiply-add) of one window.

        conv1 + conv2 + per block (QKV, out_proj, fc1, fc2 and the full
        non-causal score square plus P.V).
        """
        T_in, T, d, F = self.n_frames, self.n_ctx, self.d_model, self.d_ff
        stem = 2 * T_in * d * 3 * self.n_mels + 2 * T * d * 3 * d
        block = 2 * T * d * (3 * d) + 2 * T * d * d + 2 * T * d * F * 2 + 4 * T * T * d
        return stem + self.n_layer * block

    def with_(self, **kw) -> "EncoderConfig":
        return dataclasses.replace(self, **kw)


CONFIGS = {
    "c0": EncoderConfig("c0", batch=1, n_mels=80, d_model=384, n_head=6, d_ff=1536, n_layer=1, seed=1000),
    "c1": EncoderConfig("c1", batch=1, n_mels=80, d_model=384, n_head=6, d_ff=1536, n_layer=4, seed=1001),
    "c2": EncoderConfig("c2", batch=8, n_mels=80, d_model=512, n_head=8, d_ff=2048, n_layer=6, seed=1002),
    "c3": EncoderConfig("c3", batch=16, n_mels=80, d_model=768, n_head=12, d_ff=3072, n_layer=12, seed=1003),
    "c4": EncoderConfig("c4", batch=16, n_mels=128, d_model=1280, n_head=20, d_ff=5120, n_layer=32, seed=1004),
}

# Human-readable workload names (used in bench output).
WORKLOAD_NAMES = {
    "c0": "whisper-tiny-shaped 1-block encoder, batch 1",
    "c1": "whisper-tiny-shaped 4-block encoder, batch 1",
    "c2": "whisper-base-shaped 6-block encoder, batch 8",
    "c3": "whisper-small-shaped 12-block encoder, batch 16",
    "c4": "whisper-large-v3-shaped 32-block encoder, batch 16",
}
