"""fp64 CPU oracle of the Whisper audio-encoder forward pass.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import it.  The product path (the HIP
library and its binding) never calls it and shares no code with it.
"""
from .encoder import (  # noqa: F401
    attention,
    conv1d,
    cross_attend,
    cross_kv,
    encode,
    encoder_block,
    gelu,
    greedy_argmax,
    layer_norm,
    mha,
    softmax_rows,
)
from .frontend import hann_periodic, log_mel, mel_filters, stft_power  # noqa: F401,E402
