"""wenc: the Whisper audio-encoder forward pass as hand-written HIP for gfx950.

The compute lives in ``libwenc.so`` (C ABI, declared in ``include/wenc.h``);
``whisper_audio_encoder_amd.wenc`` is the ctypes binding.  Importing this
package does not load the library: ``configs`` and ``synth`` stay usable on a
machine without a GPU.
"""
from .configs import CONFIGS, EncoderConfig  # noqa: F401

__all__ = ["CONFIGS", "EncoderConfig"]
