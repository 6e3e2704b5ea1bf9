"""MI355X-native (gfx950) Kimi Delta Attention token mixer.

The computation lives in ``libkda.so`` (C ABI declared in ``include/kda.h``,
hand-written HIP kernels); ``kda`` is its thin ctypes binding and ``synth``
draws seeded synthetic inputs.
"""
from . import synth  # noqa: F401
from .kda import (KDAError, kda_conv_prefill, kda_conv_state_bytes, kda_conv_state_update,  # noqa: F401
                  kda_decode_step, kda_gate_prologue, kda_gemm, kda_last_error,
                  kda_output_norm_gate, kda_prefill, kda_prefill_workspace_bytes, kda_state_bytes,
                  kda_version)
