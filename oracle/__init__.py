"""fp64 CPU oracle of the GEMM -> residual -> RMSNorm -> GEMM(+SwiGLU) chain.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU
baseline leg of ``bench.py`` may import this package.  The library in
``gemm_epilogue_transformer_amd`` never imports it, and this package never imports the
library: the two share no code (only ``synth_inputs`` serves both).
"""
from .oracle import *  # noqa: F401,F403
