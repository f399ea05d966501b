"""CPU fp64 oracle for the forward pass of one Llama decoder block.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path imports, calls or links
this package: only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` use it.  It shares no code, table or
helper with the HIP kernels in ``llama_decoder_block_amd/csrc``; both sides
receive the same seeded inputs and nothing else.

Every function is the plain definition from the pages, evaluated in float64
with numpy, with no blocking, fusion or reordering beyond what the definition
states.  Pages cited (by title, section and equation; no line numbers):

  [LA] "Llama Architecture: RMSNorm, SwiGLU, RoPE, GQA, and PyTorch
       Implementation" (ailinkdeeptech.com/research/llama)
  [RN] "RMSNorm: Root Mean Square Layer Normalization" study note
       (ai-engineer-exhaustive.pages.dev/research/llama/llama-rmsnorm)
  [L3] "LLaMA-3 8B 现代 LLM 架构、计算规模与能耗" (ienjoy.github.io/llama3-8b.html)
  [MA] "LLaMA Architecture > Model Architecture"
       (mbrenndoerfer.com/writing/llama-architecture-design-training-efficiency/model-architecture)

The 8-bit KV-cache model (``oracle.fp8``: E4M3 codes with one fp32 scale per
cache row) is pinned against the format definition in
``tests/test_oracle_kvcache_pins.py``.

Parity status: every function here is pinned by a ``-m "not gpu"`` test in
``tests/test_oracle_pins.py`` (closed forms, the [L3] worked example,
invariants, library special cases and brute force).  The bf16 storage-point
variant (``bf16_storage=True``) is a reading of where the bf16 path rounds;
the pages do not fix those points, so that variant is "parity unpinned" as a
reading (its rounding helper itself is pinned against a library routine).
"""

from .reference import (  # noqa: F401
    rmsnorm,
    rope_inv_freq,
    rope,
    linear,
    silu,
    softmax_last,
    gqa_attention,
    swiglu_ffn,
    block_forward,
    block_forward_rows,
    decode_step,
)
from .bf16 import round_bf16  # noqa: F401
from . import fp8  # noqa: F401
from . import paged  # noqa: F401
from . import head  # noqa: F401
from . import bruteforce  # noqa: F401
