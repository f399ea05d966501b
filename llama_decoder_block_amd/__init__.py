"""MI355X-native forward pass of one Llama decoder block.

The compute lives in hand-written HIP kernels for gfx950 behind the C-ABI
library ``libllama_block.so`` (declared in ``include/llama_block.h``).  The
Python layer in :mod:`llama_decoder_block_amd.binding` only marshals torch
tensors (device memory and the current stream) into that ABI.
"""

__all__ = ["binding", "synth"]
