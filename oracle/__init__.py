"""CPU oracle for non-causal DiT attention (dense, SAGE-quantized, Skip-Softmax).

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call or
link anything in this package: only the test suite, the smoke check of the
build entry point and the CPU-baseline leg of the benchmark use it.  It shares
no code with the HIP path and imports nothing from it.

The oracle is plain numpy.  Floating point is float64 except where a step is
pinned to IEEE binary32 (so that a GPU implementation can reproduce it bit
for bit); those steps use numpy float32 arithmetic, which is correctly rounded
binary32.

Sources (page titles as published):
  * "TRTLLM Attention" (vllm-omni user guide): sections "Dense mode",
    "Skip-Softmax", "SAGE quantization".
  * "Diffusion Attention Backends" (vllm-omni user guide): sections
    "TRTLLM_ATTN Backend and Skip-Softmax", "TRTLLM_ATTN SAGE Quantization".
  * "SAGE + Skip-Softmax - API Design & Test Plan" (vllm-omni design doc):
    Part 1 section 4, the knob to kernel-argument table.
  * "VisualGen Quantized Attention (Beta)" (TensorRT-LLM docs): sections
    "Recipes" and "SageAttention in the TRTLLM backend".

Parity status per function is listed in each module's header.
"""
from .codecs import (bf16_round, e4m3_decode, e4m3_encode, f32, int8_code,
                     E4M3_MAX, INT8_MAX)
from .attention import (exact_attention, sage_quantize, sage_attention,
                        sage_skip_attention, skip_attention, skip_gate_enabled,
                        k_channel_mean)

__all__ = [
    "bf16_round", "e4m3_decode", "e4m3_encode", "f32", "int8_code", "E4M3_MAX",
    "INT8_MAX", "exact_attention", "sage_quantize", "sage_attention", "sage_skip_attention",
    "skip_attention", "skip_gate_enabled", "k_channel_mean",
]
