"""CPU oracle for exact attention with a per-token int8 KV cache.

TEST INFRASTRUCTURE ONLY.  Nothing in the library imports this package; only
the tests, the smoke check and the CPU-baseline leg of the benchmark call it.
It is deliberately plain and slow: fp64 numpy, the full score matrix is
materialised (row blocks for long sequences), no tiling, no online softmax.
It shares no code, constants or helpers with the HIP path.

Modules
  attention  -- softmax(Q K^T * scale) V with causal / window / GQA masks, the
                Mul/Add epilogue, log-sum-exp, dequantization of int8 K/V, and
                the merge of results over disjoint key sets by log-sum-exp.
  quantize   -- the per-token absmax/127 int8 quantizer (numpy fp32), the
                closed-form compression ratio, the decode-time cache write and
                the rotate-half RoPE applied to K in that write.
  turboquant -- the 2-4-bit TurboQuant codec: randomized Hadamard rotation, L2
                normalisation, Lloyd-Max codebooks for Beta(d/2, d/2), packing, and
                decode attention over a cache held as such codes.

Every function is pinned by tests in tests/test_oracle_pins.py and
tests/test_oracle_turboquant.py (brute force, a library cross-check, invariants
and closed forms).  No function here is
"parity unpinned".
"""
from .attention import attention, apply_epilogue, dequantize, visible_mask, decode, merge_lse  # noqa: F401
from .quantize import quantize_per_token, compression_ratio, append_kv, rope_rotate_half  # noqa: F401
from .turboquant import (hadamard, beta_codebook, tq_encode, tq_decode, tq_pack, tq_unpack,  # noqa: F401
                         tq_compression_ratio, tq_attention_decode)
