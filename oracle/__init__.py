"""CPU oracle of the UFP4 hot path (RHT + blockwise 4-bit quantization +
block-scaled 4-bit GEMMs).

THIS PACKAGE IS TEST INFRASTRUCTURE.  Only tests/, __graft_entry__.smoke() and
the cpu_baseline leg of bench.py may import it.  The product path
(rht_bit_block_amd) never imports, calls or links anything here, and nothing
here imports the product path: the two share no code.

Parity status per function (pins live in tests/test_oracle_*.py):
  philox4x32_10     pinned to rocRAND's Philox4x32-10 engine (independent library)
  bf16_bits_to_f32  pinned to torch's bfloat16 -> float32 cast
  rht_signs/rht     pinned: H^T H = I, equality with scipy.linalg.hadamard,
                    X W^T = (X H')(W H')^T, fp32 error bound, closed forms
  scale_*           pinned: 1-ulp bound, exact power-of-two bracket (Fractions),
                    E1M2 == INT4 / 4, S(B) = S(B^T)
  round_*           pinned: rint-based and frexp-based reformulations, bin-bias
                    closed form, exact SR probabilities, SR mean error
  encode/pack       pinned: round trip of every level, canonical zero
  E4M3 (MXFP8)      pinned: level set and RNE rounding equal torch's
                    float8_e4m3fn, error bound, lossless on-grid values
  dequant/gemm_ref  pinned: brute-force triple loop, lossless on-grid case
  level_stats       pinned: exact brute force (Fractions, exhaustive nearest
                    level) on tiny inputs, SR unbiasedness, bin-asymmetry
                    values of tests/golden/bin_bias.txt
"""
from .ufp4 import *  # noqa: F401,F403
from .philox import philox4x32_10, split_seed  # noqa: F401
