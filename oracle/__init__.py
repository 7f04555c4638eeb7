"""Plain CPU oracle for the quantized linear projection.

TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the CPU-baseline
leg of the benchmark may import this package.  The product path (the HIP
library and its Python binding) never calls it, and the two share no code.

What it computes, in the order the pages give it (FoldQuantVLA abstract:
channel scaling, then block Hadamard, then dynamic per-token quantization, then
native integer execution; Omega-QVLA "Rotazione Composita", "Implementazione a
Blocchi"; LoopQ abstract for plain RTN weights and the W4A16 weight-only form):

  fold            x / s, w * s                         (channel scaling)
  rotate          v @ blockdiag(H_b / sqrt(b))          (dense f64 matmul per block)
  quantize        per-row symmetric, round-half-even   (per-token dynamic / RTN)
  integer GEMM    int64 dot products of the codes
  E2M3 storage    int4-grid codes (-7 .. 7) as FP6 E2M3 fields packed densely
                  (OCP MX v1.0 element encoding): the same integers, a second
                  storage form of the W4A4 operands
  epilogue        acc * s_x[m] * s_w[n]  -> f32 -> f16/bf16 (RNE)
  GeGLU epilogue  gate|up rows interleaved in blocks of 32; h = gelu(g) * u
                  from the bf16-rounded dequantized g, u (the fused form of the
                  backbone MLP's gated GeLU)
  W4A16 GEMV      f64 dot products against q * s16[group]
  composite rot.  (Omega-QVLA "Rotazione SVD" / "Implementazione a Blocchi")
                  zigzag permutation of the input channels by weight norms,
                  per block R_j = U_j H_b / sqrt(b) with U_j the eigenvectors
                  of the block's weight Gram matrix
  per-step table  (Omega-QVLA "Scalatura delle Attivazioni DiT per Passo")
                  s_t[c] = max |rotated calibration activations| / qmax per
                  step; static codes v / s_t[c]; s_t folded into that step's
                  weights before their RTN

Floating point is float64 throughout, integers are int64.  Every function is
pinned by tests that do not re-use its own formula (closed forms, brute force,
independent library routines); the one function with no such pin for its
variant choice is named in ``UNPINNED``.
"""

from .qlin_ref import (  # noqa: F401
    sylvester_hadamard,
    block_rotation_matrix,
    rotate_blocks,
    calibrate_fold,
    quantize_rows,
    quantize_groups_w4a16,
    pack_int4,
    unpack_int4,
    e2m3_value,
    e2m3_code_of_int,
    pack_e2m3,
    unpack_e2m3,
    gelu,
    geglu,
    rotate_quant_act,
    quantize_weights,
    calibrate_step_scales,
    rotate_quant_act_static,
    quantize_weights_step,
    zigzag_permutation,
    composite_rotations,
    rotate_composite,
    rotate_quant_act_composite,
    quantize_weights_composite,
    int_gemm,
    dequant_epilogue,
    gemm,
    GEGLU_BLOCK,
    interleave_gate_up,
    split_gate_up,
    gemm_geglu,
    gemv_w4a16,
    round_to_bf16_bits,
    bf16_bits_to_f64,
    round_to_f16,
    round_output,
    qmax_of,
)
from .compare import (  # noqa: F401
    compare_codes,
    compare_scales,
    compare_outputs,
    CompareResult,
)

# The GeLU variant (exact erf form vs tanh form) is not fixed by the pages; the
# oracle takes the erf form.  Its values are pinned against a library GeLU, but
# the choice of variant itself is a reading, not a pin.
UNPINNED = ("gelu variant choice (erf form taken)",)
