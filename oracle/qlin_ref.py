"""Reference definitions of every step of the quantized linear projection.

TEST INFRASTRUCTURE ONLY (see the package docstring).  NumPy, float64 and
int64, no blocking, fusion or reordering beyond what each definition states.

Sources (page title, section):
  [FQ]  FoldQuantVLA: Native Low-Bit Quantization of Vision-Language-Action
        Models via Consistent Folding -- abstract (channel scaling, block
        Hadamard transform, dynamic per-token quantization, W4A4 integer
        execution, o_proj/down_proj kept at W8A8).
  [OQ]  Omega-QVLA technical summary -- Metodologia 1, "Rotazione Composita
        SVD-Hadamard" (normalised Hadamard matrix H) and "Implementazione a
        Blocchi" (block approximation of the C_in x C_in rotation).
  [LQ]  LoopQ: Fair, Closed-Loop Evaluation of Quantized VLA Models --
        abstract (plain round-to-nearest weights; weight-only 4-bit kernels at
        batch 1; memory-bound action expert).
  [QV]  QuantVLA technical summary -- Methodology B/C (per-head and per-layer
        scalars folded into the dequantization scale, no extra runtime op).
  [OR]  Omega-QVLA technical summary -- Metodologia 1, "Rotazione SVD",
        "Rotazione Hadamard" (R = R_SVD * H) and "Implementazione a Blocchi"
        (block form, zigzag permutation of the channels by weight norms).
  [OS]  Omega-QVLA technical summary -- Metodologia 2, "Scalatura delle
        Attivazioni DiT per Passo" (a precomputed scale table per denoising
        step, per layer and per channel, derived from calibration
        trajectories and looked up at inference in place of a single static
        scale).

Readings where the pages leave a step open are stated at each function.
"""

from __future__ import annotations

import math

import numpy as np

# --------------------------------------------------------------------------
# Hadamard rotation  [OQ] Rotazione Composita / Implementazione a Blocchi,
#                    [FQ] abstract ("block Hadamard transforms")
# --------------------------------------------------------------------------


def _is_pow2(b: int) -> bool:
    return b >= 1 and (b & (b - 1)) == 0


def sylvester_hadamard(b: int) -> np.ndarray:
    """Unnormalised Hadamard matrix of order b in Sylvester (natural) order.

    H_b[i, j] = (-1) ** popcount(i & j), entries +-1, int64.  The pages only
    say "normalised Hadamard matrix"; the natural order is the reading taken.
    """
    if not _is_pow2(b):
        raise ValueError(f"Hadamard order must be a power of two, got {b}")
    i = np.arange(b, dtype=np.int64)[:, None]
    j = np.arange(b, dtype=np.int64)[None, :]
    a = i & j
    parity = np.zeros_like(a)
    while np.any(a):
        parity ^= a & 1
        a >>= 1
    return np.where(parity == 0, 1, -1).astype(np.int64)


def block_rotation_matrix(k: int, b: int) -> np.ndarray:
    """Dense k x k block-diagonal rotation blockdiag(H_b / sqrt(b)), float64.

    b in {0, 1} means no rotation (identity).  Used only at small k: the
    pages replace the dense C_in x C_in rotation by this block form.
    """
    if b in (0, 1):
        return np.eye(k, dtype=np.float64)
    if k % b:
        raise ValueError("k must be a multiple of the Hadamard block")
    hb = sylvester_hadamard(b).astype(np.float64) / math.sqrt(b)
    r = np.zeros((k, k), dtype=np.float64)
    for j in range(k // b):
        r[j * b:(j + 1) * b, j * b:(j + 1) * b] = hb
    return r


def rotate_blocks(v: np.ndarray, b: int) -> np.ndarray:
    """Row-wise rotation v @ blockdiag(H_b / sqrt(b)) over contiguous k-blocks.

    A dense float64 matmul per block of b input channels (no fast transform).
    """
    v = np.asarray(v, dtype=np.float64)
    if b in (0, 1):
        return v.copy()
    k = v.shape[-1]
    if k % b:
        raise ValueError("k must be a multiple of the Hadamard block")
    hb = sylvester_hadamard(b).astype(np.float64) / math.sqrt(b)
    out = np.empty_like(v)
    for j in range(k // b):
        out[..., j * b:(j + 1) * b] = v[..., j * b:(j + 1) * b] @ hb
    return out


# --------------------------------------------------------------------------
# Channel-scale fold  [FQ] abstract ("channel scaling")
# --------------------------------------------------------------------------


def calibrate_fold(x: np.ndarray, w: np.ndarray) -> np.ndarray:
    """Per-input-channel fold vector s[k] (float32).

    s_k = sqrt(max_m |X[m, k]| / max_n |W[n, k]|), evaluated in float64 and
    stored as float32.  W is [N][K] (nn.Linear layout), so the weight maximum
    is over column k.  If either maximum is zero, s_k = 1.  The formula is the
    SmoothQuant-style balance point (alpha = 1/2); the pages name channel
    scaling without its formula.
    """
    x = np.asarray(x, dtype=np.float64)
    w = np.asarray(w, dtype=np.float64)
    if x.shape[1] != w.shape[1]:
        raise ValueError("x and w must share the input dimension")
    ax = np.max(np.abs(x), axis=0)
    aw = np.max(np.abs(w), axis=0)
    s = np.ones(x.shape[1], dtype=np.float64)
    ok = (ax > 0) & (aw > 0)
    s[ok] = np.sqrt(ax[ok] / aw[ok])
    return s.astype(np.float32)


# --------------------------------------------------------------------------
# Symmetric round-to-nearest quantization
#   [FQ] abstract ("dynamic per-token quantization"), [LQ] abstract ("RTN")
# --------------------------------------------------------------------------


def qmax_of(bits: int) -> int:
    if bits not in (4, 8):
        raise ValueError("bits must be 4 or 8")
    return (1 << (bits - 1)) - 1


def quantize_rows(v: np.ndarray, bits: int):
    """Per-row symmetric quantization with a dynamic scale.

    amax_m = max_k |v[m, k]|; scale_m = float32(amax_m / qmax);
    r = v / float64(scale_m); q = clamp(round_half_even(r), -qmax, qmax).
    A zero row gives scale 0 and codes 0.  qmax = 7 (int4) or 127 (int8): the
    grid is symmetric, so -8 / -128 never occur.  Codes are computed with the
    stored (float32) scale.

    Returns (q int64, scale float32, r float64 -- the pre-rounding values).
    """
    qmax = qmax_of(bits)
    v = np.asarray(v, dtype=np.float64)
    amax = np.max(np.abs(v), axis=1)
    scale = (amax / qmax).astype(np.float32)
    s64 = scale.astype(np.float64)
    r = np.zeros_like(v)
    nz = s64 > 0
    r[nz] = v[nz] / s64[nz, None]
    q = np.clip(np.rint(r), -qmax, qmax).astype(np.int64)
    return q, scale, r


def quantize_groups_w4a16(w: np.ndarray, group: int):
    """Weight-only int4 with one fp16 scale per (row, group of input channels).

    For row n and group g (input channels [g*group, (g+1)*group)):
    s16 = fp16_rne(amax / 7); q = clamp(rne(w / float64(s16)), -7, 7);
    s16 == 0 gives q = 0.  Symmetric, no zero point, no fold, no rotation
    ([LQ] abstract: 4-bit weight-only kernels, plain RTN).

    Returns (q int64 [N][K], s16 float16 [N][K/group], r float64 [N][K]).
    """
    w = np.asarray(w, dtype=np.float64)
    n, k = w.shape
    if k % group:
        raise ValueError("k must be a multiple of the group size")
    ng = k // group
    wg = w.reshape(n, ng, group)
    amax = np.max(np.abs(wg), axis=2)
    s16 = (amax / 7.0).astype(np.float16)  # float64 -> float16 directly, RNE
    s64 = s16.astype(np.float64)
    r = np.zeros_like(wg)
    nz = s64 > 0
    r[nz] = wg[nz] / s64[nz][:, None]
    q = np.clip(np.rint(r), -7, 7).astype(np.int64)
    return q.reshape(n, k), s16, r.reshape(n, k)


def pack_int4(q: np.ndarray) -> np.ndarray:
    """Two int4 codes per byte along the last axis: element 2j in the low
    nibble, element 2j+1 in the high nibble, two's complement."""
    q = np.asarray(q, dtype=np.int64)
    if q.shape[-1] % 2:
        raise ValueError("int4 packing needs an even last dimension")
    if np.any(q < -8) or np.any(q > 7):
        raise ValueError("int4 code out of range")
    lo = q[..., 0::2] & 0xF
    hi = q[..., 1::2] & 0xF
    return (lo | (hi << 4)).astype(np.uint8)


def unpack_int4(p: np.ndarray) -> np.ndarray:
    """Inverse of pack_int4: sign-extended nibbles, int64."""
    p = np.asarray(p, dtype=np.uint8).astype(np.int64)
    lo = p & 0xF
    hi = (p >> 4) & 0xF
    lo = np.where(lo >= 8, lo - 16, lo)
    hi = np.where(hi >= 8, hi - 16, hi)
    out = np.empty(p.shape[:-1] + (p.shape[-1] * 2,), dtype=np.int64)
    out[..., 0::2] = lo
    out[..., 1::2] = hi
    return out


# --------------------------------------------------------------------------
# FP6 E2M3 storage of int4-grid codes
#   [FQ] abstract (W4A4 integer execution): the codes and their products are
#   those of the int4 path; only their storage differs.  The encoding is the
#   FP6 E2M3 element of the OCP Microscaling Formats (MX) v1.0 specification:
#   1 sign bit, 2 exponent bits (bias 1), 3 mantissa bits, subnormals at
#   exponent 0, no infinities or NaN.  Every integer -7 .. 7 is exact in it,
#   so a dot product of two such code vectors accumulated in fp32 (|sum| <
#   2^24 for k < 2^18) equals the integer dot product.
# --------------------------------------------------------------------------


def e2m3_value(code: int) -> float:
    """Real value of a 6-bit E2M3 code (bit 5 sign, bits 4..3 exponent field,
    bits 2..0 mantissa field): subnormal m/8 at exponent field 0, else
    2^(e - 1) * (1 + m/8)."""
    if not 0 <= code < 64:
        raise ValueError("E2M3 codes are 6 bits")
    s = -1.0 if code & 0x20 else 1.0
    e = (code >> 3) & 3
    m = code & 7
    mag = m / 8.0 if e == 0 else 2.0 ** (e - 1) * (1.0 + m / 8.0)
    return s * mag


def e2m3_code_of_int(v: int) -> int:
    """The E2M3 code whose value is the integer v (-7 .. 7), found by search
    over the 32 non-negative codes (+0 for zero)."""
    if not -7 <= v <= 7:
        raise ValueError("only -7 .. 7 are codes of the int4 grid")
    for c in range(32):
        if e2m3_value(c) == abs(v):
            return c | (0x20 if v < 0 else 0)
    raise AssertionError("unreachable: every integer 0 .. 7 is an E2M3 value")


def pack_e2m3(q: np.ndarray) -> np.ndarray:
    """Int4-grid codes (-7 .. 7) along the last axis as E2M3 codes packed
    densely, little-endian: code j occupies bits 6j .. 6j+5 of the row's bit
    string, bit b of byte i being bit 8i + b.  Last axis a multiple of 4
    (3 bytes per 4 codes)."""
    q = np.asarray(q, dtype=np.int64)
    if q.shape[-1] % 4:
        raise ValueError("E2M3 packing needs a last dimension divisible by 4")
    if np.any(q < -7) or np.any(q > 7):
        raise ValueError("E2M3 storage holds the int4 grid -7 .. 7")
    table = np.array([e2m3_code_of_int(v) for v in range(-7, 8)], dtype=np.int64)
    codes = table[q + 7]
    bits = ((codes[..., None] >> np.arange(6)) & 1).astype(np.uint8)
    bits = bits.reshape(q.shape[:-1] + (q.shape[-1] * 6,))
    return np.packbits(bits, axis=-1, bitorder="little")


def unpack_e2m3(p: np.ndarray) -> np.ndarray:
    """Inverse of pack_e2m3: the integer value of every 6-bit field, int64
    (a field whose value is not an integer raises)."""
    p = np.asarray(p, dtype=np.uint8)
    bits = np.unpackbits(p, axis=-1, bitorder="little").astype(np.int64)
    k = bits.shape[-1] // 6
    fields = bits[..., :6 * k].reshape(p.shape[:-1] + (k, 6))
    codes = np.sum(fields << np.arange(6), axis=-1)
    values = np.array([e2m3_value(c) for c in range(64)])[codes]
    if np.any(values != np.rint(values)):
        raise ValueError("field is not an integer E2M3 value")
    return np.rint(values).astype(np.int64)


# --------------------------------------------------------------------------
# GeGLU glue between the gate/up and down projections of an MLP block
# --------------------------------------------------------------------------

_erf = np.vectorize(math.erf, otypes=[np.float64])


def gelu(t: np.ndarray) -> np.ndarray:
    """Exact GeLU t * (1 + erf(t / sqrt 2)) / 2 in float64 with the host libm
    erf.  The variant (erf vs tanh form) is a reading; the pages are silent."""
    t = np.asarray(t, dtype=np.float64)
    return t * 0.5 * (1.0 + _erf(t / math.sqrt(2.0)))


def geglu(x: np.ndarray, k: int) -> np.ndarray:
    """h = gelu(gate) * up for x = [gate | up] along the last axis (width 2k)."""
    x = np.asarray(x, dtype=np.float64)
    return gelu(x[..., :k]) * x[..., k:2 * k]


# --------------------------------------------------------------------------
# Whole stages, as the library's entry points expose them
# --------------------------------------------------------------------------


def rotate_quant_act(x, fold_s, had_block: int, bits: int, preop: str = "none"):
    """Online activation path: (optional GeGLU) -> x / s -> block Hadamard ->
    per-token dynamic symmetric quantization ([FQ] abstract).

    x: [M][K] (or [M][2K] with preop='geglu'); fold_s: float32 [K] or None.
    Returns (q int64 [M][K], scale float32 [M], r float64 [M][K]).
    """
    x = np.asarray(x, dtype=np.float64)
    if preop == "geglu":
        k = x.shape[1] // 2
        v = geglu(x, k)
    elif preop == "none":
        v = x
    else:
        raise ValueError(preop)
    if fold_s is not None:
        v = v / np.asarray(fold_s, dtype=np.float32).astype(np.float64)[None, :]
    v = rotate_blocks(v, had_block)
    return quantize_rows(v, bits)


def quantize_weights(w, fold_s, had_block: int, bits: int, group: int = 0):
    """Offline weight path.

    group == 0: w * s -> block Hadamard on the rows -> per-output-channel
    symmetric RTN (the consistent counterpart of the activation path, so that
    (x/s) H (w s H)^T = x w^T).  Returns (q, scale float32 [N], r).
    group > 0 : W4A16 group quantization (bits must be 4, no fold, no
    rotation).  Returns (q, s16 float16 [N][K/group], r).
    """
    w = np.asarray(w, dtype=np.float64)
    if group:
        if bits != 4 or fold_s is not None or had_block not in (0, 1):
            raise ValueError("group quantization is int4 with no fold/rotation")
        return quantize_groups_w4a16(w, group)
    if fold_s is not None:
        w = w * np.asarray(fold_s, dtype=np.float32).astype(np.float64)[None, :]
    w = rotate_blocks(w, had_block)
    return quantize_rows(w, bits)


# --------------------------------------------------------------------------
# Per-step static activation scales  [OS] Metodologia 2
#
# Reading (the page gives no formula): the table entry of a (step, layer)
# pair is one scale per input channel of the projection, in the channel
# space where activations are quantized (after the fold and the block
# Hadamard), set RTN-style from the calibration tokens of that step:
#     s_t[c] = float32( max_m |v_t[m, c]| / qmax ).
# At inference the activation codes take it in place of the per-token
# dynamic scale:  q[m, c] = clamp(rne(v[m, c] / s_t[c]), -qmax, qmax)
# (code 0 where s_t[c] = 0).  A per-channel scale cannot be pulled out of the
# integer dot product, so it is folded into that step's weights before their
# per-output-channel RTN:  w_t = RTN_rows( rotate(w * s) * s_t ).  Then
#     s_w_t[n] * sum_c q[m, c] qw_t[n, c]  ~  sum_c (v[m, c] / s_t[c]) (w_rot[n, c] s_t[c])
# = x w^T, with the activation scale 1 in the GEMM's epilogue.  One weight
# copy per step is the cost.
# --------------------------------------------------------------------------


def _rotated(x, fold_s, had_block: int, fold_op: str) -> np.ndarray:
    v = np.asarray(x, dtype=np.float64)
    if fold_s is not None:
        f = np.asarray(fold_s, dtype=np.float32).astype(np.float64)[None, :]
        v = v / f if fold_op == "div" else v * f
    return rotate_blocks(v, had_block)


def calibrate_step_scales(x_cal, fold_s, had_block: int, bits: int) -> np.ndarray:
    """Table row s_t[c] (float32 [K]) from the calibration tokens x_cal
    [M][K] of one denoising step: the activation path up to the rotation
    (x / s, block Hadamard), then float32(max_m |v[m, c]| / qmax)."""
    v = _rotated(x_cal, fold_s, had_block, "div")
    return (np.max(np.abs(v), axis=0) / qmax_of(bits)).astype(np.float32)


def rotate_quant_act_static(x, fold_s, had_block: int, bits: int, step_scale):
    """Activation codes at one step with its static per-channel scales:
    v = rotate(x / s); r = v / float64(s_t[c]); q = clamp(rne(r), +-qmax);
    channels with s_t[c] = 0 give code 0.  Returns (q int64 [M][K], r)."""
    qmax = qmax_of(bits)
    v = _rotated(x, fold_s, had_block, "div")
    st = np.asarray(step_scale, dtype=np.float32).astype(np.float64)
    r = np.zeros_like(v)
    nz = st > 0
    r[:, nz] = v[:, nz] / st[None, nz]
    q = np.clip(np.rint(r), -qmax, qmax).astype(np.int64)
    return q, r


def quantize_weights_step(w, fold_s, had_block: int, bits: int, step_scale):
    """One step's weights: rotate(w * s) with column c multiplied by s_t[c]
    (float32 value, product in float64), then per-output-channel symmetric
    RTN.  Returns (q int64 [N][K], scale float32 [N], r)."""
    v = _rotated(w, fold_s, had_block, "mul")
    v = v * np.asarray(step_scale, dtype=np.float32).astype(np.float64)[None, :]
    return quantize_rows(v, bits)


# --------------------------------------------------------------------------
# SVD-Hadamard composite rotation with the zigzag permutation  [OR]
#
# Readings (the page is garbled on sides and conventions):
#  * The page writes y = x W with W of shape C_in x C_out, so the U of its
#    W = U S V^T is C_in x C_in and acts on the input channels.  In the
#    [n][k] (out x in) storage used here that U is the eigenvector matrix of
#    W^T W; in the block form, of the block's Gram matrix
#    G_j = W[:, B_j]^T W[:, B_j] (b x b), eigenvectors ordered by descending
#    eigenvalue, each with its largest-magnitude entry positive (the first
#    such entry on ties).
#  * The composite rotation of block j is R_j = U_j (H_b / sqrt(b)): x is
#    multiplied by U_j, then by the normalised Hadamard matrix.
#  * The zigzag permutation: input channels sorted by descending L2 norm of
#    their weight column (lower index first on ties) are dealt to the k / b
#    blocks in snake order -- rank r, round t = r // nb, i = r % nb goes to
#    block i on even rounds and nb - 1 - i on odd rounds, at slot t.
#  * The permutation is applied first (a gather of input channels), on both
#    sides: x[:, perm] R and W[:, perm] R, so x W^T is unchanged.
# --------------------------------------------------------------------------


def zigzag_permutation(w, had_block: int) -> np.ndarray:
    """perm[c'] = the input channel placed at position c' (int64 [K])."""
    w = np.asarray(w, dtype=np.float64)
    k = w.shape[1]
    b = had_block
    if b < 1 or k % b:
        raise ValueError("k must be a multiple of the block")
    nb = k // b
    norms = np.sqrt(np.sum(w * w, axis=0))
    order = np.lexsort((np.arange(k), -norms))   # descending norm, then index
    perm = np.empty(k, dtype=np.int64)
    for r, c in enumerate(order):
        t, i = divmod(r, nb)
        j = i if t % 2 == 0 else nb - 1 - i
        perm[j * b + t] = c
    return perm


def _sign_fixed(u: np.ndarray) -> np.ndarray:
    u = u.copy()
    for c in range(u.shape[1]):
        i = int(np.argmax(np.abs(u[:, c])))
        if u[i, c] < 0:
            u[:, c] = -u[:, c]
    return u


def composite_rotations(w, perm, had_block: int) -> np.ndarray:
    """R [k/b][b][b] float64: R_j = U_j (H_b / sqrt(b)) from the Gram matrix
    of block j of the permuted weight columns."""
    w = np.asarray(w, dtype=np.float64)[:, np.asarray(perm)]
    b = had_block
    nb = w.shape[1] // b
    hb = sylvester_hadamard(b).astype(np.float64) / math.sqrt(b)
    out = np.empty((nb, b, b), dtype=np.float64)
    for j in range(nb):
        blk = w[:, j * b:(j + 1) * b]
        evals, evecs = np.linalg.eigh(blk.T @ blk)
        order = np.argsort(-evals, kind="stable")
        out[j] = _sign_fixed(evecs[:, order]) @ hb
    return out


def rotate_composite(v, perm, rot) -> np.ndarray:
    """v[:, perm], then block j of the permuted channels times rot[j]
    (rot as given, float32 values taken exactly)."""
    v = np.asarray(v, dtype=np.float64)[:, np.asarray(perm)]
    rot = np.asarray(rot).astype(np.float64)
    nb, b, _ = rot.shape
    out = np.empty_like(v)
    for j in range(nb):
        out[:, j * b:(j + 1) * b] = v[:, j * b:(j + 1) * b] @ rot[j]
    return out


def rotate_quant_act_composite(x, fold_s, perm, rot, bits: int):
    """x / s (optional fold, on the original channels) -> gather -> per-block
    composite rotation -> per-token dynamic quantization."""
    v = np.asarray(x, dtype=np.float64)
    if fold_s is not None:
        v = v / np.asarray(fold_s, dtype=np.float32).astype(np.float64)[None, :]
    return quantize_rows(rotate_composite(v, perm, rot), bits)


def quantize_weights_composite(w, fold_s, perm, rot, bits: int):
    """w * s -> gather -> per-block composite rotation -> per-row RTN."""
    v = np.asarray(w, dtype=np.float64)
    if fold_s is not None:
        v = v * np.asarray(fold_s, dtype=np.float32).astype(np.float64)[None, :]
    return quantize_rows(rotate_composite(v, perm, rot), bits)


def int_gemm(qx: np.ndarray, qw: np.ndarray) -> np.ndarray:
    """acc[m, n] = sum_k qx[m, k] * qw[n, k] in int64 ([FQ]: native integer
    execution).  Checks that the result fits the int32 accumulator."""
    qx = np.asarray(qx, dtype=np.int64)
    qw = np.asarray(qw, dtype=np.int64)
    acc = qx @ qw.T
    if acc.size and np.max(np.abs(acc)) >= 2 ** 31:
        raise OverflowError("accumulator exceeds int32")
    return acc


def dequant_epilogue(acc, x_scale, w_scale) -> np.ndarray:
    """y32 = float32(acc * s_x[m] * s_w[n]) with the product in float64.

    Per-head / per-layer calibration scalars ([QV] Methodology B, C) are
    pre-multiplied into s_w and need no separate step.
    """
    acc = np.asarray(acc, dtype=np.int64).astype(np.float64)
    sx = np.asarray(x_scale, dtype=np.float32).astype(np.float64)
    sw = np.asarray(w_scale, dtype=np.float32).astype(np.float64)
    return (acc * sx[:, None] * sw[None, :]).astype(np.float32)


def round_to_bf16_bits(y32: np.ndarray) -> np.ndarray:
    """float32 -> bfloat16 with round-half-to-even, as uint16 bit patterns.

    NumPy has no bfloat16: add 0x7FFF plus the lowest kept bit to the float32
    pattern and drop the low 16 bits.  Finite inputs only.
    """
    u = np.ascontiguousarray(y32, dtype=np.float32).view(np.uint32).astype(np.uint64)
    lsb = (u >> 16) & 1
    return (((u + 0x7FFF + lsb) >> 16) & 0xFFFF).astype(np.uint16)


def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    """Exact widening of bfloat16 bit patterns to float64."""
    u = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    return u.view(np.float32).astype(np.float64)


def round_to_f16(y32: np.ndarray) -> np.ndarray:
    """float32 -> float16 with round-half-to-even (NumPy's cast)."""
    return np.asarray(y32, dtype=np.float32).astype(np.float16)


def round_output(y32: np.ndarray, dtype: str) -> np.ndarray:
    """The reference output: the float32 result rounded to the output dtype,
    returned widened to float64 for comparison."""
    if dtype == "f16":
        return round_to_f16(y32).astype(np.float64)
    if dtype == "bf16":
        return bf16_bits_to_f64(round_to_bf16_bits(y32))
    if dtype == "f32":
        return np.asarray(y32, dtype=np.float32).astype(np.float64)
    raise ValueError(dtype)


def gemm(qx, x_scale, qw, w_scale, out_dtype: str):
    """Integer GEMM followed by the dequantizing epilogue.

    Returns (acc int64, y32 float32, y_ref float64 rounded to out_dtype).
    """
    acc = int_gemm(qx, qw)
    y32 = dequant_epilogue(acc, x_scale, w_scale)
    return acc, y32, round_output(y32, out_dtype)


# --------------------------------------------------------------------------
# Fused gate|up projection with the GeGLU epilogue
# --------------------------------------------------------------------------

GEGLU_BLOCK = 32   # gate and up rows alternate in blocks of this many rows


def interleave_gate_up(gate: np.ndarray, up: np.ndarray, block: int = GEGLU_BLOCK) -> np.ndarray:
    """Rows of the fused gate|up weight (or its per-row scales): block j of
    gate rows (rows block*j .. block*j + block - 1) followed by the same block
    of up rows.  gate and up have f rows each, f a multiple of block."""
    gate = np.asarray(gate)
    up = np.asarray(up)
    f = gate.shape[0]
    if up.shape[0] != f or f % block:
        raise ValueError("gate and up need the same row count, a multiple of the block")
    tail = gate.shape[1:]
    g = gate.reshape((f // block, block) + tail)
    u = up.reshape((f // block, block) + tail)
    return np.concatenate([g, u], axis=1).reshape((2 * f,) + tail)


def split_gate_up(y: np.ndarray, block: int = GEGLU_BLOCK):
    """Inverse of interleave_gate_up along the last axis (output columns)."""
    y = np.asarray(y)
    n2 = y.shape[-1]
    v = y.reshape(y.shape[:-1] + (n2 // (2 * block), 2, block))
    return v[..., 0, :].reshape(y.shape[:-1] + (n2 // 2,)), v[..., 1, :].reshape(y.shape[:-1] + (n2 // 2,))


def gemm_geglu(qx, x_scale, qw, w_scale, out_dtype: str, block: int = GEGLU_BLOCK):
    """Gate|up projection with GeGLU in the epilogue (the fused form of the
    backbone MLP's gated GeLU).  qw / w_scale hold the gate and up rows
    interleaved (interleave_gate_up).  Reading: the dequantized gate and up
    values are rounded to bfloat16 first, as the unfused chain stores them,
    then h = gelu(g) * u in float64, float32, then out_dtype (RNE).

    Returns (acc int64 [M][2F], h32 float32 [M][F], h_ref float64).
    """
    acc = int_gemm(qx, qw)
    y32 = dequant_epilogue(acc, x_scale, w_scale)
    g32, u32 = split_gate_up(y32, block)
    g = bf16_bits_to_f64(round_to_bf16_bits(g32))
    u = bf16_bits_to_f64(round_to_bf16_bits(u32))
    h32 = (gelu(g) * u).astype(np.float32)
    return acc, h32, round_output(h32, out_dtype)


def gemv_w4a16(x, qw, s16, group: int):
    """Weight-only product y[m, n] = sum_k x[m, k] * q[n, k] * s16[n, k//group]
    in float64, then float32, then float16 (RNE).  [LQ] abstract: batch-1
    weight-only kernels of the memory-bound action expert.

    Returns (y32 float32, y_ref float64 holding the float16 values).
    """
    x = np.asarray(x, dtype=np.float64)
    q = np.asarray(qw, dtype=np.int64).astype(np.float64)
    s = np.asarray(s16, dtype=np.float16).astype(np.float64)
    n, k = q.shape
    wdq = q * np.repeat(s, group, axis=1)[:, :k]
    y32 = (x @ wdq.T).astype(np.float32)
    return y32, round_output(y32, "f16")
