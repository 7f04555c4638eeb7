"""Stage-wise parity of the HIP path against the CPU oracle (GPU only).

Each GPU stage is compared with the oracle run on that stage's GPU inputs:
codes equal up to boundary flips, scales to 1e-6, integer accumulators
bit-exact, fp16/bf16/f32 outputs within 1e-2 max / 1e-3 RMS of the oracle's
fp32 result rounded to the output dtype.

Method: FoldQuantVLA abstract (fold, block Hadamard, per-token dynamic
quantization, W4A4/W8A8 integer GEMM); LoopQ abstract (RTN, W4A16 GEMV).
"""

import sys

import numpy as np
import pytest
import torch

import bit_ptq_vla_amd as q
import oracle
from bit_ptq_vla_amd import synth

pytestmark = pytest.mark.gpu
DEV = "cuda"
SEED = 1234

DT = {"f16": torch.float16, "bf16": torch.bfloat16, "f32": torch.float32}


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def codes_np(t: torch.Tensor, bits: int) -> np.ndarray:
    a = t.cpu().numpy()
    if bits == 6:
        return oracle.unpack_e2m3(a).astype(np.int64)
    return oracle.unpack_int4(a) if bits == 4 else a.astype(np.int64)


def f64(t: torch.Tensor) -> np.ndarray:
    return t.detach().cpu().to(torch.float64).numpy()


def assert_ok(res, what):
    assert res.ok, f"{what}: {res.detail}"


# ---------------------------------------------------------------- activation stage

ACT_CASES = [
    # m, k, b, bits, dtype, fold
    (16, 512, 64, 4, "f16", True),      # single W4A4 linear
    (37, 2048, 128, 4, "bf16", True),   # backbone hidden, ragged m
    (5, 16384, 128, 8, "bf16", True),   # down-projection input width
    (50, 1024, 64, 4, "f16", True),     # action-expert width
    (3, 11008, 0, 8, "f16", False),     # no rotation, k not a power of two
    (7, 64, 8, 4, "f32", True),
    (33, 4096, 256, 8, "f16", True),
    (2, 128, 2, 4, "bf16", False),
    (300, 256, 128, 4, "bf16", True),   # several rows per block
    (3, 14336, 128, 8, "bf16", True),   # 512 lanes, chunk count 4 (not a power-of-two row)
    (4, 32768, 128, 4, "bf16", True),   # longest rows: 1024 lanes, 4 chunks
    # many rows (m * k >= 2^21): k / 32 lanes per row, four chunks each
    (1030, 2048, 128, 4, "bf16", True),   # one wave per row, ragged row groups
    (2049, 1024, 256, 8, "bf16", True),   # 32 lanes = one Hadamard block of 256
    (513, 4096, 64, 6, "f16", True),      # E2M3 storage, 128 lanes
    (1024, 2048, 128, 8, "f32", False),
]


@pytest.mark.parametrize("m,k,b,bits,dtype,fold", ACT_CASES)
def test_rotate_quant_act_parity(m, k, b, bits, dtype, fold):
    say(f"act m={m} k={k} b={b} bits={bits} {dtype} fold={fold}")
    x = synth.normal_tensor(SEED, f"act/{m}/{k}/{b}", (m, k), dtype=dtype, outliers=max(1, k // 100),
                            outlier_scale=25.0)
    x[m // 2] = 0  # one all-zero token
    s = None
    if fold:
        s = synth.random_scales(SEED, f"fold/{k}", k) * 100.0
    xd = x.to(DEV)
    inv_s = (1.0 / s).to(DEV) if fold else None
    xq, xs = q.qlin_rotate_quant_act(xd, fold_inv_s=inv_s, had_block=b, bits=bits)
    torch.cuda.synchronize()
    # E2M3 storage (bits 6) holds the codes of the int4 grid
    q_ref, s_ref, r_ref = oracle.rotate_quant_act(synth.to_f64(x), s.numpy() if fold else None, b,
                                                  4 if bits == 6 else bits)
    assert_ok(oracle.compare_scales(xs.cpu().numpy(), s_ref), "scales")
    assert_ok(oracle.compare_codes(codes_np(xq, bits), q_ref, r_ref), "codes")
    assert xs[m // 2].item() == 0.0 and np.all(codes_np(xq, bits)[m // 2] == 0)


@pytest.mark.parametrize("m,k,dtype", [(9, 2048, "bf16"), (4, 16384, "bf16"), (6, 512, "f16"),
                                       (1100, 2048, "bf16"), (1030, 1024, "f16")])
def test_rotate_quant_act_geglu_parity(m, k, dtype):
    say(f"act geglu m={m} k={k} {dtype}")
    gu = synth.normal_tensor(SEED, f"geglu/{m}/{k}", (m, 2 * k), dtype=dtype)
    s = synth.random_scales(SEED, f"gfold/{k}", k) * 100.0
    xq, xs = q.qlin_rotate_quant_act(gu.to(DEV), k=k, fold_inv_s=(1.0 / s).to(DEV), had_block=128,
                                     bits=8, pre=q.QLIN_PRE_GEGLU)
    torch.cuda.synchronize()
    q_ref, s_ref, r_ref = oracle.rotate_quant_act(synth.to_f64(gu), s.numpy(), 128, 8, preop="geglu")
    assert_ok(oracle.compare_scales(xs.cpu().numpy(), s_ref), "scales")
    assert_ok(oracle.compare_codes(codes_np(xq, 8), q_ref, r_ref), "codes")


# ---------------------------------------------------------------- per-step static table

TABLE_CASES = [
    # m (calibration and evaluation rows), k, b, bits, dtype, fold
    (50, 1024, 64, 4, "f16", True),      # action-expert width
    (50, 4096, 64, 4, "f16", True),      # action-expert down input (1024 lanes)
    (200, 2048, 128, 8, "bf16", True),   # several row groups per block
    (7, 512, 0, 8, "f32", False),        # no rotation
    (33, 256, 256, 4, "bf16", True),     # Hadamard block = k
    (3, 32768, 128, 4, "bf16", True),    # longest rows: 1024 lanes, 4 chunks
]


def _zero_block(k, b):
    return b > 1 and k >= 2 * b


def _table_inputs(m, k, b, dtype, fold, tag):
    xc = synth.normal_tensor(SEED, f"tcal/{tag}/{m}/{k}", (m, k), dtype=dtype, outliers=max(1, k // 100),
                             outlier_scale=10.0)
    xe = synth.normal_tensor(SEED, f"teval/{tag}/{m}/{k}", (m, k), dtype=dtype, outliers=max(1, k // 100),
                             outlier_scale=10.0)
    if _zero_block(k, b):
        xc[:, :b] = 0          # a whole zero Hadamard block: table entries 0
        xe[:, :b] = 1          # ... whose codes must still be 0
    s = synth.random_scales(SEED, f"tfold/{k}", k) * 100.0 if fold else None
    return xc, xe, s


def _assert_table(got, ref, xc, s, b, bits):
    """A calibrated table against the oracle's.  The kernel rotates in fp32:
    a butterfly stage adds at most one rounding (u = 2^-24) relative to the
    magnitudes it adds, so a rotated value is off by at most
    (log2 b + 2) u sum_block |x / s| / sqrt(b) (+2 for the fold's fp32
    reciprocal).  A channel's maximum over a few tokens can sit on a
    cancelling sum, where this exceeds the 1e-6 of a row's maximum."""
    m, k = xc.shape
    xf = synth.to_f64(xc) / (s.numpy().astype(np.float64)[None, :] if s is not None else 1.0)
    bb = max(b, 1)
    blk = np.abs(xf).reshape(m, k // bb, bb).sum(axis=2) / np.sqrt(bb)        # [m][blocks]
    amag = np.repeat(blk.max(axis=0), bb) / (7 if bits == 4 else 127)
    bound = (np.log2(bb) + 2) * 2.0 ** -24 * amag + 2.0 ** -23 * np.abs(ref)
    assert np.all(np.abs(got - ref) <= bound), float(np.max(np.abs(got - ref) / np.maximum(bound, 1e-300)))
    assert_ok(oracle.compare_scales(got, ref, rtol=1e-5), "table")


@pytest.mark.parametrize("m,k,b,bits,dtype,fold", TABLE_CASES)
def test_calibrate_step_scales_parity(m, k, b, bits, dtype, fold):
    say(f"step table calibrate m={m} k={k} b={b} bits={bits} {dtype}")
    xc, _, s = _table_inputs(m, k, b, dtype, fold, "c")
    inv = (1.0 / s).to(DEV) if fold else None
    table = q.qlin_calibrate_step_scales(xc.to(DEV), fold_inv_s=inv, had_block=b, bits=bits)
    torch.cuda.synchronize()
    ref = oracle.calibrate_step_scales(synth.to_f64(xc), s.numpy() if fold else None, b, bits)
    got = table.cpu().numpy().astype(np.float64)
    _assert_table(got, ref, xc, s, b, bits)
    if _zero_block(k, b):
        assert np.all(got[:b] == 0)


@pytest.mark.parametrize("m,k,b,bits,dtype,fold", TABLE_CASES)
def test_rotate_quant_act_static_parity(m, k, b, bits, dtype, fold):
    """Evaluation tokens quantized with a table from other (calibration)
    tokens: codes against the oracle's, clipping included; the same table
    (the oracle's) enters both sides."""
    say(f"step table static codes m={m} k={k} b={b} bits={bits} {dtype}")
    xc, xe, s = _table_inputs(m, k, b, dtype, fold, "s")
    sg = s.numpy() if fold else None
    table = oracle.calibrate_step_scales(synth.to_f64(xc), sg, b, bits) * np.float32(0.8)   # some clipping
    inv = (1.0 / s).to(DEV) if fold else None
    xq = q.qlin_rotate_quant_act_static(xe.to(DEV), torch.from_numpy(table).to(DEV), fold_inv_s=inv,
                                        had_block=b, bits=bits)
    torch.cuda.synchronize()
    q_ref, r_ref = oracle.rotate_quant_act_static(synth.to_f64(xe), sg, b, bits, table)
    got = codes_np(xq, bits)
    assert_ok(oracle.compare_codes(got, q_ref, r_ref), "codes")
    qmax = 7 if bits == 4 else 127
    assert np.count_nonzero(np.abs(got) == qmax) > 0          # the clipped range is reached
    if _zero_block(k, b):
        assert np.all(got[:, :b] == 0)


@pytest.mark.parametrize("n,k,b,bits,dtype,fold", [(96, 1024, 64, 4, "f16", True), (40, 2048, 128, 8, "bf16", True),
                                                    (17, 512, 0, 4, "f32", False), (8, 16384, 128, 8, "bf16", True)])
def test_quantize_weights_step_parity(n, k, b, bits, dtype, fold):
    say(f"step table weights n={n} k={k} b={b} bits={bits} {dtype}")
    w = synth.normal_tensor(SEED, f"tw/{n}/{k}", (n, k), std=0.02, dtype=dtype)
    table = synth.random_scales(SEED, f"ttab/{k}", k)
    table[: max(b, 8)] = 0                                       # zero entries zero those columns
    s = synth.random_scales(SEED, f"twfold/{k}", k) * 10.0 if fold else None
    wq, ws = q.qlin_quantize_weights_step(w.to(DEV), table.to(DEV), fold_s=s.to(DEV) if fold else None,
                                          had_block=b, bits=bits)
    torch.cuda.synchronize()
    q_ref, s_ref, r_ref = oracle.quantize_weights_step(synth.to_f64(w), s.numpy() if fold else None, b, bits,
                                                       table.numpy())
    assert_ok(oracle.compare_codes(codes_np(wq, bits), q_ref, r_ref), "codes")
    assert_ok(oracle.compare_scales(ws.cpu().numpy(), s_ref), "scales")


# ---------------------------------------------------------------- composite rotation

COMPOSITE_CASES = [
    # m, k, b, bits, dtype, fold
    (50, 1024, 64, 4, "f16", True),      # action-expert width
    (37, 2048, 128, 4, "bf16", True),    # backbone hidden
    (5, 16384, 128, 8, "bf16", True),    # down input width: one row per block
    (300, 512, 32, 8, "f32", False),     # several row groups per block
    (9, 256, 16, 4, "f16", False),
    # four rows per thread (grids of >= 256 blocks), ragged last row tile
    (816, 2048, 128, 4, "bf16", True),   # the backbone MLP input
    (700, 2048, 64, 4, "f16", True),
    (600, 4096, 32, 8, "bf16", False),
    (1100, 1024, 16, 4, "f32", True),
]


def _composite_weights(n, k, dtype, tag):
    w = synth.normal_tensor(SEED, f"cw/{tag}/{n}/{k}", (n, k), std=0.02, dtype=dtype)
    # channel norms spread over two decades, so the zigzag deal matters
    spread = torch.from_numpy((10.0 ** np.random.default_rng(k).uniform(-1, 1, size=k)).astype(np.float32))
    return (w.float() * spread[None, :]).to(w.dtype)


U32 = 2.0 ** -24


def _composite_bounded(v_gpu, q_gpu, s_gpu, vin, perm, rot, bits, what):
    """The composite path's results against the oracle within the stated
    error bound: every rotated value within
        E = (gamma_b + 3u) sum_i |v_i| |R_ij| + u |v_ref|,   u = 2^-24,
    of the exact product of the oracle's fold (gamma_b: b fp32 roundings of
    the matrix-core sum; 3u: the fp32 fold product and 1/s; u |v|: the final
    fp32 rounding of the b = 16 path's fp64 sum); scales within the row's
    largest E over qmax (+2 ulp); a code differing by at most one, and only
    where the oracle's quotient lies within the propagated bound of a
    rounding boundary (half-integer)."""
    b = rot.shape[-1]
    qmax = oracle.qmax_of(bits)
    gamma = b * U32 / (1 - b * U32)
    v_ref = oracle.rotate_composite(vin, perm, rot)
    mag = oracle.rotate_composite(np.abs(vin), perm, np.abs(rot.astype(np.float64)))
    bound = (gamma + 3 * U32) * mag + U32 * np.abs(v_ref) + 1e-30
    dv = np.abs(v_gpu.astype(np.float64) - v_ref)
    worst = np.max(dv / bound)
    assert worst <= 1.0, f"{what}: rotated value off by {worst:.3f} x the bound"
    q_ref, s_ref, r_ref = oracle.quantize_rows(v_ref, bits)
    row_e = np.max(bound, axis=1)
    s64 = s_gpu.astype(np.float64)
    assert np.all(np.abs(s64 - s_ref) <= row_e / qmax + 2 * U32 * s_ref + 1e-45), f"{what}: scale beyond the bound"
    d = q_gpu.astype(np.int64) - q_ref
    assert np.max(np.abs(d)) <= 1, f"{what}: a code differs by more than one"
    zero = s_ref == 0                      # all-zero rows: scale 0 and codes 0 on both sides
    assert np.all(s64[zero] == 0) and not np.any(q_gpu[zero]), f"{what}: zero row not quantized to zeros"
    if np.any(d):
        sref = np.where(zero, 1.0, s_ref)[:, None]
        tol = bound / sref + np.abs(r_ref) * (row_e[:, None] / (sref * qmax) + 4 * U32)
        tol = np.maximum(tol, 1e-5 * np.maximum(1.0, np.abs(r_ref)))   # the quantizer's own tie window
        dist = np.abs(np.abs(r_ref - np.floor(r_ref)) - 0.5)
        far = (d != 0) & (dist > tol)
        assert not np.any(far), f"{what}: {int(np.count_nonzero(far))} code flips away from a rounding boundary"
    return int(np.count_nonzero(d))


@pytest.mark.parametrize("m,k,b,bits,dtype,fold", COMPOSITE_CASES)
def test_composite_quant_parity(m, k, b, bits, dtype, fold):
    """Activations and weights with the oracle's permutation and rotations
    (fp32) as inputs: rotated rows, scales and codes against the oracle within
    the stated error bound of the rotation's arithmetic."""
    say(f"composite quant m={m} k={k} b={b} bits={bits} {dtype}")
    x = synth.normal_tensor(SEED, f"cx/{m}/{k}", (m, k), dtype=dtype, outliers=max(1, k // 100), outlier_scale=25.0)
    x[m // 2] = 0
    w = _composite_weights(64, k, dtype, "q")
    s = synth.random_scales(SEED, f"cfold/{k}", k) * 100.0 if fold else None
    sg = s.numpy() if fold else None
    wf = synth.to_f64(w) * (sg.astype(np.float64)[None, :] if fold else 1.0)
    perm = oracle.zigzag_permutation(wf, b)
    rot = oracle.composite_rotations(wf, perm, b).astype(np.float32)
    pd, rd = torch.from_numpy(perm.astype(np.int32)).to(DEV), torch.from_numpy(rot).to(DEV)
    inv = (1.0 / s).to(DEV) if fold else None
    xwork = torch.empty(m * k, dtype=torch.float32, device=DEV)
    wwork = torch.empty(64 * k, dtype=torch.float32, device=DEV)
    xq, xs = q.qlin_rotate_quant_act_composite(x.to(DEV), pd, rd, fold_inv_s=inv, bits=bits, work=xwork)
    wq, ws = q.qlin_quantize_weights_composite(w.to(DEV), pd, rd, fold_s=s.to(DEV) if fold else None, bits=bits,
                                               work=wwork)
    torch.cuda.synchronize()
    xin = synth.to_f64(x) / (sg.astype(np.float64)[None, :] if fold else 1.0)
    _composite_bounded(xwork.view(m, k).cpu().numpy(), codes_np(xq, bits), xs.cpu().numpy(), xin, perm, rot, bits,
                       "activations")
    assert xs[m // 2].item() == 0.0
    _composite_bounded(wwork.view(64, k).cpu().numpy(), codes_np(wq, bits), ws.cpu().numpy(), wf, perm, rot, bits,
                       "weights")


@pytest.mark.parametrize("n,k,b,dtype,fold", [(96, 1024, 64, "f16", True), (256, 2048, 128, "bf16", True),
                                               (40, 512, 16, "f32", False), (64, 256, 32, "f16", False)])
def test_calibrate_composite_parity(n, k, b, dtype, fold):
    """The zigzag permutation equals the oracle's; each rotation is
    orthogonal, turns its block's weight columns into orthogonal columns
    with the oracle's eigenvalues as energies, and matches the oracle's
    rotation column for column where the eigenvalue is well separated."""
    say(f"composite calibrate n={n} k={k} b={b} {dtype}")
    w = _composite_weights(n, k, dtype, "c")
    s = synth.random_scales(SEED, f"ccfold/{k}", k) * 100.0 if fold else None
    perm, rot = q.qlin_calibrate_composite(w.to(DEV), b, fold_s=s.to(DEV) if fold else None)
    torch.cuda.synchronize()
    wf = synth.to_f64(w) * (s.numpy().astype(np.float64)[None, :] if fold else 1.0)
    perm_ref = oracle.zigzag_permutation(wf, b)
    assert np.array_equal(perm.cpu().numpy().astype(np.int64), perm_ref)
    rot_ref = oracle.composite_rotations(wf, perm_ref, b)
    h = oracle.sylvester_hadamard(b) / np.sqrt(b)
    got = rot.cpu().numpy().astype(np.float64)
    tol = 1e-5 if b <= 64 else 1e-4          # fp64 Jacobi up to b = 64, fp32 at 128
    wp = wf[:, perm_ref]
    for j in range(k // b):
        r = got[j]
        assert np.abs(r @ r.T - np.eye(b)).max() < tol, f"block {j} not orthogonal"
        u = r @ h.T
        blk = wp[:, j * b:(j + 1) * b]
        z = blk @ u
        ev = np.linalg.eigvalsh(blk.T @ blk)[::-1]
        energies = (z * z).sum(axis=0)
        assert np.abs(energies - ev).max() <= tol * ev[0] * 10, f"block {j} energies"
        u_ref = rot_ref[j] @ h.T
        gap = np.minimum(np.abs(np.diff(ev, prepend=np.inf)), np.abs(np.diff(ev, append=-np.inf)))
        sep = gap > 1e-2 * ev[0]
        assert np.abs(u[:, sep] - u_ref[:, sep]).max() < 1e-2, f"block {j} eigenvectors"


def test_composite_linear_end_to_end():
    """Calibrate on the GPU, quantize both sides with the GPU's permutation
    and rotations, W4A4 GEMM: each stage against the oracle on the same
    inputs, and the projection against x w^T."""
    say("composite linear 50x1024x1024")
    wl = synth.CFG3
    pr = wl.projs[0]
    w = synth.weight(wl, pr)
    x = synth.activation(wl, pr, 50, tag="/t0", std=synth.cfg3_sigma(0))
    perm, rot = q.qlin_calibrate_composite(w.to(DEV), 64)
    xwork = torch.empty(50 * pr.k, dtype=torch.float32, device=DEV)
    wwork = torch.empty(pr.n * pr.k, dtype=torch.float32, device=DEV)
    xq, xs = q.qlin_rotate_quant_act_composite(x.to(DEV), perm, rot, bits=4, work=xwork)
    wq, ws = q.qlin_quantize_weights_composite(w.to(DEV), perm, rot, bits=4, work=wwork)
    y = q.qlin_gemm_w4a4(xq, xs, wq, ws, pr.k, y_dtype=torch.float16)
    torch.cuda.synchronize()
    pg, rg = perm.cpu().numpy().astype(np.int64), rot.cpu().numpy()
    _composite_bounded(xwork.view(50, pr.k).cpu().numpy(), codes_np(xq, 4), xs.cpu().numpy(), synth.to_f64(x), pg,
                       rg, 4, "activations")
    rws = _sample_rows(pr.n, 32)
    _composite_bounded(wwork.view(pr.n, pr.k).cpu().numpy()[rws], codes_np(wq, 4)[rws], ws.cpu().numpy()[rws],
                       synth.to_f64(w[rws]), pg, rg, 4, "weights")
    _, _, y_ref = oracle.gemm(codes_np(xq, 4), xs.cpu().numpy(), codes_np(wq, 4), ws.cpu().numpy(), "f16")
    assert_ok(oracle.compare_outputs(f64(y), y_ref), "output")
    y_true = synth.to_f64(x) @ synth.to_f64(w).T
    assert np.linalg.norm(f64(y) - y_true) / np.linalg.norm(y_true) < 0.3


def test_rotate_quant_act_strided_rows():
    say("act strided ldx")
    x = synth.normal_tensor(SEED, "strided", (12, 1536), dtype="f16")
    view = x.to(DEV)[:, 256:1280]  # k = 1024 inside rows of 1536
    xq, xs = q.qlin_rotate_quant_act(view, had_block=64, bits=4)
    torch.cuda.synchronize()
    q_ref, s_ref, r_ref = oracle.rotate_quant_act(synth.to_f64(x)[:, 256:1280], None, 64, 4)
    assert_ok(oracle.compare_scales(xs.cpu().numpy(), s_ref), "scales")
    assert_ok(oracle.compare_codes(codes_np(xq, 4), q_ref, r_ref), "codes")


@pytest.mark.parametrize("k,b,bits", [(1024, 64, 4), (4096, 128, 4), (2048, 64, 8)])
def test_rotate_quant_act_bf16_path_rounds_like_f32(k, b, bits):
    """bf16 rows take their own kernel at b = 64 / 128; fed the same values
    as f32 (exact), the general kernel must give the same codes and scales
    bit for bit: each fold product is rounded to fp32 before the first
    butterfly in both (a product fused into that add would differ by an ulp
    in some rows)."""
    say(f"act bf16 vs f32 k={k} b={b} bits={bits}")
    x = synth.normal_tensor(SEED, f"bf16f32/{k}", (37, k), dtype="bf16", outliers=k // 100, outlier_scale=20.0)
    inv = (1.0 / (synth.random_scales(SEED, f"bf16f32/fold/{k}", k) * 100.0)).to(DEV)
    xq1, xs1 = q.qlin_rotate_quant_act(x.to(DEV), fold_inv_s=inv, had_block=b, bits=bits)
    xq2, xs2 = q.qlin_rotate_quant_act(x.float().to(DEV), fold_inv_s=inv, had_block=b, bits=bits)
    torch.cuda.synchronize()
    assert torch.equal(xs1.view(torch.int32), xs2.view(torch.int32))
    assert torch.equal(xq1, xq2)


# ---------------------------------------------------------------- weight stage

WQ_CASES = [
    (512, 512, 64, 4, "f16", True),
    (300, 2048, 128, 4, "f16", True),
    (64, 16384, 128, 8, "f16", True),
    (257, 4096, 0, 8, "bf16", False),
    (40, 1024, 64, 8, "f32", True),
]


@pytest.mark.parametrize("n,k,b,bits,dtype,fold", WQ_CASES)
def test_quantize_weights_parity(n, k, b, bits, dtype, fold):
    say(f"wq n={n} k={k} b={b} bits={bits} {dtype}")
    w = synth.normal_tensor(SEED, f"w/{n}/{k}", (n, k), std=0.02, dtype=dtype)
    w[3] = 0
    s = synth.random_scales(SEED, f"wfold/{k}", k) * 100.0 if fold else None
    wq, ws = q.qlin_quantize_weights(w.to(DEV), fold_s=s.to(DEV) if fold else None, had_block=b, bits=bits)
    torch.cuda.synchronize()
    q_ref, s_ref, r_ref = oracle.quantize_weights(synth.to_f64(w), s.numpy() if fold else None, b, bits)
    assert_ok(oracle.compare_scales(ws.cpu().numpy(), s_ref), "scales")
    assert_ok(oracle.compare_codes(codes_np(wq, bits), q_ref, r_ref), "codes")


@pytest.mark.parametrize("n,k,dtype", [(96, 4096, "f16"), (33, 11008, "f16"), (16, 256, "bf16")])
def test_quantize_weights_group128_parity(n, k, dtype):
    say(f"wq g128 n={n} k={k}")
    w = synth.normal_tensor(SEED, f"wg/{n}/{k}", (n, k), std=0.015, dtype=dtype)
    w[1, :128] = 0  # an all-zero group
    wq, ws = q.qlin_quantize_weights(w.to(DEV), bits=4, group=128)
    torch.cuda.synchronize()
    q_ref, s_ref, r_ref = oracle.quantize_weights(synth.to_f64(w), None, 0, 4, group=128)
    assert np.array_equal(ws.cpu().numpy().view(np.uint16), s_ref.view(np.uint16)), "fp16 group scales differ"
    assert_ok(oracle.compare_codes(codes_np(wq, 4), q_ref, r_ref), "codes")


# ---------------------------------------------------------------- integer GEMM

GEMM_SHAPES = [
    # up to 64 rows: the 16-column kernel (one to four 16-row tiles, k over eight waves)
    (16, 512, 512),      # single linear
    (50, 1024, 4096),
    (64, 256, 16384),
    (1, 96, 128),        # one token, fewer k pieces than waves
    (33, 64, 192),       # k % 128 == 64: a half-full last int4 piece (w4a8 needs k % 128 == 0)
    (40, 100, 4096),
    (17, 99, 2048),      # odd n: ragged last column strip
    (5, 1000, 1024),
    (50, 4096, 1024),
    # more rows: the large-tile GEMM
    (300, 520, 1024),    # ragged M and N tiles
    (257, 256, 2048),    # split-K
    (80, 100, 4096),     # split-K, n % 8 == 4: four outputs per reduce lane
    (70, 99, 2048),      # split-K, odd n: one output per reduce lane
    (65, 256, 16384),    # split-K
    (1000, 1800, 4160),  # int8 x int8: two K splits, one block per CU (240 CUs); ragged M and N (k past
                         # 64 stages: the 64 x 64 two-round plan does not apply)
    (250, 4000, 256),    # int8 x int8: 64 x 64 tiles, one per CU (252); ragged M and N
    (300, 520, 320),     # k % 128 == 64 on the large-tile GEMM: a half-full last int4 stage
    (70, 99, 4160),      # ... with split-K: 33 stages in two splits, the half stage in the last
]


# scheme -> (activation bits, weight bits, entry point)
SCHEMES = {"w4a4": (4, 4, "qlin_gemm_w4a4"), "w8a8": (8, 8, "qlin_gemm_w8a8"), "w4a8": (8, 4, "qlin_gemm_w4a8")}


def scheme_codes(scheme, tag, m, n, k):
    abits, wbits, fn = SCHEMES[scheme]
    a = synth.random_codes(SEED, f"A{tag}/{m}/{k}/{abits}", m, k, abits)
    b = synth.random_codes(SEED, f"B{tag}/{n}/{k}/{wbits}", n, k, wbits)
    return a, b, abits, wbits, getattr(q, fn)


def workspace_for(scheme, m, n, k):
    """The split-K workspace of qlin_gemm_ws for this shape (None: no split)."""
    return q.gemm_workspace({"w4a4": q.QLIN_W4A4, "w8a8": q.QLIN_W8A8, "w4a8": q.QLIN_W4A8}[scheme], m, n, k, DEV)


@pytest.mark.parametrize("ws", [False, True], ids=["plain", "workspace"])
@pytest.mark.parametrize("m,n,k", GEMM_SHAPES)
@pytest.mark.parametrize("scheme", ["w4a4", "w8a8", "w4a8"])
def test_gemm_raw_accumulators_bit_exact(scheme, m, n, k, ws):
    """Plain entry points (never split k) and qlin_gemm_ws with its workspace
    (split-K on the shapes marked so): raw int32 accumulators, bit-exact."""
    say(f"gemm i32 {scheme} {m}x{n}x{k} ws={ws}")
    if scheme == "w4a8" and k % 128:
        pytest.skip("W4A8 takes k in multiples of 128")
    work = workspace_for(scheme, m, n, k) if ws else None
    if ws and work is None:
        pytest.skip("no split-K at this shape: the workspace call is the plain call")
    a, b, abits, wbits, fn = scheme_codes(scheme, "", m, n, k)
    acc = fn(a.to(DEV), None, b.to(DEV), None, k, y_dtype=torch.int32, workspace=work)
    torch.cuda.synchronize()
    ref = oracle.int_gemm(codes_np(a, abits), codes_np(b, wbits))
    got = acc.cpu().numpy().astype(np.int64)
    assert np.array_equal(got, ref), f"{np.count_nonzero(got != ref)} accumulators differ"


# Grids above one block per CU (256 CUs): the launch with two resident blocks
# per CU and the shorter DMA ring; the smaller shapes above take the one-block
# deep-ring launch.  Sampled rows (first, last, random) against the oracle.
BIG_GRID_SHAPES = [
    ("w8a8", 1100, 3968, 256),    # 9 x 31 tiles of 128 x 128
    ("w4a4", 1100, 3968, 256),    # 9 x 31 tiles of 128 x 128
    ("w4a4", 2100, 4096, 256),    # 17 x 16 tiles of 128 x 256
    ("w4a8", 1100, 3968, 512),    # 9 x 31 tiles of 128 x 128
    # at least one 256 x 256 tile per CU: int8 and W4A8 operands take the
    # one-block-per-CU 256 x 256 launch with tiles in groups of 4 tile rows,
    # W4A4 the 128 x 256 launch in groups of 8 (ragged last group, ragged M
    # and N edges)
    ("w8a8", 4100, 4000, 512),    # 17 x 16 tiles of 256 x 256
    ("w4a4", 4100, 4000, 512),    # 33 x 16 tiles of 128 x 256
    ("w4a8", 4100, 4096, 256),
    ("w8a8", 6528, 2560, 1024),   # 26 x 10 tiles, the last tile row half empty
    ("w8a8", 6528, 2048, 1024),   # 208 tiles of 256 x 256 on 256 CUs (at least 3/4 of them: still this plan)
    ("w4a8", 6100, 2000, 512),    # 24 x 8 = 192 tiles, exactly 3/4 of the CUs; ragged M and N
    ("w8a8", 4100, 4096, 192),    # 3 k-stages: one zero-filled stage pads the 4-stage ring
    ("w4a4", 4352, 4096, 384),    # 34 x 16 tiles of 128 x 256, 3 k-stages
    ("w4a8", 4352, 4096, 512),    # 4 k-stages, padded to 6 (3-stage ring)
    ("w8a8", 256, 4096, 2048),    # the 7B decoder's 256 tokens: 64 x 64 tiles, one per CU
    ("w8a8", 816, 2048, 2048),    # short k: 416 tiles of 64 x 64, two rounds
    ("w8a8", 600, 2000, 1024),    # short k: 10 x 32 tiles of 64 x 64, ragged M and N
    ("w8a8", 256, 11008, 512),    # 172 tiles of 128 x 128 (the deep ring), not 64 x 64
    ("w4a4", 2100, 4096, 320),    # 128 x 256 tiles, a half-full last int4 stage
]


@pytest.mark.parametrize("scheme,m,n,k", BIG_GRID_SHAPES)
def test_gemm_big_grid_sampled_rows(scheme, m, n, k):
    say(f"gemm i32 big grid {scheme} {m}x{n}x{k}")
    a, b, abits, wbits, fn = scheme_codes(scheme, "big", m, n, k)
    acc = fn(a.to(DEV), None, b.to(DEV), None, k, y_dtype=torch.int32)
    torch.cuda.synchronize()
    rows = _sample_rows(m, 24)
    ref = oracle.int_gemm(codes_np(a, abits)[rows], codes_np(b, wbits))
    got = acc.cpu().numpy().astype(np.int64)[rows]
    assert np.array_equal(got, ref), f"{np.count_nonzero(got != ref)} accumulators differ"


# 256 x 256 grids whose last round would fill at most half of the 256 CUs:
# the full rounds run as 256 x 256 tiles and the last rows as 128 x 128
# tiles (two blocks per CU) in a second launch.
TAIL_SHAPES = [
    ("w8a8", 9316, 2048, 512),    # 37 tile rows of 8: 32 in full rounds, a ragged tail of 1124 rows
    ("w4a8", 9316, 2048, 512),
    ("w8a8", 8300, 4096, 256),    # 33 tile rows of 16: a tail of 108 rows
]


@pytest.mark.parametrize("out", ["i32", "bf16"])
@pytest.mark.parametrize("scheme,m,n,k", TAIL_SHAPES)
def test_gemm_256_grid_with_small_tile_tail(scheme, m, n, k, out):
    """Rows on both sides of the split, the first and last rows and random
    ones: raw accumulators bit-exact, dequantized outputs within tolerance,
    against the oracle."""
    say(f"gemm 256 + tail {scheme} {m}x{n}x{k} {out}")
    a, b, abits, wbits, fn = scheme_codes(scheme, "tail", m, n, k)
    tm, per_round = (m + 255) // 256, 256 // ((n + 255) // 256)
    split = tm // per_round * per_round * 256
    rows = np.array(sorted(set(_sample_rows(m, 24).tolist()) | set(range(split - 3, split + 3))))
    ac, bc = codes_np(a, abits), codes_np(b, wbits)
    if out == "i32":
        acc = fn(a.to(DEV), None, b.to(DEV), None, k, y_dtype=torch.int32)
        torch.cuda.synchronize()
        got = acc.cpu().numpy().astype(np.int64)[rows]
        ref = oracle.int_gemm(ac[rows], bc)
        assert np.array_equal(got, ref), f"{np.count_nonzero(got != ref)} accumulators differ"
    else:
        sx = synth.random_scales(SEED, f"sxt/{m}", m)
        sw = synth.random_scales(SEED, f"swt/{n}", n)
        y = fn(a.to(DEV), sx.to(DEV), b.to(DEV), sw.to(DEV), k, y_dtype=torch.bfloat16)
        torch.cuda.synchronize()
        _, _, y_ref = oracle.gemm(ac[rows], sx.numpy()[rows], bc, sw.numpy(), "bf16")
        assert_ok(oracle.compare_outputs(f64(y)[rows], y_ref), "output")


@pytest.mark.parametrize("m,f,k", [(1100, 1984, 256), (2100, 2048, 256), (4100, 2048, 512), (2050, 8192, 256),
                                   (1100, 2048, 192)])
def test_gemm_geglu_big_grid_sampled_rows(m, f, k):
    say(f"gemm geglu big grid {m}x{f}x{k}")
    n2 = 2 * f
    a = synth.random_codes(SEED, f"Agbig/{m}/{k}", m, k, 4)
    b = synth.random_codes(SEED, f"Bgbig/{n2}/{k}", n2, k, 4)
    sx = synth.random_scales(SEED, f"sxgbig/{m}", m)
    sw = synth.random_scales(SEED, f"swgbig/{n2}", n2)
    h = q.qlin_gemm_w4a4_geglu(a.to(DEV), sx.to(DEV), b.to(DEV), sw.to(DEV), k, h_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    rows = _sample_rows(m, 24)
    _, _, h_ref = oracle.gemm_geglu(codes_np(a, 4)[rows], sx.numpy()[rows], codes_np(b, 4), sw.numpy(), "bf16")
    assert_ok(oracle.compare_outputs(f64(h)[rows], h_ref), "h")


@pytest.mark.parametrize("out", ["f16", "bf16", "f32"])
@pytest.mark.parametrize("scheme,m,n,k", [("w4a4", 300, 520, 1024), ("w8a8", 129, 384, 4096),
                                          ("w8a8", 64, 256, 16384), ("w4a4", 16, 512, 512),
                                          ("w8a8", 40, 100, 4096), ("w4a4", 17, 99, 2048),
                                          ("w4a8", 300, 520, 1024), ("w4a8", 64, 256, 16384),
                                          ("w4a8", 17, 99, 2048), ("w4a4", 50, 1024, 1024),
                                          ("w8a8", 80, 100, 4096), ("w4a8", 9, 1000, 1024),
                                          ("w8a8", 250, 4000, 256), ("w4a4", 300, 520, 320),
                                          ("w4a4", 33, 64, 192)])
def test_gemm_dequant_epilogue(scheme, m, n, k, out):
    say(f"gemm {out} {scheme} {m}x{n}x{k}")
    a, b, abits, wbits, fn = scheme_codes(scheme, "e", m, n, k)
    sx = synth.random_scales(SEED, f"sx/{m}", m)
    sw = synth.random_scales(SEED, f"sw/{n}", n)
    a, b, sx, sw = a.to(DEV), b.to(DEV), sx.to(DEV), sw.to(DEV)
    y = fn(a, sx, b, sw, k, y_dtype=DT[out])
    work = workspace_for(scheme, m, n, k)
    y_ws = fn(a, sx, b, sw, k, y_dtype=DT[out], workspace=work) if work is not None else y
    torch.cuda.synchronize()
    _, _, y_ref = oracle.gemm(codes_np(a.cpu(), abits), sx.cpu().numpy(), codes_np(b.cpu(), wbits),
                              sw.cpu().numpy(), out)
    assert_ok(oracle.compare_outputs(f64(y), y_ref), "output")
    # the split-K reduction applies the same epilogue arithmetic: bit-identical outputs
    bits = torch.int32 if out == "f32" else torch.int16
    assert torch.equal(y.view(bits), y_ws.view(bits))


GEGLU_SHAPES = [
    # m, f (h columns; n2 = 2 f interleaved weight rows), k
    (50, 64, 256),       # 128-wide tiles
    (130, 2048, 512),    # 128-wide tiles (256-wide ones would not fill the CUs), ragged m
    (1, 32, 128),        # one token, one gate/up pair, ragged n tile
    (300, 4096, 1024),
]


@pytest.mark.parametrize("out", ["bf16", "f16", "f32"])
@pytest.mark.parametrize("m,f,k", GEGLU_SHAPES)
def test_gemm_w4a4_geglu(m, f, k, out):
    say(f"gemm geglu {out} {m}x{f}x{k}")
    n2 = 2 * f
    a = synth.random_codes(SEED, f"Ag/{m}/{k}", m, k, 4)
    b = synth.random_codes(SEED, f"Bg/{n2}/{k}", n2, k, 4)   # any codes: rows already in fused order
    sx = synth.random_scales(SEED, f"sxg/{m}", m)
    sw = synth.random_scales(SEED, f"swg/{n2}", n2)
    h = q.qlin_gemm_w4a4_geglu(a.to(DEV), sx.to(DEV), b.to(DEV), sw.to(DEV), k, h_dtype=DT[out])
    torch.cuda.synchronize()
    assert h.shape == (m, f)
    _, _, h_ref = oracle.gemm_geglu(codes_np(a, 4), sx.numpy(), codes_np(b, 4), sw.numpy(), out)
    assert_ok(oracle.compare_outputs(f64(h), h_ref), "h")


def test_interleave_binding_matches_oracle():
    g = torch.arange(64 * 3, dtype=torch.int32).reshape(64, 3)
    u = -g
    got = q.interleave_gate_up(g, u).numpy()
    assert np.array_equal(got, oracle.interleave_gate_up(g.numpy(), u.numpy()))


@pytest.mark.parametrize("m", [3, 65])
@pytest.mark.parametrize("scheme", ["w4a4", "w8a8", "w4a8"])
def test_gemm_extreme_codes_at_max_k(scheme, m):
    """Every code at the most negative value (-8 int4, -128 int8) and the
    largest k the entry points take (131072 - 128): the largest accumulator
    magnitudes the kernels can meet, bit-exact (3 rows: the 16-column kernel;
    65: the large-tile GEMM)."""
    abits, wbits, fn = SCHEMES[scheme]
    fn = getattr(q, fn)
    n, k = 96, 131072 - 128
    def extreme(rows, bits):
        if bits == 8:
            return torch.full((rows, k), -128, dtype=torch.int8)
        return torch.full((rows, k // 2), 0x88, dtype=torch.uint8)   # two -8 nibbles
    a, b = extreme(m, abits), extreme(n, wbits)
    b[1] = 0x77 if wbits == 4 else 127                                # a row of +7 / +127
    acc = fn(a.to(DEV), None, b.to(DEV), None, k, y_dtype=torch.int32)
    torch.cuda.synchronize()
    ref = oracle.int_gemm(codes_np(a, abits), codes_np(b, wbits))
    assert np.array_equal(acc.cpu().numpy().astype(np.int64), ref)


@pytest.mark.parametrize("m", [40, 700])
def test_gemm_w4a4_stacked_weights_equal_separate(m):
    """q, k, v weights stacked along n (one GEMM over their shared activation
    codes): outputs equal the three separate GEMMs' outputs bit for bit, on the
    small-M and the large-tile kernels."""
    say(f"gemm stacked qkv m={m}")
    k, ns = 2048, (2048, 512, 1024)
    x = synth.normal_tensor(SEED, f"stk/x/{m}", (m, k), dtype="bf16", outliers=20, outlier_scale=20.0).to(DEV)
    xq, xs = q.qlin_rotate_quant_act(x, had_block=128, bits=4)
    parts = [q.qlin_quantize_weights(synth.normal_tensor(SEED, f"stk/w/{i}", (n, k), std=0.02, dtype="bf16").to(DEV),
                                     had_block=128, bits=4) for i, n in enumerate(ns)]
    y = q.qlin_gemm_w4a4(xq, xs, torch.cat([t[0] for t in parts]), torch.cat([t[1] for t in parts]), k,
                         y_dtype=torch.bfloat16)
    ys = [q.qlin_gemm_w4a4(xq, xs, a, b, k, y_dtype=torch.bfloat16) for a, b in parts]
    torch.cuda.synchronize()
    assert torch.equal(y.view(torch.int16), torch.cat(ys, dim=1).view(torch.int16))


@pytest.mark.parametrize("scheme", ["w4a4", "w8a8", "w4a8"])
def test_gemm_small_m_matches_large_tile_epilogue(scheme):
    """Rows 0..63 computed alone (16-column kernel) equal the same rows of a
    129-row call (large-tile GEMM) bit for bit: the two share the epilogue
    arithmetic, float(acc) * s_x * (s_w * 2^-shift)."""
    say(f"gemm small-m vs large-tile {scheme}")
    m, n, k = 129, 520, 2048
    a, b, abits, wbits, fn = scheme_codes(scheme, "cmp", m, n, k)
    sx = synth.random_scales(SEED, f"sxc/{m}", m).to(DEV)
    sw = synth.random_scales(SEED, f"swc/{n}", n).to(DEV)
    a, b = a.to(DEV), b.to(DEV)
    for dt in (torch.float16, torch.bfloat16, torch.float32):
        big = fn(a, sx, b, sw, k, y_dtype=dt)
        small = fn(a[:64].contiguous(), sx[:64].contiguous(), b, sw, k, y_dtype=dt)
        torch.cuda.synchronize()
        bits = torch.int32 if dt == torch.float32 else torch.int16
        assert torch.equal(big[:64].contiguous().view(bits), small.view(bits)), str(dt)


def test_gemm_deterministic():
    say("gemm determinism")
    a = synth.random_codes(SEED, "Ad", 129, 16384, 8).to(DEV)
    b = synth.random_codes(SEED, "Bd", 256, 16384, 8).to(DEV)
    sx = synth.random_scales(SEED, "sxd", 129).to(DEV)
    sw = synth.random_scales(SEED, "swd", 256).to(DEV)
    work = workspace_for("w8a8", 129, 256, 16384)
    y1 = q.qlin_gemm_w8a8(a, sx, b, sw, 16384, workspace=work)
    y2 = q.qlin_gemm_w8a8(a, sx, b, sw, 16384, workspace=work)
    torch.cuda.synchronize()
    assert torch.equal(y1.view(torch.int16), y2.view(torch.int16))


# ---------------------------------------------------------------- W4A16 GEMV

GEMV_CASES = [(1, 4096, 4096), (1, 11008, 4096), (1, 4096, 11008), (3, 520, 1024), (50, 1024, 4096),
              (64, 256, 256), (17, 1000, 2048),
              # every chunk-slot count (k up to 32768), token-row pass size and rows-per-wave choice,
              # ragged n and m
              (1, 300, 128), (2, 77, 32768), (5, 130, 20480), (9, 333, 16384), (4, 250, 12288),
              (8, 8200, 2048), (1, 9000, 5120), (64, 40, 1024), (50, 1030, 4096),
              # from four rows on the matrix-core kernel: one to four 16-row tiles, one group
              # per k slice or several (odd counts, 1 to 32 per slice), idle slices (k = 128, 384),
              # row tiles of 4..16 valid rows
              (50, 1024, 1024), (33, 4096, 1024), (47, 520, 128), (12, 200, 384), (16, 1000, 1664),
              (64, 100, 32768), (25, 96, 2560), (49, 17, 1152), (4, 1024, 4096), (7, 4096, 1024),
              (3, 4096, 4096)]


@pytest.mark.parametrize("m,n,k", GEMV_CASES)
def test_gemv_w4a16_parity(m, n, k):
    say(f"gemv {m}x{n}x{k}")
    x = synth.normal_tensor(SEED, f"gx/{m}/{k}", (m, k), dtype="f16")
    w = synth.normal_tensor(SEED, f"gw/{n}/{k}", (n, k), std=0.015, dtype="f16")
    wq, ws = q.qlin_quantize_weights(w.to(DEV), bits=4, group=128)
    y = q.qlin_gemv_w4a16(x.to(DEV), wq, ws)
    torch.cuda.synchronize()
    y32, y_ref = oracle.gemv_w4a16(synth.to_f64(x), codes_np(wq, 4), ws.cpu().numpy(), 128)
    assert_ok(oracle.compare_outputs(f64(y), y_ref), "output")


@pytest.mark.parametrize("nbytes", [16, 4096 + 16, 8 * 2 ** 20 + 256 * 1024, 46 * 2 ** 20 + 48])
def test_stream_read_reads_every_word_once(nbytes):
    """The streaming-read reference folds every 16-byte word it reads into
    the sink by xor, so the xor of the sink equals the xor of the bytes read."""
    say(f"stream read {nbytes} bytes")
    g = torch.Generator().manual_seed(nbytes)
    src = torch.randint(-2 ** 31, 2 ** 31 - 1, (nbytes // 4 + 64,), dtype=torch.int32, generator=g)
    sink = torch.zeros(q.QLIN_STREAM_READ_SINK_WORDS, dtype=torch.int32, device=DEV)
    q.qlin_stream_read(src.to(DEV), nbytes, sink=sink)
    torch.cuda.synchronize()
    want = np.bitwise_xor.reduce(src[: nbytes // 4].numpy())
    assert np.bitwise_xor.reduce(sink.cpu().numpy()) == want


@pytest.mark.parametrize("m", [2, 20])
def test_gemv_w4a16_subnormal_and_large_x(m):
    # fp16 subnormal, zero and near-maximum activations (the vector kernel folds a
    # per-chunk sum of x into its accumulation, which must see the same values;
    # at 20 rows the matrix cores take them as operands)
    say(f"gemv subnormal/large x m={m}")
    n, k = 520, 4096
    x = synth.normal_tensor(SEED, "gx/sub", (m, k), dtype="f16")
    x[0, ::3] = torch.tensor(3.0e-6, dtype=torch.float16)     # subnormal
    x[0, 1::7] = 0
    x[1, ::5] = torch.tensor(-2.0e3, dtype=torch.float16)     # large
    x[1, 0], x[1, k - 1] = 6.0e4, -6.0e4                        # near the fp16 maximum
    x[m - 1, 2::9] = torch.tensor(-6.1e-5, dtype=torch.float16)  # smallest normals
    w = synth.normal_tensor(SEED, "gw/sub", (n, k), std=0.015, dtype="f16")
    wq, ws = q.qlin_quantize_weights(w.to(DEV), bits=4, group=128)
    y = q.qlin_gemv_w4a16(x.to(DEV), wq, ws)
    torch.cuda.synchronize()
    y32, y_ref = oracle.gemv_w4a16(synth.to_f64(x), codes_np(wq, 4), ws.cpu().numpy(), 128)
    for i in range(m):  # each row on its own scale
        assert_ok(oracle.compare_outputs(f64(y)[i:i + 1], y_ref[i:i + 1]), f"output row {i}")


@pytest.mark.parametrize("m,n,k", [(50, 1024, 4096), (9, 300, 1024)])
def test_gemv_w4a16_repeatable(m, n, k):
    # the k slices' partial tiles are added in a fixed order: two calls agree bit for bit
    say(f"gemv repeat {m}x{n}x{k}")
    x = synth.normal_tensor(SEED, f"gx/{m}/{k}", (m, k), dtype="f16").to(DEV)
    w = synth.normal_tensor(SEED, f"gw/{n}/{k}", (n, k), std=0.015, dtype="f16")
    wq, ws = q.qlin_quantize_weights(w.to(DEV), bits=4, group=128)
    y1 = q.qlin_gemv_w4a16(x, wq, ws)
    y2 = q.qlin_gemv_w4a16(x, wq, ws)
    torch.cuda.synchronize()
    assert torch.equal(y1.view(torch.int16), y2.view(torch.int16))


@pytest.mark.parametrize("m,k,ns", [(1, 4096, (4096, 4096, 4096)), (1, 4096, (11008, 11008)), (20, 1024, (520, 96))])
def test_gemv_w4a16_merged_rows_equal_separate(m, k, ns):
    """Weights of projections that read one input stacked along n (q|k|v,
    gate|up): the merged call's outputs are the separate calls' outputs, bit
    for bit (every output row is computed from its own weight row alone)."""
    say(f"gemv merged m={m} k={k} n={ns}")
    x = synth.normal_tensor(SEED, f"gmx/{m}/{k}", (m, k), dtype="f16").to(DEV)
    parts = []
    for i, n in enumerate(ns):
        w = synth.normal_tensor(SEED, f"gmw/{i}/{n}/{k}", (n, k), std=0.015, dtype="f16")
        parts.append(q.qlin_quantize_weights(w.to(DEV), bits=4, group=128))
    wq = torch.cat([t[0] for t in parts])
    ws = torch.cat([t[1] for t in parts])
    y = q.qlin_gemv_w4a16(x, wq, ws)
    ys = [q.qlin_gemv_w4a16(x, a, b) for a, b in parts]
    torch.cuda.synchronize()
    assert torch.equal(y.view(torch.int16), torch.cat(ys, dim=1).view(torch.int16))


# ---------------------------------------------------------------- fold calibration


@pytest.mark.parametrize("pre", [q.QLIN_PRE_NONE, q.QLIN_PRE_GEGLU])
def test_calibrate_fold_parity(pre):
    say(f"calibrate pre={pre}")
    m, k, n = 100, 2048, 300
    width = 2 * k if pre == q.QLIN_PRE_GEGLU else k
    x = synth.normal_tensor(SEED, f"cx/{pre}", (m, width), dtype="bf16", outliers=20, outlier_scale=30.0)
    w = synth.normal_tensor(SEED, f"cw/{pre}", (n, k), std=0.02, dtype="f16")
    x[:, 5] = 0  # channel with zero maximum -> s = 1
    if pre == q.QLIN_PRE_GEGLU:
        x[:, k + 5] = 0
    s, inv_s = q.qlin_calibrate_fold(x.to(DEV), w.to(DEV), pre=pre)
    torch.cuda.synchronize()
    xf = synth.to_f64(x)
    act = oracle.geglu(xf, k) if pre == q.QLIN_PRE_GEGLU else xf
    s_ref = oracle.calibrate_fold(act, synth.to_f64(w))
    assert_ok(oracle.compare_scales(s.cpu().numpy(), s_ref), "fold s")
    assert s.cpu().numpy()[5] == 1.0
    np.testing.assert_array_equal(inv_s.cpu().numpy(), (np.float32(1.0) / s.cpu().numpy()).astype(np.float32))


# ---------------------------------------------------------------- whole projections


def test_single_w4a4_linear_end_to_end():
    """16x512x512, 4 outlier channels x20, W ~ N(0, 0.02), fold, b = 64, W4A4, fp16 out."""
    wl = synth.CFG1
    proj = wl.projs[0]
    say("single W4A4 linear")
    x = synth.activation(wl, proj, 16)
    w = synth.weight(wl, proj)
    xd, wd = x.to(DEV), w.to(DEV)
    s, inv_s = q.qlin_calibrate_fold(xd, wd)
    wq, ws = q.qlin_quantize_weights(wd, fold_s=s, had_block=64, bits=4)
    xq, xs = q.qlin_rotate_quant_act(xd, fold_inv_s=inv_s, had_block=64, bits=4)
    y = q.qlin_gemm_w4a4(xq, xs, wq, ws, 512, y_dtype=torch.float16)
    torch.cuda.synchronize()
    xf, wf = synth.to_f64(x), synth.to_f64(w)
    s_ref = oracle.calibrate_fold(xf, wf)
    assert_ok(oracle.compare_scales(s.cpu().numpy(), s_ref), "fold")
    sg = s.cpu().numpy()
    qw_ref, sw_ref, rw = oracle.quantize_weights(wf, sg, 64, 4)
    assert_ok(oracle.compare_codes(codes_np(wq, 4), qw_ref, rw), "weight codes")
    assert_ok(oracle.compare_scales(ws.cpu().numpy(), sw_ref), "weight scales")
    qx_ref, sx_ref, rx = oracle.rotate_quant_act(xf, sg, 64, 4)
    assert_ok(oracle.compare_codes(codes_np(xq, 4), qx_ref, rx), "act codes")
    assert_ok(oracle.compare_scales(xs.cpu().numpy(), sx_ref), "act scales")
    acc, _, y_ref = oracle.gemm(codes_np(xq, 4), xs.cpu().numpy(), codes_np(wq, 4), ws.cpu().numpy(), "f16")
    assert_ok(oracle.compare_outputs(f64(y), y_ref), "output")
    # the quantized projection approximates the float one (reported bound, generous)
    ref = xf @ wf.T
    assert np.linalg.norm(f64(y) - ref) / np.linalg.norm(ref) < 0.35


def _sample_rows(m, count, seed=7):
    rng = np.random.default_rng(seed)
    rows = set(rng.choice(m, size=min(count, m), replace=False).tolist())
    rows.update({0, m - 1})
    return np.array(sorted(rows))


@pytest.mark.slow
def test_backbone_mlp_block_stagewise_full_size():
    """M = 816 backbone MLP block at full size: gate|up W4A4 (N = 32768,
    K = 2048) -> GeGLU pre-op -> int8 -> down W8A8 (N = 2048, K = 16384),
    bf16, b = 128.  Launch configuration as timed by the benchmark; sampled
    rows are checked stage by stage."""
    wl = synth.CFG2
    gu, dn = wl.projs
    m = 816
    say("backbone MLP block: generate")
    x = synth.activation(wl, gu, m)
    w_gu = synth.weight(wl, gu)
    w_dn = synth.weight(wl, dn)
    xd, wgd, wdd = x.to(DEV), w_gu.to(DEV), w_dn.to(DEV)
    say("backbone MLP block: gpu path")
    s1, inv1 = q.qlin_calibrate_fold(xd, wgd)
    wq1, ws1 = q.qlin_quantize_weights(wgd, fold_s=s1, had_block=128, bits=4)
    xq1, xs1 = q.qlin_rotate_quant_act(xd, fold_inv_s=inv1, had_block=128, bits=4)
    y1 = q.qlin_gemm_w4a4(xq1, xs1, wq1, ws1, 2048, y_dtype=torch.bfloat16)
    s2, inv2 = q.qlin_calibrate_fold(y1, wdd, pre=q.QLIN_PRE_GEGLU)
    wq2, ws2 = q.qlin_quantize_weights(wdd, fold_s=s2, had_block=128, bits=8)
    hq, hs = q.qlin_rotate_quant_act(y1, k=16384, fold_inv_s=inv2, had_block=128, bits=8, pre=q.QLIN_PRE_GEGLU)
    y2 = q.qlin_gemm_w8a8(hq, hs, wq2, ws2, 16384, y_dtype=torch.bfloat16,
                          workspace=workspace_for("w8a8", m, dn.n, 16384))
    torch.cuda.synchronize()
    say("backbone MLP block: oracle checks")
    xf = synth.to_f64(x)
    s1g = s1.cpu().numpy()
    assert_ok(oracle.compare_scales(s1g, oracle.calibrate_fold(xf, synth.to_f64(w_gu))), "fold gate|up")
    rows_w = _sample_rows(32768, 48)
    qw, sw, rw = oracle.quantize_weights(synth.to_f64(w_gu[rows_w]), s1g, 128, 4)
    assert_ok(oracle.compare_codes(codes_np(wq1, 4)[rows_w], qw, rw), "gate|up weight codes")
    assert_ok(oracle.compare_scales(ws1.cpu().numpy()[rows_w], sw), "gate|up weight scales")
    rows = _sample_rows(m, 6)
    qx, sx, rx = oracle.rotate_quant_act(xf[rows], s1g, 128, 4)
    assert_ok(oracle.compare_codes(codes_np(xq1, 4)[rows], qx, rx), "act codes")
    assert_ok(oracle.compare_scales(xs1.cpu().numpy()[rows], sx), "act scales")
    xq1n, wq1n = codes_np(xq1, 4), codes_np(wq1, 4)
    _, _, y1_ref = oracle.gemm(xq1n[rows], xs1.cpu().numpy()[rows], wq1n, ws1.cpu().numpy(), "bf16")
    assert_ok(oracle.compare_outputs(f64(y1)[rows], y1_ref), "gate|up output")
    y1f = f64(y1)
    s2g = s2.cpu().numpy()
    assert_ok(oracle.compare_scales(s2g, oracle.calibrate_fold(oracle.geglu(y1f, 16384), synth.to_f64(w_dn))),
              "fold down")
    rows_d = _sample_rows(2048, 12)
    qw2, sw2, rw2 = oracle.quantize_weights(synth.to_f64(w_dn[rows_d]), s2g, 128, 8)
    assert_ok(oracle.compare_codes(codes_np(wq2, 8)[rows_d], qw2, rw2), "down weight codes")
    qh, sh, rh = oracle.rotate_quant_act(y1f[rows], s2g, 128, 8, preop="geglu")
    assert_ok(oracle.compare_codes(codes_np(hq, 8)[rows], qh, rh), "GeGLU act codes")
    assert_ok(oracle.compare_scales(hs.cpu().numpy()[rows], sh), "GeGLU act scales")
    _, _, y2_ref = oracle.gemm(codes_np(hq, 8)[rows], hs.cpu().numpy()[rows], codes_np(wq2, 8),
                               ws2.cpu().numpy(), "bf16")
    assert_ok(oracle.compare_outputs(f64(y2)[rows], y2_ref), "down output")


@pytest.mark.slow
def test_backbone_mlp_block_fused_geglu_full_size():
    """The benchmark's chain: X -> int4 -> gate|up W4A4 GEMM with the GeGLU
    epilogue (weights interleaved in blocks of 32 rows) -> h bf16 -> fold,
    Hadamard 128, int8 -> down W8A8 -> bf16; sampled rows stage by stage."""
    wl = synth.CFG2
    gu, dn = wl.projs
    m, f = 816, dn.k
    say("fused MLP block: generate")
    x = synth.activation(wl, gu, m)
    w_gu = synth.weight(wl, gu)
    w_dn = synth.weight(wl, dn)
    w_int = q.interleave_gate_up(w_gu[:f], w_gu[f:])
    xd, wgd, wdd = x.to(DEV), w_int.to(DEV), w_dn.to(DEV)
    say("fused MLP block: gpu path")
    s1, inv1 = q.qlin_calibrate_fold(xd, wgd)
    wq1, ws1 = q.qlin_quantize_weights(wgd, fold_s=s1, had_block=128, bits=4)
    xq1, xs1 = q.qlin_rotate_quant_act(xd, fold_inv_s=inv1, had_block=128, bits=4)
    h = q.qlin_gemm_w4a4_geglu(xq1, xs1, wq1, ws1, 2048, h_dtype=torch.bfloat16)
    s2, inv2 = q.qlin_calibrate_fold(h, wdd)
    wq2, ws2 = q.qlin_quantize_weights(wdd, fold_s=s2, had_block=128, bits=8)
    hq, hs = q.qlin_rotate_quant_act(h, fold_inv_s=inv2, had_block=128, bits=8)
    y2 = q.qlin_gemm_w8a8(hq, hs, wq2, ws2, f, y_dtype=torch.bfloat16, workspace=workspace_for("w8a8", m, dn.n, f))
    torch.cuda.synchronize()
    say("fused MLP block: oracle checks")
    rows = _sample_rows(m, 6)
    xq1n, wq1n = codes_np(xq1, 4), codes_np(wq1, 4)
    _, _, h_ref = oracle.gemm_geglu(xq1n[rows], xs1.cpu().numpy()[rows], wq1n, ws1.cpu().numpy(), "bf16")
    assert_ok(oracle.compare_outputs(f64(h)[rows], h_ref), "h")
    hf = f64(h)
    s2g = s2.cpu().numpy()
    assert_ok(oracle.compare_scales(s2g, oracle.calibrate_fold(hf, synth.to_f64(w_dn))), "fold down")
    qh, sh, rh = oracle.rotate_quant_act(hf[rows], s2g, 128, 8)
    assert_ok(oracle.compare_codes(codes_np(hq, 8)[rows], qh, rh), "h codes")
    assert_ok(oracle.compare_scales(hs.cpu().numpy()[rows], sh), "h scales")
    _, _, y2_ref = oracle.gemm(codes_np(hq, 8)[rows], hs.cpu().numpy()[rows], codes_np(wq2, 8),
                               ws2.cpu().numpy(), "bf16")
    assert_ok(oracle.compare_outputs(f64(y2)[rows], y2_ref), "down output")


def _check_linear(x, w, s, b, bits, out, rows=None, scheme_fn=None):
    """One quantized projection on the GPU, checked stage by stage against the
    oracle: weight codes and scales, activation codes and scales, output (on
    sampled rows when `rows` is given)."""
    xd, wd = x.to(DEV), w.to(DEV)
    sd = None if s is None else s.to(DEV)
    inv = None if s is None else (1.0 / s).to(DEV)
    wq, ws = q.qlin_quantize_weights(wd, fold_s=sd, had_block=b, bits=bits)
    xq, xs = q.qlin_rotate_quant_act(xd, fold_inv_s=inv, had_block=b, bits=bits)
    fn = scheme_fn or (q.qlin_gemm_w4a4 if bits == 4 else q.qlin_gemm_w8a8)
    y = fn(xq, xs, wq, ws, x.shape[1], y_dtype=DT[out])
    torch.cuda.synchronize()
    sg = None if s is None else s.numpy()
    r = np.arange(x.shape[0]) if rows is None else rows
    rd = torch.as_tensor(r, device=DEV)
    rw = _sample_rows(w.shape[0], 32)
    qw_ref, sw_ref, rr = oracle.quantize_weights(synth.to_f64(w[rw]), sg, b, bits)
    assert_ok(oracle.compare_codes(codes_np(wq, bits)[rw], qw_ref, rr), "weight codes")
    assert_ok(oracle.compare_scales(ws.cpu().numpy()[rw], sw_ref), "weight scales")
    qx_ref, sx_ref, rx = oracle.rotate_quant_act(synth.to_f64(x[r]), sg, b, bits)
    xq_r = codes_np(xq[rd], bits)
    xs_r = xs[rd].cpu().numpy()
    assert_ok(oracle.compare_codes(xq_r, qx_ref, rx), "act codes")
    assert_ok(oracle.compare_scales(xs_r, sx_ref), "act scales")
    _, _, y_ref = oracle.gemm(xq_r, xs_r, codes_np(wq, bits), ws.cpu().numpy(), out)
    assert_ok(oracle.compare_outputs(f64(y[rd]), y_ref), "output")


@pytest.mark.slow
def test_action_expert_denoising_steps():
    """Action expert (M = 50; q, k, v, o 1024x1024, up 4096x1024, down
    1024x4096) at denoising steps 0, 4 and 9: X_t ~ N(0, sigma_t^2) per
    projection and step, the fold calibrated on step 0, W4A4 with b = 64,
    fp16 out; and the W4A16 g128 GEMV on the same weights and inputs."""
    wl = synth.CFG3
    for proj in wl.projs:
        w = synth.weight(wl, proj)
        x0 = synth.activation(wl, proj, 50, tag="/t0", std=synth.cfg3_sigma(0))
        s = oracle.calibrate_fold(synth.to_f64(x0), synth.to_f64(w)).astype(np.float32)
        wq16, ws16 = q.qlin_quantize_weights(w.to(DEV), bits=4, group=128)
        for t in (0, 4, 9):
            say(f"action expert {proj.name} step {t}")
            x = synth.activation(wl, proj, 50, tag=f"/t{t}", std=synth.cfg3_sigma(t))
            _check_linear(x, w, torch.from_numpy(s), 64, 4, "f16")
            y16 = q.qlin_gemv_w4a16(x.to(DEV), wq16, ws16)
            torch.cuda.synchronize()
            _, y16_ref = oracle.gemv_w4a16(synth.to_f64(x), codes_np(wq16, 4), ws16.cpu().numpy(), 128)
            assert_ok(oracle.compare_outputs(f64(y16), y16_ref), "W4A16 output")


def test_action_expert_merged_qkv():
    """q, k, v of the action expert reading one input with their weights
    stacked along n (3072 x 1024, one fold calibrated on the stacked weights):
    the whole W4A4 linear against the oracle at steps 0 and 9."""
    wl = synth.CFG3
    pr = {p.name: p for p in wl.projs}
    w = torch.cat([synth.weight(wl, pr[n]) for n in ("q", "k", "v")])
    x0 = synth.activation(wl, pr["q"], 50, tag="/t0", std=synth.cfg3_sigma(0))
    s = oracle.calibrate_fold(synth.to_f64(x0), synth.to_f64(w)).astype(np.float32)
    for t in (0, 9):
        say(f"action expert merged qkv step {t}")
        x = synth.activation(wl, pr["q"], 50, tag=f"/t{t}", std=synth.cfg3_sigma(t))
        _check_linear(x, w, torch.from_numpy(s), 64, 4, "f16")


def test_action_expert_per_step_static_tables():
    """Action expert at steps 0, 4 and 9 with per-step static tables: each
    step's table calibrated (on the GPU) from that step's calibration tokens,
    the step's weights with the table folded in, the evaluation tokens
    quantized with the table, W4A4 GEMM with x_scale = 1.  Tables, codes and
    outputs against the oracle; and the per-step outputs track x w^T."""
    from bit_ptq_vla_amd.workload import ActionExpert
    ae = ActionExpert(DEV)
    ae.build_static()
    wl = synth.CFG3
    for (pr, xs, inv, per_step, xq, y), s in zip(ae.static, ae.fold_s):
        w = synth.weight(wl, pr)
        sg = s.cpu().numpy()
        rw = _sample_rows(pr.n, 32)
        for t in (0, 4, 9):
            say(f"action expert static {pr.name} step {t}")
            table, wq_t, ws_t = per_step[t]
            xc = synth.activation(wl, pr, 50, tag=f"/cal{t}", std=synth.cfg3_sigma(t))
            t_ref = oracle.calibrate_step_scales(synth.to_f64(xc), sg, 64, 4)
            _assert_table(table.cpu().numpy().astype(np.float64), t_ref, xc, s.cpu(), 64, 4)
            tg = table.cpu().numpy()
            qw_ref, sw_ref, rr = oracle.quantize_weights_step(synth.to_f64(w[rw]), sg, 64, 4, tg)
            assert_ok(oracle.compare_codes(codes_np(wq_t, 4)[rw], qw_ref, rr), "weight codes")
            assert_ok(oracle.compare_scales(ws_t.cpu().numpy()[rw], sw_ref), "weight scales")
            xq_t = q.qlin_rotate_quant_act_static(xs[t], table, fold_inv_s=inv, had_block=64, bits=4)
            yt = q.qlin_gemm_w4a4(xq_t, ae.ones, wq_t, ws_t, pr.k, y_dtype=torch.float16)
            torch.cuda.synchronize()
            x = xs[t].cpu()
            qx_ref, rx = oracle.rotate_quant_act_static(synth.to_f64(x), sg, 64, 4, tg)
            assert_ok(oracle.compare_codes(codes_np(xq_t, 4), qx_ref, rx), "act codes")
            _, _, y_ref = oracle.gemm(codes_np(xq_t, 4), np.ones(50, np.float32), codes_np(wq_t, 4),
                                      ws_t.cpu().numpy(), "f16")
            assert_ok(oracle.compare_outputs(f64(yt), y_ref), "output")
            # the method's end: the per-step quantized projection tracks x w^T
            # (W4A4 on Gaussian tokens: about 0.21 relative error, dynamic or static)
            y_true = synth.to_f64(x) @ synth.to_f64(w).T
            assert np.linalg.norm(f64(yt) - y_true) / np.linalg.norm(y_true) < 0.3


@pytest.mark.slow
def test_decoder7b_w8a8_m256():
    """7B-decoder projections at M = 256, W8A8 per-token / per-channel (no
    fold, no rotation), fp16 out; sampled rows."""
    wl = synth.CFG4
    for proj in wl.projs[3:]:   # o 4096x4096, gate and up 11008x4096, down 4096x11008
        say(f"decoder W8A8 {proj.name} {proj.n}x{proj.k}")
        x = synth.activation(wl, proj, 256)
        w = synth.weight(wl, proj)
        _check_linear(x, w, None, 0, 8, "f16", rows=_sample_rows(256, 12))


@pytest.mark.slow
def test_sweep_layer_e2m3_storage_equals_int4():
    """The benchmark's sweep layer with the W4A4 codes in E2M3 storage (q|k|v
    and the fused gate|up GEMM on the FP6 matrix cores, the two-blocks-per-CU
    GeGLU kernel at this size) gives the int4 layer's outputs bit for bit:
    q|k|v, h and the down projection."""
    from bit_ptq_vla_amd.workload import SweepModel

    m = 6528
    say(f"sweep layer E2M3 storage M={m}")
    model = SweepModel(DEV, m, layers=1, e2m3=True)
    L = model.layer[0]
    outs = []
    for e6 in (False, True):
        model.use_e2m3 = e6
        model.run_layer(L, m)
        torch.cuda.synchronize()
        outs.append([t.clone() for t in (model.y_qkv, model.h, model.y_dn)])
    for name, a, b in zip(("q|k|v", "h", "down"), outs[0], outs[1]):
        assert torch.equal(a.view(torch.int16), b.view(torch.int16)), f"{name} differs between storages"
    del model
    torch.cuda.empty_cache()


@pytest.mark.parametrize("m", [6528, 52224])
def test_backbone_sweep_layer_large_m(m):
    """One layer of the 18-layer backbone sweep at M = 6528 and 52224: q (W4A4
    2048x2048), o (W8A8 2048x2048) and the fused gate|up GeGLU GEMM (W4A4
    32768x2048 interleaved) -> int8 h -> down (W8A8 2048x16384); b = 128,
    bf16; sampled rows, stage by stage."""
    wl = synth.CFG5
    projs = {p.name: p for p in wl.projs}
    rows = _sample_rows(m, 8)
    rd = torch.as_tensor(rows, device=DEV)
    for name in ("q", "o"):
        p = projs[name]
        say(f"sweep M={m} {name}")
        x = synth.activation(wl, p, m, tag="/L0")
        w = synth.weight(wl, p, tag="/L0")
        s = oracle.calibrate_fold(synth.to_f64(x), synth.to_f64(w)).astype(np.float32)
        _check_linear(x, w, torch.from_numpy(s), 128, 4 if p.scheme == "w4a4" else 8, "bf16", rows=rows)
    gu, dn = projs["gate_up"], projs["down"]
    f = dn.k
    say(f"sweep M={m} gate|up GeGLU")
    x = synth.activation(wl, gu, m, tag="/L0")
    w_gu = synth.weight(wl, gu, tag="/L0")
    w_int = q.interleave_gate_up(w_gu[:f], w_gu[f:])
    xd, wd = x.to(DEV), w_int.to(DEV)
    s1, inv1 = q.qlin_calibrate_fold(xd, wd)
    wq1, ws1 = q.qlin_quantize_weights(wd, fold_s=s1, had_block=128, bits=4)
    xq1, xs1 = q.qlin_rotate_quant_act(xd, fold_inv_s=inv1, had_block=128, bits=4)
    h = q.qlin_gemm_w4a4_geglu(xq1, xs1, wq1, ws1, gu.k, h_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    _, _, h_ref = oracle.gemm_geglu(codes_np(xq1[rd], 4), xs1[rd].cpu().numpy(), codes_np(wq1, 4),
                                    ws1.cpu().numpy(), "bf16")
    assert_ok(oracle.compare_outputs(f64(h[rd]), h_ref), "h")
    say(f"sweep M={m} down")
    w_dn = synth.weight(wl, dn, tag="/L0")
    wdd = w_dn.to(DEV)
    s2, inv2 = q.qlin_calibrate_fold(h, wdd)
    wq2, ws2 = q.qlin_quantize_weights(wdd, fold_s=s2, had_block=128, bits=8)
    hq, hs = q.qlin_rotate_quant_act(h, fold_inv_s=inv2, had_block=128, bits=8)
    y = q.qlin_gemm_w8a8(hq, hs, wq2, ws2, f, y_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    hf = f64(h[rd])
    qh, sh, rh = oracle.rotate_quant_act(hf, s2.cpu().numpy(), 128, 8)
    hq_r = codes_np(hq[rd], 8)
    assert_ok(oracle.compare_codes(hq_r, qh, rh), "h codes")
    assert_ok(oracle.compare_scales(hs[rd].cpu().numpy(), sh), "h scales")
    _, _, y_ref = oracle.gemm(hq_r, hs[rd].cpu().numpy(), codes_np(wq2, 8), ws2.cpu().numpy(), "bf16")
    assert_ok(oracle.compare_outputs(f64(y[rd]), y_ref), "down output")
