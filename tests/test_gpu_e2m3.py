"""Parity of the E2M3 storage path (GPU only).

W4A4 codes stored as FP6 E2M3 fields run on the FP6 matrix cores.  The codes
are the int4 grid's and the products exact, so:
  - GEMM raw accumulators equal the oracle's integer GEMM bit for bit, and
    dequantized outputs equal the packed-int4 GEMM's outputs bit for bit on
    the same codes (and the oracle's within the output tolerance);
  - the quantizers' E2M3 codes decode to exactly the codes of their packed
    int4 output on the same input (same rounding), and match the oracle up to
    rounding-boundary flips, with identical scales.
Inputs: seeded synthetic codes in -7 .. 7 stored by the oracle's pack_e2m3 and
pack_int4; seeded normals for the quantizers.

Method: FoldQuantVLA abstract (W4A4 integer execution of the projections).
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
SEED = 4321
E = q.QLIN_BITS_E2M3


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def f64(t: torch.Tensor) -> np.ndarray:
    return t.detach().cpu().to(torch.float64).numpy()


def assert_ok(res, what):
    assert res.ok, f"{what}: {res.detail}"


def sample_rows(m, count, seed=7):
    rng = np.random.default_rng(seed)
    rows = set(rng.choice(m, size=min(count, m), replace=False).tolist())
    rows.update({0, m - 1})
    return np.array(sorted(rows))


def operands(tag, m, n, k):
    """Grid codes a [m][k], b [n][k] (int64) and their E2M3 and packed int4
    device storage."""
    a = synth.random_grid_codes(SEED, f"A{tag}/{m}/{k}", m, k).astype(np.int64)
    b = synth.random_grid_codes(SEED, f"B{tag}/{n}/{k}", n, k).astype(np.int64)
    a6 = torch.from_numpy(oracle.pack_e2m3(a)).to(DEV)
    b6 = torch.from_numpy(oracle.pack_e2m3(b)).to(DEV)
    a4 = torch.from_numpy(oracle.pack_int4(a)).to(DEV)
    b4 = torch.from_numpy(oracle.pack_int4(b)).to(DEV)
    return a, b, a6, b6, a4, b4


# ---------------------------------------------------------------- GEMM

E2M3_SHAPES = [
    # 128 x 128 tiles (grids below one 256 x 256 tile per CU)
    (16, 512, 512),      # single linear
    (1, 96, 128),        # one token, one k-stage (padded to two)
    (50, 1024, 4096),    # action-expert shape
    (300, 520, 1024),    # ragged M and N tiles
    (17, 99, 2048),      # odd n
    (65, 256, 16384),    # long k
    (129, 200, 384),     # three k-stages (one zero-filled pad stage)
    (1000, 1800, 4096),
]


@pytest.mark.parametrize("m,n,k", E2M3_SHAPES)
def test_gemm_e2m3_raw_accumulators_bit_exact(m, n, k):
    say(f"e2m3 gemm i32 {m}x{n}x{k}")
    a, b, a6, b6, _, _ = operands("r", m, n, k)
    acc = q.qlin_gemm_e2m3(a6, None, b6, None, k, y_dtype=torch.int32)
    torch.cuda.synchronize()
    ref = oracle.int_gemm(a, b)
    got = acc.cpu().numpy().astype(np.int64)
    assert np.array_equal(got, ref), f"{np.count_nonzero(got != ref)} accumulators differ"


# at least one 256 x 256 tile per CU: the one-block-per-CU launch, tiles in
# groups of 4 tile rows (ragged last group and edges); sampled rows
E2M3_BIG = [
    (4100, 4000, 512),   # 17 x 16 tiles
    (4352, 4096, 384),   # three k-stages, padded to four
    (6528, 2560, 1024),  # the last tile row half empty
    (4096, 4352, 128),   # one k-stage, padded to two
    (8100, 8000, 256),   # 32 x 32 tiles, ragged M and N edges
]


@pytest.mark.parametrize("m,n,k", E2M3_BIG)
def test_gemm_e2m3_big_grid_sampled_rows(m, n, k):
    say(f"e2m3 gemm i32 big grid {m}x{n}x{k}")
    a, b, a6, b6, _, _ = operands("big", m, n, k)
    acc = q.qlin_gemm_e2m3(a6, None, b6, None, k, y_dtype=torch.int32)
    torch.cuda.synchronize()
    rows = sample_rows(m, 24)
    ref = oracle.int_gemm(a[rows], b)
    got = acc.cpu().numpy().astype(np.int64)[rows]
    assert np.array_equal(got, ref), f"{np.count_nonzero(got != ref)} accumulators differ"


@pytest.mark.parametrize("m", [3, 300])
def test_gemm_e2m3_extreme_codes_at_max_k(m):
    """|acc| = 49 k at the largest k (all codes +-7): 6.4e6 < 2^24, exact."""
    k, n = 131072 - 128, 64
    say(f"e2m3 gemm extreme codes m={m} k={k}")
    a = np.full((m, k), 7, dtype=np.int64)
    a[1::2] = -7
    b = np.full((n, k), 7, dtype=np.int64)
    b[1:, 1::3] = -7     # row 0 stays all +7: acc[0][0] = 49 k
    acc = q.qlin_gemm_e2m3(torch.from_numpy(oracle.pack_e2m3(a)).to(DEV), None,
                           torch.from_numpy(oracle.pack_e2m3(b)).to(DEV), None, k, y_dtype=torch.int32)
    torch.cuda.synchronize()
    ref = oracle.int_gemm(a, b)
    assert np.array_equal(acc.cpu().numpy().astype(np.int64), ref)
    assert np.max(np.abs(ref)) == 49 * k


@pytest.mark.parametrize("out", ["bf16", "f16", "f32"])
@pytest.mark.parametrize("m,n,k", [(300, 520, 1024), (16, 512, 512), (4100, 4000, 512)])
def test_gemm_e2m3_epilogue_equals_int4_path(m, n, k, out):
    say(f"e2m3 gemm {out} {m}x{n}x{k}")
    dt = {"bf16": torch.bfloat16, "f16": torch.float16, "f32": torch.float32}[out]
    a, b, a6, b6, a4, b4 = operands("e", m, n, k)
    sx = synth.random_scales(SEED, f"sx/{m}", m).to(DEV)
    sw = synth.random_scales(SEED, f"sw/{n}", n).to(DEV)
    y6 = q.qlin_gemm_e2m3(a6, sx, b6, sw, k, y_dtype=dt)
    y4 = q.qlin_gemm_w4a4(a4, sx, b4, sw, k, y_dtype=dt)
    torch.cuda.synchronize()
    bits = torch.int32 if out == "f32" else torch.int16
    assert torch.equal(y6.view(bits), y4.view(bits)), "E2M3 and packed-int4 outputs differ"
    rows = sample_rows(m, 16)
    _, _, y_ref = oracle.gemm(a[rows], sx.cpu().numpy()[rows], b, sw.cpu().numpy(), out)
    assert_ok(oracle.compare_outputs(f64(y6)[rows], y_ref), "output")


def test_gemm_e2m3_static_scratch_entry_point():
    m, n, k = 300, 520, 1024
    say("e2m3 gemm through qlin_gemm_static_ws")
    _, _, a6, b6, _, _ = operands("s", m, n, k)
    sx = synth.random_scales(SEED, f"sxs/{m}", m).to(DEV)
    sw = synth.random_scales(SEED, f"sws/{n}", n).to(DEV)
    y1 = q.qlin_gemm_e2m3(a6, sx, b6, sw, k)
    y2 = q.qlin_gemm_static_ws(q.QLIN_W4A4_E2M3, a6, sx, b6, sw, k)
    torch.cuda.synchronize()
    assert torch.equal(y1.view(torch.int16), y2.view(torch.int16))


@pytest.mark.parametrize("out", ["bf16", "f16", "f32"])
@pytest.mark.parametrize("m,f,k", [(50, 64, 256), (130, 2048, 512), (1, 32, 128), (300, 4096, 1024),
                                   (4100, 2048, 512), (2050, 8192, 256), (4100, 2080, 384)])
def test_gemm_geglu_e2m3_equals_int4_path(m, f, k, out):
    # the last three grids fill the chip: 128 x 256 tiles, two blocks per CU
    # (4100 x 4160: ragged last tile row and column; 3 k-stages padded to 4)
    say(f"e2m3 gemm geglu {out} {m}x{f}x{k}")
    dt = {"bf16": torch.bfloat16, "f16": torch.float16, "f32": torch.float32}[out]
    n2 = 2 * f
    a, b, a6, b6, a4, b4 = operands("g", m, n2, k)
    sx = synth.random_scales(SEED, f"sxg/{m}", m).to(DEV)
    sw = synth.random_scales(SEED, f"swg/{n2}", n2).to(DEV)
    h6 = q.qlin_gemm_geglu(q.QLIN_W4A4_E2M3, a6, sx, b6, sw, k, h_dtype=dt)
    h4 = q.qlin_gemm_w4a4_geglu(a4, sx, b4, sw, k, h_dtype=dt)
    torch.cuda.synchronize()
    assert h6.shape == (m, f)
    bits = torch.int32 if out == "f32" else torch.int16
    assert torch.equal(h6.view(bits), h4.view(bits)), "E2M3 and packed-int4 GeGLU outputs differ"
    rows = sample_rows(m, 12)
    _, _, h_ref = oracle.gemm_geglu(a[rows], sx.cpu().numpy()[rows], b, sw.cpu().numpy(), out)
    assert_ok(oracle.compare_outputs(f64(h6)[rows], h_ref), "h")


# ---------------------------------------------------------------- quantizers


def decode6(t: torch.Tensor) -> np.ndarray:
    return oracle.unpack_e2m3(t.cpu().numpy())


ACT_CASES = [
    # m, k, b, dtype, pre
    (37, 2048, 128, "bf16", q.QLIN_PRE_NONE),    # bfloat16 fast path, ragged m
    (4, 16384, 128, "bf16", q.QLIN_PRE_NONE),    # fast path, four chunks per lane
    (16, 512, 64, "f16", q.QLIN_PRE_NONE),       # row kernel
    (9, 1024, 0, "f32", q.QLIN_PRE_NONE),        # no rotation
    (300, 256, 128, "bf16", q.QLIN_PRE_NONE),    # several rows per block
    (3, 32768, 128, "bf16", q.QLIN_PRE_NONE),    # longest rows
    (9, 2048, 128, "bf16", q.QLIN_PRE_GEGLU),    # GeGLU pre-op (the down projection's input form)
    (6, 512, 64, "f16", q.QLIN_PRE_GEGLU),
]


@pytest.mark.parametrize("m,k,b,dtype,pre", ACT_CASES)
def test_rotate_quant_act_e2m3(m, k, b, dtype, pre):
    say(f"e2m3 act m={m} k={k} b={b} {dtype} pre={pre}")
    width = 2 * k if pre == q.QLIN_PRE_GEGLU else k
    x = synth.normal_tensor(SEED, f"act6/{m}/{k}/{pre}", (m, width), dtype=dtype, outliers=max(1, k // 100),
                            outlier_scale=25.0)
    x[m // 2] = 0
    s = synth.random_scales(SEED, f"fold6/{k}", k) * 100.0
    xd, inv = x.to(DEV), (1.0 / s).to(DEV)
    xq6, xs6 = q.qlin_rotate_quant_act(xd, k=k, fold_inv_s=inv, had_block=b, bits=E, pre=pre)
    xq4, xs4 = q.qlin_rotate_quant_act(xd, k=k, fold_inv_s=inv, had_block=b, bits=4, pre=pre)
    torch.cuda.synchronize()
    assert xq6.shape == (m, k * 3 // 4)
    c6 = decode6(xq6)
    assert np.array_equal(c6, oracle.unpack_int4(xq4.cpu().numpy())), "E2M3 codes differ from the int4 codes"
    assert torch.equal(xs6, xs4)
    q_ref, s_ref, r_ref = oracle.rotate_quant_act(synth.to_f64(x), s.numpy(), b, 4,
                                                  preop="geglu" if pre == q.QLIN_PRE_GEGLU else "none")
    assert_ok(oracle.compare_scales(xs6.cpu().numpy(), s_ref), "scales")
    assert_ok(oracle.compare_codes(c6, q_ref, r_ref), "codes")
    assert np.all(c6[m // 2] == 0)


@pytest.mark.parametrize("n,k,b,dtype", [(96, 1024, 64, "f16"), (256, 2048, 128, "bf16"), (40, 512, 0, "f32")])
def test_quantize_weights_e2m3(n, k, b, dtype):
    say(f"e2m3 weights n={n} k={k} b={b} {dtype}")
    w = synth.normal_tensor(SEED, f"w6/{n}/{k}", (n, k), std=0.02, dtype=dtype)
    s = synth.random_scales(SEED, f"wfold6/{k}", k) * 10.0
    wd, sd = w.to(DEV), s.to(DEV)
    wq6, ws6 = q.qlin_quantize_weights(wd, fold_s=sd, had_block=b, bits=E)
    wq4, ws4 = q.qlin_quantize_weights(wd, fold_s=sd, had_block=b, bits=4)
    torch.cuda.synchronize()
    c6 = decode6(wq6)
    assert np.array_equal(c6, oracle.unpack_int4(wq4.cpu().numpy()))
    assert torch.equal(ws6, ws4)
    q_ref, s_ref, r_ref = oracle.quantize_weights(synth.to_f64(w), s.numpy(), b, 4)
    assert_ok(oracle.compare_scales(ws6.cpu().numpy(), s_ref), "scales")
    assert_ok(oracle.compare_codes(c6, q_ref, r_ref), "codes")


def test_static_and_composite_quantizers_e2m3():
    m, k, b = 50, 1024, 64
    say("e2m3 static-table and composite quantizers")
    xc = synth.normal_tensor(SEED, "t6cal", (m, k), dtype="f16")
    xe = synth.normal_tensor(SEED, "t6eval", (m, k), dtype="f16")
    xcd, xed = xc.to(DEV), xe.to(DEV)
    table = q.qlin_calibrate_step_scales(xcd, had_block=b, bits=E)
    t4 = q.qlin_calibrate_step_scales(xcd, had_block=b, bits=4)
    xq6 = q.qlin_rotate_quant_act_static(xed, table, had_block=b, bits=E)
    xq4 = q.qlin_rotate_quant_act_static(xed, table, had_block=b, bits=4)
    w = synth.normal_tensor(SEED, "c6w", (96, k), std=0.02, dtype="f16").to(DEV)
    perm, rot = q.qlin_calibrate_composite(w, b)
    cq6, cs6 = q.qlin_rotate_quant_act_composite(xed, perm, rot, bits=E)
    cq4, cs4 = q.qlin_rotate_quant_act_composite(xed, perm, rot, bits=4)
    wq6, ws6 = q.qlin_quantize_weights_composite(w, perm, rot, bits=E)
    wq4, ws4 = q.qlin_quantize_weights_composite(w, perm, rot, bits=4)
    sq6, ss6 = q.qlin_quantize_weights_step(w, table, had_block=b, bits=E)
    sq4, ss4 = q.qlin_quantize_weights_step(w, table, had_block=b, bits=4)
    torch.cuda.synchronize()
    assert torch.equal(table, t4), "the table's qmax is the int4 grid's"
    for got, ref in ((xq6, xq4), (cq6, cq4), (wq6, wq4), (sq6, sq4)):
        assert np.array_equal(decode6(got), oracle.unpack_int4(ref.cpu().numpy()))
    for got, ref in ((cs6, cs4), (ws6, ws4), (ss6, ss4)):
        assert torch.equal(got, ref)


def test_w4a4_linear_e2m3_end_to_end_equals_int4():
    """x -> fold + Hadamard + per-token codes -> GEMM: the E2M3 and packed
    int4 paths give the same output bits (single-linear workload, 16 x 512 x 512)."""
    say("e2m3 linear end to end")
    wl = synth.CFG1
    p = wl.projs[0]
    x = synth.activation(wl, p, 16).to(DEV)
    w = synth.weight(wl, p).to(DEV)
    s, inv = q.qlin_calibrate_fold(x, w)
    outs = []
    for bits, scheme in ((4, q.QLIN_W4A4), (E, q.QLIN_W4A4_E2M3)):
        wq, ws = q.qlin_quantize_weights(w, fold_s=s, had_block=64, bits=bits)
        xq, xs = q.qlin_rotate_quant_act(x, fold_inv_s=inv, had_block=64, bits=bits)
        if scheme == q.QLIN_W4A4:
            outs.append(q.qlin_gemm_w4a4(xq, xs, wq, ws, p.k, y_dtype=torch.float16))
        else:
            outs.append(q.qlin_gemm_e2m3(xq, xs, wq, ws, p.k, y_dtype=torch.float16))
    torch.cuda.synchronize()
    assert torch.equal(outs[0].view(torch.int16), outs[1].view(torch.int16))
