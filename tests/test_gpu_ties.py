"""Exact rounding ties and the hand-worked vectors through the HIP path (GPU only).

Random normal inputs almost never land on a rounding boundary, so the
stage-wise parity tests cannot tell round-half-to-even from other tie rules.
Here every input is built so that the value to be rounded is exactly a
half-integer (a code) or exactly halfway between two representable outputs
(fp16 / bf16), and the HIP result must equal the oracle's with no flip
allowed.  The expected values are also checked against Python's own
round-half-even (``round``) or torch's float casts, which share nothing with
the oracle.

Method: FoldQuantVLA abstract (channel scaling, block Hadamard, dynamic
per-token symmetric quantization, integer GEMM with a dequantizing epilogue);
LoopQ abstract (plain round-to-nearest weights, batch-1 weight-only W4A16);
the hand-worked vectors are tests/golden/hand_worked.json.

Construction of tied activations: a row of target values v whose entries are
half-integers j + 1/2 (|v| < qmax) plus one entry at +-qmax, so that the
per-token scale is exactly 1 and v / scale is exactly a tie; the input is
x = v @ blockdiag(H_b / sqrt(b)) for b in {1, 4, 16, 64, 256}, where
1/sqrt(b) is a power of two and x is exact in the input dtype (checked), so
the rotation returns v exactly.
"""

import json
import os
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
GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "hand_worked.json")
TDT = {"f16": torch.float16, "bf16": torch.bfloat16, "f32": torch.float32}


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def golden():
    with open(GOLDEN) as f:
        return json.load(f)


def codes_np(t: torch.Tensor, bits: int) -> np.ndarray:
    a = t.cpu().numpy()
    return oracle.unpack_int4(a) if bits == 4 else a.astype(np.int64)


def py_rne(r: float) -> int:
    """Round half to even with Python's built-in round (independent of NumPy)."""
    return int(round(float(r)))


def exact_tensor(a: np.ndarray, dtype: str) -> torch.Tensor:
    """float64 values -> a tensor of the storage dtype, asserting that the
    cast is exact."""
    t = torch.from_numpy(np.ascontiguousarray(a)).to(TDT[dtype])
    assert np.array_equal(t.to(torch.float64).numpy(), a), f"values are not exact in {dtype}"
    return t


# ---------------------------------------------------------------- hand-worked vectors


def test_golden_act_b4_int4():
    """act_b4_int4: k = 8, b = 4, int4; row 0 without a fold, row 1 with the
    fold vector [2,2,2,2,1,1,1,1] (the kernel multiplies by 1/s), row 2 zero."""
    g = golden()["act_b4_int4"]
    x = exact_tensor(np.array(g["x"], dtype=np.float64), "f32")
    codes = np.array(g["codes"], dtype=np.int64)
    scale = np.array(g["scale"], dtype=np.float32)
    packed = np.array(g["packed"], dtype=np.uint8)
    inv_s = torch.tensor([1.0 / v for v in g["fold_s"]], dtype=torch.float32, device=DEV)
    for dtype in ("f32", "f16", "bf16"):
        xd = x.to(TDT[dtype]).to(DEV)
        xq_plain, xs_plain = q.qlin_rotate_quant_act(xd, had_block=g["had_block"], bits=g["bits"])
        xq_fold, xs_fold = q.qlin_rotate_quant_act(xd, fold_inv_s=inv_s, had_block=g["had_block"], bits=g["bits"])
        torch.cuda.synchronize()
        for r in range(3):
            xq, xs = (xq_fold, xs_fold) if r in g["fold_rows"] else (xq_plain, xs_plain)
            assert np.array_equal(xq.cpu().numpy()[r], packed[r]), f"{dtype} row {r} packed bytes"
            assert np.array_equal(codes_np(xq, 4)[r], codes[r]), f"{dtype} row {r} codes"
            assert np.float32(xs.cpu().numpy()[r]) == scale[r], f"{dtype} row {r} scale"


def test_golden_act_ties_int8():
    """act_ties_int8: b = 1, amax 127 (scale 1), values +-0.5, +-1.5, +-2.5, 3.5."""
    g = golden()["act_ties_int8"]
    x = np.array(g["x"], dtype=np.float64)
    want = np.array(g["codes"], dtype=np.int64)
    assert [py_rne(v) for v in x[0]] == list(want[0])
    for dtype in ("f32", "f16", "bf16"):
        xq, xs = q.qlin_rotate_quant_act(exact_tensor(x, dtype).to(DEV), had_block=g["had_block"], bits=g["bits"])
        torch.cuda.synchronize()
        assert np.array_equal(codes_np(xq, 8), want), dtype
        assert np.array_equal(xs.cpu().numpy(), np.array(g["scale"], dtype=np.float32)), dtype


def test_golden_w4a16_group_rebuilt_in_group128():
    """w4a16_group4's groups rebuilt inside 128-wide groups: the first group
    holds 0.5, -0.25, 0.125 and zeros (s16 = fp16(0.5/7), codes 7, -4, 2);
    the second is all zero (s16 0, codes 0); the third holds -1 (code -7)."""
    g = golden()["w4a16_group4"]
    w = np.zeros((1, 384), dtype=np.float64)
    w[0, :3] = [0.5, -0.25, 0.125]
    w[0, 256] = -1.0
    wq, ws = q.qlin_quantize_weights(exact_tensor(w, "f16").to(DEV), bits=4, group=128)
    torch.cuda.synchronize()
    codes = codes_np(wq, 4)[0]
    want = np.zeros(384, dtype=np.int64)
    want[:3] = g["codes"][0][:3]
    want[256] = g["codes"][0][8]
    assert np.array_equal(codes, want)
    s16 = ws.cpu().to(torch.float64).numpy()[0]
    assert list(s16) == g["s16"][0]


@pytest.mark.parametrize("m", [2, 130])
@pytest.mark.parametrize("scheme", ["w4a4", "w8a8", "w4a8"])
def test_golden_gemm_2x2x4_zero_padded(scheme, m):
    """gemm_2x2x4 with k zero-padded to a legal length (64 for W8A8, 128 with
    int4 operands); m = 2 runs the small-M kernel, m = 130 (rows repeated)
    the large-tile GEMM.  The -8 activation code is kept (int4 nibble 0x8)."""
    g = golden()["gemm_2x2x4"]
    abits, wbits = {"w4a4": (4, 4), "w8a8": (8, 8), "w4a8": (8, 4)}[scheme]
    k = 64 if scheme == "w8a8" else 128
    qx = np.zeros((m, k), dtype=np.int64)
    qx[:, :4] = np.array(g["qx"])[np.arange(m) % 2]
    qw = np.zeros((2, k), dtype=np.int64)
    qw[:, :4] = g["qw"]
    sx = np.array(g["x_scale"], dtype=np.float32)[np.arange(m) % 2]
    sw = np.array(g["w_scale"], dtype=np.float32)

    def dev_codes(c, bits):
        if bits == 8:
            return torch.from_numpy(c.astype(np.int8)).to(DEV)
        return torch.from_numpy(oracle.pack_int4(c)).to(DEV)

    fn = getattr(q, f"qlin_gemm_{scheme}")
    a, b = dev_codes(qx, abits), dev_codes(qw, wbits)
    acc = fn(a, None, b, None, k, y_dtype=torch.int32)
    outs = {dt: fn(a, torch.from_numpy(sx).to(DEV), b, torch.from_numpy(sw).to(DEV), k, y_dtype=TDT[dt])
            for dt in ("f16", "bf16", "f32")}
    torch.cuda.synchronize()
    rows = np.arange(m) % 2
    assert np.array_equal(acc.cpu().numpy(), np.array(g["acc"])[rows])
    for dt, y in outs.items():
        assert np.array_equal(y.cpu().to(torch.float64).numpy(), np.array(g["y"])[rows]), dt


# ---------------------------------------------------------------- activation ties


def tied_rows(rng, m, k, bits, b, per_block=None):
    """(x float64 [m][k], v float64 [m][k]): v rows of half-integer ties with
    one +-qmax entry each; x = v @ blockdiag(H_b / sqrt(b)).  per_block keeps
    only that many nonzero entries in each Hadamard block (fewer terms per
    rotated value keep x exact in bfloat16)."""
    qmax = 7 if bits == 4 else 127
    j = rng.integers(-qmax, qmax, size=(m, k))            # j + 0.5 in (-qmax, qmax)
    v = j.astype(np.float64) + 0.5
    if per_block is not None:
        blk = max(b, 1)
        keep = np.zeros((m, k), dtype=bool)
        for r in range(m):
            for c0 in range(0, k, blk):
                keep[r, c0 + rng.choice(blk, size=per_block, replace=False)] = True
        v *= keep
        pos = np.array([rng.choice(np.flatnonzero(keep[r])) for r in range(m)])
    else:
        pos = rng.integers(0, k, size=m)
    v[np.arange(m), pos] = qmax * np.where(rng.random(m) < 0.5, -1.0, 1.0)
    x = oracle.rotate_blocks(v, b) if b > 1 else v.copy()   # H / sqrt(b) is symmetric and its own inverse
    assert np.array_equal(oracle.rotate_blocks(x, b) if b > 1 else x, v), "rotation not exact"
    return x, v


ACT_TIE_CASES = [
    # m, k, b, bits, dtype, nonzeros per Hadamard block (None: all), fold (powers of two)
    (64, 2048, 1, 4, "bf16", None, False),
    (64, 4096, 1, 8, "f16", None, False),
    (40, 2048, 64, 4, "f32", None, False),    # general row kernel
    (40, 2048, 64, 8, "f32", None, True),
    (33, 2048, 64, 4, "bf16", 8, False),      # bfloat16 fast kernel (Hadamard 64); sparse keeps x exact
    (33, 4096, 64, 8, "bf16", 1, False),
    (24, 1024, 4, 4, "bf16", None, False),
    (24, 1024, 16, 8, "f32", None, True),
    (9, 4096, 256, 8, "f32", None, False),
    (3, 16384, 64, 8, "f32", None, False),    # down-projection input width
    (5, 32768, 256, 4, "f32", None, True),    # longest rows
]


@pytest.mark.parametrize("m,k,b,bits,dtype,per_block,fold", ACT_TIE_CASES)
def test_rotate_quant_act_exact_ties(m, k, b, bits, dtype, per_block, fold):
    say(f"ties act m={m} k={k} b={b} bits={bits} {dtype} fold={fold}")
    rng = synth.rng_for(SEED, f"tie/{m}/{k}/{b}/{bits}/{dtype}")
    x, v = tied_rows(rng, m, k, bits, b, per_block)
    inv_s = None
    s_np = None
    if fold:
        s_np = np.exp2(rng.integers(-2, 3, size=k)).astype(np.float32)
        x = x * s_np.astype(np.float64)                       # the kernel multiplies by 1/s
        inv_s = torch.from_numpy((1.0 / s_np).astype(np.float32)).to(DEV)
    xt = exact_tensor(x, dtype)
    xq, xs = q.qlin_rotate_quant_act(xt.to(DEV), fold_inv_s=inv_s, had_block=b, bits=bits)
    torch.cuda.synchronize()
    q_ref, s_ref, r_ref = oracle.rotate_quant_act(xt.to(torch.float64).numpy(), s_np, b, bits)
    assert np.all(s_ref == 1.0) and np.array_equal(r_ref, v)
    want = np.vectorize(py_rne)(v)
    assert np.array_equal(q_ref, want)
    assert np.array_equal(xs.cpu().numpy(), np.ones(m, dtype=np.float32))
    res = oracle.compare_codes(codes_np(xq, bits), q_ref, r_ref, max_frac=0.0)
    assert res.ok, res.detail


@pytest.mark.parametrize("bits,b", [(4, 64), (8, 16), (8, 1)])
def test_quantize_weights_exact_ties(bits, b):
    """Per-output-channel RTN of the weights on exact ties (fold by powers of two)."""
    say(f"ties weights bits={bits} b={b}")
    n, k = 96, 2048
    rng = synth.rng_for(SEED, f"tiew/{bits}/{b}")
    w, v = tied_rows(rng, n, k, bits, b)
    s_np = np.exp2(rng.integers(-2, 3, size=k)).astype(np.float32)
    w = w / s_np.astype(np.float64)                           # the weight path multiplies by s
    wt = exact_tensor(w, "f32")
    wq, ws = q.qlin_quantize_weights(wt.to(DEV), fold_s=torch.from_numpy(s_np).to(DEV), had_block=b, bits=bits)
    torch.cuda.synchronize()
    q_ref, s_ref, r_ref = oracle.quantize_weights(wt.to(torch.float64).numpy(), s_np, b, bits)
    assert np.all(s_ref == 1.0) and np.array_equal(r_ref, v)
    assert np.array_equal(q_ref, np.vectorize(py_rne)(v))
    assert np.array_equal(ws.cpu().numpy(), np.ones(n, dtype=np.float32))
    res = oracle.compare_codes(codes_np(wq, bits), q_ref, r_ref, max_frac=0.0)
    assert res.ok, res.detail


def test_quantize_weights_group128_exact_ties():
    """W4A16 group quantization: each 128-group has max |w| = 7 * 2^e, so
    s16 = 2^e exactly and w / s16 = j + 1/2 is a tie; one group is all zero."""
    say("ties w4a16 groups")
    n, k = 40, 1024
    rng = synth.rng_for(SEED, "tieg")
    e = rng.integers(-8, 2, size=(n, k // 128)).astype(np.float64)
    j = rng.integers(-7, 7, size=(n, k)) + 0.5
    pos = rng.integers(0, 128, size=(n, k // 128))
    for gi in range(k // 128):
        j[np.arange(n), gi * 128 + pos[:, gi]] = 7.0 * np.where(rng.random(n) < 0.5, -1, 1)
    w = j * np.repeat(np.exp2(e), 128, axis=1)
    w[3, 256:384] = 0.0
    wt = exact_tensor(w, "f16")
    wq, ws = q.qlin_quantize_weights(wt.to(DEV), bits=4, group=128)
    torch.cuda.synchronize()
    q_ref, s_ref, r_ref = oracle.quantize_weights(wt.to(torch.float64).numpy(), None, 0, 4, group=128)
    want = np.vectorize(py_rne)(np.where(w == 0, 0.0, j))
    assert np.array_equal(q_ref, want)
    assert np.array_equal(codes_np(wq, 4), q_ref)
    assert np.array_equal(ws.cpu().numpy().view(np.uint16), np.asarray(s_ref, dtype=np.float16).view(np.uint16))


@pytest.mark.parametrize("bits", [4, 8])
def test_static_table_codes_exact_ties(bits):
    """Per-step static table codes: table entries powers of two, v / table[c]
    exactly a half-integer."""
    say(f"ties static table bits={bits}")
    m, k, b = 50, 1024, 64
    rng = synth.rng_for(SEED, f"ties/static/{bits}")
    qmax = 7 if bits == 4 else 127
    table = np.exp2(rng.integers(-3, 3, size=k)).astype(np.float32)
    t = rng.integers(-qmax, qmax, size=(m, k)) + 0.5
    v = t * table.astype(np.float64)
    x = oracle.rotate_blocks(v, b)
    xt = exact_tensor(x, "f32")
    xq = q.qlin_rotate_quant_act_static(xt.to(DEV), torch.from_numpy(table).to(DEV), had_block=b, bits=bits)
    torch.cuda.synchronize()
    q_ref, r_ref = oracle.rotate_quant_act_static(xt.to(torch.float64).numpy(), None, b, bits, table)
    assert np.array_equal(r_ref, t)
    assert np.array_equal(q_ref, np.vectorize(py_rne)(t))
    res = oracle.compare_codes(codes_np(xq, bits), q_ref, r_ref, max_frac=0.0)
    assert res.ok, res.detail


@pytest.mark.parametrize("bits", [4, 8])
def test_composite_codes_exact_ties(bits):
    """Composite-rotation quantizer with a caller-given permutation and
    rotation blocks H_64 / 8: the gathered, rotated rows are exact ties."""
    say(f"ties composite bits={bits}")
    m, k, b = 24, 1024, 64
    rng = synth.rng_for(SEED, f"ties/comp/{bits}")
    perm = rng.permutation(k)
    x_perm, v = tied_rows(rng, m, k, bits, b)
    x = np.empty_like(x_perm)
    x[:, perm] = x_perm                                    # x[:, perm] == x_perm
    rot = np.stack([oracle.sylvester_hadamard(b) / 8.0] * (k // b)).astype(np.float32)
    xt = exact_tensor(x, "f32")
    xq, xs = q.qlin_rotate_quant_act_composite(xt.to(DEV), torch.from_numpy(perm.astype(np.int32)).to(DEV),
                                               torch.from_numpy(rot).to(DEV), bits=bits)
    torch.cuda.synchronize()
    q_ref, s_ref, r_ref = oracle.rotate_quant_act_composite(xt.to(torch.float64).numpy(), None, perm,
                                                            rot.astype(np.float64), bits)
    assert np.all(s_ref == 1.0) and np.array_equal(r_ref, v)
    assert np.array_equal(q_ref, np.vectorize(py_rne)(v))
    res = oracle.compare_codes(codes_np(xq, bits), q_ref, r_ref, max_frac=0.0)
    assert res.ok, res.detail


# ---------------------------------------------------------------- output-rounding ties


def tie_targets(rng, shape, dtype):
    """Integers that sit exactly halfway between two neighbouring values of
    the output dtype (fp16: odd integers in [2049, 4095]; bf16: odd integers
    in [257, 511]), mixed with non-tied integers, random signs."""
    lo, hi = (2049, 4096) if dtype == "f16" else (257, 512)
    t = rng.integers(lo, hi, size=shape)
    tie = rng.random(shape) < 0.75
    t = np.where(tie, t | 1, t & ~1)
    return t * np.where(rng.random(shape) < 0.5, -1, 1)


def codes_for_targets(targets, qa, qw, per):
    """Activation and weight codes whose products sum to each target:
    output n owns `per` k-columns where its weight row holds qw (all but the
    last) and 1 (the last); each activation row then spells its target in
    base qw.  Returns (A int64 [m][k], W int64 [n][k])."""
    m, n = targets.shape
    k = n * per
    A = np.zeros((m, k), dtype=np.int64)
    W = np.zeros((n, k), dtype=np.int64)
    for c in range(n):
        cols = np.arange(c * per, (c + 1) * per)
        W[c, cols[:-1]] = qw
        W[c, cols[-1]] = 1
        for r in range(m):
            rem = int(targets[r, c])
            for col in cols[:-1]:
                a = max(-qa, min(qa, int(rem / qw)))
                A[r, col] = a
                rem -= a * qw
            assert abs(rem) <= qa, "target out of reach"
            A[r, cols[-1]] = rem
    return A, W


@pytest.mark.parametrize("m", [40, 130])
@pytest.mark.parametrize("out", ["f16", "bf16"])
@pytest.mark.parametrize("scheme", ["w4a4", "w8a8", "w4a8"])
def test_gemm_output_rounding_ties(scheme, out, m):
    """Accumulators at exact fp16 / bf16 rounding ties, with power-of-two
    scales (the fp32 product is exact): the output must be the
    round-half-even value, which torch's cast of the same fp32 number gives."""
    say(f"ties gemm out {scheme} {out} m={m}")
    abits, wbits = {"w4a4": (4, 4), "w8a8": (8, 8), "w4a8": (8, 4)}[scheme]
    qa, qw = (7 if abits == 4 else 127), (7 if wbits == 4 else 127)
    # k-columns per output: enough base-qw digits to reach 4095 (fp16) / 511 (bf16)
    hi = 4095 if out == "f16" else 511
    per = 1 + -(-(hi - qa) // (qa * qw))
    n = 64
    k = -(-(n * per) // 128) * 128
    rng = synth.rng_for(SEED, f"ties/gemm/{scheme}/{out}/{m}")
    T = tie_targets(rng, (m, n), out)
    A, W = codes_for_targets(T, qa, qw, per)
    A = np.pad(A, ((0, 0), (0, k - A.shape[1])))
    W = np.pad(W, ((0, 0), (0, k - W.shape[1])))
    assert np.array_equal(oracle.int_gemm(A, W), T)
    ex = rng.integers(-2, 2, size=m)          # |y| <= 4095 * 4 stays inside the fp16 range
    ew = rng.integers(-2, 2, size=n)
    sx = np.exp2(ex).astype(np.float32)
    sw = np.exp2(ew).astype(np.float32)

    def dev_codes(c, bits):
        if bits == 8:
            return torch.from_numpy(c.astype(np.int8)).to(DEV)
        return torch.from_numpy(oracle.pack_int4(c)).to(DEV)

    fn = getattr(q, f"qlin_gemm_{scheme}")
    y = fn(dev_codes(A, abits), torch.from_numpy(sx).to(DEV), dev_codes(W, wbits), torch.from_numpy(sw).to(DEV),
           k, y_dtype=TDT[out])
    torch.cuda.synchronize()
    _, y32, y_ref = oracle.gemm(A, sx, W, sw, out)
    want = torch.from_numpy(y32).to(TDT[out]).to(torch.float64).numpy()   # torch's RNE cast
    assert np.array_equal(y_ref, want)
    got = y.cpu().to(torch.float64).numpy()
    bad = np.argwhere(got != want)
    assert bad.size == 0, f"{len(bad)} outputs differ, first at {tuple(bad[0])}: {got[tuple(bad[0])]} vs {want[tuple(bad[0])]}"


@pytest.mark.parametrize("m", [1, 20])
def test_gemv_w4a16_output_rounding_ties(m):
    """W4A16: x = 1, group scales 1 (each group's max |w| is 7), row sums of
    codes at odd integers in (2048, 4096): fp16 ties, round-half-even."""
    say(f"ties gemv m={m}")
    n, k = 96, 1024
    rng = synth.rng_for(SEED, f"ties/gemv/{m}")
    T = tie_targets(rng, (n,), "f16")
    codes = np.zeros((n, k), dtype=np.int64)
    for r in range(n):
        rem = int(T[r])
        for g in range(k // 128):
            codes[r, g * 128] = 7                    # group scale fp16(7 / 7) = 1
            rem -= 7
        for c in range(k):
            if c % 128 == 0:
                continue
            a = max(-7, min(7, rem))
            codes[r, c] = a
            rem -= a
        assert rem == 0
    w = exact_tensor(codes.astype(np.float64), "f16")
    wq, ws = q.qlin_quantize_weights(w.to(DEV), bits=4, group=128)
    x = torch.ones((m, k), dtype=torch.float16, device=DEV)
    y = q.qlin_gemv_w4a16(x, wq, ws)
    torch.cuda.synchronize()
    assert np.array_equal(codes_np(wq, 4), codes)
    assert np.all(ws.cpu().to(torch.float64).numpy() == 1.0)
    y32, y_ref = oracle.gemv_w4a16(np.ones((m, k)), codes, ws.cpu().numpy(), 128)
    want = torch.from_numpy(np.tile(T.astype(np.float32), (m, 1))).to(torch.float16).to(torch.float64).numpy()
    assert np.array_equal(y_ref, want)
    assert np.array_equal(y.cpu().to(torch.float64).numpy(), want)
