"""Pins for the oracle's quantizers, packing, integer GEMM, epilogue, GEMV
and GeGLU (CPU only).

Quantization: FoldQuantVLA abstract (dynamic per-token symmetric activations,
W4A4/W8A8 native integer execution); LoopQ abstract (plain RTN weights,
weight-only 4-bit at batch 1).  Epilogue scalars: QuantVLA technical summary,
Methodology B and C (folded into the dequantization scale).
"""

import json
import math
import os

import numpy as np
import pytest
import torch

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "hand_worked.json")


def _g():
    with open(GOLDEN) as f:
        return json.load(f)


# ---------------------------------------------------------------- golden


def test_golden_act_b4_int4():
    g = _g()["act_b4_int4"]
    x = np.array(g["x"], dtype=np.float64)
    s = np.array(g["fold_s"], dtype=np.float32)
    for row in range(x.shape[0]):
        fold = s if row in g["fold_rows"] else None
        q, sc, _ = oracle.rotate_quant_act(x[row:row + 1], fold, g["had_block"], g["bits"])
        assert q[0].tolist() == g["codes"][row]
        assert float(sc[0]) == g["scale"][row]
        assert oracle.pack_int4(q)[0].tolist() == g["packed"][row]


def test_golden_act_ties_int8():
    g = _g()["act_ties_int8"]
    q, sc, _ = oracle.rotate_quant_act(np.array(g["x"]), None, g["had_block"], g["bits"])
    assert q.tolist() == g["codes"]
    assert sc.tolist() == g["scale"]


def test_golden_w4a16_group():
    g = _g()["w4a16_group4"]
    w = np.array(g["w"], dtype=np.float64)
    q, s16, _ = oracle.quantize_weights(w, None, 0, 4, group=g["group"])
    assert q.tolist() == g["codes"]
    assert s16.astype(np.float64).tolist() == g["s16"]


def test_golden_gemm():
    g = _g()["gemm_2x2x4"]
    acc, y32, yref = oracle.gemm(np.array(g["qx"]), np.array(g["x_scale"], np.float32),
                                 np.array(g["qw"]), np.array(g["w_scale"], np.float32), "f32")
    assert acc.tolist() == g["acc"]
    assert y32.astype(np.float64).tolist() == g["y"]


# ---------------------------------------------------------------- quantizer


@pytest.mark.parametrize("bits", [4, 8])
def test_on_grid_round_trip(bits):
    qmax = oracle.qmax_of(bits)
    rng = np.random.default_rng(10)
    q = rng.integers(-qmax, qmax + 1, size=(12, 40))
    q[np.arange(12), rng.integers(0, 40, 12)] = rng.choice([-qmax, qmax], 12)  # amax on grid
    sigma = (2.0 ** rng.integers(-8, 4, 12)) * rng.choice([1.0, 1.25, 0.75], 12)
    x = q * sigma[:, None]
    got_q, got_s, _ = oracle.quantize_rows(x, bits)
    assert np.array_equal(got_q, q)
    assert np.array_equal(got_s.astype(np.float64), sigma)


@pytest.mark.parametrize("bits", [4, 8])
def test_brute_force_nearest_code_8x8(bits):
    qmax = oracle.qmax_of(bits)
    rng = np.random.default_rng(11 + bits)
    x = rng.standard_normal((8, 8)) * rng.uniform(0.1, 10.0, (8, 1))
    q, s, _ = oracle.quantize_rows(x, bits)
    codes = np.arange(-qmax, qmax + 1)
    for m in range(8):
        amax = max(abs(x[m]))
        assert s[m] == np.float32(amax / qmax)
        sm = float(s[m])
        for k in range(8):
            d = np.abs(x[m, k] - codes * sm)
            best = codes[d == d.min()]
            expect = best[0] if len(best) == 1 else best[best % 2 == 0][0]
            assert q[m, k] == expect, (m, k)


@pytest.mark.parametrize("bits", [4, 8])
def test_power_of_two_equivariance(bits):
    rng = np.random.default_rng(12)
    x = rng.standard_normal((6, 64))
    q0, s0, _ = oracle.rotate_quant_act(x, None, 64, bits)
    for e in (-7, -1, 3, 12):
        q1, s1, _ = oracle.rotate_quant_act(x * 2.0 ** e, None, 64, bits)
        assert np.array_equal(q0, q1)
        assert np.array_equal(s1.astype(np.float64), s0.astype(np.float64) * 2.0 ** e)


@pytest.mark.parametrize("bits,b", [(4, 64), (8, 128), (4, 8)])
def test_one_hot_rows_closed_form(bits, b):
    qmax = oracle.qmax_of(bits)
    x = np.zeros((3, 2 * b))
    x[0, 1] = 5.0
    x[1, b + 2] = -0.75
    x[2, 0] = 1e-3
    q, s, _ = oracle.rotate_quant_act(x, None, b, bits)
    for m, (c, blk) in enumerate([(5.0, 0), (-0.75, 1), (1e-3, 0)]):
        assert s[m] == np.float32(abs(c) / math.sqrt(b) / qmax)
        assert np.all(np.abs(q[m, blk * b:(blk + 1) * b]) == qmax)
        other = np.delete(np.arange(2 * b), np.arange(blk * b, (blk + 1) * b))
        assert np.all(q[m, other] == 0)


def test_zero_rows_and_grid_symmetry():
    x = np.zeros((2, 16))
    x[1, 3] = -1.0
    q, s, _ = oracle.quantize_rows(x, 4)
    assert s[0] == 0 and np.all(q[0] == 0)
    assert q[1, 3] == -7 and q.min() >= -7


def test_fold_direction_consistency():
    """Activation divides by s, weight multiplies: the 8-bit quantized product
    approximates x w^T; the opposite direction would not."""
    rng = np.random.default_rng(13)
    x = rng.standard_normal((32, 256))
    x[:, [7, 100]] *= 25.0
    w = rng.standard_normal((48, 256)) * 0.02
    s = oracle.calibrate_fold(x, w)
    qx, sx, _ = oracle.rotate_quant_act(x, s, 64, 8)
    qw, sw, _ = oracle.quantize_weights(w, s, 64, 8)
    _, y32, _ = oracle.gemm(qx, sx, qw, sw, "f32")
    ref = x @ w.T
    assert np.linalg.norm(y32 - ref) / np.linalg.norm(ref) < 0.02
    bad_w = w / s.astype(np.float64)  # wrong direction for the weights
    qw2, sw2, _ = oracle.quantize_weights(bad_w, None, 64, 8)
    _, y2, _ = oracle.gemm(qx, sx, qw2, sw2, "f32")
    assert np.linalg.norm(y2 - ref) / np.linalg.norm(ref) > 0.5


def test_w4a16_group_equals_k_is_per_channel_with_fp16_scale():
    rng = np.random.default_rng(14)
    w = rng.standard_normal((10, 128)) * 0.02
    q, s16, _ = oracle.quantize_groups_w4a16(w, 128)
    amax = np.max(np.abs(w), axis=1)
    assert np.array_equal(s16[:, 0], (amax / 7).astype(np.float16))
    # brute force nearest code under the stored scale
    codes = np.arange(-7, 8)
    for n in range(10):
        sc = float(s16[n, 0])
        for k in range(0, 128, 17):
            d = np.abs(w[n, k] - codes * sc)
            best = codes[d == d.min()]
            expect = best[0] if len(best) == 1 else best[best % 2 == 0][0]
            assert q[n, k] == expect


# ---------------------------------------------------------------- packing


def test_pack_all_bytes_round_trip():
    allb = np.arange(256, dtype=np.uint8)[None, :]
    q = oracle.unpack_int4(allb)
    assert q.min() == -8 and q.max() == 7
    assert np.array_equal(oracle.pack_int4(q), allb)
    assert oracle.pack_int4(np.array([[-1, 7, -8, 0, 3, -2]])).tolist() == [[0x7F, 0x08, 0xE3]]
    with pytest.raises(ValueError):
        oracle.pack_int4(np.array([[1, 9]]))


# ---------------------------------------------------------------- GEMM


def test_int_gemm_triple_loop_8x8x8():
    rng = np.random.default_rng(15)
    qx = rng.integers(-127, 128, (8, 8))
    qw = rng.integers(-127, 128, (8, 8))
    acc = oracle.int_gemm(qx, qw)
    for m in range(8):
        for n in range(8):
            t = 0
            for k in range(8):
                t += int(qx[m, k]) * int(qw[n, k])
            assert acc[m, n] == t


def test_int_gemm_k_split_and_overflow():
    rng = np.random.default_rng(16)
    qx = rng.integers(-127, 128, (5, 512))
    qw = rng.integers(-127, 128, (7, 512))
    acc = oracle.int_gemm(qx, qw)
    parts = sum(oracle.int_gemm(qx[:, i:i + 64], qw[:, i:i + 64]) for i in range(0, 512, 64))
    assert np.array_equal(acc, parts)
    perm = rng.permutation(512)
    assert np.array_equal(oracle.int_gemm(qx[:, perm], qw[:, perm]), acc)
    big = np.full((1, 140000), 127)
    with pytest.raises(OverflowError):
        oracle.int_gemm(big, big)


def test_textbook_w8a8_special_case():
    """b = 1, no fold: per-token / per-channel symmetric int8 -- the product of
    the dequantized matrices, computed in the other order."""
    rng = np.random.default_rng(17)
    x = rng.standard_normal((9, 96))
    w = rng.standard_normal((11, 96)) * 0.015
    qx, sx, _ = oracle.rotate_quant_act(x, None, 1, 8)
    qw, sw, _ = oracle.quantize_weights(w, None, 1, 8)
    _, y32, _ = oracle.gemm(qx, sx, qw, sw, "f32")
    xd = qx * sx.astype(np.float64)[:, None]
    wd = qw * sw.astype(np.float64)[:, None]
    np.testing.assert_allclose(y32, xd @ wd.T, rtol=3e-7, atol=1e-30)


# ---------------------------------------------------------------- output rounding


def test_bf16_rounding_matches_library_cast():
    rng = np.random.default_rng(18)
    v = (rng.standard_normal(200000) * 3.7).astype(np.float32)
    # exact ties and near-ties in the bf16 grid
    base = v[:1000].view(np.uint32) & np.uint32(0xFFFF0000)
    ties = (base | np.uint32(0x8000)).view(np.float32)
    near = (base | np.uint32(0x7FFF)).view(np.float32)
    v = np.concatenate([v, ties, near, np.array([0.0, -0.0, 1e-40, 3e38], np.float32)])
    got = oracle.round_to_bf16_bits(v)
    ref = torch.from_numpy(v).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(got, ref)
    np.testing.assert_array_equal(oracle.bf16_bits_to_f64(got),
                                  torch.from_numpy(v).to(torch.bfloat16).to(torch.float64).numpy())


def test_f16_rounding_matches_library_cast():
    rng = np.random.default_rng(19)
    v = (rng.standard_normal(100000) * 50).astype(np.float32)
    got = oracle.round_output(v, "f16")
    ref = torch.from_numpy(v).to(torch.float16).to(torch.float64).numpy()
    np.testing.assert_array_equal(got, ref)


# ---------------------------------------------------------------- GEMV


def test_gemv_on_grid_weights_is_exact_float_gemv():
    rng = np.random.default_rng(20)
    n, k, g = 24, 512, 128
    q = rng.integers(-7, 8, (n, k))
    q[:, ::g] = 7   # every group reaches the grid maximum
    s16 = (2.0 ** rng.integers(-10, -4, (n, k // g))).astype(np.float16)
    w = q * np.repeat(s16.astype(np.float64), g, axis=1)
    q2, s2, _ = oracle.quantize_groups_w4a16(w, g)
    assert np.array_equal(q2, q) and np.array_equal(s2, s16)
    x = rng.standard_normal((3, k)).astype(np.float16).astype(np.float64)
    y32, yref = oracle.gemv_w4a16(x, q2, s2, g)
    np.testing.assert_array_equal(y32, (x @ w.T).astype(np.float32))
    np.testing.assert_array_equal(yref, (x @ w.T).astype(np.float32).astype(np.float16))


# ---------------------------------------------------------------- GeLU


def test_gelu_matches_library_and_identities():
    t = np.linspace(-8, 8, 2001)
    ref = torch.nn.functional.gelu(torch.from_numpy(t), approximate="none").numpy()
    np.testing.assert_allclose(oracle.gelu(t), ref, rtol=1e-13, atol=1e-15)
    assert oracle.gelu(np.array([0.0]))[0] == 0.0
    np.testing.assert_allclose(oracle.gelu(t) - oracle.gelu(-t), t, atol=1e-14)
    g, u = t[990:1000], t[1500:1510]
    x = np.concatenate([g, u])[None, :]
    np.testing.assert_allclose(oracle.geglu(x, 10)[0], oracle.gelu(g) * u, rtol=1e-15)


# ---------------------------------------------------------------- fused gate|up + GeGLU


def test_interleave_gate_up_order():
    # hand-built order at block 2: gate rows 0,1 | up rows 0,1 | gate rows 2,3 | up rows 2,3
    gate = np.array([[0], [1], [2], [3]])
    up = np.array([[10], [11], [12], [13]])
    got = oracle.interleave_gate_up(gate, up, block=2)[:, 0]
    assert got.tolist() == [0, 1, 10, 11, 2, 3, 12, 13]
    g2, u2 = oracle.split_gate_up(got[None, :], block=2)
    assert g2[0].tolist() == [0, 1, 2, 3] and u2[0].tolist() == [10, 11, 12, 13]
    with pytest.raises(ValueError):
        oracle.interleave_gate_up(gate[:3], up[:3], block=2)


def test_gemm_geglu_matches_torch_composition():
    # against torch: int64 matmul, float64 scaling, torch bf16 casts and torch's erf GeLU
    rng = np.random.default_rng(7)
    m, f, k = 5, 64, 96
    qx = rng.integers(-7, 8, size=(m, k))
    qg = rng.integers(-7, 8, size=(f, k))
    qu = rng.integers(-7, 8, size=(f, k))
    sx = (rng.random(m) * 0.1 + 0.01).astype(np.float32)
    sg = (rng.random(f) * 0.01 + 0.001).astype(np.float32)
    su = (rng.random(f) * 0.01 + 0.001).astype(np.float32)
    qw = oracle.interleave_gate_up(qg, qu)
    sw = oracle.interleave_gate_up(sg[:, None], su[:, None])[:, 0]
    acc, h32, h_ref = oracle.gemm_geglu(qx, sx, qw, sw, "bf16")

    def deq(q, s):
        a = torch.from_numpy(qx).to(torch.int64) @ torch.from_numpy(q).to(torch.int64).T
        return (a.double() * torch.from_numpy(sx).double()[:, None] * torch.from_numpy(s).double()[None, :]).float()

    g = deq(qg, sg).to(torch.bfloat16).double()
    u = deq(qu, su).to(torch.bfloat16).double()
    h = (torch.nn.functional.gelu(g, approximate="none") * u).float()
    np.testing.assert_allclose(h32, h.numpy(), rtol=2.5e-7, atol=1e-30)
    ref = h.to(torch.bfloat16).double().numpy()
    # equal except where the float32 values straddle a bfloat16 rounding point
    assert np.mean(h_ref != ref) < 0.01
    np.testing.assert_allclose(h_ref, ref, rtol=2 ** -7)
    # the accumulators are the plain integer products in the interleaved column order
    g_acc, u_acc = oracle.split_gate_up(acc)
    assert np.array_equal(g_acc, qx @ qg.T) and np.array_equal(u_acc, qx @ qu.T)


# ---------------------------------------------------------------- compare rules


def test_compare_codes_rules():
    r = np.array([[0.5 + 1e-7, 2.0, -3.4999999, 100.5]])
    q_ref = np.rint(r).astype(np.int64)
    q_gpu = q_ref.copy()
    assert oracle.compare_codes(q_gpu, q_ref, r).ok
    q_gpu[0, 0] -= 1                       # flip at a boundary: allowed only under the count limit
    res = oracle.compare_codes(q_gpu, q_ref, r, max_frac=0.5)
    assert res.ok, res.detail
    assert not oracle.compare_codes(q_gpu, q_ref, r).ok   # floor(1e-4 * 4) = 0
    q_gpu = q_ref.copy()
    q_gpu[0, 1] += 1                       # flip far from a boundary
    assert not oracle.compare_codes(q_gpu, q_ref, r, max_frac=0.5).ok
    q_gpu = q_ref.copy()
    q_gpu[0, 3] += 2
    assert not oracle.compare_codes(q_gpu, q_ref, r, max_frac=0.5).ok


def test_compare_outputs_rules():
    y = np.linspace(-1, 1, 1000)
    assert oracle.compare_outputs(y, y).ok
    z = y.copy()
    z[3] += 0.005
    assert oracle.compare_outputs(z, y).ok
    z[3] += 0.02
    assert not oracle.compare_outputs(z, y).ok
    assert not oracle.compare_outputs(y * 1.01, y).ok
    assert oracle.compare_scales(np.array([1.0, 0.0]), np.array([1.0 + 1e-7, 0.0])).ok
    assert not oracle.compare_scales(np.array([1.0, 1e-9]), np.array([1.0, 0.0])).ok
