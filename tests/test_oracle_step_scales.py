"""Pins of the oracle's per-step static activation scales (Omega-QVLA
technical summary, Metodologia 2, "Scalatura delle Attivazioni DiT per
Passo"): hand-computed values, reductions to the dynamic per-row quantizer,
calibration invariants, and the error bound of the folded composition."""

import numpy as np
import pytest

import oracle


def _rows(*rows):
    return np.array(rows, dtype=np.float64)


# ---- hand-computed, k = b = 4 (H_4 / 2 in Sylvester order), int4 -----------
# x [1,1,1,1] rotates to [2,0,0,0]; [1,-1,1,-1] to [0,2,0,0].

def test_calibration_table_by_hand():
    cal = _rows([1, 1, 1, 1], [3, -3, 3, -3])          # v: [2,0,0,0], [0,6,0,0]
    s = oracle.calibrate_step_scales(cal, None, 4, 4)
    assert s.dtype == np.float32
    assert np.array_equal(s, np.array([2 / 7, 6 / 7, 0, 0], dtype=np.float32))


def test_static_codes_by_hand():
    s = np.array([2 / 7, 6 / 7, 0, 0], dtype=np.float32)
    x = _rows([0.25] * 4,                 # v [0.5,0,0,0]: 0.5 / (2/7) = 1.75 -> 2
              [0.5, -0.5, 0.5, -0.5],     # v [0,1,0,0]: 1 / (6/7) = 1.17 -> 1
              [1, 0, 0, 0],               # v [.5,.5,.5,.5]: 1.75, 0.58, (s 0), (s 0)
              [10, 10, 10, 10],           # v [20,0,0,0]: 70 -> clipped to 7
              [-1, -1, -1, -1])           # v [-2,0,0,0]: -7
    q, _ = oracle.rotate_quant_act_static(x, None, 4, 4, s)
    assert q.tolist() == [[2, 0, 0, 0], [0, 1, 0, 0], [2, 1, 0, 0], [7, 0, 0, 0], [-7, 0, 0, 0]]


def test_static_codes_fold_divides():
    # x / s before the rotation: a fold of 2 on every channel halves v
    s = np.array([2 / 7, 6 / 7, 0, 0], dtype=np.float32)
    fold = np.full(4, 2.0, dtype=np.float32)
    q, _ = oracle.rotate_quant_act_static(_rows([1.2, 1.2, 1.2, 1.2]), fold, 4, 4, s)   # v [1.2,0,0,0]
    assert q.tolist() == [[4, 0, 0, 0]]                                              # 4.2 -> 4


# ---- reductions to the dynamic per-row quantizer -----------------------------

@pytest.mark.parametrize("bits", [4, 8])
def test_constant_table_is_dynamic_row_quantization(bits):
    # one token, a table holding its own dynamic scale in every channel: the
    # static codes are the per-token dynamic codes
    rng = np.random.default_rng(7)
    x = rng.standard_normal((1, 256)) * 3
    fold = (rng.random(256) + 0.5).astype(np.float32)
    q_dyn, s_dyn, _ = oracle.rotate_quant_act(x, fold, 64, bits)
    table = np.full(256, s_dyn[0], dtype=np.float32)
    q_st, _ = oracle.rotate_quant_act_static(x, fold, 64, bits, table)
    assert np.array_equal(q_st, q_dyn)


def test_unit_table_weights_are_plain_rtn():
    rng = np.random.default_rng(8)
    w = rng.standard_normal((24, 128))
    fold = (rng.random(128) + 0.5).astype(np.float32)
    q1, s1, _ = oracle.quantize_weights(w, fold, 32, 4)
    q2, s2, _ = oracle.quantize_weights_step(w, fold, 32, 4, np.ones(128, dtype=np.float32))
    assert np.array_equal(q1, q2) and np.array_equal(s1, s2)
    # a power-of-two table: same codes, scales times that power
    q3, s3, _ = oracle.quantize_weights_step(w, fold, 32, 4, np.full(128, 8.0, dtype=np.float32))
    assert np.array_equal(q1, q3) and np.array_equal(s3, s1 * np.float32(8))


# ---- calibration invariants ----------------------------------------------------

@pytest.mark.parametrize("bits", [4, 8])
def test_calibration_tokens_fill_the_grid(bits):
    rng = np.random.default_rng(9)
    qmax = 7 if bits == 4 else 127
    x = rng.standard_normal((40, 512)) * np.linspace(0.5, 4, 512)[None, :]
    x[:, 128:192] = 0                                  # one whole Hadamard block of zeros
    fold = (rng.random(512) + 0.5).astype(np.float32)
    s = oracle.calibrate_step_scales(x, fold, 64, bits)
    assert np.all(s[128:192] == 0) and np.all(s[:64] > 0)
    q, _ = oracle.rotate_quant_act_static(x, fold, 64, bits, s)
    assert np.abs(q).max() <= qmax
    live = s > 0
    assert np.all(np.abs(q[:, live]).max(axis=0) == qmax)   # each channel's max reaches qmax
    assert np.all(q[:, ~live] == 0)


# ---- the folded composition -----------------------------------------------------

@pytest.mark.parametrize("bits", [4, 8])
def test_folded_step_weights_error_bound(bits):
    """s_w_t[n] sum_c q[m,c] qw_t[n,c] against x w^T, for the calibration
    tokens (no clipping): with e_x = v/s_t - q (|e_x| <= 1/2) and
    e_w = w_rot s_t - qw s_w (|e_w| <= s_w / 2),
        |y - y_hat| <= sum_c ( |qw_t s_w| / 2 + |q| s_w / 2 + s_w / 4 )."""
    rng = np.random.default_rng(10)
    m, n, k, b = 16, 24, 256, 64
    x = rng.standard_normal((m, k)) * (1 + 3 * rng.random(k))[None, :]
    w = rng.standard_normal((n, k)) * 0.05
    fold = (rng.random(k) + 0.5).astype(np.float32)
    s_t = oracle.calibrate_step_scales(x, fold, b, bits)
    q, _ = oracle.rotate_quant_act_static(x, fold, b, bits, s_t)
    qw, sw, _ = oracle.quantize_weights_step(w, fold, b, bits, s_t)
    acc = oracle.int_gemm(q, qw).astype(np.float64)
    sw64 = sw.astype(np.float64)
    y_hat = acc * sw64[None, :]
    y = x @ w.T
    what = np.abs(qw).astype(np.float64) * sw64[:, None]                  # |qw_t s_w| [n][k]
    bound = (0.5 * what.sum(axis=1)[None, :]
             + 0.5 * np.abs(q).astype(np.float64) @ np.broadcast_to(sw64[:, None], (n, k)).T
             + 0.25 * k * sw64[None, :])
    err = np.abs(y - y_hat)
    assert np.all(err <= bound * (1 + 1e-9) + 1e-12)
    # and the composition is the right one: folding 1 / s_t into the weights
    # instead (the wrong direction) misses by far more
    rel = np.linalg.norm(y - y_hat) / np.linalg.norm(y)
    assert rel < (0.3 if bits == 4 else 0.02)
    qw2, sw2, _ = oracle.quantize_weights_step(w, fold, b, bits, (1 / s_t.astype(np.float64)).astype(np.float32))
    y2 = oracle.int_gemm(q, qw2).astype(np.float64) * sw2.astype(np.float64)[None, :]
    assert np.linalg.norm(y - y2) / np.linalg.norm(y) > 2 * rel


def test_per_step_tables_absorb_drift():
    """Activations whose range grows over the steps (sigma_t = 0.5 + 0.1 t):
    each step's own table quantizes that step's tokens with less error than a
    single table calibrated on every step (the page's reason for the table)."""
    rng = np.random.default_rng(11)
    k, b, bits = 256, 64, 4
    steps = [rng.standard_normal((32, k)) * (0.5 + 0.1 * t) for t in range(10)]
    pooled = oracle.calibrate_step_scales(np.concatenate(steps), None, b, bits)
    for t in (0, 3):
        own = oracle.calibrate_step_scales(steps[t], None, b, bits)
        v = oracle.rotate_blocks(steps[t], b)

        def err(table):
            q, _ = oracle.rotate_quant_act_static(steps[t], None, b, bits, table)
            return np.linalg.norm(q * table.astype(np.float64)[None, :] - v) / np.linalg.norm(v)
        assert err(own) < err(pooled)
