"""Pins for the oracle's rotation and fold (CPU only).

Block Hadamard: Omega-QVLA technical summary, Metodologia 1 ("Rotazione
Composita", "Implementazione a Blocchi"); FoldQuantVLA abstract.
Channel fold: FoldQuantVLA abstract ("channel scaling").
"""

import json
import math
import os

import numpy as np
import pytest
import scipy.linalg

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "hand_worked.json")


def _fwht_butterfly(v):
    """Iterative in-place butterfly (a different algorithm from the oracle's
    dense matmul): pairs (i, i + h) become (a + b, a - b) for h = 1, 2, 4, ..."""
    v = np.array(v, dtype=np.float64, copy=True)
    b = v.shape[-1]
    h = 1
    while h < b:
        for start in range(0, b, 2 * h):
            a = v[..., start:start + h].copy()
            c = v[..., start + h:start + 2 * h].copy()
            v[..., start:start + h] = a + c
            v[..., start + h:start + 2 * h] = a - c
        h *= 2
    return v


@pytest.mark.parametrize("b", [1, 2, 4, 8, 16, 32, 64, 128, 256])
def test_hadamard_orthogonal_and_symmetric(b):
    h = oracle.sylvester_hadamard(b)
    assert h.dtype == np.int64
    assert np.array_equal(h @ h.T, b * np.eye(b, dtype=np.int64))
    assert np.array_equal(h, h.T)
    assert set(np.unique(h)) <= {-1, 1}


@pytest.mark.parametrize("b", [1, 2, 4, 8, 16, 64, 128, 256])
def test_hadamard_matches_library_sylvester(b):
    # scipy's construction is the Kronecker recursion [[H, H], [H, -H]].
    assert np.array_equal(oracle.sylvester_hadamard(b), scipy.linalg.hadamard(b))


def test_hadamard_hand_worked():
    g = json.load(open(GOLDEN))
    assert np.array_equal(oracle.sylvester_hadamard(4), np.array(g["hadamard_4"]["H"]))


def test_hadamard_rejects_non_pow2():
    with pytest.raises(ValueError):
        oracle.sylvester_hadamard(12)


@pytest.mark.parametrize("b", [2, 8, 64, 128])
def test_rotation_equals_butterfly(b):
    rng = np.random.default_rng(1)
    k = 4 * b
    v = rng.standard_normal((5, k))
    got = oracle.rotate_blocks(v, b)
    ref = np.concatenate([_fwht_butterfly(v[:, j * b:(j + 1) * b]) for j in range(k // b)], axis=1)
    ref /= math.sqrt(b)
    np.testing.assert_allclose(got, ref, rtol=0, atol=1e-12)


@pytest.mark.parametrize("b", [4, 64, 128])
def test_rotation_orthonormal_and_product_preserving(b):
    rng = np.random.default_rng(2)
    k = 2 * b
    x = rng.standard_normal((7, k))
    w = rng.standard_normal((9, k))
    xr = oracle.rotate_blocks(x, b)
    wr = oracle.rotate_blocks(w, b)
    np.testing.assert_allclose(np.linalg.norm(xr, axis=1), np.linalg.norm(x, axis=1), rtol=1e-13)
    np.testing.assert_allclose(xr @ wr.T, x @ w.T, rtol=0, atol=1e-11)
    r = oracle.block_rotation_matrix(k, b)
    np.testing.assert_allclose(r @ r.T, np.eye(k), atol=1e-14)
    np.testing.assert_allclose(x @ r, xr, atol=1e-13)


@pytest.mark.parametrize("b", [8, 64])
def test_rotation_one_hot_and_constant(b):
    h = scipy.linalg.hadamard(b)
    for j in (0, 3, b - 1):
        e = np.zeros((1, 2 * b))
        e[0, b + j] = 1.0          # one-hot in the second block
        got = oracle.rotate_blocks(e, b)
        assert np.all(got[0, :b] == 0)
        np.testing.assert_allclose(got[0, b:], h[j] / math.sqrt(b), atol=1e-15)
    c = np.full((1, b), 3.0)
    got = oracle.rotate_blocks(c, b)
    np.testing.assert_allclose(got[0, 0], 3.0 * math.sqrt(b), rtol=1e-15)
    np.testing.assert_allclose(got[0, 1:], 0.0, atol=1e-13)


def test_rotation_identity_cases():
    x = np.arange(12.0).reshape(2, 6)
    assert np.array_equal(oracle.rotate_blocks(x, 0), x)
    assert np.array_equal(oracle.rotate_blocks(x, 1), x)
    with pytest.raises(ValueError):
        oracle.rotate_blocks(x, 4)


def test_rotation_spreads_outlier_and_lowers_int4_error():
    """The block rotation spreads a dominant channel over its block, so int4
    per-token quantization error drops on outlier-heavy activations."""
    rng = np.random.default_rng(3)
    x = rng.standard_normal((64, 512))
    x[:, [5, 77, 300, 411]] *= 30.0
    errs = {}
    for b in (0, 64):
        v = oracle.rotate_blocks(x, b)
        q, s, _ = oracle.quantize_rows(v, 4)
        vhat = q * s.astype(np.float64)[:, None]
        errs[b] = np.mean((oracle.rotate_blocks(vhat, b) - x) ** 2)  # rotate back (H symmetric, orthonormal)
    assert errs[64] < 0.5 * errs[0]


def test_fold_closed_form_8x8():
    x = np.zeros((8, 8))
    w = np.zeros((8, 8))
    for k in range(8):
        x[k, k] = -(k + 1) * 4.0       # max |X_k| = 4 (k+1)
        w[(k + 3) % 8, k] = (k + 1.0)  # max |W_k| = k + 1
    x[0, 7] = 100.0                    # column 7: max(32, 100) = 100
    s = oracle.calibrate_fold(x, w)
    expect = np.full(8, 2.0)
    expect[7] = math.sqrt(100.0 / 8.0)
    assert s.dtype == np.float32
    np.testing.assert_array_equal(s, expect.astype(np.float32))


def test_fold_zero_column_guard_and_product():
    rng = np.random.default_rng(4)
    x = rng.standard_normal((16, 32))
    w = rng.standard_normal((24, 32)) * 0.02
    x[:, 3] = 0.0
    w[:, 9] = 0.0
    s = oracle.calibrate_fold(x, w)
    assert s[3] == 1.0 and s[9] == 1.0
    s64 = s.astype(np.float64)
    np.testing.assert_allclose((x / s64) @ (w * s64).T, x @ w.T, rtol=0, atol=1e-12)
    # after the fold, activation and weight column maxima are balanced
    ok = np.ones(32, bool)
    ok[[3, 9]] = False
    ax = np.max(np.abs(x / s64), axis=0)[ok]
    aw = np.max(np.abs(w * s64), axis=0)[ok]
    np.testing.assert_allclose(ax, aw, rtol=1e-6)
