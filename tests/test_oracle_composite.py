"""Pins of the oracle's SVD-Hadamard composite rotation and zigzag
permutation (Omega-QVLA technical summary, Metodologia 1, "Rotazione SVD",
"Rotazione Hadamard", "Implementazione a Blocchi"): a hand-dealt
permutation, the balance it is for, the SVD's singular values from an
independent routine, the reduction to the plain block Hadamard, and the
invariance of x w^T."""

import numpy as np
import pytest

import oracle


def test_zigzag_by_hand():
    # input-channel norms 8 1 7 2 6 3 5 4, two blocks of 4: ranks c0 c2 c4 c6
    # c7 c5 c3 c1 dealt 0 1 | 1 0 | 0 1 | 1 0 (snake order)
    w = np.zeros((3, 8))
    w[0] = [8, 1, 7, 2, 6, 3, 5, 4]
    assert oracle.zigzag_permutation(w, 4).tolist() == [0, 6, 7, 1, 2, 4, 5, 3]
    # ties go to the lower index first
    assert oracle.zigzag_permutation(np.ones((2, 8)), 4).tolist() == [0, 3, 4, 7, 1, 2, 5, 6]


def test_zigzag_is_a_balanced_permutation():
    rng = np.random.default_rng(3)
    k, b = 1024, 64
    w = rng.standard_normal((96, k)) * (10.0 ** rng.uniform(-2, 1, size=k))[None, :]
    perm = oracle.zigzag_permutation(w, b)
    assert sorted(perm.tolist()) == list(range(k))
    norms = np.sqrt((w * w).sum(axis=0))
    per_block = norms[perm].reshape(k // b, b).sum(axis=1)
    # snake dealing: any two blocks differ by at most the largest norm
    assert per_block.max() - per_block.min() <= norms.max()
    # against contiguous blocks of the unpermuted channels, far more even
    plain = norms.reshape(k // b, b).sum(axis=1)
    assert per_block.std() < 0.2 * plain.std()


def test_composite_rotation_is_svd_then_hadamard():
    rng = np.random.default_rng(4)
    n, k, b = 40, 64, 16
    w = rng.standard_normal((n, k)) * rng.uniform(0.1, 3, size=k)[None, :]
    perm = oracle.zigzag_permutation(w, b)
    rot = oracle.composite_rotations(w, perm, b)
    h = oracle.sylvester_hadamard(b) / np.sqrt(b)
    wp = w[:, perm]
    for j in range(k // b):
        r = rot[j]
        assert np.allclose(r @ r.T, np.eye(b), atol=1e-12)
        u = r @ h.T                                          # undo the Hadamard factor
        blk = wp[:, j * b:(j + 1) * b]
        z = blk @ u                                          # rotated weight columns
        energies = (z * z).sum(axis=0)
        sv = np.linalg.svd(blk, compute_uv=False)            # an independent routine
        assert np.allclose(energies, sv ** 2, rtol=1e-10, atol=1e-9)   # descending spectrum
        assert np.allclose(z.T @ z, np.diag(energies), atol=1e-8)      # orthogonal columns
        big = np.argmax(np.abs(u), axis=0)
        assert np.all(u[big, np.arange(b)] > 0)              # sign convention


def test_diagonal_gram_reduces_to_block_hadamard():
    # weight columns already orthogonal with distinct decreasing norms in
    # every block: U = I, so the composite is the plain block Hadamard
    n, k, b = 32, 32, 8
    w = np.zeros((n, k))
    for c in range(k):
        w[c, c] = 100.0 - c                                   # distinct norms, orthogonal columns
    perm = np.arange(k)
    rot = oracle.composite_rotations(w, perm, b)
    x = np.random.default_rng(5).standard_normal((6, k))
    assert np.allclose(oracle.rotate_composite(x, perm, rot), oracle.rotate_blocks(x, b), atol=1e-12)


def test_projection_is_unchanged():
    rng = np.random.default_rng(6)
    m, n, k, b = 12, 48, 256, 64
    x = rng.standard_normal((m, k))
    w = rng.standard_normal((n, k)) * rng.uniform(0.05, 2, size=k)[None, :]
    perm = oracle.zigzag_permutation(w, b)
    rot = oracle.composite_rotations(w, perm, b)
    y = oracle.rotate_composite(x, perm, rot) @ oracle.rotate_composite(w, perm, rot).T
    assert np.allclose(y, x @ w.T, rtol=1e-10, atol=1e-10)


@pytest.mark.parametrize("bits", [4, 8])
def test_quantized_composite_tracks_the_projection(bits):
    rng = np.random.default_rng(7)
    m, n, k, b = 16, 64, 512, 64
    x = rng.standard_normal((m, k))
    x[:, rng.choice(k, 5, replace=False)] *= 30.0            # outlier input channels
    w = rng.standard_normal((n, k)) * 0.05
    fold = (rng.random(k) + 0.5).astype(np.float32)
    perm = oracle.zigzag_permutation(w * fold[None, :], b)
    rot = oracle.composite_rotations(w * fold[None, :], perm, b).astype(np.float32)
    qx, sx, _ = oracle.rotate_quant_act_composite(x, fold, perm, rot, bits)
    qw, sw, _ = oracle.quantize_weights_composite(w, fold, perm, rot, bits)
    y = oracle.int_gemm(qx, qw) * sx.astype(np.float64)[:, None] * sw.astype(np.float64)[None, :]
    yt = x @ w.T
    rel = np.linalg.norm(y - yt) / np.linalg.norm(yt)
    assert rel < (0.4 if bits == 4 else 0.03)
    # and it spreads the outlier channels: better than quantizing unrotated
    qx0, sx0, _ = oracle.rotate_quant_act(x, fold, 0, bits)
    qw0, sw0, _ = oracle.quantize_weights(w, fold, 0, bits)
    y0 = oracle.int_gemm(qx0, qw0) * sx0.astype(np.float64)[:, None] * sw0.astype(np.float64)[None, :]
    assert rel < np.linalg.norm(y0 - yt) / np.linalg.norm(yt)
    # a float32 rotation is orthogonal to float32 accuracy, so the float
    # projection through it is unchanged to that accuracy
    yf = oracle.rotate_composite(x / fold, perm, rot) @ oracle.rotate_composite(w * fold, perm, rot).T
    assert np.linalg.norm(yf - yt) / np.linalg.norm(yt) < 1e-5
