"""Pins for the oracle's transform builder (CPU only)."""

import json
import os

import numpy as np
import pytest
import scipy.linalg

from oracle import transforms as tr
from synth.gen import random_case, CONFIGS, make_weights, make_activations

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


@pytest.mark.parametrize("d", [2, 4, 16, 32, 256])
def test_hadamard_is_sylvester_and_orthogonal(d):
    H = tr.hadamard(d)
    assert np.array_equal(H, scipy.linalg.hadamard(d).astype(float))
    assert np.array_equal(H @ H.T, d * np.eye(d))
    Hn = tr.hadamard_normalized(d)
    assert np.allclose(Hn @ Hn.T, np.eye(d), atol=1e-14)


def _case(bs=32, d_in=128, d_out=96, n=200, seed=0):
    W, X = random_case(seed, n, d_in, d_out)
    A = tr.weight_moments(W, bs)
    B = tr.activation_moments(X, bs)
    return W, X, A, B


def test_moments_definition():
    W, X, A, B = _case()
    # brute force: explicit loops over a block
    b = 1
    Wb = W[:, 32:64].astype(np.float64)
    Xb = X[:, 32:64].astype(np.float64)
    Abf = sum(np.outer(Wb[o], Wb[o]) for o in range(Wb.shape[0]))
    Bbf = sum(np.outer(Xb[t], Xb[t]) for t in range(Xb.shape[0])) / Xb.shape[0]
    assert np.allclose(A[b], Abf, rtol=1e-12, atol=0)
    assert np.allclose(B[b], Bbf, rtol=1e-12, atol=1e-14)


def test_cholesky_and_eigh_reconstruct():
    _, _, A, B = _case()
    for b in range(A.shape[0]):
        L, eps = tr.cholesky_damped(A[b])
        assert eps == 0.0
        assert np.allclose(L @ L.T, A[b], rtol=1e-12, atol=1e-12 * np.abs(A[b]).max())
        assert np.allclose(L, np.tril(L))
        C = L.T @ B[b] @ L
        lam, U = tr.eig_desc(0.5 * (C + C.T))
        assert np.all(np.diff(lam) <= 0)
        assert np.allclose(U @ np.diag(lam) @ U.T, C, atol=1e-10 * np.abs(C).max())
        assert np.allclose(U.T @ U, np.eye(U.shape[0]), atol=1e-12)
        piv = np.argmax(np.abs(U), axis=0)
        assert np.all(U[piv, np.arange(U.shape[1])] > 0)


def test_damping_ladder_on_rank_deficient_block():
    # 8 output rows cannot make a 32x32 moment full rank
    rng = np.random.default_rng(7)
    W = rng.standard_normal((8, 32))
    A = tr.weight_moments(W, 32)[0]
    L, eps = tr.cholesky_damped(A)
    assert eps > 0
    assert np.allclose(L @ L.T, A + eps * np.trace(A) / 32 * np.eye(32), rtol=1e-10, atol=1e-10)


@pytest.mark.parametrize("kind", tr.KINDS)
def test_transform_pair_is_inverse_transpose(kind):
    W, X, A, B = _case()
    Tx32, Tw32, Tx, Tw = tr.build_transforms(kind, W, B.astype(np.float32), 32)
    for b in range(Tx.shape[0]):
        assert np.allclose(Tw[b].T @ Tx[b], np.eye(32), atol=1e-11)
    # unquantized product is unchanged:  (T_W W)^T (T_X X) = W^T X
    nb = Tx.shape[0]
    Wd = W.astype(np.float64).reshape(W.shape[0], nb, 32)
    Xd = X.astype(np.float64).reshape(X.shape[0], nb, 32)
    Wt_ = np.einsum("bij,obj->obi", Tw, Wd).reshape(W.shape)
    Xt_ = np.einsum("bij,tbj->tbi", Tx, Xd).reshape(X.shape)
    ref = X.astype(np.float64) @ W.astype(np.float64).T
    assert np.allclose(Xt_ @ Wt_.T, ref, rtol=1e-10, atol=1e-10 * np.abs(ref).max())
    assert Tx32.dtype == np.float32 and np.array_equal(Tx32, Tx.astype(np.float32))


@pytest.mark.parametrize("kind", ["wus", "wush"])
def test_balanced_moments(kind):
    _, _, A, B = _case(seed=3)
    Bf = B.astype(np.float32).astype(np.float64)
    for b in range(A.shape[0]):
        Tx, Tw = tr.block_transform(kind, A[b], Bf[b])
        Wp, U, sig = tr.block_factors(A[b], Bf[b])
        mw = Tw @ A[b] @ Tw.T
        mx = Tx @ Bf[b] @ Tx.T
        scale = np.abs(mw).max()
        assert np.allclose(mw, mx, atol=1e-9 * scale)
        if kind == "wus":
            assert np.allclose(mw, np.diag(sig), atol=1e-9 * scale)
        else:
            # Hadamard backbone equalises the per-coordinate energy: constant diagonal
            assert np.allclose(np.diag(mw), sig.sum() / 32, rtol=1e-9)
            H = tr.hadamard_normalized(32)
            assert np.allclose(mw, H @ np.diag(sig) @ H.T, atol=1e-9 * scale)


def test_proxy_loss_closed_form_and_cauchy_schwarz():
    _, _, A, B = _case(seed=4)
    for b in range(A.shape[0]):
        Tx, Tw = tr.block_transform("wush", A[b], B[b])
        _, _, sig = tr.block_factors(A[b], B[b])
        j_wush = tr.proxy_loss(Tw, A[b], B[b])
        assert np.isclose(j_wush, sig.sum() ** 2, rtol=1e-9)
        j_id = tr.proxy_loss(np.eye(32), A[b], B[b])
        assert np.isclose(j_id, np.trace(A[b]) * np.trace(B[b]), rtol=1e-12)
        assert j_wush <= j_id * (1 + 1e-12)
        j_wus = tr.proxy_loss(tr.block_transform("wus", A[b], B[b])[1], A[b], B[b])
        assert np.isclose(j_wus, j_wush, rtol=1e-9)
        j_h = tr.proxy_loss(tr.hadamard_normalized(32), A[b], B[b])
        assert np.isclose(j_h, j_id, rtol=1e-9)           # orthogonal T leaves J unchanged


def test_proxy_optimum_brute_force_2x2():
    """No 2x2 invertible T on a grid beats the closed-form optimum."""
    rng = np.random.default_rng(11)
    for trial in range(5):
        G = rng.standard_normal((2, 6))
        A = G @ G.T
        K = rng.standard_normal((2, 9))
        B = K @ K.T / 9
        _, Tw = tr.block_transform("wush", A, B)
        j_opt = tr.proxy_loss(Tw, A, B)
        grid = np.linspace(-2, 2, 17)
        best = np.inf
        for a in grid:
            for b in grid:
                for c in grid:
                    for d in grid:
                        T = np.array([[a, b], [c, d]])
                        if abs(np.linalg.det(T)) < 1e-3:
                            continue
                        best = min(best, tr.proxy_loss(T, A, B))
        assert best >= j_opt * (1 - 1e-9)
        assert best <= j_opt * 1.2                      # the grid does get close


def test_golden_2x2_hand_example():
    with open(os.path.join(GOLDEN, "wush_2x2.json")) as f:
        g = json.load(f)
    A = np.array(g["A"], float)
    B = np.array(g["B"], float)
    Tx, Tw = tr.block_transform("wush", A, B)
    assert np.allclose(Tx, np.array(g["Tx"]), atol=1e-14)
    assert np.allclose(Tw, np.array(g["Tw"]), atol=1e-14)
    Tx, Tw = tr.block_transform("wus", A, B)
    assert np.allclose(Tx, np.array(g["Tx_wus"]), atol=1e-14)
    assert np.allclose(Tw, np.array(g["Tw_wus"]), atol=1e-14)


def test_tiny_workload_builds():
    w = CONFIGS["tiny"]
    W = make_weights(w)
    X = make_activations(w)
    B = tr.activation_moments(X, 32).astype(np.float32)
    for kind in ("identity", "hadamard", "wush"):
        Tx, Tw, _, _ = tr.build_transforms(kind, W, B, 32)
        assert Tx.shape == (8, 32, 32) and np.all(np.isfinite(Tx)) and np.all(np.isfinite(Tw))
