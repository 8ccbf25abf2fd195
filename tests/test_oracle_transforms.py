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


# ---------------------------------------------------------------------------
# Hadamard-diagonal variant (the pages' diagonal approximation of the
# data-aware component; reading in the oracle's transforms module)


def test_hd_scales_are_the_optimal_diagonal_and_inverse_transpose():
    W, X, A, B = _case(seed=31)
    dx, dw, dx64, dw64 = tr.build_hd(W, B.astype(np.float32), 32)
    Tx = tr.hd_dense(dx64, 32)
    Tw = tr.hd_dense(dw64, 32)
    for b in range(A.shape[0]):
        a, bb = np.diag(A[b]), np.diag(B[b].astype(np.float32).astype(np.float64))
        # T_W^T T_X = I
        assert np.allclose(Tw[b].T @ Tx[b], np.eye(32), atol=1e-12)
        # the proxy reaches the Cauchy-Schwarz bound (sum sqrt(a b))^2 ...
        J = tr.proxy_loss(Tw[b], A[b], B[b].astype(np.float32).astype(np.float64))
        J_diag_bound = np.sum(np.sqrt(a * bb)) ** 2
        # ... which only holds for the diagonal of the moments; with the full
        # moments J is tr(E A E) tr(E^-1 B E^-1) evaluated on the off-diagonals too
        E = np.diag(dw64.reshape(-1, 32)[b] * np.sqrt(32))
        Ei = np.linalg.inv(E)
        assert np.isclose(J, np.trace(E @ A[b] @ E) * np.trace(Ei @ B[b].astype(np.float32).astype(np.float64) @ Ei),
                          rtol=1e-10)
        assert np.isclose(np.sum(np.diag(E) ** 2 * a) * np.sum(bb / np.diag(E) ** 2), J_diag_bound, rtol=1e-10)
        # no other diagonal does better on the diagonal model
        rng = np.random.default_rng(b)
        for _ in range(20):
            e = np.diag(E) * np.exp(0.3 * rng.standard_normal(32))
            assert np.sum(e ** 2 * a) * np.sum(bb / e ** 2) >= J_diag_bound * (1 - 1e-12)


def test_hd_sits_between_wush_and_hadamard():
    W, X, A, B = _case(seed=32)
    B32 = B.astype(np.float32)
    _, _, dx64, dw64 = tr.build_hd(W, B32, 32)
    Tw_hd = tr.hd_dense(dw64, 32)
    for b in range(A.shape[0]):
        Bb = B32[b].astype(np.float64)
        _, Tw_w = tr.block_transform("wush", A[b], Bb, 32)
        _, Tw_h = tr.block_transform("hadamard", A[b], Bb, 32)
        j_w = tr.proxy_loss(Tw_w, A[b], Bb)
        j_h = tr.proxy_loss(Tw_h, A[b], Bb)
        # the diagonal model's optimum, evaluated on the diagonal moments
        a, bb = np.diag(A[b]), np.diag(Bb)
        assert j_w <= tr.proxy_loss(Tw_hd[b], A[b], Bb) * (1 + 1e-9)
        assert np.sum(np.sqrt(a * bb)) ** 2 <= np.sum(a) * np.sum(bb) * (1 + 1e-12)
        assert j_h == pytest.approx(np.trace(A[b]) * np.trace(Bb), rel=1e-9)


def test_hd_equals_wush_on_diagonal_moments():
    # with diagonal moments the full construction has nothing off the diagonal
    # to exploit: both reach (sum sqrt(a b))^2
    rng = np.random.default_rng(33)
    a = rng.uniform(0.1, 10, 32)
    bb = rng.uniform(0.1, 10, 32)
    A, B = np.diag(a), np.diag(bb)
    _, Tw_w = tr.block_transform("wush", A, B, 32)
    dx, dw = tr.hd_block_scales(a, bb, 32)
    Tw = tr.hd_dense(dw, 32)[0]
    bound = np.sum(np.sqrt(a * bb)) ** 2
    assert tr.proxy_loss(Tw, A, B) == pytest.approx(bound, rel=1e-12)
    assert tr.proxy_loss(Tw_w, A, B) == pytest.approx(bound, rel=1e-9)
    # the scales themselves: closed form (a / b)^(1/4) / sqrt(32)
    assert np.allclose(dx, (a / bb) ** 0.25 / np.sqrt(32), rtol=1e-15)
    assert np.allclose(dx * dw, np.full(32, 1.0 / 32), rtol=1e-15)


def test_hd_floors_and_zero_blocks():
    a = np.array([4.0, 0.0] + [1.0] * 30)
    bb = np.array([0.0, 2.0] + [1.0] * 30)
    dx, dw = tr.hd_block_scales(a, bb, 32)
    assert np.all(np.isfinite(dx)) and np.all(np.isfinite(dw)) and np.all(dx > 0)
    assert dx[0] == pytest.approx((4.0 / (1e-12 * 2.0)) ** 0.25 / np.sqrt(32))
    dx0, dw0 = tr.hd_block_scales(a, np.zeros(32), 32)       # all-zero activations: b = 1
    assert np.allclose(dx0, np.sqrt(np.sqrt(np.maximum(a, 4e-12))) / np.sqrt(32))
    with pytest.raises(np.linalg.LinAlgError):
        tr.hd_block_scales(np.zeros(32), bb, 32)


# ---------------------------------------------------------------------------
# shared-transform variant

def test_shared_with_one_block_per_group_is_the_per_block_build():
    Wt, X = random_case(41, 96, 128, 40)
    bs = 32
    Sx = tr.activation_moments(X, bs)
    for kind in ("wus", "wush"):
        _, _, tx, tw = tr.build_transforms(kind, Wt, Sx, bs)
        _, _, sx, sw = tr.build_shared(kind, Wt, Sx, bs, np.arange(4), 4)
        assert np.array_equal(sx, tx) and np.array_equal(sw, tw)


def test_shared_is_invariant_to_duplicated_blocks():
    # k copies of one block's data: A_G = k A_b and B_G = k B_b, and the
    # construction is unchanged by a common positive scale of A and B
    rng = np.random.default_rng(42)
    bs, k = 16, 3
    Wb = rng.standard_normal((40, bs))
    Xb = rng.standard_normal((60, bs)) * np.linspace(0.5, 4.0, bs)
    Wt = np.tile(Wb, (1, k)).astype(np.float32)
    X = np.tile(Xb, (1, k)).astype(np.float32)
    Sx = tr.activation_moments(X, bs)
    _, _, one_x, one_w = tr.build_transforms("wush", Wt[:, :bs], Sx[:1], bs)
    _, _, sx, sw = tr.build_shared("wush", Wt, Sx, bs, np.zeros(k, dtype=int), 1)
    assert np.allclose(sx[0], one_x[0], rtol=1e-9, atol=1e-12)
    assert np.allclose(sw[0], one_w[0], rtol=1e-9, atol=1e-12)


def test_shared_pair_is_inverse_transpose_and_keeps_the_product():
    Wt, X = random_case(43, 80, 192, 24)
    bs = 32
    Sx = tr.activation_moments(X, bs)
    group = np.array([0, 1, 0, 2, 1, 0])
    _, _, gx, gw = tr.build_shared("wush", Wt, Sx, bs, group, 3)
    for gi in range(3):
        assert np.allclose(gw[gi].T @ gx[gi], np.eye(bs), atol=1e-9)
    Tx, Tw = tr.expand_shared(gx, group), tr.expand_shared(gw, group)
    W64, X64 = Wt.astype(np.float64), X.astype(np.float64)
    Y = np.zeros((X.shape[0], Wt.shape[0]))
    for b in range(len(group)):
        sl = slice(b * bs, (b + 1) * bs)
        Y += (X64[:, sl] @ Tx[b].T) @ (W64[:, sl] @ Tw[b].T).T
    assert np.allclose(Y, X64 @ W64.T, rtol=1e-9, atol=1e-9)


def test_shared_group_minimises_its_pooled_proxy():
    # the group's matrix beats the members' own matrices on the pooled moments
    Wt, X = random_case(44, 120, 96, 48)
    bs = 32
    Sx = tr.activation_moments(X, bs).astype(np.float64)
    A = tr.weight_moments(Wt, bs)
    # J takes the weight-side matrix T_W (the activation side is T_W^{-T})
    _, _, _, gw = tr.build_shared("wush", Wt, Sx, bs, np.zeros(3, dtype=int), 1)
    _, _, _, pw = tr.build_transforms("wush", Wt, Sx, bs)
    J = lambda T: tr.proxy_loss(T, A.sum(axis=0), Sx.sum(axis=0))
    assert all(J(gw[0]) < J(pw[b]) * (1 - 1e-9) for b in range(3))
    assert J(gw[0]) < J(tr.hadamard_normalized(bs))


def test_shared_rejects_bad_groups():
    Wt, X = random_case(45, 40, 64, 8)
    Sx = tr.activation_moments(X, 32)
    with pytest.raises(ValueError):
        tr.build_shared("wush", Wt, Sx, 32, np.array([0, 2]), 2)
    with pytest.raises(ValueError):
        tr.build_shared("wush", Wt, Sx, 32, np.array([0, 0]), 2)
