"""Per-block transforms: identity, Hadamard, WUS, WUSH (test infrastructure only).

Source: "WUSH" news article (chain.bitekongjian.com), paragraph on the
construction: the transform is assembled from a Cholesky factor of weight
statistics (W), the U and S factors of an SVD, and a Hadamard matrix (H); it
is non-orthogonal and block-diagonal, and it is built from second moments of
weights and activations.  Paragraph on deployment: moments come from
calibration data or an existing Hessian; Cholesky and SVD run per block, in
parallel; at inference only the activations are transformed.  "WUSH:
Near-Optimal Adaptive Transforms for LLM Quantization" (AI Radio episode),
"Problem Setup and Goal": T_W and T_X are chosen to minimise the layer loss of
q(T_W W)^T q(T_X X) against W^T X, so T_X = T_W^{-T} keeps the unquantized
product unchanged.

The pages name the factors but print no formula.  Reading used here (the
plainest one consistent with every stated property; derivation in the design
notes):

    A_b = W_b W_b^T           (weights restricted to block b; not normalised)
    B_b = X_b X_b^T / n       (activation second moment of block b)
    A_b = W' W'^T             (Cholesky, W' lower triangular)
    C_b = W'^T B_b W' = U diag(lam) U^T   (eigh; = K K^T with K = W'^T X_b/sqrt(n),
                                           so U, S = sqrt(lam) are K's SVD factors)
    T_W = H^ S^{+1/2} U^T W'^{-1}
    T_X = H^ S^{-1/2} U^T W'^T            (= T_W^{-T})

with H^ the orthonormal Sylvester Hadamard matrix (WUSH) or the identity (WUS).
It minimises the first-order proxy  J(T) = tr(T A T^T) * tr(T^{-T} B T^{-1})
(quantization noise proportional to signal energy, as the article's paragraph
on FP optimality states), whose minimum is (sum sigma_i)^2.
"""

import numpy as np

KINDS = ("identity", "hadamard", "wus", "wush")     # the dense kinds; build_hd is the diagonal variant
DAMPING = (0.0, 1e-10, 1e-8, 1e-6, 1e-4, 1e-2)
SIGMA_FLOOR = 1e-12


def hadamard(d):
    """Sylvester Hadamard matrix, natural order: H[i, j] = (-1)**popcount(i & j)."""
    i = np.arange(d)
    bits = np.bitwise_and(i[:, None], i[None, :])
    pop = np.zeros_like(bits)
    for s in range(int(np.log2(d)) + 1):
        pop += (bits >> s) & 1
    return np.where(pop % 2 == 0, 1.0, -1.0)


def hadamard_normalized(d):
    """H / sqrt(d): orthogonal."""
    return hadamard(d) / np.sqrt(d)


def weight_moments(Wt, bs):
    """A_b = W_b W_b^T in fp64 for every block.  Wt is [d_out][d_in] (nn.Linear)."""
    Wt = np.asarray(Wt, dtype=np.float64)
    d_out, d_in = Wt.shape
    Wb = Wt.reshape(d_out, d_in // bs, bs).transpose(1, 2, 0)   # [b][i][o]
    return Wb @ Wb.transpose(0, 2, 1)


def activation_moments(Xt, bs):
    """B_b = X_b X_b^T / n in fp64 for every block.  Xt is [n][d_in] (token-major)."""
    Xt = np.asarray(Xt, dtype=np.float64)
    n, d_in = Xt.shape
    Xb = Xt.reshape(n, d_in // bs, bs).transpose(1, 2, 0)       # [b][i][t]
    return (Xb @ Xb.transpose(0, 2, 1)) / n


def cholesky_damped(A):
    """Lower Cholesky factor of A, retrying with A + eps*(tr A/bs)*I on failure.

    Returns (L, eps_used).  Raises np.linalg.LinAlgError when every rung of the
    damping ladder fails.
    """
    bs = A.shape[0]
    t = np.trace(A) / bs
    for eps in DAMPING:
        try:
            return np.linalg.cholesky(A + eps * t * np.eye(bs)), eps
        except np.linalg.LinAlgError:
            continue
    raise np.linalg.LinAlgError("block moment not positive definite after damping")


def eig_desc(C):
    """Symmetric eigen-decomposition with eigenvalues in descending order.

    Each eigenvector is signed so that its entry of largest magnitude is
    positive (the lowest index wins a tie in magnitude).
    """
    lam, U = np.linalg.eigh(C)
    order = np.argsort(-lam, kind="stable")
    lam = lam[order]
    U = U[:, order]
    piv = np.argmax(np.abs(U), axis=0)                 # first max-|.| index per column
    sgn = np.sign(U[piv, np.arange(U.shape[1])])
    sgn[sgn == 0] = 1.0
    return lam, U * sgn


def block_factors(A, B):
    """W', U, sigma for one block (fp64)."""
    Wp, _ = cholesky_damped(A)
    C = Wp.T @ B @ Wp
    C = 0.5 * (C + C.T)
    lam, U = eig_desc(C)
    sig = np.sqrt(np.maximum(lam, 0.0))
    sig = np.maximum(sig, SIGMA_FLOOR * sig[0]) if sig[0] > 0 else np.ones_like(sig)
    return Wp, U, sig


def block_transform(kind, A, B, bs=None):
    """(T_X, T_W) for one block, fp64.  A / B may be None for identity / hadamard."""
    bs = bs if bs is not None else A.shape[0]
    if kind == "identity":
        eye = np.eye(bs)
        return eye, eye.copy()
    if kind == "hadamard":
        H = hadamard_normalized(bs)
        return H, H.copy()
    Wp, U, sig = block_factors(A, B)
    left_x = np.diag(sig ** -0.5) @ U.T                # S^{-1/2} U^T
    left_w = np.diag(sig ** 0.5) @ U.T                 # S^{+1/2} U^T
    Tx = left_x @ Wp.T
    Tw = left_w @ np.linalg.inv(Wp)
    if kind == "wush":
        H = hadamard_normalized(bs)
        Tx = H @ Tx
        Tw = H @ Tw
    elif kind != "wus":
        raise ValueError(kind)
    return Tx, Tw


def build_transforms(kind, Wt, Sx, bs):
    """All blocks: returns (Tx, Tw) as float32 [nblk][bs][bs] and the fp64 versions.

    Wt: [d_out][d_in] weights; Sx: [nblk][bs][bs] activation moments (may be
    None for identity / hadamard).
    """
    d_in = np.asarray(Wt).shape[1]
    nblk = d_in // bs
    A = weight_moments(Wt, bs) if kind in ("wus", "wush") else None
    Tx64 = np.empty((nblk, bs, bs))
    Tw64 = np.empty((nblk, bs, bs))
    for b in range(nblk):
        Ab = A[b] if A is not None else None
        Bb = np.asarray(Sx[b], dtype=np.float64) if Sx is not None else None
        Tx64[b], Tw64[b] = block_transform(kind, Ab, Bb, bs)
    return Tx64.astype(np.float32), Tw64.astype(np.float32), Tx64, Tw64


# ---------------------------------------------------------------------------
# Shared-transform variant.  The news article's paragraph on deployment
# limits proposes sharing one transform among similar blocks.  The pages give
# no rule for grouping or for building the shared matrix.  Reading used here:
# the caller assigns every block a group id; a group's matrix is the
# construction above applied to the group's summed moments
#     A_G = sum_{b in G} W_b W_b^T,   B_G = sum_{b in G} B_b,
# i.e. the group's blocks are treated as further samples of one block.  It
# minimises J(T; A_G, B_G), which bounds the group's summed per-block proxies
# sum_b J(T; A_b, B_b) from above (a sum of products of non-negative terms is
# at most the product of the sums).  T_X = T_W^{-T} still holds per group, so
# the unquantized product is unchanged.

def build_shared(kind, Wt, Sx, bs, group, ngroups):
    """Per-group (Tx, Tw) as float32 [ngroups][bs][bs] and the fp64 versions.

    group: [nblk] ints in [0, ngroups); every group must own a block.
    """
    d_in = np.asarray(Wt).shape[1]
    nblk = d_in // bs
    group = np.asarray(group)
    if group.shape != (nblk,) or group.min() < 0 or group.max() >= ngroups:
        raise ValueError("group ids must be one per block, in [0, ngroups)")
    if len(np.unique(group)) != ngroups:
        raise ValueError("every group must own at least one block")
    A = weight_moments(Wt, bs) if kind in ("wus", "wush") else None
    Tx64 = np.empty((ngroups, bs, bs))
    Tw64 = np.empty((ngroups, bs, bs))
    for gi in range(ngroups):
        members = np.flatnonzero(group == gi)
        Ag = A[members].sum(axis=0) if A is not None else None
        Bg = np.asarray(Sx, dtype=np.float64)[members].sum(axis=0) if Sx is not None else None
        Tx64[gi], Tw64[gi] = block_transform(kind, Ag, Bg, bs)
    return Tx64.astype(np.float32), Tw64.astype(np.float32), Tx64, Tw64


def expand_shared(Tg, group):
    """Per-block matrices [nblk][bs][bs] from the per-group ones."""
    return np.asarray(Tg)[np.asarray(group)]


# ---------------------------------------------------------------------------
# Hadamard-diagonal variant.  The news article's paragraphs on deployment and
# on limitations propose approximating the data-aware component by a diagonal
# matrix.  Reading used here: keep the orthonormal Hadamard and replace
# S^{-1/2} U^T W'^T by what the same construction gives for diagonal moments
# a_i = (W_b W_b^T)_ii and b_i = (B_b)_ii (W' = diag(sqrt a), U = I,
# lam = a b):
#     T_X = H^ diag((a_i / b_i)^{1/4}),   T_W = H^ diag((b_i / a_i)^{1/4}) = T_X^{-T}.
# Among T_W = H^ E with E diagonal it minimises the proxy J, because
# J = (sum e_i^2 a_i)(sum b_i / e_i^2) >= (sum sqrt(a_i b_i))^2 (Cauchy-Schwarz)
# with equality at e_i^4 proportional to b_i / a_i.  Moments below 1e-12 of
# the block's largest are floored; an all-zero activation block uses b = 1 (as
# the full builder's sigma fallback does) and an all-zero weight block is an
# error (as the full builder's Cholesky is).  The scales carry the Hadamard's
# 1/sqrt(bs): d = sqrt(sqrt(ratio)) / sqrt(bs), so that T = H diag(d) with H
# the +-1 Sylvester matrix.

HD_FLOOR = 1e-12


def hd_block_scales(a, b, bs):
    """(d_x, d_w) of one block from the moment diagonals a, b (fp64, length bs)."""
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    if not a.max() > 0:
        raise np.linalg.LinAlgError("block weights are all zero")
    a = np.maximum(a, HD_FLOOR * a.max())
    b = np.maximum(b, HD_FLOOR * b.max()) if b.max() > 0 else np.ones_like(b)
    inv = 1.0 / np.sqrt(bs)
    return np.sqrt(np.sqrt(a / b)) * inv, np.sqrt(np.sqrt(b / a)) * inv


def build_hd(Wt, Sx, bs):
    """Per-channel scales (dx, dw): float32 [d_in] each, plus their fp64 values."""
    A = weight_moments(Wt, bs)
    a = np.diagonal(A, axis1=1, axis2=2)
    b = np.diagonal(np.asarray(Sx, dtype=np.float64), axis1=1, axis2=2)
    dx = np.empty(a.shape)
    dw = np.empty(a.shape)
    for k in range(a.shape[0]):
        dx[k], dw[k] = hd_block_scales(a[k], b[k], bs)
    dx, dw = dx.reshape(-1), dw.reshape(-1)
    return dx.astype(np.float32), dw.astype(np.float32), dx, dw


def hd_dense(d, bs):
    """The block matrices H diag(d_b) that per-channel scales d [d_in] stand for (fp64)."""
    d = np.asarray(d, dtype=np.float64).reshape(-1, bs)
    return hadamard(bs)[None, :, :] * d[:, None, :]


def proxy_loss(T, A, B):
    """First-order loss model J(T) = tr(T A T^T) * tr(T^{-T} B T^{-1})."""
    Ti = np.linalg.inv(T)
    return np.trace(T @ A @ T.T) * np.trace(Ti.T @ B @ Ti)
