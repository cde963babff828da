"""Pins of the oracle's backward pass (App. F.2.2, eq. 10-12, Algorithm 3).

Paper: "MoRE: Scaling mixture of experts with hardware-aware low-rank routing".
The backward returns the gradients of
    F = sum_{n,c} tvbar[n,c] * l[n, idx[n,c]] + sum_i pbar_i * psum_i
with the selection idx held fixed.  The pins differentiate F numerically
(central differences in fp64, F evaluated with the oracle's forward functions
logits() and softmax_colsum(), which share no code with the backward), and
check the invariances the softmax Jacobian of eq. (11) implies.
"""
import numpy as np
import pytest


def setup(seed, N=5, h=8, r=4, M=7, k=2, bias=True):
    rng = np.random.default_rng(seed)
    X = rng.standard_normal((N, h))
    R1 = rng.standard_normal((h, r)) / np.sqrt(h)
    R2 = rng.standard_normal((r, M)) / np.sqrt(r)
    # bias on a 2^-8 grid, so that the fp32 bias and its +-2^-10 steps are exact
    b = (np.round(rng.standard_normal(M) * 0.7 * 256) / 256).astype(np.float32) if bias else None
    idx = np.stack([rng.permutation(M)[:k] for _ in range(N)]).astype(np.int32)
    tv = rng.standard_normal((N, k))
    pb = rng.standard_normal(M) * 2.0
    return X, R1, R2, b, idx, tv, pb


def F(oracle_lib, X, R1, R2, b, idx, tv, pb):
    L = oracle_lib.logits(X, R1, R2, b)
    sel = np.take_along_axis(L, idx.astype(np.int64), axis=1)
    return float((tv * sel).sum() + np.dot(pb, oracle_lib.softmax_colsum(X, R1, R2, b)))


def numgrad(f, A, eps):
    G = np.zeros_like(A, dtype=np.float64)
    it = np.nditer(A, flags=["multi_index"])
    for _ in it:
        i = it.multi_index
        a0 = A[i]
        A[i] = a0 + eps
        fp = f()
        A[i] = a0 - eps
        fm = f()
        A[i] = a0
        G[i] = (fp - fm) / (2 * eps)
    return G


@pytest.mark.parametrize("seed,bias", [(0, True), (1, False), (2, True)])
def test_gradients_match_central_differences(oracle_lib, seed, bias):
    X, R1, R2, b, idx, tv, pb = setup(seed, bias=bias)
    g = oracle_lib.backward_lowrank(X, R1, R2, b, idx, tv, pb)
    f = lambda: F(oracle_lib, X, R1, R2, b, idx, tv, pb)
    for name, A in (("xbar", X), ("r1bar", R1), ("r2bar", R2)):
        num = numgrad(f, A, 1e-6)
        assert np.allclose(g[name], num, rtol=1e-6, atol=1e-7), name
    if b is not None:
        num = numgrad(f, b, np.float32(2.0 ** -10))
        # central difference on a quadratic-free step: error O(eps^2 F''') ~ 1e-7
        assert np.allclose(g["bbar"], num, rtol=1e-4, atol=1e-5)


def test_balance_gradient_ignores_a_constant_shift_of_pbar(oracle_lib):
    """eq. (12): the logit gradient is P (pbar - g) with g the P-mean of pbar,
    so pbar + c gives the same gradients."""
    X, R1, R2, b, idx, tv, pb = setup(3)
    a = oracle_lib.backward_lowrank(X, R1, R2, b, idx, tv, pb)
    c = oracle_lib.backward_lowrank(X, R1, R2, b, idx, tv, pb + 3.25)
    for key in a:
        assert np.allclose(a[key], c[key], rtol=1e-12, atol=1e-12), key


def test_bias_gradient_totals_the_selected_gradients(oracle_lib):
    """sum_j P_j (pbar_j - g) = 0 for every token, so the bias gradient sums
    to the sum of tvbar."""
    X, R1, R2, b, idx, tv, pb = setup(4, N=9, M=11, k=3)
    g = oracle_lib.backward_lowrank(X, R1, R2, b, idx, tv, pb)
    assert abs(g["bbar"].sum() - tv.sum()) < 1e-12


def test_linear_in_the_incoming_gradients(oracle_lib):
    X, R1, R2, b, idx, tv, pb = setup(5)
    rng = np.random.default_rng(9)
    tv2, pb2 = rng.standard_normal(tv.shape), rng.standard_normal(pb.shape)
    s = oracle_lib.backward_lowrank(X, R1, R2, b, idx, tv + tv2, pb + pb2)
    a = oracle_lib.backward_lowrank(X, R1, R2, b, idx, tv, pb)
    c = oracle_lib.backward_lowrank(X, R1, R2, b, idx, tv2, pb2)
    for key in s:
        assert np.allclose(s[key], a[key] + c[key], rtol=1e-12, atol=1e-12), key


def test_selected_only_gradient_by_hand(oracle_lib):
    """pbar = 0, one token, one selected expert e with tvbar = 1: F = l_e, so
    dF/dR2[:, e] = z, dF/dX = R1 R2[:, e], dF/db_e = 1, nothing else."""
    X, R1, R2, b, _, _, _ = setup(6, N=1, k=1)
    e = 3
    g = oracle_lib.backward_lowrank(X, R1, R2, b, np.array([[e]], np.int32), np.array([[1.0]]), None)
    z = X[0] @ R1
    expect_r2 = np.zeros_like(R2)
    expect_r2[:, e] = z
    assert np.allclose(g["r2bar"], expect_r2, atol=1e-14)
    assert np.allclose(g["xbar"][0], R1 @ R2[:, e], atol=1e-14)
    assert np.allclose(g["r1bar"], np.outer(X[0], R2[:, e]), atol=1e-14)
    assert np.allclose(g["bbar"], np.eye(R2.shape[1])[e], atol=1e-14)
