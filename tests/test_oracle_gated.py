"""Pins of the oracle's gated (SwiGLU) shard and of the reduce-scatter layout of the block tail.

Pages cited, as [tag section]:
  [Z] zwjcode.cn, "一层 MLP 太宽而放不下时怎样切？列并行、行并行与块尾归约"

Each oracle function is checked against something other than its own formula: closed-form
identities of SiLU, numpy matmul, torch autograd, central finite differences, the page's
channel-numbering check [Z 10], and torch.chunk for the token slices.
"""
import math

import numpy as np
import pytest
import torch

import oracle


def _silu_tanh(z):
    # sigmoid(z) = (1 + tanh(z / 2)) / 2, an identity independent of the oracle's exp form
    z = np.asarray(z, dtype=np.float64)
    return z * 0.5 * (1.0 + np.tanh(0.5 * z))


# ---------------------------------------------------------------- SiLU


def test_silu_matches_tanh_identity():
    z = np.linspace(-30.0, 30.0, 10001)
    # atol covers the reference's own cancellation in 1 + tanh(z / 2) for very negative z
    np.testing.assert_allclose(oracle.silu(z), _silu_tanh(z), rtol=1e-14, atol=1e-14)


def test_silu_special_values_and_odd_part():
    assert oracle.silu([0.0])[0] == 0.0
    z = np.linspace(-20.0, 20.0, 4001)
    # silu(z) - silu(-z) = z (sigmoid(z) + sigmoid(-z) = 1)
    np.testing.assert_allclose(oracle.silu(z) - oracle.silu(-z), z, rtol=0, atol=2e-14)
    assert abs(oracle.silu([40.0])[0] / 40.0 - 1.0) < 1e-15
    assert abs(oracle.silu([-40.0])[0]) < 1e-15
    assert abs(oracle.silu([1.0])[0] - 1.0 / (1.0 + math.exp(-1.0))) < 1e-16


def test_silu_derivative_by_central_differences():
    z = np.linspace(-8.0, 8.0, 321)
    h = 1e-5
    fd = (_silu_tanh(z + h) - _silu_tanh(z - h)) / (2 * h)
    np.testing.assert_allclose(oracle.silu_deriv(z), fd, rtol=0, atol=1e-9)
    assert abs(oracle.silu_deriv([0.0])[0] - 0.5) < 1e-16


# ---------------------------------------------------------------- gated shard forward


def _weights(seed, N=9, D=12, F=16):
    rng = np.random.default_rng(seed)
    X = rng.standard_normal((N, D))
    Wg = rng.standard_normal((D, F)) * 0.3
    Wu = rng.standard_normal((D, F)) * 0.3
    W2 = rng.standard_normal((F, D)) * 0.3
    return X, Wg, Wu, W2


@pytest.mark.parametrize("T,r", [(1, 0), (2, 1), (4, 2), (8, 7)])
def test_gated_shard_matches_numpy(T, r):
    X, Wg, Wu, W2 = _weights(1)
    Fs = Wg.shape[1] // T
    c = slice(r * Fs, (r + 1) * Fs)
    G, U, H, P = oracle.swiglu_shard_fwd(X, Wg, Wu, W2, T, r)
    Gn = X @ Wg[:, c]
    Un = X @ Wu[:, c]
    Hn = _silu_tanh(Gn) * Un
    np.testing.assert_allclose(G, Gn, rtol=1e-13, atol=1e-13)
    np.testing.assert_allclose(U, Un, rtol=1e-13, atol=1e-13)
    np.testing.assert_allclose(H, Hn, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(P, Hn @ W2[c, :], rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("T", [1, 2, 4, 8])
def test_gated_sharded_sum_equals_unsharded(T):
    # [Z 08]: gate and up cut at the same columns, down cut at the matching rows, partials summed.
    X, Wg, Wu, W2 = _weights(2)
    Y = oracle.partial_sum([oracle.swiglu_shard_fwd(X, Wg, Wu, W2, T, r)[3] for r in range(T)])
    Yd = oracle.swiglu_dense_fwd(X, Wg, Wu, W2)
    Yn = (_silu_tanh(X @ Wg) * (X @ Wu)) @ W2
    np.testing.assert_allclose(Y, Yd, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(Yd, Yn, rtol=1e-12, atol=1e-12)


def test_gated_channel_numbers_line_up():
    # [Z 10]: give the gate and up projections recognisable channel numbers and check that
    # every shard sees the same channel in the same position. One token x = [1], one input
    # feature, column c of both weights carries c + 1.
    T, F = 4, 12
    X = np.ones((1, 1))
    ids = np.arange(1, F + 1, dtype=np.float64)[None, :]
    W2 = np.ones((F, 1))
    for r in range(T):
        G, U, H, _ = oracle.swiglu_shard_fwd(X, ids, ids, W2, T, r)
        want = np.arange(r * F // T + 1, (r + 1) * F // T + 1, dtype=np.float64)
        assert np.array_equal(G[0], want) and np.array_equal(U[0], want)
        np.testing.assert_allclose(H[0], _silu_tanh(want) * want, rtol=1e-14)


def test_misaligned_gate_and_up_shards_are_caught():
    # [Z 08]: if the two up-projections use different shard orders the shapes still match but
    # the channels do not. Planted on the CPU from the oracle's own shard pieces: rank r takes
    # the gate of shard r with the up of shard (r + 1) mod T.
    X, Wg, Wu, W2 = _weights(3)
    T = 4
    Fs = Wg.shape[1] // T
    parts = [oracle.swiglu_shard_fwd(X, Wg, Wu, W2, T, r) for r in range(T)]
    good = sum(p[3] for p in parts)
    bad = sum((oracle.silu(parts[r][0]) * parts[(r + 1) % T][1]) @ W2[r * Fs:(r + 1) * Fs]
              for r in range(T))
    assert np.abs(good - bad).max() > 1e-3
    np.testing.assert_allclose(good, oracle.swiglu_dense_fwd(X, Wg, Wu, W2), rtol=1e-12,
                               atol=1e-12)


# ---------------------------------------------------------------- gated shard backward


def _torch_gated(X, Wg, Wu, W2, dY, T, r):
    Fs = Wg.shape[1] // T
    c = slice(r * Fs, (r + 1) * Fs)
    t = {k: torch.tensor(v, dtype=torch.float64, requires_grad=True)
         for k, v in dict(X=X, Wg=Wg[:, c], Wu=Wu[:, c], W2=W2[c, :]).items()}
    G = t["X"] @ t["Wg"]
    H = torch.nn.functional.silu(G) * (t["X"] @ t["Wu"])
    P = H @ t["W2"]
    (P * torch.tensor(dY)).sum().backward()
    return {k: v.grad.numpy() for k, v in t.items()}


@pytest.mark.parametrize("T,r", [(1, 0), (2, 0), (4, 3)])
def test_gated_backward_matches_autograd(T, r):
    X, Wg, Wu, W2 = _weights(4)
    dY = np.random.default_rng(5).standard_normal((X.shape[0], X.shape[1]))
    g = oracle.swiglu_shard_bwd(X, Wg, Wu, W2, dY, T, r)
    ref = _torch_gated(X, Wg, Wu, W2, dY, T, r)
    np.testing.assert_allclose(g["dX"], ref["X"], rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(g["dWg"], ref["Wg"], rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(g["dWu"], ref["Wu"], rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(g["dW2"], ref["W2"], rtol=1e-11, atol=1e-12)


def test_gated_backward_by_finite_differences():
    # Loss <dY, Y> with Y the sum of all shards: dX summed over shards, and each shard's
    # weight gradients, against central differences of the unsharded forward.
    X, Wg, Wu, W2 = _weights(6, N=4, D=5, F=8)
    dY = np.random.default_rng(7).standard_normal((4, 5))
    T = 2
    loss = lambda X_, Wg_, Wu_, W2_: float((oracle.swiglu_dense_fwd(X_, Wg_, Wu_, W2_) * dY).sum())
    g = [oracle.swiglu_shard_bwd(X, Wg, Wu, W2, dY, T, r) for r in range(T)]
    dX = g[0]["dX"] + g[1]["dX"]
    h = 1e-6
    for (n, k) in [(0, 0), (1, 3), (3, 4)]:
        Xp, Xm = X.copy(), X.copy()
        Xp[n, k] += h
        Xm[n, k] -= h
        fd = (loss(Xp, Wg, Wu, W2) - loss(Xm, Wg, Wu, W2)) / (2 * h)
        assert abs(dX[n, k] - fd) < 1e-7
    Fs = 4
    for (k, j) in [(0, 1), (2, 6), (4, 7)]:
        r, jj = j // Fs, j % Fs
        for name, W in (("dWg", Wg), ("dWu", Wu)):
            Wp, Wm = W.copy(), W.copy()
            Wp[k, j] += h
            Wm[k, j] -= h
            args_p = (X, Wp, Wu, W2) if name == "dWg" else (X, Wg, Wp, W2)
            args_m = (X, Wm, Wu, W2) if name == "dWg" else (X, Wg, Wm, W2)
            fd = (loss(*args_p) - loss(*args_m)) / (2 * h)
            assert abs(g[r][name][k, jj] - fd) < 1e-7
    for (j, d) in [(0, 0), (5, 2), (7, 4)]:
        r, jj = j // Fs, j % Fs
        Wp, Wm = W2.copy(), W2.copy()
        Wp[j, d] += h
        Wm[j, d] -= h
        fd = (loss(X, Wg, Wu, Wp) - loss(X, Wg, Wu, Wm)) / (2 * h)
        assert abs(g[r]["dW2"][jj, d] - fd) < 1e-7


# ---------------------------------------------------------------- reduce-scatter layout


@pytest.mark.parametrize("N,T", [(10, 4), (8, 8), (3, 8), (4096, 8), (7, 1), (0, 3)])
def test_token_slices_follow_torch_chunk(N, T):
    chunks = torch.arange(N).chunk(T) if N else ()
    got = [oracle.token_slice(N, T, r) for r in range(T)]
    for r, (row0, rows) in enumerate(got):
        if r < len(chunks):
            assert (row0, rows) == (int(chunks[r][0]), len(chunks[r]))
        else:
            assert rows == 0
    assert sum(rows for _, rows in got) == N


@pytest.mark.parametrize("N,D,T", [(10, 6, 4), (64, 64, 2), (3, 5, 8)])
def test_scattered_tail_reassembles_the_full_tail(N, D, T):
    # [Z 04]: the reduce-scatter form changes where the rows live, not the sum. Integer data:
    # every order of summation is exact, so the slices concatenate to the all-reduce result
    # bit for bit, with b2 added once.
    rng = np.random.default_rng(N * 131 + T)
    Ps = [rng.integers(-50, 51, size=(N, D)).astype(np.float64) for _ in range(T)]
    b2 = rng.integers(-3, 4, size=D).astype(np.float64)
    Y = oracle.partial_sum(Ps, b2)
    slices = [oracle.partial_reduce_scatter(Ps, r, b2) for r in range(T)]
    assert np.array_equal(np.concatenate(slices, axis=0), Y)
    for r in range(T):
        row0, rows = oracle.token_slice(N, T, r)
        assert np.array_equal(slices[r] - sum(P[row0:row0 + rows] for P in Ps), np.tile(b2, (rows, 1)))


def test_scatter_argument_errors():
    P = [np.zeros((4, 3))] * 2
    with pytest.raises(oracle.OracleError):
        oracle.partial_reduce_scatter(P, 2)
    with pytest.raises(oracle.OracleError):
        oracle.token_slice(4, 0, 0)
