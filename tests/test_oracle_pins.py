"""Pins of the fp64 CPU oracle against what the pages and the mathematics fix.

Every oracle function is pinned by something other than itself: values printed on the pages
(tests/golden), library routines (numpy matmul, torch's gelu, scipy's normal cdf), closed-form
identities, brute-force finite differences and invariants the pages state. A plausible mistake
(a dropped bias, a wrong sign, a transposed operand, b2 added per shard, a wrong shard slice)
fails at least one of them.

Pages cited:
  [Z] zwjcode.cn, "一层 MLP 太宽而放不下时怎样切？列并行、行并行与块尾归约"
  [C] charliedreemur.github.io, "TP:Column / Row Parallel Linear 怎么切? MLP 和 attention 怎么切?"
  [U] unpurerationalist.github.io, "LLM Systems 16: Model Parallel Training"
"""
import json
import math
import os

import numpy as np
import pytest
import scipy.special
import torch

import oracle
from tensor_mlp_block_amd import synth
from tensor_mlp_block_amd.workloads import Workload

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
ACTS = ("identity", "relu", "gelu_tanh", "gelu_erf", "gelu_sigmoid")


def _golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def _normal_case(N, D, F, seed, b_std=0.3, w_std=0.5):
    w = Workload("pin", N=N, D=D, F=F, T=1, act="gelu_tanh", dtype="f32", seed=seed,
                 dist="normal", w_std=w_std, b_std=b_std)
    return (synth.gen_X(w).double().numpy(), synth.gen_W1(w).double().numpy(),
            synth.gen_b1(w).double().numpy(), synth.gen_W2(w).double().numpy(),
            synth.gen_b2(w).double().numpy())


def _int_case(N, D, F, seed):
    w = Workload("pin", N=N, D=D, F=F, T=1, act="relu", dtype="f32", seed=seed, dist="int")
    return (synth.gen_X(w).double().numpy(), synth.gen_W1(w).double().numpy(),
            synth.gen_b1(w).double().numpy(), synth.gen_W2(w).double().numpy(),
            synth.gen_b2(w).double().numpy())


def _torch_act(name, z):
    """The activation by library routines only (torch / numpy / scipy), fp64."""
    t = torch.as_tensor(z, dtype=torch.float64)
    if name == "identity":
        return t.numpy().copy()
    if name == "relu":
        return torch.relu(t).numpy()
    if name == "gelu_erf":
        return torch.nn.functional.gelu(t).numpy()
    if name == "gelu_tanh":
        return torch.nn.functional.gelu(t, approximate="tanh").numpy()
    if name == "gelu_sigmoid":
        return (t * torch.sigmoid(1.702 * t)).numpy()
    raise ValueError(name)


def _torch_act_deriv(name, z):
    t = torch.as_tensor(z, dtype=torch.float64).clone().requires_grad_(True)
    y = torch.as_tensor(_torch_act_graph(name, t))
    y.sum().backward()
    return t.grad.numpy()


def _torch_act_graph(name, t):
    if name == "identity":
        return t * 1.0
    if name == "relu":
        return torch.relu(t)
    if name == "gelu_erf":
        return torch.nn.functional.gelu(t)
    if name == "gelu_tanh":
        return torch.nn.functional.gelu(t, approximate="tanh")
    if name == "gelu_sigmoid":
        return t * torch.sigmoid(1.702 * t)
    raise ValueError(name)


# --------------------------------------------------------------------------------------------
# Values printed on the pages
# --------------------------------------------------------------------------------------------

def test_worked_example_forward_matches_printed_values():
    """[Z 03]: x=[1,2], the 2x4 W1 and 4x2 W2 under ReLU give [4,5] sharded and unsharded."""
    g = _golden("worked_example_fwd.json")
    x, W1, W2, T = np.array(g["x"], float), np.array(g["W1"], float), np.array(g["W2"], float), g["T"]
    partials = []
    for r in range(T):
        Z, H, P = oracle.shard_fwd(x, W1, None, W2, T, r, act=g["act"])
        assert np.array_equal(Z, np.array(g["pre_activation_per_rank"][r], float))
        assert np.array_equal(H, np.array(g["h_per_rank"][r], float))
        assert np.array_equal(P, np.array(g["partial_per_rank"][r], float))
        partials.append(P)
    assert np.array_equal(oracle.partial_sum(partials), np.array(g["Y_sharded"], float))
    assert np.array_equal(oracle.block_fwd(x, W1, None, W2, None, T, act="relu"),
                          np.array(g["Y_sharded"], float))
    assert np.array_equal(oracle.dense_fwd(x, W1, None, W2, None, act="relu"),
                          np.array(g["Y_unsharded"], float))


def test_worked_example_with_b2_adds_it_once():
    """[Z 05]: adding b2 on every rank before the sum gives Y + T*b2. With b2=[1,-1] on the
    worked example (a variant derived here; the page prints no numbers for it) the correct
    result is [5,4] and the per-rank mistake gives [6,3]."""
    g = _golden("worked_example_fwd.json")
    x, W1, W2 = np.array(g["x"], float), np.array(g["W1"], float), np.array(g["W2"], float)
    b2 = np.array([1.0, -1.0])
    Y = oracle.block_fwd(x, W1, None, W2, b2, 2, act="relu")
    assert np.array_equal(Y, [[5.0, 4.0]])
    partials = [oracle.shard_fwd(x, W1, None, W2, 2, r, act="relu")[2] for r in range(2)]
    wrong = oracle.partial_sum([p + b2 for p in partials])
    assert np.array_equal(wrong, [[6.0, 3.0]])
    assert not np.array_equal(wrong, Y)


def test_column_backward_example_is_a_sum_not_a_concatenation():
    """[C 推导 / 关键公式]: X=[1,2], A=[[1,2],[3,4]], dY=[1,1] on two cards give dX
    contributions [1,3] and [2,4]; dX = [3,7]. The column-parallel layer alone is the MLP
    with the identity activation and W2 = I, so the shard backward's dX partial is exactly
    that card's contribution."""
    g = _golden("column_backward_example.json")
    X, A, dY, T = (np.array(g["X"], float), np.array(g["A"], float), np.array(g["dY"], float),
                   g["T"])
    I = np.eye(2)
    parts = []
    for r in range(T):
        out = oracle.shard_bwd(X, A, None, I, dY, T, r, act="identity")
        assert np.array_equal(out["dX"], np.array(g["dX_per_card"][r], float))
        parts.append(out["dX"])
    total = oracle.partial_sum(parts)
    assert np.array_equal(total, np.array(g["dX"], float))
    assert total.size != len(g["not_dX"])
    assert np.array_equal(oracle.dense_bwd(X, A, None, I, dY, act="identity")["dX"],
                          np.array(g["dX"], float))


# --------------------------------------------------------------------------------------------
# Activations: library routines, identities, finite differences
# --------------------------------------------------------------------------------------------

@pytest.mark.parametrize("name", ACTS)
def test_activation_matches_library_routine(name):
    z = np.linspace(-10.0, 10.0, 10001)
    np.testing.assert_allclose(oracle.act(name, z), _torch_act(name, z), rtol=1e-14, atol=1e-15)


def test_gelu_erf_is_z_times_normal_cdf():
    z = np.linspace(-12.0, 12.0, 4801)
    np.testing.assert_allclose(oracle.act("gelu_erf", z), z * scipy.special.ndtr(z),
                               rtol=1e-13, atol=1e-15)


def test_gelu_tanh_close_to_exact_gelu():
    """The tanh form approximates z*Phi(z) closely (absolute gap well under 1e-3)."""
    z = np.linspace(-8.0, 8.0, 3201)
    gap = np.max(np.abs(oracle.act("gelu_tanh", z) - z * scipy.special.ndtr(z)))
    assert 0.0 < gap < 1e-3


@pytest.mark.parametrize("name", ("gelu_tanh", "gelu_erf", "gelu_sigmoid"))
def test_gelu_identities(name):
    """phi(0)=0; phi(z) - phi(-z) = z for every form (the squashing part is odd);
    phi(z)/z -> 1 for large z and phi(z) -> 0 for very negative z."""
    z = np.linspace(-6.0, 6.0, 1201)
    assert oracle.act(name, np.array([0.0]))[0] == 0.0
    np.testing.assert_allclose(oracle.act(name, z) - oracle.act(name, -z), z, rtol=0,
                               atol=1e-14)
    big = oracle.act(name, np.array([40.0, -40.0]))
    assert abs(big[0] / 40.0 - 1.0) < 1e-12 and abs(big[1]) < 1e-12


@pytest.mark.parametrize("name", ACTS)
def test_activation_derivative_by_finite_differences(name):
    z = np.linspace(-5.0, 5.0, 2001)
    z = z[np.abs(z) > 1e-3]  # ReLU has a kink at 0
    h = 1e-6
    fd = (oracle.act(name, z + h) - oracle.act(name, z - h)) / (2 * h)
    np.testing.assert_allclose(oracle.act_deriv(name, z), fd, rtol=0, atol=2e-8)


@pytest.mark.parametrize("name", ACTS)
def test_activation_derivative_matches_autograd(name):
    z = np.linspace(-7.0, 7.0, 1401)
    z = z[np.abs(z) > 1e-9]
    np.testing.assert_allclose(oracle.act_deriv(name, z), _torch_act_deriv(name, z),
                               rtol=1e-12, atol=1e-14)


def test_relu_derivative_at_zero_is_zero():
    """Reading: the gradient passes only where Z > 0."""
    assert oracle.act_deriv("relu", np.array([0.0]))[0] == 0.0


# --------------------------------------------------------------------------------------------
# Forward: library routines, sharded = unsharded, T-invariance, bias ownership
# --------------------------------------------------------------------------------------------

@pytest.mark.parametrize("name", ACTS)
@pytest.mark.parametrize("T", (1, 2, 4))
def test_shard_forward_matches_numpy_matmul(name, T):
    """Each shard step by library routines: numpy fp64 matmul for both projections and the
    library activation. Catches a transposed operand, a wrong shard slice or a lost b1."""
    X, W1, b1, W2, _ = _normal_case(7, 12, 20, seed=11)
    fs = 20 // T
    for r in range(T):
        c = slice(r * fs, (r + 1) * fs)
        Z, H, P = oracle.shard_fwd(X, W1, b1, W2, T, r, act=name)
        Zr = X @ W1[:, c] + b1[c]
        np.testing.assert_allclose(Z, Zr, rtol=1e-13, atol=1e-13)
        Hr = _torch_act(name, Zr)
        np.testing.assert_allclose(H, Hr, rtol=1e-12, atol=1e-13)
        np.testing.assert_allclose(P, Hr @ W2[c, :], rtol=1e-12, atol=1e-12)


def test_identity_t1_reduces_to_two_matmuls():
    X, W1, b1, W2, b2 = _normal_case(9, 16, 24, seed=12)
    Y = oracle.dense_fwd(X, W1, b1, W2, b2, act="identity")
    np.testing.assert_allclose(Y, (X @ W1 + b1) @ W2 + b2, rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("name", ACTS)
@pytest.mark.parametrize("T", (1, 2, 4, 8))
def test_sharded_sum_equals_unsharded(name, T):
    """[Z 02], [C 代码]: the sum of the row-parallel partials plus b2 is the unsharded MLP."""
    X, W1, b1, W2, b2 = _normal_case(6, 10, 32, seed=13)
    Ys = oracle.block_fwd(X, W1, b1, W2, b2, T, act=name)
    Yd = oracle.dense_fwd(X, W1, b1, W2, b2, act=name)
    np.testing.assert_allclose(Ys, Yd, rtol=1e-12, atol=1e-12)


def test_t_invariance_is_exact_on_integer_data():
    """[Z 11]: results must not change with T. Integer data make every order exact."""
    X, W1, b1, W2, b2 = _int_case(16, 16, 64, seed=14)
    ref = oracle.dense_fwd(X, W1, b1, W2, b2, act="relu")
    for T in (1, 2, 4, 8):
        assert np.array_equal(oracle.block_fwd(X, W1, b1, W2, b2, T, act="relu"), ref)


def test_b2_added_exactly_once_and_mutation_is_caught():
    """[Z 05], [U 3.8]: Y - sum_r P^(r) == b2 exactly. The per-shard-b2 mutation yields
    Y + (T-1) b2 and fails the same check."""
    X, W1, b1, W2, b2 = _int_case(16, 16, 64, seed=15)
    assert np.any(b2 != 0)
    T = 4
    partials = [oracle.shard_fwd(X, W1, b1, W2, T, r, act="relu")[2] for r in range(T)]
    Y = oracle.block_fwd(X, W1, b1, W2, b2, T, act="relu")
    raw = oracle.partial_sum(partials)
    assert np.array_equal(Y - raw, np.broadcast_to(b2, Y.shape))
    mutant = oracle.partial_sum([p + b2 for p in partials])
    assert np.array_equal(mutant - Y, np.broadcast_to((T - 1) * b2, Y.shape))
    assert not np.array_equal(mutant - raw, np.broadcast_to(b2, Y.shape))


def test_bias_share_worked_example():
    """[Z 05], the alternative to adding b2 once: every rank adds b2/T to its own partial.
    On the worked example [Z 03] with b2 = [1,-1] (the derived variant above), rank 0
    contributes [1,2] + [0.5,-0.5] = [1.5,1.5], rank 1 [3,3] + [0.5,-0.5] = [3.5,2.5] (by
    hand), and the sum is [5,4], the b2-once result."""
    g = _golden("worked_example_fwd.json")
    parts = [np.array(p, float) for p in g["partial_per_rank"]]
    b2 = np.array([1.0, -1.0])
    assert np.array_equal(oracle.partial_sum_bias_share(parts[:1], b2, 2), [[1.5, 1.5]])
    assert np.array_equal(oracle.partial_sum_bias_share(parts[1:], b2, 2), [[3.5, 2.5]])
    assert np.array_equal(oracle.partial_sum_bias_share(parts, b2, 2), [[5.0, 4.0]])
    assert np.array_equal(oracle.partial_sum_bias_share(parts, None, 2),
                          np.array(g["Y_sharded"], float))


@pytest.mark.parametrize("T", (1, 2, 4, 8))
def test_bias_share_equals_b2_once_for_power_of_two_T(T):
    """[Z 05]: with b2/T on every rank the tail holds b2 exactly once. On integer data and T a
    power of two, b2/T is a short binary fraction, so the result equals the b2-once block
    exactly; forgetting the division (Y + (T-1) b2) or adding the share on one rank only
    (Y - (T-1) b2/T) would not."""
    X, W1, b1, W2, b2 = _int_case(16, 16, 64, seed=16)
    assert np.any(b2 != 0)
    partials = [oracle.shard_fwd(X, W1, b1, W2, T, r, act="relu")[2] for r in range(T)]
    once = oracle.block_fwd(X, W1, b1, W2, b2, T, act="relu")
    share = oracle.partial_sum_bias_share(partials, b2, T)
    assert np.array_equal(share, once)
    assert np.array_equal(share - oracle.partial_sum(partials), np.broadcast_to(b2, share.shape))
    # one rank's contribution carries exactly a 1/T share
    c0 = oracle.partial_sum_bias_share(partials[:1], b2, T)
    assert np.array_equal((c0 - partials[0]) * T, np.broadcast_to(b2, c0.shape))


@pytest.mark.parametrize("T", (3, 6))
def test_bias_share_at_other_T_differs_only_by_rounding(T):
    """For T not a power of two b2/T is inexact; the tail then differs from the b2-once block by
    rounding only (a few fp64 ulps of the largest value), far below the per-rank mistake."""
    X, W1, b1, W2, b2 = _int_case(16, 16, 96, seed=17)
    partials = [oracle.shard_fwd(X, W1, b1, W2, T, r, act="relu")[2] for r in range(T)]
    once = oracle.block_fwd(X, W1, b1, W2, b2, T, act="relu")
    share = oracle.partial_sum_bias_share(partials, b2, T)
    bound = 4 * T * np.finfo(float).eps * np.max(np.abs(once))
    assert np.max(np.abs(share - once)) <= bound
    mutant = oracle.partial_sum([p + b2 for p in partials])
    assert np.max(np.abs(mutant - once)) > 1e6 * bound


def test_b1_shards_concatenate_to_unsharded_preactivation():
    """[Z 05]: the up-projection bias splits with W1's columns, so concatenating every
    shard's Z gives X W1 + b1 (numpy), exactly on integer data."""
    X, W1, b1, W2, _ = _int_case(8, 8, 32, seed=16)
    T = 4
    Zs = [oracle.shard_fwd(X, W1, b1, W2, T, r, act="relu")[0] for r in range(T)]
    assert np.array_equal(np.concatenate(Zs, axis=1), X @ W1 + b1)


@pytest.mark.parametrize("name", ("relu", "gelu_tanh", "gelu_sigmoid"))
def test_row_first_split_counterexample(name):
    """[C MLP 为什么先 column 后 row], [U 3.2]: splitting X by columns and W1 by rows, then
    applying the activation per part, does not give phi(X W1); the linear case does."""
    X, W1, _, _, _ = _normal_case(4, 8, 32, seed=17, w_std=1.0)
    full = oracle.act(name, X @ W1)
    bad = sum(oracle.act(name, X[:, i * 4:(i + 1) * 4] @ W1[i * 4:(i + 1) * 4, :])
              for i in range(2))
    assert not np.allclose(bad, full)
    lin = sum(X[:, i * 4:(i + 1) * 4] @ W1[i * 4:(i + 1) * 4, :] for i in range(2))
    np.testing.assert_allclose(lin, X @ W1, rtol=1e-12, atol=1e-12)


# --------------------------------------------------------------------------------------------
# Backward: brute-force finite differences, library routines, shard identities
# --------------------------------------------------------------------------------------------

def _fd_grads(X, W1, b1, W2, b2, dY, act, h=1e-6):
    """Central differences of the scalar loss <dY, Y(X, W1, b1, W2, b2)> (brute force)."""
    def loss(X_, W1_, b1_, W2_, b2_):
        return float(np.sum(dY * oracle.dense_fwd(X_, W1_, b1_, W2_, b2_, act=act)))

    args = [X, W1, b1, W2, b2]
    grads = []
    for i, a in enumerate(args):
        g = np.zeros_like(a)
        it = np.nditer(a, flags=["multi_index"])
        for _ in it:
            idx = it.multi_index
            plus = [x.copy() for x in args]
            minus = [x.copy() for x in args]
            plus[i][idx] += h
            minus[i][idx] -= h
            g[idx] = (loss(*plus) - loss(*minus)) / (2 * h)
        grads.append(g)
    return dict(zip(("dX", "dW1", "db1", "dW2", "db2"), grads))


@pytest.mark.parametrize("name", ACTS)
def test_dense_backward_matches_finite_differences(name):
    X, W1, b1, W2, b2 = _normal_case(3, 4, 6, seed=18, w_std=0.8, b_std=0.5)
    if name == "relu":  # keep every pre-activation away from the kink
        Z = X @ W1 + b1
        assert np.min(np.abs(Z)) > 1e-3
    dY = _normal_case(3, 4, 6, seed=19)[0]
    fd = _fd_grads(X, W1, b1, W2, b2, dY, name)
    g = oracle.dense_bwd(X, W1, b1, W2, dY, act=name)
    for k in ("dX", "dW1", "db1", "dW2", "db2"):
        np.testing.assert_allclose(g[k], fd[k], rtol=1e-6, atol=1e-7, err_msg=k)


@pytest.mark.parametrize("name", ACTS)
@pytest.mark.parametrize("T", (1, 2, 4))
def test_shard_backward_matches_numpy(name, T):
    """Every backward step by library routines (numpy matmul, torch autograd for phi')."""
    X, W1, b1, W2, _ = _normal_case(7, 12, 20, seed=20)
    dY = _normal_case(7, 12, 20, seed=21)[0]
    fs = 20 // T
    for r in range(T):
        c = slice(r * fs, (r + 1) * fs)
        g = oracle.shard_bwd(X, W1, b1, W2, dY, T, r, act=name)
        Z = X @ W1[:, c] + b1[c]
        H = _torch_act(name, Z)
        dZ = (dY @ W2[c, :].T) * _torch_act_deriv(name, Z)
        np.testing.assert_allclose(g["dZ"], dZ, rtol=1e-11, atol=1e-12)
        np.testing.assert_allclose(g["dW2"], H.T @ dY, rtol=1e-11, atol=1e-12)
        np.testing.assert_allclose(g["dW1"], X.T @ dZ, rtol=1e-11, atol=1e-12)
        np.testing.assert_allclose(g["db1"], dZ.sum(axis=0), rtol=1e-11, atol=1e-12)
        np.testing.assert_allclose(g["dX"], dZ @ W1[:, c].T, rtol=1e-11, atol=1e-12)


@pytest.mark.parametrize("T", (2, 4, 8))
def test_shard_backward_slices_and_sums_to_dense(T):
    """[Z 06], [U 3.6.1]: each shard's weight gradients are slices of the dense ones (no
    exchange); the dX partials sum to the dense dX (the column-parallel all-reduce)."""
    X, W1, b1, W2, _ = _normal_case(5, 8, 32, seed=22)
    dY = _normal_case(5, 8, 32, seed=23)[0]
    dense = oracle.dense_bwd(X, W1, b1, W2, dY, act="gelu_tanh")
    fs = 32 // T
    parts = []
    for r in range(T):
        c = slice(r * fs, (r + 1) * fs)
        g = oracle.shard_bwd(X, W1, b1, W2, dY, T, r, act="gelu_tanh")
        np.testing.assert_allclose(g["dW1"], dense["dW1"][:, c], rtol=1e-12, atol=1e-13)
        np.testing.assert_allclose(g["dW2"], dense["dW2"][c, :], rtol=1e-12, atol=1e-13)
        np.testing.assert_allclose(g["db1"], dense["db1"][c], rtol=1e-12, atol=1e-13)
        parts.append(g["dX"])
    np.testing.assert_allclose(oracle.partial_sum(parts), dense["dX"], rtol=1e-12, atol=1e-12)


def test_negative_number_relu_exercise():
    """[Z 14] exercise 3: the worked example with negative entries under ReLU; the full path
    and the two-card path agree, and dY0/dx from the oracle's backward (dY = e0) matches
    brute-force finite differences. The page prints no answer, so the pin is the FD check."""
    x = np.array([[1.0, -2.0]])
    W1 = np.array([[1.0, 0.0, 1.0, 2.0], [0.0, 1.0, 1.0, -1.0]])
    W2 = np.array([[1.0, 0.0], [0.0, 1.0], [1.0, 1.0], [2.0, -1.0]])
    Ys = oracle.block_fwd(x, W1, None, W2, None, 2, act="relu")
    Yd = oracle.dense_fwd(x, W1, None, W2, None, act="relu")
    assert np.array_equal(Ys, Yd)
    # pre-activations [1,-2,-1,4]: relu -> [1,0,0,4]; Y = [1+8, -4] = [9,-4]
    assert np.array_equal(Yd, [[9.0, -4.0]])
    e0 = np.array([[1.0, 0.0]])
    parts = [oracle.shard_bwd(x, W1, None, W2, e0, 2, r, act="relu")["dX"] for r in range(2)]
    dx = oracle.partial_sum(parts)
    h = 1e-6
    fd = np.array([[(oracle.dense_fwd(x + h * np.eye(2)[i], W1, None, W2, None, act="relu")[0, 0]
                     - oracle.dense_fwd(x - h * np.eye(2)[i], W1, None, W2, None, act="relu")[0, 0])
                    / (2 * h) for i in range(2)]])
    np.testing.assert_allclose(dx, fd, rtol=1e-9, atol=1e-9)
    assert np.array_equal(dx, [[5.0, -2.0]])


# --------------------------------------------------------------------------------------------
# Argument checking
# --------------------------------------------------------------------------------------------

def test_oracle_rejects_bad_arguments():
    X, W1, b1, W2, _ = _normal_case(2, 4, 6, seed=24)
    with pytest.raises(oracle.OracleError, match="-3"):
        oracle.shard_fwd(X, W1, b1, W2, 4, 0)          # 4 does not divide F=6 [U 3.8]
    with pytest.raises(oracle.OracleError, match="-2"):
        oracle.shard_fwd(X, W1, b1, W2, 2, 2)          # r outside [0, T)
    with pytest.raises(oracle.OracleError):
        oracle.act("swish", np.zeros(3))


def test_shape_examples_from_the_pages():
    """[C 先弄清楚]: W [8192, 32768] split 8 ways by columns is [8192, 4096] per card, and
    A [8, 32] split 2 ways is [8, 16]. The oracle's shard outputs carry that width."""
    X = np.ones((1, 8))
    A = np.ones((8, 32))
    B = np.ones((32, 8))
    Z, H, P = oracle.shard_fwd(X, A, None, B, 2, 1, act="identity")
    assert Z.shape == (1, 16) and P.shape == (1, 8)
    assert math.prod((8192, 32768)) // 8 == 8192 * 4096
