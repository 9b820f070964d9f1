"""Pins of the CPU oracle against things other than itself.

The oracle (oracle/moe_oracle.cc) is the parity reference for the GPU library,
so each of its functions is tied here to brute force, closed forms, library
routines on special cases, or invariants that a plausible slip (a transposed
operand, a swapped gate/up branch, a wrong sign, a lost tie rule, an
off-by-one in the permutation) would break.  Pages (by title):
"Step 3.5 Flash: Open Frontier-Level Intelligence with 11B Active Parameters"
(§2.2, §2.2.2, §4.1.2) and "Step 3.5 Flash 技术论文深度解读" (architecture
table; SwiGLU gate/up branches in the activation-explosion causes).
"""
import itertools

import numpy as np
import pytest
import scipy.special
import torch
import torch.nn.functional as F

import oracle
from tests._util import from_bf16, rand_bf16, rel_l2, to_bf16


def _beta(scores, bias):
    # Biased score in float32, as the routing definition adds them.
    return (scores.astype(np.float32) + bias.astype(np.float32)).astype(np.float32)


def _brute_force_topk(beta_row, k):
    """Best k-subset by total biased score; among equal totals the
    lexicographically smallest sorted index tuple (= lower index wins)."""
    best, best_sum = None, None
    for sub in itertools.combinations(range(len(beta_row)), k):
        s = float(np.sum(beta_row[list(sub)].astype(np.float64)))
        if best is None or s > best_sum:
            best, best_sum = sub, s
    return np.array(best, np.int32)


# ---------------------------------------------------------------- routing --

@pytest.mark.parametrize("E,k", [(5, 1), (8, 2), (8, 3), (16, 2), (12, 3)])
def test_route_matches_brute_force_subsets(E, k):
    rng = np.random.default_rng(100 + E * 10 + k)
    T, d = 24, 64
    x = rand_bf16(rng, (T, d))
    wr = rand_bf16(rng, (E, d), 0.05)
    b = rng.uniform(-0.05, 0.05, E).astype(np.float32)
    ids, w, gap, s = oracle.route(x, wr, b, k, want_scores=True)
    beta = _beta(s, b)
    for t in range(T):
        np.testing.assert_array_equal(ids[t], _brute_force_topk(beta[t], k))
        srt = np.sort(beta[t].astype(np.float64))[::-1]
        assert gap[t] == np.float32(srt[k - 1] - srt[k])


def test_route_tie_goes_to_lower_index():
    # Experts 1 and 4 (and 2 and 6) get identical router rows and biases, so
    # their biased scores tie exactly; the lower index must win.
    rng = np.random.default_rng(7)
    T, d, E, k = 16, 64, 8, 3
    x = rand_bf16(rng, (T, d))
    wr = rand_bf16(rng, (E, d), 0.05)
    wr[4] = wr[1]
    wr[6] = wr[2]
    b = np.zeros(E, np.float32)
    ids, _, gap, s = oracle.route(x, wr, b, k, want_scores=True)
    beta = _beta(s, b)
    assert np.all(beta[:, 1] == beta[:, 4])
    for t in range(T):
        np.testing.assert_array_equal(ids[t], _brute_force_topk(beta[t], k))
    # All experts tied: the first k indices are chosen.
    ids0, w0, gap0, _ = oracle.route(np.zeros((3, d), np.uint16), wr, b, k)
    np.testing.assert_array_equal(ids0, np.tile(np.arange(k), (3, 1)))
    np.testing.assert_array_equal(gap0, 0.0)
    np.testing.assert_allclose(w0, 1.0 / k, rtol=1e-7)


@pytest.mark.parametrize("E,k", [(64, 8), (288, 8), (288, 16)])
def test_route_many_ties_at_full_expert_count(E, k):
    # x = 0 makes every score 0.5, so the biased scores tie in whole groups
    # (bias drawn from a handful of values); the chosen set must be the k
    # best bias values with the lowest indices inside the tied group.
    rng = np.random.default_rng(E + k)
    d = 64
    wr = rand_bf16(rng, (E, d), 0.05)
    b = (rng.integers(0, 4, E) * 0.125).astype(np.float32)
    x = np.zeros((4, d), np.uint16)
    ids, w, gap, _ = oracle.route(x, wr, b, k)
    order = np.lexsort((np.arange(E), -b.astype(np.float64)))
    for t in range(4):
        np.testing.assert_array_equal(ids[t], np.sort(order[:k]))


def test_route_scores_are_library_sigmoid_of_logits():
    rng = np.random.default_rng(11)
    T, d, E, k = 32, 256, 16, 2
    x = rand_bf16(rng, (T, d))
    wr = rand_bf16(rng, (E, d), 0.02)
    b = np.zeros(E, np.float32)
    c = rng.uniform(-1, 1, E).astype(np.float32)
    _, _, _, s = oracle.route(x, wr, b, k, logit_bias=c, want_scores=True)
    z = from_bf16(x).astype(np.float64) @ from_bf16(wr).astype(np.float64).T + c.astype(np.float64)
    np.testing.assert_allclose(s, scipy.special.expit(z), rtol=0, atol=3e-7)


def test_route_one_hot_router_closed_form():
    # Router row e is a_e times the unit vector at column pi(e) (pi not an
    # involution), so z[t,e] = a_e * x[t, pi(e)] exactly: a transposed router
    # or a wrong sign would select different experts.
    rng = np.random.default_rng(12)
    T, d, E, k = 40, 64, 10, 3
    pi = rng.permutation(d)[:E]
    a = np.linspace(0.5, 2.0, E).astype(np.float32)
    wr_f = np.zeros((E, d), np.float32)
    wr_f[np.arange(E), pi] = a
    wr = to_bf16(wr_f)
    x = rand_bf16(rng, (T, d))
    b = rng.uniform(-0.1, 0.1, E).astype(np.float32)
    ids, w, _, s = oracle.route(x, wr, b, k, want_scores=True)
    z = from_bf16(x)[:, pi].astype(np.float64) * from_bf16(wr)[np.arange(E), pi].astype(np.float64)
    np.testing.assert_allclose(s, scipy.special.expit(z), rtol=0, atol=1e-7)
    beta = _beta(s, b)
    for t in range(T):
        order = np.lexsort((np.arange(E), -beta[t].astype(np.float64)))
        np.testing.assert_array_equal(ids[t], np.sort(order[:k]))
        np.testing.assert_allclose(w[t], s[t, ids[t]] / s[t, ids[t]].astype(np.float64).sum(), rtol=1e-6)


def test_forced_selection_by_bias():
    # Scores lie in (0, 1), so +1 on a k-set forces that set for every token.
    rng = np.random.default_rng(13)
    T, d, E, k = 50, 128, 16, 3
    S = np.array([2, 9, 14])
    x = rand_bf16(rng, (T, d))
    wr = rand_bf16(rng, (E, d), 0.05)
    b = np.zeros(E, np.float32)
    b[S] = 1.0
    ids, w, _, s = oracle.route(x, wr, b, k, want_scores=True)
    np.testing.assert_array_equal(ids, np.tile(S, (T, 1)))
    # Weights use the unbiased scores of the chosen set.
    expect = s[:, S] / s[:, S].astype(np.float64).sum(1, keepdims=True)
    np.testing.assert_allclose(w, expect, rtol=1e-6)


def test_all_tokens_to_one_expert_and_k1_weight_is_one():
    rng = np.random.default_rng(14)
    T, d, E = 33, 64, 8
    x = rand_bf16(rng, (T, d))
    wr = rand_bf16(rng, (E, d), 0.05)
    b = np.zeros(E, np.float32)
    b[5] = 10.0
    ids, w, gap, _ = oracle.route(x, wr, b, 1)
    assert np.all(ids == 5)
    assert np.all(w == 1.0)
    assert np.all(gap > 8.0)
    b2 = rng.uniform(-0.05, 0.05, E).astype(np.float32)
    _, w2, _, _ = oracle.route(x, wr, b2, 1)
    assert np.all(w2 == 1.0)


def test_bias_is_used_for_selection_only():
    rng = np.random.default_rng(15)
    T, d, E, k = 30, 128, 12, 3
    x = rand_bf16(rng, (T, d))
    wr = rand_bf16(rng, (E, d), 0.05)
    b = rng.uniform(-0.05, 0.05, E).astype(np.float32)
    ids, w, gap, _ = oracle.route(x, wr, b, k)
    # Shift all biases by the same amount: the set cannot change (up to
    # rounding of beta, which the gap bounds), and the weights must not move.
    for shift in (0.25, -0.125, 0.0625):
        ids2, w2, _, _ = oracle.route(x, wr, b + np.float32(shift), k)
        safe = gap > 1e-6
        np.testing.assert_array_equal(ids2[safe], ids[safe])
        np.testing.assert_array_equal(w2[safe], w[safe])
    # Lower the bias of every expert outside each token's set: same set, same
    # weights, bit for bit.
    for t in range(T):
        b3 = b.copy()
        out = np.setdiff1d(np.arange(E), ids[t])
        b3[out] -= 0.5
        ids3, w3, _, _ = oracle.route(x[t:t + 1], wr, b3, k)
        np.testing.assert_array_equal(ids3[0], ids[t])
        np.testing.assert_array_equal(w3[0], w[t])


def test_k_equals_E_weights_are_normalised_library_sigmoids():
    rng = np.random.default_rng(16)
    T, d, E = 20, 64, 6
    x = rand_bf16(rng, (T, d))
    wr = rand_bf16(rng, (E, d), 0.1)
    b = rng.uniform(-0.1, 0.1, E).astype(np.float32)
    ids, w, gap, _ = oracle.route(x, wr, b, E)
    np.testing.assert_array_equal(ids, np.tile(np.arange(E), (T, 1)))
    assert np.all(np.isinf(gap))
    z = from_bf16(x).astype(np.float64) @ from_bf16(wr).astype(np.float64).T
    s = scipy.special.expit(z)
    np.testing.assert_allclose(w, s / s.sum(1, keepdims=True), rtol=2e-6)


@pytest.mark.parametrize("T,d,E,k,bias", [(64, 256, 16, 2, 0.05), (48, 512, 288, 8, 0.1)])
def test_route_invariants(T, d, E, k, bias):
    rng = np.random.default_rng(T + E)
    x = rand_bf16(rng, (T, d))
    wr = rand_bf16(rng, (E, d), 0.02)
    b = rng.uniform(-bias, bias, E).astype(np.float32)
    ids, w, gap, _ = oracle.route(x, wr, b, k)
    assert ids.shape == (T, k)
    assert np.all((ids >= 0) & (ids < E))
    assert np.all(np.diff(ids, axis=1) > 0)          # distinct and ascending
    assert np.all(w >= 0)
    np.testing.assert_allclose(w.astype(np.float64).sum(1), 1.0, atol=1e-6)
    assert np.all(gap >= 0)


# ------------------------------------------------------------ permutation --

def _random_ids(rng, T, E, k):
    return np.stack([np.sort(rng.choice(E, k, replace=False)) for _ in range(T)]).astype(np.int32).reshape(T, k)


@pytest.mark.parametrize("T,E,k", [(0, 8, 2), (1, 8, 8), (37, 16, 2), (200, 64, 8), (513, 288, 8)])
def test_permute_is_stable_counting_sort(T, E, k):
    rng = np.random.default_rng(T * 7 + E)
    ids = _random_ids(rng, T, E, k) if T else np.zeros((0, k), np.int32)
    counts, offsets, perm, pos = oracle.permute(ids, E)
    flat = ids.ravel()
    np.testing.assert_array_equal(counts, np.bincount(flat, minlength=E))
    np.testing.assert_array_equal(offsets, np.concatenate([[0], np.cumsum(np.bincount(flat, minlength=E))]))
    np.testing.assert_array_equal(perm, np.argsort(flat, kind="stable"))
    # Invariants: bijection, inverse, grouping.
    assert counts.sum() == T * k and offsets[-1] == T * k
    assert np.all(np.diff(offsets) >= 0)
    np.testing.assert_array_equal(np.sort(perm), np.arange(T * k))
    np.testing.assert_array_equal(pos[perm], np.arange(T * k))
    for e in range(E):
        rows = perm[offsets[e]:offsets[e + 1]]
        assert np.all(flat[rows] == e)
        assert np.all(np.diff(rows // k) > 0)            # ascending token order


def test_permute_skewed_loads():
    T, E, k = 100, 16, 2
    ids = np.zeros((T, k), np.int32)
    ids[:, 0] = 3
    ids[:, 1] = 7
    counts, offsets, perm, pos = oracle.permute(ids, E)
    assert counts[3] == T and counts[7] == T and counts.sum() == 2 * T
    np.testing.assert_array_equal(perm[:T], np.arange(T) * 2)
    np.testing.assert_array_equal(perm[T:], np.arange(T) * 2 + 1)


# ----------------------------------------------------------------- experts --

def _torch_swiglu(x, w_gu, w_d):
    """Textbook SwiGLU with library routines, float64: W_d (silu(W_g x) * W_u x)."""
    xt = torch.from_numpy(from_bf16(x).astype(np.float64))
    gu = torch.from_numpy(from_bf16(w_gu).astype(np.float64))
    wd = torch.from_numpy(from_bf16(w_d).astype(np.float64))
    h = gu.shape[0] // 2
    a = F.silu(xt @ gu[:h].T) * (xt @ gu[h:].T)
    return (a @ wd.T).numpy()


def test_expert_permutation_matrix_closed_form():
    # W_g row j = c_j e_{pi(j)}, W_u row j = e_{rho(j)}, W_d row i = e_{tau(i)}:
    # out_i = silu(c_tau(i) x_{pi(tau(i))}) * x_{rho(tau(i))}.  Swapping the
    # gate and up halves, transposing any matrix or flipping SiLU's sign
    # changes the result.
    rng = np.random.default_rng(21)
    d, h = 64, 32
    pi = rng.permutation(d)[:h]
    rho = rng.permutation(d)[:h]
    tau = rng.integers(0, h, d)
    c = np.linspace(-3, 3, h).astype(np.float32)
    gu = np.zeros((2 * h, d), np.float32)
    gu[np.arange(h), pi] = c
    gu[h + np.arange(h), rho] = 1.0
    wd = np.zeros((d, h), np.float32)
    wd[np.arange(d), tau] = 1.0
    x = rand_bf16(rng, d)
    out = oracle.expert(x, to_bf16(gu), to_bf16(wd))
    xf = from_bf16(x).astype(np.float64)
    cf = from_bf16(to_bf16(c)).astype(np.float64)
    g = cf[tau] * xf[pi[tau]]
    expect = F.silu(torch.from_numpy(g)).numpy() * xf[rho[tau]]
    np.testing.assert_allclose(out, expect, rtol=1e-6, atol=1e-30)


def test_expert_clamped_closed_form():
    # The permutation-matrix expert again: out_i is one hidden activation, so
    # clipping shows up element by element as numpy's clip of the closed form.
    # A clamp above every activation changes nothing.
    rng = np.random.default_rng(23)
    d, h = 64, 32
    pi = rng.permutation(d)[:h]
    rho = rng.permutation(d)[:h]
    tau = rng.integers(0, h, d)
    c = np.linspace(-3, 3, h).astype(np.float32)
    gu = np.zeros((2 * h, d), np.float32)
    gu[np.arange(h), pi] = c
    gu[h + np.arange(h), rho] = 2.5
    wd = np.zeros((d, h), np.float32)
    wd[np.arange(d), tau] = 1.0
    x = rand_bf16(rng, d, 2.0)
    xf = from_bf16(x).astype(np.float64)
    cf = from_bf16(to_bf16(c)).astype(np.float64)
    act = F.silu(torch.from_numpy(cf[tau] * xf[pi[tau]])).numpy() * 2.5 * xf[rho[tau]]
    for clamp in (0.05, 0.5, 2.0):
        out = oracle.expert_clamped(x, to_bf16(gu), to_bf16(wd), clamp)
        np.testing.assert_allclose(out, np.clip(act, -clamp, clamp), rtol=1e-6, atol=1e-30)
        assert np.any(np.abs(act) > clamp)
    big = float(np.abs(act).max()) * 2
    np.testing.assert_array_equal(oracle.expert_clamped(x, to_bf16(gu), to_bf16(wd), big),
                                  oracle.expert(x, to_bf16(gu), to_bf16(wd)))
    with pytest.raises(ValueError):
        oracle.expert_clamped(x, to_bf16(gu), to_bf16(wd), 0.0)


def test_expert_matches_library_swiglu():
    rng = np.random.default_rng(22)
    d, h = 128, 64
    gu = rand_bf16(rng, (2 * h, d), 0.05)
    wd = rand_bf16(rng, (d, h), 0.05)
    for _ in range(4):
        x = rand_bf16(rng, d)
        out = oracle.expert(x, gu, wd)
        ref = _torch_swiglu(x[None], gu, wd)[0]
        assert rel_l2(out, ref) < 1e-6


def test_expert_zero_input_gives_zero():
    rng = np.random.default_rng(23)
    d, h = 64, 32
    out = oracle.expert(np.zeros(d, np.uint16), rand_bf16(rng, (2 * h, d)), rand_bf16(rng, (d, h)))
    assert np.all(out == 0)


# ------------------------------------------------------------- whole layer --

def _layer_inputs(rng, T, d, E, k, h, hs, bias=0.05):
    x = rand_bf16(rng, (T, d))
    wr = rand_bf16(rng, (E, d), 0.05)
    b = rng.uniform(-bias, bias, E).astype(np.float32)
    gu = [rand_bf16(rng, (2 * h, d), 0.05) for _ in range(E)]
    wd = [rand_bf16(rng, (d, h), 0.05) for _ in range(E)]
    sgu = rand_bf16(rng, (2 * hs, d), 0.05) if hs else None
    swd = rand_bf16(rng, (d, hs), 0.05) if hs else None
    return x, wr, b, gu, wd, sgu, swd


def test_layer_identical_experts_closed_form():
    # Every expert has the same weights, so the routed part is
    # routed_scale * SwiGLU(x) (weights sum to one) whatever the routing.
    rng = np.random.default_rng(31)
    T, d, E, k, h, hs = 12, 64, 8, 3, 32, 16
    x, wr, b, gu, wd, sgu, swd = _layer_inputs(rng, T, d, E, k, h, hs)
    gu = [gu[0]] * E
    wd = [wd[0]] * E
    for lam in (1.0, 0.5):
        _, _, _, y = oracle.layer(x, wr, b, k, gu, wd, sgu, swd, routed_scale=lam)
        ref = lam * _torch_swiglu(x, gu[0], wd[0]) + _torch_swiglu(x, sgu, swd)
        assert rel_l2(y, ref) < 2e-6


def test_layer_single_expert_is_dense_swiglu_plus_shared():
    rng = np.random.default_rng(32)
    T, d, E, k, h, hs = 9, 128, 1, 1, 64, 32
    x, wr, b, gu, wd, sgu, swd = _layer_inputs(rng, T, d, E, k, h, hs)
    ids, w, _, y = oracle.layer(x, wr, b, k, gu, wd, sgu, swd)
    assert np.all(ids == 0) and np.all(w == 1.0)
    ref = _torch_swiglu(x, gu[0], wd[0]) + _torch_swiglu(x, sgu, swd)
    assert rel_l2(y, ref) < 1e-6


def test_layer_weighted_sum_over_chosen_experts():
    # Output = shared + sum_j w_j * expert_j(x) with w from library sigmoids of
    # the chosen experts; experts pinned by the tests above.
    rng = np.random.default_rng(33)
    T, d, E, k, h, hs = 10, 64, 6, 2, 32, 32
    x, wr, b, gu, wd, sgu, swd = _layer_inputs(rng, T, d, E, k, h, hs)
    ids, w, _, y = oracle.layer(x, wr, b, k, gu, wd, sgu, swd)
    z = from_bf16(x).astype(np.float64) @ from_bf16(wr).astype(np.float64).T
    s = scipy.special.expit(z)
    ref_sh = _torch_swiglu(x, sgu, swd)
    for t in range(T):
        sel = ids[t]
        wt = s[t, sel] / s[t, sel].sum()
        np.testing.assert_allclose(w[t], wt, rtol=2e-6)
        routed = sum(wt[j] * _torch_swiglu(x[t:t + 1], gu[e], wd[e])[0] for j, e in enumerate(sel))
        assert rel_l2(y[t], ref_sh[t] + routed) < 2e-6


def test_layer_zero_input_and_shared_off():
    rng = np.random.default_rng(34)
    T, d, E, k, h, hs = 6, 64, 8, 2, 32, 32
    x, wr, b, gu, wd, sgu, swd = _layer_inputs(rng, T, d, E, k, h, hs)
    ids0, w0, _, y0 = oracle.layer(np.zeros_like(x), wr, b, k, gu, wd, sgu, swd)
    assert np.all(y0 == 0)
    # z = 0 gives equal scores: selection is by bias alone, weights equal.
    order = np.lexsort((np.arange(E), -b.astype(np.float64)))
    np.testing.assert_array_equal(ids0, np.tile(np.sort(order[:k]), (T, 1)))
    np.testing.assert_allclose(w0, 1.0 / k, rtol=1e-7)
    # Shared expert off = full output minus the shared expert's output.
    _, _, _, y_full = oracle.layer(x, wr, b, k, gu, wd, sgu, swd)
    _, _, _, y_routed = oracle.layer(x, wr, b, k, gu, wd)
    assert rel_l2(y_full - y_routed, _torch_swiglu(x, sgu, swd)) < 2e-6
    # routed_scale = 0 leaves only the shared expert.
    _, _, _, y_sh = oracle.layer(x, wr, b, k, gu, wd, sgu, swd, routed_scale=0.0)
    assert rel_l2(y_sh, _torch_swiglu(x, sgu, swd)) < 1e-6


def test_layer_token_subset_matches_full():
    rng = np.random.default_rng(35)
    T, d, E, k, h, hs = 16, 64, 8, 2, 32, 32
    x, wr, b, gu, wd, sgu, swd = _layer_inputs(rng, T, d, E, k, h, hs)
    ids, w, gap, y = oracle.layer(x, wr, b, k, gu, wd, sgu, swd)
    sub = np.array([15, 3, 7])
    ids2, w2, gap2, y2 = oracle.layer(x, wr, b, k, gu, wd, sgu, swd, tokens=sub)
    np.testing.assert_array_equal(ids2, ids[sub])
    np.testing.assert_array_equal(y2, y[sub])
    # Missing weights for a selected expert is an error, not a silent zero.
    gu_missing = list(gu)
    gu_missing[int(ids[0, 0])] = None
    wd_missing = list(wd)
    wd_missing[int(ids[0, 0])] = None
    with pytest.raises(ValueError):
        oracle.layer(x, wr, b, k, gu_missing, wd_missing, sgu, swd, tokens=np.array([0]))


# ------------------------------------------------ layer under given routing --
# [Blog] §2.2.2: the output is defined by the top-K set S_t and its mask; the
# oracle's forward_given_routing takes S_t as an input.

def _perm_expert(rng, d, h, scale):
    """A permutation-matrix expert (see test_expert_permutation_matrix_closed_form)
    and its closed form as a function of x (float64)."""
    pi = rng.permutation(d)[:h]
    rho = rng.permutation(d)[:h]
    tau = rng.integers(0, h, d)
    c = (np.linspace(-2, 2, h) * scale).astype(np.float32)
    gu = np.zeros((2 * h, d), np.float32)
    gu[np.arange(h), pi] = c
    gu[h + np.arange(h), rho] = 1.0
    wd = np.zeros((d, h), np.float32)
    wd[np.arange(d), tau] = 1.0
    cf = from_bf16(to_bf16(c)).astype(np.float64)

    def closed(xf):
        return F.silu(torch.from_numpy(cf[tau] * xf[pi[tau]])).numpy() * xf[rho[tau]]
    return to_bf16(gu), to_bf16(wd), closed


def test_given_routing_equals_layer_on_its_own_sets():
    rng = np.random.default_rng(61)
    T, d, E, k, h, hs = 14, 64, 8, 3, 32, 16
    x, wr, b, gu, wd, sgu, swd = _layer_inputs(rng, T, d, E, k, h, hs)
    c = rng.uniform(-0.5, 0.5, E).astype(np.float32)
    ids, w, _, y = oracle.layer(x, wr, b, k, gu, wd, sgu, swd, routed_scale=0.75, logit_bias=c)
    w2, y2 = oracle.forward_given_routing(x, wr, ids, gu, wd, sgu, swd, routed_scale=0.75, logit_bias=c)
    np.testing.assert_array_equal(w2, w)
    np.testing.assert_array_equal(y2, y)
    sub = np.array([9, 2])
    _, y3 = oracle.forward_given_routing(x, wr, ids[sub], gu, wd, sgu, swd, routed_scale=0.75, logit_bias=c,
                                         tokens=sub)
    np.testing.assert_array_equal(y3, y[sub])


def test_given_routing_one_expert_is_that_expert_plus_shared():
    # k = 1 with a set the router would not pick: weight exactly 1, output
    # the chosen expert plus the shared expert (library SwiGLU).
    rng = np.random.default_rng(62)
    T, d, E, k, h, hs = 7, 128, 6, 1, 32, 32
    x, wr, b, gu, wd, sgu, swd = _layer_inputs(rng, T, d, E, k, h, hs)
    own, _, _, _ = oracle.route(x, wr, b, 1)
    ids = ((own + 3) % E).astype(np.int32)
    w, y = oracle.forward_given_routing(x, wr, ids, gu, wd, sgu, swd)
    assert np.all(w == 1.0)
    for t in range(T):
        e = int(ids[t, 0])
        ref = _torch_swiglu(x[t:t + 1], gu[e], wd[e])[0] + _torch_swiglu(x[t:t + 1], sgu, swd)[0]
        assert rel_l2(y[t], ref) < 1e-6


def test_given_routing_selects_the_named_experts_closed_form():
    # Every expert is a different permutation-matrix expert, so each output
    # element names which expert produced it; the given sets are arbitrary
    # (not the router's), the weights library sigmoids of those experts'
    # logits renormalised over the set.  Using slot j's expert for slot j+1,
    # the router's own set, biased scores or unnormalised weights all fail.
    rng = np.random.default_rng(63)
    T, d, E, k, h = 10, 64, 7, 3, 32
    experts = [_perm_expert(rng, d, h, 1.0 + 0.3 * e) for e in range(E)]
    gu = [e[0] for e in experts]
    wd = [e[1] for e in experts]
    x = rand_bf16(rng, (T, d))
    wr = rand_bf16(rng, (E, d), 0.2)
    c = rng.uniform(-1, 1, E).astype(np.float32)
    ids = np.stack([np.sort(rng.choice(E, k, replace=False)) for _ in range(T)]).astype(np.int32)
    w, y = oracle.forward_given_routing(x, wr, ids, gu, wd, routed_scale=1.5, logit_bias=c)
    z = from_bf16(x).astype(np.float64) @ from_bf16(wr).astype(np.float64).T + c.astype(np.float64)
    s = scipy.special.expit(z)
    for t in range(T):
        wt = s[t, ids[t]] / s[t, ids[t]].sum()
        np.testing.assert_allclose(w[t], wt, rtol=2e-6)
        xf = from_bf16(x[t]).astype(np.float64)
        ref = 1.5 * sum(wt[j] * experts[e][2](xf) for j, e in enumerate(ids[t]))
        np.testing.assert_allclose(y[t], ref, rtol=2e-6, atol=1e-7)


def test_given_routing_rejects_invalid_sets():
    rng = np.random.default_rng(64)
    T, d, E, k, h, hs = 2, 64, 6, 2, 32, 0
    x, wr, b, gu, wd, _, _ = _layer_inputs(rng, T, d, E, k, h, hs)
    for bad in ([[1, 1], [0, 2]], [[2, 1], [0, 2]], [[0, 6], [1, 2]], [[-1, 3], [1, 2]]):
        with pytest.raises(ValueError):
            oracle.forward_given_routing(x, wr, np.array(bad, np.int32), gu, wd)


# ---------------------------------------------------------------- combine --

def test_combine_closed_forms():
    rng = np.random.default_rng(51)
    T, d, k = 20, 64, 4
    P = T * k
    # Row r of y_perm holds the value r in every column (exact in bf16 up to
    # 256), so a gather through the wrong index shows up as a wrong value.
    y_perm = to_bf16(np.repeat(np.arange(P, dtype=np.float32)[:, None], d, axis=1))
    pos = rng.permutation(P).astype(np.int32)
    # One-hot weights pick exactly one slot.
    for j in range(k):
        w = np.zeros((T, k), np.float32)
        w[:, j] = 1.0
        y = oracle.combine(y_perm, pos, w)
        np.testing.assert_array_equal(y, np.repeat(pos.reshape(T, k)[:, j:j + 1].astype(np.float32), d, axis=1))
    # Equal weights give the mean of the gathered row indices; shared adds;
    # routed_scale scales only the routed part.
    w = np.full((T, k), 1.0 / k, np.float32)
    sh = rng.standard_normal((T, d)).astype(np.float32)
    y = oracle.combine(y_perm, pos, w, sh, routed_scale=2.0)
    expect = sh.astype(np.float64) + 2.0 * pos.reshape(T, k).mean(1)[:, None]
    np.testing.assert_allclose(y, expect, rtol=1e-6)
    # Random rows and weights: linear in the weights.
    y_perm2 = rand_bf16(rng, (P, d))
    w2 = rng.random((T, k)).astype(np.float32)
    a = oracle.combine(y_perm2, pos, w2)
    b = oracle.combine(y_perm2, pos, (2 * w2).astype(np.float32))
    np.testing.assert_allclose(b, 2 * a, rtol=1e-6)


def test_combine_residual_is_added_once():
    # The skip connection: zero expert outputs give the residual back exactly;
    # otherwise the residual adds to the output of the call without it (the
    # two differ only by the final f32 rounding).
    rng = np.random.default_rng(52)
    T, d, k = 12, 64, 3
    P = T * k
    pos = rng.permutation(P).astype(np.int32)
    res = rand_bf16(rng, (T, d), 2.0)
    w = rng.random((T, k)).astype(np.float32)
    zero = np.zeros((P, d), np.uint16)
    np.testing.assert_array_equal(oracle.combine(zero, pos, w, residual=res), from_bf16(res))
    y_perm = rand_bf16(rng, (P, d))
    sh = rng.standard_normal((T, d)).astype(np.float32)
    a = oracle.combine(y_perm, pos, w, sh, routed_scale=0.5)
    b = oracle.combine(y_perm, pos, w, sh, routed_scale=0.5, residual=res)
    np.testing.assert_allclose(b, a.astype(np.float64) + from_bf16(res), rtol=2e-7, atol=1e-6)
    # The residual is not scaled with the routed part.
    c = oracle.combine(y_perm, pos, w, None, routed_scale=0.0, residual=res)
    np.testing.assert_array_equal(c, from_bf16(res))


# ---------------------------------------------------------------- rmsnorm --

def test_rmsnorm_matches_library_and_is_scale_invariant():
    rng = np.random.default_rng(41)
    T, d = 16, 256
    v = rand_bf16(rng, (T, d), 3.0)
    out = oracle.rmsnorm(v, eps=0.0)
    ref = F.rms_norm(torch.from_numpy(from_bf16(v).astype(np.float64)), (d,), eps=0.0)
    ref_bf16 = to_bf16(ref.numpy().astype(np.float32))
    diff = np.abs(out.astype(np.int32) - ref_bf16.astype(np.int32))
    assert diff.max() <= 1 and (diff == 0).mean() > 0.999
    # Power-of-two scaling of the input is exact, so the output is unchanged.
    v4 = to_bf16(from_bf16(v) * 4.0)
    np.testing.assert_array_equal(oracle.rmsnorm(v4, eps=0.0), out)
    # Zero-centred gain: weight (1 + gamma).
    gamma = np.full(d, 1.0, np.float32)
    out2 = oracle.rmsnorm(v, gamma=gamma, eps=0.0)
    np.testing.assert_array_equal(from_bf16(out2), from_bf16(out) * 2.0)
    rms = np.sqrt((from_bf16(out).astype(np.float64) ** 2).mean(1))
    np.testing.assert_allclose(rms, 1.0, atol=4e-3)


def test_rmsnorm_eps_inside_the_square_root():
    # A constant row of value v gives v / sqrt(v^2 + eps) * (1 + gamma_i).
    # With eps of the order of v^2 the place of eps matters: outside the root,
    # v / (|v| + eps), the result would be near 1 instead of 1/sqrt(2).
    d = 64
    gamma = np.linspace(-0.5, 0.5, d).astype(np.float32)
    for v, eps in ((0.01, 1e-4), (0.25, 0.0625), (-3.0, 9.0), (0.5, 1e-6)):
        row = to_bf16(np.full((3, d), v, np.float32))
        vb = float(from_bf16(row[0, 0]))
        for g in (None, gamma):
            out = from_bf16(oracle.rmsnorm(row, gamma=g, eps=eps)).astype(np.float64)
            gain = 1.0 if g is None else 1.0 + g.astype(np.float64)
            expect = vb / np.sqrt(vb * vb + np.float64(np.float32(eps))) * gain
            np.testing.assert_allclose(out, np.broadcast_to(expect, (3, d)), rtol=2 ** -8, atol=0)
    # Random rows whose mean square is comparable to eps, against the library
    # in float64 (at most one bf16 ulp apart: both round once).
    rng = np.random.default_rng(45)
    T = 16
    v = rand_bf16(rng, (T, d), 0.02)
    for eps in (1e-4, 4e-4, 1e-3):
        out = oracle.rmsnorm(v, eps=eps)
        ref = F.rms_norm(torch.from_numpy(from_bf16(v).astype(np.float64)), (d,), eps=float(np.float32(eps)))
        diff = np.abs(out.astype(np.int32) - to_bf16(ref.numpy().astype(np.float32)).astype(np.int32))
        assert diff.max() <= 1


# ------------------------------------------------------------ diagnostics --
# [Blog] §2.2.2 (p_e, f_e, group sums, L_EP over G expert groups), §5.2.3
# (routing confidence), §4.1.2 / Figure 4 (per-expert activation norms).

def _route_with_scores(x, wr, b, k, logit_bias=None):
    ids, _, _, s = oracle.route(x, wr, b, k, logit_bias=logit_bias, want_scores=True)
    return ids, s


@pytest.mark.parametrize("G", [1, 2, 4, 8])
def test_diag_uniform_scores_closed_form(G):
    # x = 0 makes every logit 0, every score 1/2 and every p_{t,e} = 1/E,
    # whatever the selection bias picks; then p_g = 1/G and L_EP = sum_g f_g = 1.
    rng = np.random.default_rng(40 + G)
    T, d, E, k = 37, 64, 16, 3
    x = np.zeros((T, d), np.uint16)
    wr = rand_bf16(rng, (E, d), 0.05)
    b = rng.uniform(-0.3, 0.3, E).astype(np.float32)
    ids, s = _route_with_scores(x, wr, b, k)
    p_e, f_e, l_ep, conf = oracle.route_diag(s, ids, G)
    np.testing.assert_allclose(p_e, 1.0 / E, rtol=1e-14)
    assert l_ep == pytest.approx(1.0, rel=1e-14)
    assert conf == pytest.approx(k / E, rel=1e-14)
    # f_e counts the bias-chosen set: ids are the same for every token here.
    expect_f = np.zeros(E)
    expect_f[ids[0]] = 1.0 / k
    np.testing.assert_array_equal(f_e, expect_f)


def test_diag_two_groups_closed_form_from_logit_bias():
    # x = 0 and a per-expert logit term: s_e = expit(c_e) for every token, so
    # p_e = expit(c_e) / sum expit(c).  A selection bias of +1 on expert 0 with
    # k = 1 gives f = (1, 0, 0, 0).  With contiguous groups {0,1} {2,3},
    # L_EP = 2 * (p_0 + p_1); p_1 != p_2 separates this from interleaved groups.
    T, d, E, k = 9, 64, 4, 1
    c = np.array([0.3, 1.5, -2.0, 0.7], np.float32)
    x = np.zeros((T, d), np.uint16)
    wr = to_bf16(np.ones((E, d)))
    b = np.array([1.0, 0, 0, 0], np.float32)
    ids, s = _route_with_scores(x, wr, b, k, logit_bias=c)
    assert np.all(ids == 0)
    p_e, f_e, l_ep, conf = oracle.route_diag(s, ids, 2)
    sig = scipy.special.expit(c.astype(np.float64))
    p = sig / sig.sum()
    np.testing.assert_allclose(p_e, p, rtol=1e-7)
    np.testing.assert_array_equal(f_e, [1.0, 0, 0, 0])
    assert l_ep == pytest.approx(2 * (p[0] + p[1]), rel=1e-7)
    assert conf == pytest.approx(p[0], rel=1e-7)
    # One group: L_EP = 1 whatever f and p are.  E groups of one: E * f_0 p_0.
    assert oracle.route_diag(s, ids, 1)[2] == pytest.approx(1.0, rel=1e-14)
    assert oracle.route_diag(s, ids, E)[2] == pytest.approx(E * p[0], rel=1e-7)


def test_diag_all_experts_chosen_has_full_confidence():
    rng = np.random.default_rng(43)
    T, d, E = 21, 64, 6
    x = rand_bf16(rng, (T, d))
    wr = rand_bf16(rng, (E, d), 0.1)
    b = rng.uniform(-0.1, 0.1, E).astype(np.float32)
    ids, s = _route_with_scores(x, wr, b, E)
    p_e, f_e, _, conf = oracle.route_diag(s, ids, 3)
    assert conf == pytest.approx(1.0, rel=1e-12)
    np.testing.assert_allclose(f_e, 1.0 / E, rtol=1e-14)
    # p_e is the token mean of the library sigmoids normalised per token.
    z = from_bf16(x).astype(np.float64) @ from_bf16(wr).astype(np.float64).T
    sg = scipy.special.expit(z)
    np.testing.assert_allclose(p_e, (sg / sg.sum(1, keepdims=True)).mean(0), rtol=2e-6)


@pytest.mark.parametrize("T,d,E,k,G", [(64, 256, 16, 2, 4), (48, 512, 288, 8, 8)])
def test_diag_invariants(T, d, E, k, G):
    rng = np.random.default_rng(T * E + G)
    x = rand_bf16(rng, (T, d))
    wr = rand_bf16(rng, (E, d), 0.05)
    ids, s = _route_with_scores(x, wr, np.zeros(E, np.float32), k)
    p_e, f_e, l_ep, conf = oracle.route_diag(s, ids, G)
    assert p_e.sum() == pytest.approx(1.0, rel=1e-12)
    assert f_e.sum() == pytest.approx(1.0, rel=1e-12)
    assert np.all(p_e > 0) and np.all(f_e >= 0)
    # f_e is the selection histogram over T k picks.
    np.testing.assert_array_equal(f_e * T * k, np.bincount(ids.ravel(), minlength=E))
    # Without a selection bias the chosen experts are each token's k largest
    # p_{t,e}, so their mass is at least the uniform share k / E, and below 1.
    assert k / E <= conf < 1.0
    # Confidence is not the renormalised weight mass (which is 1).
    assert conf < 0.99
    assert l_ep > 0
    # T = 0: everything is zero.
    z = oracle.route_diag(np.zeros((0, E), np.float32), np.zeros((0, k), np.int32), G)
    assert not z[0].any() and not z[1].any() and z[2] == 0.0 and z[3] == 0.0


def test_diag_rejects_uneven_groups():
    s = np.full((2, 6), 0.5, np.float32)
    ids = np.array([[0], [1]], np.int32)
    with pytest.raises(ValueError):
        oracle.route_diag(s, ids, 4)


def test_activation_rms_closed_forms():
    rng = np.random.default_rng(44)
    rows = rng.standard_normal((7, 96)).astype(np.float32)
    r = oracle.activation_rms(rows)
    assert r == pytest.approx(float(torch.linalg.vector_norm(torch.from_numpy(rows).double()) / np.sqrt(7 * 96)),
                              rel=1e-14)
    assert oracle.activation_rms(2 * rows) == pytest.approx(2 * r, rel=1e-14)
    assert oracle.activation_rms(np.full((3, 8), -0.75, np.float32)) == pytest.approx(0.75, rel=1e-15)
    assert oracle.activation_rms(np.zeros((0, 8), np.float32)) == 0.0
    # Rows with equal mean squares: the RMS is that of any one of them.
    one = rng.standard_normal(64).astype(np.float32)
    assert oracle.activation_rms(np.stack([one, -one, one[::-1]])) == pytest.approx(
        oracle.activation_rms(one[None]), rel=1e-14)


def test_expert_rms_groups_rows_and_ratio_closed_form():
    # Expert e's rows all hold the constant c_e, so its RMS is |c_e|; expert 2
    # gets no rows and is left out of the median.  Used RMS (1, 2, 3, 4):
    # median 2.5, ratios 0.4 and 1.6.
    d = 16
    counts = np.array([2, 1, 0, 3, 1])
    c = np.array([-1.0, 2.0, 9.0, 3.0, -4.0])
    offsets = np.concatenate([[0], np.cumsum(counts)])
    rows = np.concatenate([np.full((n, d), v, np.float32) for n, v in zip(counts, c)])
    shared = np.full((4, d), 0.5, np.float32)
    rms, ratio = oracle.expert_rms(to_bf16(rows), offsets, shared)
    np.testing.assert_allclose(rms, [1, 2, 0, 3, 4, 0.5], rtol=1e-15)
    np.testing.assert_allclose(ratio, [0.4, 1.6], rtol=1e-15)
    # Odd count: the middle value.  Drop expert 4's row.
    counts2 = np.array([2, 1, 0, 3, 0])
    offsets2 = np.concatenate([[0], np.cumsum(counts2)])
    rms2, ratio2 = oracle.expert_rms(to_bf16(rows[:6]), offsets2)
    np.testing.assert_allclose(ratio2, [0.5, 1.5], rtol=1e-15)
    assert rms2[5] == 0.0
    # No rows at all.
    rms3, ratio3 = oracle.expert_rms(np.zeros((0, d), np.uint16), np.zeros(4, np.int64))
    assert not rms3.any() and not ratio3.any()
