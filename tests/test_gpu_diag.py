"""Parity of the diagnostic calls (moe_route_diag, moe_combine_diag) with the
CPU oracle, on generator inputs.

Routing statistics: p_e within a relative 1e-5 (f32 per token, f64 across
tokens on the GPU; f64 throughout in the oracle); f_e exact where no token
is a near tie; L_EP and the routing confidence within a relative 1e-5 plus
what near-tie tokens can move.  Activation RMS and its spread within a
relative 1e-5 (f32 row sums of squares, f64 across rows).  The routing and
combine outputs of the diagnostic calls are bit-identical to the plain calls.
"""
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import pytest
import torch

import moegen
import oracle
import sparse_moe_transformer_ffn_amd as moe
from tests._util import to_bf16
from tests.gpu_harness import bf16_dev, bf16_host, check_routing, f32_dev, i32_dev, log, pool_size

pytestmark = pytest.mark.gpu

RTOL = 1e-5


def oracle_scores(x_h, wr_h, b_h, c_h, k):
    """Oracle routing with the unbiased scores, in parallel chunks."""
    T = x_h.shape[0]
    chunks = [a for a in np.array_split(np.arange(T), pool_size() * 2) if a.size]
    with ThreadPoolExecutor(pool_size()) as pool:
        parts = list(pool.map(lambda a: oracle.route(x_h[a], wr_h, b_h, k, logit_bias=c_h, want_scores=True),
                              chunks))
    return tuple(np.concatenate([p[i] for p in parts]) for i in range(4))


def run_route_diag(cfg, x_h, wr_h, b_h, c_h, G, plain_too=False):
    T, E, k = x_h.shape[0], cfg.E, cfg.k
    s = moe.make_shape(T, cfg.d, E, k, cfg.h, cfg.hs)
    n = max(T, 1)
    ids = torch.full((n, k), -7, dtype=torch.int32, device="cuda")
    w = torch.full((n, k), -1.0, device="cuda")
    gap = torch.full((n,), -1.0, device="cuda")
    cnt = torch.full((E,), 12345, dtype=torch.int32, device="cuda")
    p_e = torch.full((E,), -1.0, device="cuda")
    f_e = torch.full((E,), -1.0, device="cuda")
    summ = torch.full((2,), -1.0, device="cuda")
    ws = torch.empty(moe.moe_workspace_bytes(s), dtype=torch.uint8, device="cuda")
    x = bf16_dev(x_h if T else np.zeros((1, cfg.d), np.uint16))
    wr, b, c = bf16_dev(wr_h), f32_dev(b_h), f32_dev(c_h)
    moe.moe_route_diag(s, x, wr, b, c, ids, w, cnt, gap, G, p_e, f_e, summ, ws)
    out = [t.cpu().numpy() for t in (ids, w, gap, cnt, p_e, f_e, summ)]
    out[0], out[1], out[2] = out[0][:T], out[1][:T], out[2][:T]
    if plain_too:
        ids2, w2, gap2, cnt2 = (torch.empty_like(t) for t in (ids, w, gap, cnt))
        moe.moe_route(s, x, wr, b, c, ids2, w2, cnt2, gap2, ws)
        out += [t.cpu().numpy() for t in (ids2, w2, gap2, cnt2)]
    torch.cuda.synchronize()
    return out


def check_route_diag(g, o_ids, o_w, o_gap, o_s, E, k, G):
    g_ids, g_w, g_gap, g_cnt, g_p, g_f, g_sum = g[:7]
    T = o_ids.shape[0]
    same, near = check_routing(g_ids, g_w, g_gap, g_cnt, o_ids, o_w, o_gap, E)
    p_e, f_e, l_ep, conf = oracle.route_diag(o_s, o_ids, G)
    log(f"  G={G} near-tie tokens {near}; L_EP gpu {g_sum[0]:.7f} oracle {l_ep:.7f}; "
        f"confidence gpu {g_sum[1]:.7f} oracle {conf:.7f}")
    np.testing.assert_allclose(g_p, p_e, rtol=RTOL, atol=RTOL / E)
    # f_e is the GPU's own histogram over T k picks, and the oracle's where
    # the routings agree.
    np.testing.assert_array_equal(g_f, (g_cnt / (T * k)).astype(np.float32))
    flips = int((~same).sum())
    if flips == 0:
        np.testing.assert_array_equal(g_f, f_e.astype(np.float32))
    # A near-tie token moves one pick between two experts: f by 1/(T k) on
    # each, so L_EP by at most 2 G max_g p_g / (T k); its mass by at most 1/T.
    per = E // G
    pg_max = p_e.reshape(G, per).sum(1).max()
    assert abs(g_sum[0] - l_ep) <= RTOL * l_ep + flips * 2 * G * pg_max / (T * k)
    assert abs(g_sum[1] - conf) <= RTOL * conf + flips / T


@pytest.mark.parametrize("idx,G", [(0, 1), (0, 4), (1, 8), (1, 288), (2, 8), (3, 8)])
def test_route_diag_parity(device, idx, G):
    cfg = moegen.CONFIGS[idx]
    log(f"[route-diag] config {idx}: T={cfg.T} E={cfg.E} k={cfg.k} G={G}")
    x_h, wr_h, b_h, c_h = moegen.x(cfg), moegen.router(cfg), moegen.sel_bias(cfg), moegen.logit_bias(cfg)
    g = run_route_diag(cfg, x_h, wr_h, b_h, c_h, G, plain_too=True)
    # The diagnostic call's routing outputs are the plain call's, bit for bit.
    for a, b in zip(g[:4], g[7:]):
        np.testing.assert_array_equal(a, b[:a.shape[0]])
    o_ids, o_w, o_gap, o_s = oracle_scores(x_h, wr_h, b_h, c_h, cfg.k)
    check_route_diag(g, o_ids, o_w, o_gap, o_s, cfg.E, cfg.k, G)


@pytest.mark.parametrize("T,E,k,G,mode", [
    (1, 288, 8, 8, "normal"), (5, 5, 3, 5, "normal"), (100, 16, 16, 2, "normal"), (64, 1024, 16, 16, "normal"),
    (2047, 64, 4, 4, "normal"), (2048, 64, 4, 4, "normal"), (2051, 288, 8, 36, "normal"),
    (130, 288, 8, 8, "one_expert"), (64, 16, 2, 4, "zero_x"),
])
def test_route_diag_edge_cases(device, T, E, k, G, mode):
    # Token counts around the four-tokens-per-wave switch (2048) and ragged
    # last waves; every group count from 1 expert per group to E / 2.
    cfg = moegen.custom(0, T=T, E=E, k=k, seed=5000 + T + E + k)
    log(f"[route-diag-edge] T={T} E={E} k={k} G={G} {mode}")
    x_h, wr_h, b_h = moegen.x(cfg), moegen.router(cfg), moegen.sel_bias(cfg)
    if mode == "one_expert":
        b_h = b_h.copy()
        b_h[E // 3] = 10.0
    if mode == "zero_x":
        x_h = np.zeros_like(x_h)
    g = run_route_diag(cfg, x_h, wr_h, b_h, None, G)
    o_ids, o_w, o_gap, o_s = oracle_scores(x_h, wr_h, b_h, None, k)
    check_route_diag(g, o_ids, o_w, o_gap, o_s, E, k, G)
    if mode == "zero_x":
        # Uniform scores: p_e = 1/E, L_EP = 1, confidence k/E.
        np.testing.assert_allclose(g[4], 1.0 / E, rtol=RTOL)
        np.testing.assert_allclose(g[6], [1.0, k / E], rtol=RTOL)


def test_route_diag_zero_tokens_and_bad_groups(device):
    cfg = moegen.custom(0, T=0, E=16, k=2)
    g = run_route_diag(cfg, np.zeros((0, cfg.d), np.uint16), moegen.router(cfg), moegen.sel_bias(cfg), None, 4)
    assert np.all(g[3] == 0) and np.all(g[4] == 0) and np.all(g[5] == 0) and np.all(g[6] == 0)
    cfg = moegen.custom(0, T=8, E=16, k=2)
    for G in (0, 3, 17, -1):
        with pytest.raises(moe.MoeError):
            run_route_diag(cfg, moegen.x(cfg), moegen.router(cfg), moegen.sel_bias(cfg), None, G)


def test_route_diag_is_deterministic(device):
    cfg = moegen.CONFIGS[2]
    log(f"[route-diag-repeat] T={cfg.T}")
    args = (moegen.x(cfg), moegen.router(cfg), moegen.sel_bias(cfg), moegen.logit_bias(cfg), 8)
    a = run_route_diag(cfg, *args)
    b = run_route_diag(cfg, *args)
    for u, v in zip(a, b):
        np.testing.assert_array_equal(u, v)


# ------------------------------------------------------------- combine --

def combine_inputs(T, d, E, k, seed, spread=True, empty=()):
    """Routing ids (none on the listed experts), oracle permutation, y_perm
    rows scaled per expert so the RMS spread is not trivial, weights and a
    shared output."""
    ids = moegen.random_ids(seed, T, E - len(empty), k) if T else np.zeros((0, k), np.int32)
    keep = np.setdiff1d(np.arange(E), np.asarray(empty, np.int64))
    ids = keep[ids].astype(np.int32)
    counts, off, perm, pos = oracle.permute(ids, E)
    y = moegen.bf16_to_f32(moegen.normal_bf16(seed + 1, 320, (max(T * k, 1), d)))
    if spread and T:
        scale = 0.25 + 2.0 * moegen.uniform(seed + 2, 321, E)
        y[:T * k] *= np.repeat(scale, counts)[:, None]
    y_perm = to_bf16(y)
    w = moegen.uniform(seed + 3, 322, max(T, 1) * k).astype(np.float32).reshape(-1, k)[:T]
    ysh = (moegen.bf16_to_f32(moegen.normal_bf16(seed + 4, 323, (max(T, 1), d))) * 1.5)[:T]
    return ids, off, pos, y_perm, w, ysh


def run_combine_diag(T, d, E, k, off, pos, y_perm, w, ysh, scale, with_ratio=True, plain_too=False):
    s = moe.make_shape(T, d, E, k, 64, 64 if ysh is not None else 0)
    y = torch.full((max(T, 1), d), 7.0, dtype=torch.bfloat16, device="cuda")
    rms = torch.full((E + 1,), -1.0, device="cuda")
    ratio = torch.full((2,), -1.0, device="cuda") if with_ratio else None
    ws = torch.empty(moe.moe_workspace_bytes(s), dtype=torch.uint8, device="cuda")
    y_perm_d = bf16_dev(y_perm)
    pos_d = i32_dev(pos if T else np.zeros(1, np.int32))
    w_d = f32_dev(w if T else np.zeros((1, k), np.float32))
    ysh_d = None if ysh is None else f32_dev(ysh if T else np.zeros((1, d), np.float32))
    moe.moe_combine_diag(s, y_perm_d, pos_d, w_d, ysh_d, scale, y, i32_dev(off), rms, ratio, ws)
    plain = None
    if plain_too:
        y2 = torch.empty_like(y)
        moe.moe_combine(s, y_perm_d, pos_d, w_d, ysh_d, scale, y2)
        plain = bf16_host(y2)
    torch.cuda.synchronize()
    return (bf16_host(y), rms.cpu().numpy(), None if ratio is None else ratio.cpu().numpy(), plain)


@pytest.mark.parametrize("T,d,E,k,shared,empty", [
    (64, 4096, 288, 8, True, ()),          # the decode batch
    (2048, 4096, 288, 8, True, ()),
    (333, 1024, 64, 16, False, (5, 6)),
    (37, 256, 16, 2, True, (0, 15)),
    (1, 512, 16, 1, True, ()),             # one routed expert used: ratios (1, 1)
    (2, 64, 4, 2, False, ()),
])
def test_combine_diag_parity(device, T, d, E, k, shared, empty):
    log(f"[combine-diag] T={T} d={d} E={E} k={k} shared={shared} empty={empty}")
    ids, off, pos, y_perm, w, ysh = combine_inputs(T, d, E, k, 40 + T + E, empty=empty)
    y, rms, ratio, plain = run_combine_diag(T, d, E, k, off, pos, y_perm, w, ysh if shared else None, 0.75,
                                            plain_too=True)
    np.testing.assert_array_equal(y, plain)
    o_rms, o_ratio = oracle.expert_rms(y_perm[:T * k], off, ysh if shared else None)
    log(f"  ratio gpu {ratio} oracle {o_ratio}")
    np.testing.assert_allclose(rms, o_rms, rtol=RTOL, atol=0)
    np.testing.assert_allclose(ratio, o_ratio, rtol=RTOL, atol=0)
    for e in empty:
        assert rms[e] == 0.0
    if not shared:
        assert rms[E] == 0.0


def test_combine_diag_zero_tokens_and_no_ratio(device):
    E, d, k = 16, 128, 2
    off = np.zeros(E + 1, np.int32)
    y, rms, ratio, _ = run_combine_diag(0, d, E, k, off, None, np.zeros((1, d), np.uint16), None,
                                        np.zeros((0, d), np.float32), 1.0)
    assert np.all(rms == 0) and np.all(ratio == 0)
    ids, off, pos, y_perm, w, ysh = combine_inputs(50, d, E, k, 77)
    _, rms2, ratio2, _ = run_combine_diag(50, d, E, k, off, pos, y_perm, w, ysh, 1.0, with_ratio=False)
    o_rms, _ = oracle.expert_rms(y_perm[:50 * k], off, ysh)
    np.testing.assert_allclose(rms2, o_rms, rtol=RTOL)
    assert ratio2 is None
