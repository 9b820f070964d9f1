"""The pre-norm block's fused ends on the GPU: moe_rmsnorm_route (the
zero-centred RMSNorm in front of the layer fused into the router) and
moe_combine_residual (the skip connection fused into the combine).

moe_rmsnorm_route must equal moe_rmsnorm followed by moe_route bit for bit
(both the router that normalises as it loads, below 1024 tokens, and the
staged router fed by a normalisation pass); its x_out must be within one bf16
ulp of the oracle's RMSNorm, and its routing the oracle's routing of the
oracle's x except where a token's top-k gap is small enough for one-ulp input
differences to move it.  moe_combine_residual is checked against the
oracle's combine with the residual, and run in place.
"""
import numpy as np
import pytest
import torch

import moegen
import oracle
import sparse_moe_transformer_ffn_amd as moe
from tests._util import to_bf16
from tests.gpu_harness import (DeviceLayer, bf16_dev, bf16_host, check_output, f32_dev, i32_dev, log,
                               oracle_layer_tokens, oracle_route_all)

pytestmark = pytest.mark.gpu

# A one-ulp change of one bf16 element of x (|x| ~ 1) moves a logit by about
# 2^-8 * 0.02 and a score by a quarter of that; several such elements can add
# up.  Tokens whose oracle gap is below this may route differently.
INPUT_ULP_GAP = 1e-3


def stream_rows(cfg, scale=3.0):
    """An un-normalised residual stream: the generator's rows times `scale`."""
    return to_bf16(moegen.bf16_to_f32(moegen.x(cfg)) * scale)


def route_buffers(T, E, k):
    n = max(T, 1)
    return (torch.full((n, k), -7, dtype=torch.int32, device="cuda"), torch.full((n, k), -1.0, device="cuda"),
            torch.full((E,), 12345, dtype=torch.int32, device="cuda"), torch.full((n,), -1.0, device="cuda"))


@pytest.mark.parametrize("T,d,E,k,with_gamma", [
    (64, 4096, 288, 8, False),     # decode batch: the router normalises as it loads
    (256, 4096, 288, 8, False),    # a layer of the chained stack
    (1, 4096, 288, 8, True),
    (100, 256, 16, 2, True),
    (1024, 512, 64, 4, True),      # staged router: normalisation pass first
    (2048, 4096, 288, 8, False),
])
def test_rmsnorm_route_matches_unfused_and_oracle(device, T, d, E, k, with_gamma):
    cfg = moegen.custom(1, T=T, d=d, E=E, k=k, seed=4000 + T + d)
    log(f"[norm-route] T={T} d={d} E={E} k={k} gamma={with_gamma}")
    h_h = stream_rows(cfg)
    gamma_h = ((moegen.uniform(T + d, 330, d) - 0.5) * 0.2).astype(np.float32) if with_gamma else None
    wr_h, b_h, c_h = moegen.router(cfg), moegen.sel_bias(cfg), moegen.logit_bias(cfg)
    s = moe.make_shape(T, d, E, k, cfg.h, cfg.hs)
    ws = torch.empty(moe.moe_workspace_bytes(s), dtype=torch.uint8, device="cuda")
    h, gamma, wr, b, c = bf16_dev(h_h), f32_dev(gamma_h), bf16_dev(wr_h), f32_dev(b_h), f32_dev(c_h)
    x_out = torch.empty((T, d), dtype=torch.bfloat16, device="cuda")
    ids, w, cnt, gap = route_buffers(T, E, k)
    moe.moe_rmsnorm_route(s, h, gamma, 1e-6, wr, b, c, x_out, ids, w, cnt, gap, ws)
    x2 = torch.empty_like(x_out)
    ids2, w2, cnt2, gap2 = route_buffers(T, E, k)
    moe.moe_rmsnorm(T, d, h, gamma, 1e-6, x2)
    moe.moe_route(s, x2, wr, b, c, ids2, w2, cnt2, gap2, ws)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(bf16_host(x_out), bf16_host(x2))
    for a, z in ((ids, ids2), (w, w2), (cnt, cnt2), (gap, gap2)):
        np.testing.assert_array_equal(a.cpu().numpy(), z.cpu().numpy())
    # Against the oracle.
    x_ref = oracle.rmsnorm(h_h, gamma_h, 1e-6)
    diff = np.abs(bf16_host(x_out).astype(np.int32) - x_ref.astype(np.int32))
    assert diff.max() <= 1, diff.max()
    o_ids, o_w, o_gap, _ = oracle.route(x_ref, wr_h, b_h, k, logit_bias=c_h)
    g_ids = ids.cpu().numpy()[:T]
    same = np.all(g_ids == o_ids, axis=1)
    log(f"  x elements one ulp off: {int((diff > 0).sum())}; tokens routed differently: {int((~same).sum())}")
    assert np.all(o_gap[~same] < INPUT_ULP_GAP), o_gap[~same]
    np.testing.assert_allclose(w.cpu().numpy()[:T][same], o_w[same], rtol=1e-4, atol=1e-5)


@pytest.mark.parametrize("T,d,k,with_shared", [(64, 4096, 8, True), (300, 512, 4, False), (1, 256, 16, True)])
def test_combine_residual_parity(device, T, d, k, with_shared):
    log(f"[combine-res] T={T} d={d} k={k} shared={with_shared}")
    E = 64
    ids = moegen.random_ids(17 + T, T, E, k)
    _, _, _, pos = oracle.permute(ids, E)
    y_perm_h = moegen.normal_bf16(21 + T, 340, (T * k, d))
    w_h = moegen.uniform(22 + T, 341, T * k).astype(np.float32).reshape(T, k)
    ysh_h = moegen.bf16_to_f32(moegen.normal_bf16(23 + T, 342, (T, d))) * 2.0 if with_shared else None
    res_h = moegen.normal_bf16(24 + T, 343, (T, d), 3.0)
    s = moe.make_shape(T, d, E, k, 64, 64 if with_shared else 0)
    args = (bf16_dev(y_perm_h), i32_dev(pos), f32_dev(w_h), f32_dev(ysh_h), 0.75)
    y = torch.empty((T, d), dtype=torch.bfloat16, device="cuda")
    moe.moe_combine_residual(s, *args, bf16_dev(res_h), y)
    # In place: the residual buffer receives the block's output.
    y_in = bf16_dev(res_h)
    moe.moe_combine_residual(s, *args, y_in, y_in)
    torch.cuda.synchronize()
    got = bf16_host(y)
    np.testing.assert_array_equal(bf16_host(y_in), got)
    ref = oracle.combine(y_perm_h, pos, w_h, ysh_h, 0.75, residual=res_h)
    g = moegen.bf16_to_f32(got)
    rms = np.sqrt(np.mean(ref.astype(np.float64) ** 2))
    assert np.all(np.abs(g - ref) <= 2.0 ** -8 * np.abs(ref) + 1e-6 * rms)


@pytest.mark.parametrize("idx,stride", [(1, 4), (2, 512)])
def test_prenorm_block(device, idx, stride):
    # The whole block: h -> moe_rmsnorm_route -> permute -> experts (shared
    # fused) -> moe_combine_residual, against h + the oracle's layer on the
    # oracle's normalised rows, on sampled tokens whose routing matches: the
    # decode size (router normalising as it loads) and the prefill size
    # (normalisation pass, staged router, tiled experts).
    cfg = moegen.CONFIGS[idx]
    log(f"[prenorm-block] {cfg.name}")
    h_h = stream_rows(cfg)
    x_ref = oracle.rmsnorm(h_h, None, 1e-6)
    dl = DeviceLayer(cfg, x_host=x_ref)   # weights and router; x replaced below
    T, d, E, k = cfg.T, cfg.d, cfg.E, cfg.k
    buf = dl.buffers()
    s = buf.shape
    h = bf16_dev(h_h)
    x_out = torch.empty((T, d), dtype=torch.bfloat16, device="cuda")
    moe.moe_rmsnorm_route(s, h, None, 1e-6, dl.wr, dl.b, dl.c, x_out, buf.topk_ids, buf.topk_weights,
                          buf.expert_counts, buf.topk_gap, buf.workspace)
    moe.moe_permute(s, buf.topk_ids, buf.expert_offsets, buf.perm_pairs, buf.pair_pos, buf.workspace)
    moe.moe_expert_swiglu(s, x_out, buf.expert_offsets, buf.perm_pairs, dl.w_gu, dl.w_d, buf.y_perm, buf.workspace,
                          ws_gate_up=dl.ws_gu, ws_down=dl.ws_d, y_shared=buf.y_shared)
    y = torch.empty((T, d), dtype=torch.bfloat16, device="cuda")
    moe.moe_combine_residual(s, buf.y_perm, buf.pair_pos, buf.topk_weights, buf.y_shared, cfg.routed_scale, h, y)
    torch.cuda.synchronize()
    g_ids = buf.topk_ids.cpu().numpy()
    o_ids, _, o_gap = oracle_route_all(dl)   # dl's host rows are x_ref
    same = np.all(g_ids == o_ids, axis=1)
    assert np.all(o_gap[~same] < INPUT_ULP_GAP)
    toks = np.array([t for t in range(0, T, stride) if same[t]], np.int32)
    _, y_ffn = oracle_layer_tokens(dl, toks, o_ids[toks])
    y_ref = moegen.bf16_to_f32(h_h[toks]).astype(np.float64) + y_ffn
    check_output(moegen.bf16_to_f32(bf16_host(y))[toks], y_ref, "pre-norm block y")
