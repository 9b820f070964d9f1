"""moe_expert_swiglu_clamped: activation clipping on the SwiGLU hidden
activations, in both kernel regimes, against the oracle's clipped expert on
sampled rows (the layer's output tolerance), and bit-identical to the
unclipped call when the threshold exceeds every activation.
"""
import numpy as np
import pytest
import torch

import moegen
import oracle
import sparse_moe_transformer_ffn_amd as moe
from tests.gpu_harness import DeviceLayer, bf16_host, check_output, i32_dev, log, oracle_route_all

pytestmark = pytest.mark.gpu


def run(dl, off, perm, clamp):
    c = dl.cfg
    s = moe.make_shape(c.T, c.d, c.E, c.k, c.h, c.hs)
    ws = torch.empty(moe.moe_workspace_bytes(s), dtype=torch.uint8, device="cuda")
    y_perm = torch.zeros((c.T * c.k, c.d), dtype=torch.bfloat16, device="cuda")
    y_sh = torch.zeros((c.T, c.d), dtype=torch.float32, device="cuda")
    args = (s, dl.x, i32_dev(off), i32_dev(perm), dl.w_gu, dl.w_d, y_perm)
    kw = dict(ws_gate_up=dl.ws_gu, ws_down=dl.ws_d, y_shared=y_sh)
    if clamp is None:
        moe.moe_expert_swiglu(*args, ws, **kw)
    else:
        moe.moe_expert_swiglu_clamped(*args, clamp, ws, **kw)
    torch.cuda.synchronize()
    return bf16_host(y_perm), y_sh.cpu().numpy()


@pytest.mark.parametrize("cfg,clamp", [
    (moegen.custom(0, T=24, seed=951), 0.02),                                    # streaming kernels
    (moegen.CONFIGS[0], 0.02),                                                   # 8 rows per expert: 32-row items
    (moegen.custom(0, T=96, seed=952), 0.02),                                    # 12 rows per expert: tiled gate/up
    (moegen.CONFIGS[1], 0.5),                                                    # decode size (streaming)
    (moegen.custom(0, T=2048, d=256, E=16, k=2, h=128, hs=128, seed=950), 0.02),  # tiled kernels
])
def test_clamped_experts_parity(device, cfg, clamp):
    log(f"[clamp] T={cfg.T} d={cfg.d} E={cfg.E} h={cfg.h} clamp={clamp}")
    dl = DeviceLayer(cfg)
    o_ids, _, _ = oracle_route_all(dl)
    _, off, perm, _ = oracle.permute(o_ids, cfg.E)
    yp, ysh = run(dl, off, perm, clamp)
    yp0, ysh0 = run(dl, off, perm, None)
    # Some rows must actually change, or the test would not see the clip.
    assert np.any(yp != yp0)
    touched = np.where(np.diff(off) > 0)[0]
    pick = touched[np.linspace(0, len(touched) - 1, min(12, len(touched))).astype(int)]
    rows = sorted({r for e in pick for r in (off[e], off[e + 1] - 1)})
    ew = moegen.expert_weights_host(cfg, 0, [int(e) for e in pick])
    ref = np.stack([oracle.expert_clamped(dl.x_h[perm[r] // cfg.k],
                                          *ew[int(np.searchsorted(off, r, side="right") - 1)], clamp) for r in rows])
    check_output(moegen.bf16_to_f32(yp[rows]), ref, f"clamped y_perm rows ({len(rows)})")
    sgu, swd = moegen.shared_weights_host(cfg)
    toks = np.arange(0, cfg.T, max(1, cfg.T // 16))
    ref_sh = np.stack([oracle.expert_clamped(dl.x_h[t], sgu, swd, clamp) for t in toks])
    check_output(ysh[toks], ref_sh, "clamped y_shared")
    # A threshold above every activation clips nothing.
    yp_big, ysh_big = run(dl, off, perm, 1e30)
    np.testing.assert_array_equal(yp_big, yp0)
    np.testing.assert_array_equal(ysh_big, ysh0)


def test_clamp_must_be_positive(device):
    cfg = moegen.CONFIGS[0]
    dl = DeviceLayer(cfg)
    off = np.zeros(cfg.E + 1, np.int32)
    perm = np.zeros(cfg.T * cfg.k, np.int32)
    for bad in (0.0, -1.0, float("inf"), float("nan")):
        with pytest.raises(moe.MoeError):
            run(dl, off, perm, bad)
