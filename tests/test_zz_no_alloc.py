"""moe_expert_swiglu_noalloc (for callers that cannot allocate device memory)
against moe_expert_swiglu with a caller workspace: the same kernels, so the
same bits, on calls in a row -- each with a smaller batch than the last,
and in another kernel regime -- sharing the library's static scratch."""
import numpy as np
import pytest
import torch

import moegen
import oracle
import sparse_moe_transformer_ffn_amd as moe
from tests.gpu_harness import DeviceLayer, bf16_host, i32_dev, log

pytestmark = pytest.mark.gpu


def _routing(cfg, T, seed):
    ids = moegen.random_ids(seed, T, cfg.E, cfg.k)
    _, off, perm, _ = oracle.permute(ids, cfg.E)
    return i32_dev(off), i32_dev(perm)


def _both(dl, T, seed, shared):
    cfg = dl.cfg
    s = moe.make_shape(T, cfg.d, cfg.E, cfg.k, cfg.h, cfg.hs)
    off, perm = _routing(cfg, T, seed)
    x = dl.x[:T]
    kw = dict(ws_gate_up=dl.ws_gu, ws_down=dl.ws_d) if shared else {}
    ref = torch.full((T * cfg.k, cfg.d), 3.0, dtype=torch.bfloat16, device="cuda")
    got = torch.full_like(ref, -5.0)
    ref_sh = torch.full((T, cfg.d), 3.0, device="cuda") if shared else None
    got_sh = torch.full((T, cfg.d), -5.0, device="cuda") if shared else None
    ws = torch.empty(moe.moe_workspace_bytes(s), dtype=torch.uint8, device="cuda")
    moe.moe_expert_swiglu(s, x, off, perm, dl.w_gu, dl.w_d, ref, ws, y_shared=ref_sh, **kw)
    moe.moe_expert_swiglu_noalloc(s, x, off, perm, dl.w_gu, dl.w_d, got, y_shared=got_sh, **kw)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(bf16_host(got), bf16_host(ref))
    if shared:
        np.testing.assert_array_equal(got_sh.cpu().numpy(), ref_sh.cpu().numpy())
    return got


@pytest.mark.parametrize("shared", [True, False])
def test_noalloc_matches_workspace_call_twice(device, shared):
    # First call: 1,024 tokens of the decode layer's shape (about 28 rows per
    # expert: the tiled kernels and their work queue); then 256 tokens (7 rows
    # per expert: 32-row streaming items) and 48 (16-row streaming items),
    # into the same static scratch.
    cfg = moegen.custom(1, T=1024, seed=77)
    dl = DeviceLayer(cfg)
    log(f"[noalloc] shared={shared}: 1024 tokens, then 256, then 48")
    first = _both(dl, 1024, 5, shared)
    keep = bf16_host(first).copy()
    second = _both(dl, 256, 7, shared)
    keep2 = bf16_host(second).copy()
    _both(dl, 48, 6, shared)
    # The earlier calls' outputs are the caller's and stay as they were.
    np.testing.assert_array_equal(bf16_host(first), keep)
    np.testing.assert_array_equal(bf16_host(second), keep2)


def test_noalloc_rejects_shapes_beyond_its_scratch(device):
    # 2,000 tokens of the model's shape need 256 + 2000*8*1280*2 bytes of
    # scratch without the shared expert (40.96 MB > 32 MiB): rejected before
    # anything is enqueued.
    cfg = moegen.CONFIGS[1]
    T = 2000
    s = moe.make_shape(T, cfg.d, cfg.E, cfg.k, cfg.h, cfg.hs)
    dummy = torch.empty(16, dtype=torch.bfloat16, device="cuda")
    idx = torch.zeros(16, dtype=torch.int32, device="cuda")
    with pytest.raises(moe.MoeError) as e:
        moe.moe_expert_swiglu_noalloc(s, dummy, idx, idx, dummy, dummy, dummy)
    assert e.value.code == 4
