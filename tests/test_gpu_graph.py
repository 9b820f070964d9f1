"""The layer forward captured once into a HIP graph (torch.cuda.CUDAGraph over
the libmoe calls) and replayed: every replay must give the eager result bit
for bit, with eager work and synchronisations between replays.  No call in
the path records a memset node (counters and queues are cleared by kernels).
Covered: the decode forward (16-row streaming items), a 256-token layer
(32-row streaming items), the prefill forward (tiled kernels, work queues),
and the dense FFN with split reductions.
"""
import numpy as np
import pytest
import torch

import moegen
import sparse_moe_transformer_ffn_amd as moe
from tests.gpu_harness import DeviceLayer, bf16_host, log

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("idx", [1, 4, 2])
def test_layer_graph_replays_match_eager(device, idx):
    cfg = moegen.CONFIGS[idx]
    log(f"[graph] config {idx}: {cfg.workload}")
    dl = DeviceLayer(cfg)
    eager = dl.buffers()
    dl.forward(eager)
    torch.cuda.synchronize()
    y_ref = bf16_host(eager.y).copy()
    ids_ref = eager.topk_ids.cpu().numpy().copy()
    buf = dl.buffers()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):       # warm the persistent-grid sizes off the capture
        dl.forward(buf)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        dl.forward(buf)
    for rep in range(3):
        buf.y.zero_()
        buf.topk_ids.fill_(-1)
        graph.replay()
        torch.cuda.synchronize()
        np.testing.assert_array_equal(buf.topk_ids.cpu().numpy(), ids_ref)
        np.testing.assert_array_equal(bf16_host(buf.y), y_ref)
        # Eager work between replays.
        dl.forward(eager)
        torch.cuda.synchronize()
    np.testing.assert_array_equal(bf16_host(eager.y), y_ref)


@pytest.mark.parametrize("T", [64, 128])
def test_dense_split_graph_replays_match_eager(device, T):
    # The dense FFN with split reductions (partial sums in the workspace,
    # added by another kernel): at 64 tokens the per-CU share kernels (down
    # split four ways over the hidden reduction), at 128 the tiled ones (both
    # phases split).  Replays of the captured call must equal the eager call
    # bit for bit.
    d, H = 4096, 11264
    cfg = moegen.custom(1, T=T, hs=H, seed=777)
    log(f"[graph] dense FFN T={T} (split reductions)")
    w_gu = torch.empty((2 * H, d), dtype=torch.bfloat16, device="cuda")
    w_d = torch.empty((d, H), dtype=torch.bfloat16, device="cuda")
    moegen.fill_shared_device(cfg, 0, w_gu.data_ptr(), w_d.data_ptr(), torch.cuda.current_stream().cuda_stream)
    x = torch.from_numpy(moegen.x(cfg).view(np.int16)).view(torch.bfloat16).cuda()
    ws = torch.empty(moe.moe_dense_workspace_bytes(T, d, H), dtype=torch.uint8, device="cuda")
    y_eager = torch.empty((T, d), device="cuda")
    moe.moe_dense_swiglu(T, d, H, x, w_gu, w_d, y_eager, ws)
    torch.cuda.synchronize()
    ref = y_eager.cpu().numpy().copy()
    y = torch.empty((T, d), device="cuda")
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        moe.moe_dense_swiglu(T, d, H, x, w_gu, w_d, y, ws, side)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        moe.moe_dense_swiglu(T, d, H, x, w_gu, w_d, y, ws, torch.cuda.current_stream())
    for rep in range(3):
        y.zero_()
        graph.replay()
        torch.cuda.synchronize()
        np.testing.assert_array_equal(y.cpu().numpy(), ref)
        moe.moe_dense_swiglu(T, d, H, x, w_gu, w_d, y_eager, ws)
        torch.cuda.synchronize()
    np.testing.assert_array_equal(y_eager.cpu().numpy(), ref)
