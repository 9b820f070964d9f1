"""The layer forward captured once into a HIP graph (torch.cuda.CUDAGraph over
the libmoe calls) and replayed: every replay must give the eager result bit
for bit, with eager work and synchronisations between replays.  No call in
the path records a memset node (counters and queues are cleared by kernels).
"""
import numpy as np
import pytest
import torch

import moegen
from tests.gpu_harness import DeviceLayer, bf16_host, log

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("idx", [1, 2])
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
