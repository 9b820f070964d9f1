"""Parity of moe_dense_swiglu (the dense SwiGLU FFN of the first blocks and
the MTP heads, hidden 11,264) with the CPU oracle's SwiGLU, on generator
inputs.  The weights are the generator's shared-expert tensors of a workload
whose shared hidden size is the dense one; the oracle gets the host copy.

Both launch regimes are covered: up to 64 tokens the streaming kernels (one
M-tile of 16, 32 or 64 rows, the down reduction split over items; with a
hidden size of at least 16 units per CU, the kernels in which each CU owns a
fixed share of the weights); above
64 the LDS-tiled ones, which up to 256 tokens (one M-tile) split each weight
tile's reduction over several items when the reduction is long enough
(partial sums added afterwards in split order).  Bar: the layer's output tolerance
(relative L2 <= 5e-3, max |err| <= 3e-2 RMS), every token at the small sizes
and sampled tokens at T = 8192.
"""
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import pytest
import torch

import moegen
import oracle
import sparse_moe_transformer_ffn_amd as moe
from tests.gpu_harness import bf16_dev, check_output, log, pool_size, stream_ptr

pytestmark = pytest.mark.gpu

DENSE_HIDDEN = 11264


def run_dense(cfg, x_h, H):
    T, d = x_h.shape
    w_gu = torch.empty((2 * H, d), dtype=torch.bfloat16, device="cuda")
    w_d = torch.empty((d, H), dtype=torch.bfloat16, device="cuda")
    moegen.fill_shared_device(cfg, 0, w_gu.data_ptr(), w_d.data_ptr(), stream_ptr())
    y = torch.full((max(T, 1), d), 5.0, device="cuda")
    ws = torch.empty(moe.moe_dense_workspace_bytes(T, d, H), dtype=torch.uint8, device="cuda")
    x = bf16_dev(x_h if T else np.zeros((1, d), np.uint16))
    moe.moe_dense_swiglu(T, d, H, x, w_gu, w_d, y, ws)
    torch.cuda.synchronize()
    return y.cpu().numpy()[:max(T, 1)]


def oracle_rows(cfg, x_h, rows):
    sgu, swd = moegen.shared_weights_host(cfg)
    rows = list(rows)
    with ThreadPoolExecutor(pool_size()) as pool:
        return np.stack(list(pool.map(lambda t: oracle.expert(x_h[t], sgu, swd), rows)))


@pytest.mark.parametrize("T,d,H", [
    (1, 256, 128), (37, 256, 384), (63, 512, 256),     # streaming kernels
    (64, 256, 384),                                     # streaming, one 64-row M-tile
    (65, 256, 384), (256, 512, 256),                    # tiled, reductions too short to split
    (100, 1024, 1024), (200, 2048, 2560),               # tiled with split reductions (2 and 2; 4 and 5)
    (300, 512, 640), (1000, 256, 128),                  # tiled kernels, ragged last M-tile
    (128, 4096, DENSE_HIDDEN), (256, 4096, DENSE_HIDDEN),  # the model's size: splits 4 (gate/up) and 22 (down)
    (64, 4096, DENSE_HIDDEN),                             # streaming, one 64-row M-tile, down split 4 ways
    (16, 4096, DENSE_HIDDEN), (32, 4096, DENSE_HIDDEN),   # streaming at the model's size: 16- and 32-row
    (48, 4096, DENSE_HIDDEN),                             # M-tiles, and one 64-row M-tile
    (1, 4096, DENSE_HIDDEN), (8, 4096, DENSE_HIDDEN), (17, 4096, DENSE_HIDDEN), (63, 4096, DENSE_HIDDEN),
    # Up to 64 tokens with a hidden size of at least 16 units per CU, each CU
    # owns a fixed range of hidden units (gate/up) and of output columns over
    # a quarter of the reduction (down): ragged unit ranges (the last block
    # short), ragged reduction ranges, and waves left without K blocks.
    (64, 1024, 4352), (33, 512, 6208), (1, 256, 4096), (20, 768, 8256),
    # Tiled with one phase split while the other does not tile: down split
    # 19 and 7 ways over an odd count of 64-wide hidden chunks (hidden % 128
    # == 64: gate/up streams), gate/up split 2 ways with d % 256 != 0 (down
    # streams).  Their split scratch is sized per phase.
    (230, 1024, 10944), (165, 768, 8512), (128, 1152, 4096),
])
def test_dense_parity(device, T, d, H):
    cfg = moegen.custom(1, T=T, d=d, hs=H, seed=700 + T + H)
    log(f"[dense] T={T} d={d} H={H}")
    x_h = moegen.x(cfg)
    y = run_dense(cfg, x_h, H)
    ref = oracle_rows(cfg, x_h, range(T))
    check_output(y[:T], ref, f"dense T={T} H={H}")


def _dense_sweep(n=32, seed=20261204):
    """Seeded random dense shapes: half of them up to 64 tokens (the per-CU
    share kernels where the hidden size allows, else the streaming ones),
    half up to 300 (the tiled kernels, split or not); hidden sizes from 64 to
    12,800 units and model sizes from 64 to 1,024, all multiples of 64."""
    rng = np.random.default_rng(seed)
    shapes = []
    for i in range(n):
        T = int(rng.integers(1, 65)) if i % 2 == 0 else int(rng.integers(65, 301))
        d = 64 * int(rng.integers(1, 17))
        H = 64 * int(rng.integers(64, 201)) if rng.random() < 0.6 else 64 * int(rng.integers(1, 64))
        shapes.append((T, d, H, 9000 + i))
    return shapes


@pytest.mark.parametrize("T,d,H,seed", _dense_sweep())
def test_dense_shape_sweep(device, T, d, H, seed):
    # Every token against the oracle, at the plain bar (the output is f32).
    cfg = moegen.custom(1, T=T, d=d, hs=H, seed=seed)
    log(f"[dense-sweep] T={T} d={d} H={H} seed={seed}")
    x_h = moegen.x(cfg)
    y = run_dense(cfg, x_h, H)
    ref = oracle_rows(cfg, x_h, range(T))
    check_output(y[:T], ref, f"dense T={T} d={d} H={H}")


def test_dense_prefill_sampled_rows(device):
    T, d, H = 8192, 4096, DENSE_HIDDEN
    cfg = moegen.custom(2, hs=H, seed=2)
    log(f"[dense] T={T} d={d} H={H}, sampled rows")
    x_h = moegen.x(cfg)
    y = run_dense(cfg, x_h, H)
    rows = np.unique(np.concatenate([[0, 255, 256, T - 1], moegen.random_ids(77, 1, T, 28)[0]]))
    ref = oracle_rows(cfg, x_h, rows)
    check_output(y[rows], ref, "dense T=8192 sampled")
    assert np.all(np.isfinite(y))


def test_dense_beyond_32_bit_element_indices(device):
    # 196,608 tokens at hidden 11,264: the hidden activations hold 2.2e9
    # elements, so the rows of the last tokens sit beyond 2^31 elements.
    T, d, H = 196608, 4096, DENSE_HIDDEN
    assert T * H > 2 ** 31
    cfg = moegen.custom(2, T=T, hs=H, seed=196608)
    log(f"[dense] T={T} d={d} H={H}: hidden activations beyond 2^31 elements")
    x_h = moegen.x(cfg)
    y = run_dense(cfg, x_h, H)
    rows = np.unique(np.concatenate([[0, T // 2, T - 256, T - 1], moegen.random_ids(78, 1, T, 8)[0]]))
    assert rows[-1] * H > 2 ** 31
    ref = oracle_rows(cfg, x_h, rows)
    check_output(y[rows], ref, f"dense T={T} sampled")


def test_dense_zero_tokens_and_rejections(device):
    d, H = 256, 128
    y = torch.full((1, d), 5.0, device="cuda")
    ws = torch.empty(moe.moe_dense_workspace_bytes(0, d, H), dtype=torch.uint8, device="cuda")
    x = torch.zeros((1, d), dtype=torch.bfloat16, device="cuda")
    w = torch.zeros((2 * H, d), dtype=torch.bfloat16, device="cuda")
    moe.moe_dense_swiglu(0, d, H, x, w, w, y, ws)
    torch.cuda.synchronize()
    assert np.all(y.cpu().numpy() == 5.0)
    with pytest.raises(moe.MoeError):
        moe.moe_dense_swiglu(4, d, 100, x, w, w, y, ws)
    with pytest.raises(moe.MoeError):
        moe.moe_dense_swiglu(4096, d, H, x, w, w, y, ws)   # workspace too small
