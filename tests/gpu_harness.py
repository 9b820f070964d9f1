"""Shared pieces of the GPU parity tests: device setup of a workload from the
seeded generator, threaded calls of the CPU oracle, and the acceptance checks.

Inputs for both sides come from moegen only.  The oracle never receives a
value the GPU computed: parity of each call is checked on generator or
oracle-made inputs, and whole-layer parity compares the GPU's output with the
oracle's own forward pass of the same generator inputs.
"""
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import torch

import moegen
import oracle
import sparse_moe_transformer_ffn_amd as moe

NEAR_TIE = 1e-5          # routing gap below which either choice is correct
REL_L2_TOL = 5e-3        # whole-layer output, given the same routing
MAX_ABS_TOL = 3e-2       # times RMS of the reference output


def bf16_dev(a: np.ndarray, device="cuda") -> torch.Tensor:
    """uint16 bf16 bit patterns (host) -> torch.bfloat16 device tensor."""
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(device)


def bf16_host(t: torch.Tensor) -> np.ndarray:
    return t.detach().view(torch.int16).cpu().numpy().view(np.uint16)


def f32_dev(a, device="cuda"):
    return None if a is None else torch.from_numpy(np.ascontiguousarray(a, np.float32)).to(device)


def i32_dev(a, device="cuda"):
    return torch.from_numpy(np.ascontiguousarray(a, np.int32)).to(device)


def stream_ptr():
    return torch.cuda.current_stream().cuda_stream


def log(msg):
    print(msg, flush=True)


class DeviceLayer:
    """One layer of a workload: host copies of the small tensors (x, router,
    biases) and device copies of everything, the experts filled on the device
    by the generator (bit-identical to the host fill)."""

    def __init__(self, cfg: moegen.Config, layer: int = 0, x_host=None, device="cuda"):
        self.cfg, self.layer = cfg, layer
        self.x_h = moegen.x(cfg, layer) if x_host is None else x_host
        self.wr_h = moegen.router(cfg, layer)
        self.b_h = moegen.sel_bias(cfg, layer)
        self.c_h = moegen.logit_bias(cfg, layer)
        self.x = bf16_dev(self.x_h, device)
        self.wr = bf16_dev(self.wr_h, device)
        self.b = f32_dev(self.b_h, device)
        self.c = f32_dev(self.c_h, device)
        E, d, h, hs = cfg.E, cfg.d, cfg.h, cfg.hs
        self.w_gu = torch.empty((E, 2 * h, d), dtype=torch.bfloat16, device=device)
        self.w_d = torch.empty((E, d, h), dtype=torch.bfloat16, device=device)
        moegen.fill_experts_device(cfg, layer, self.w_gu.data_ptr(), self.w_d.data_ptr(), stream_ptr())
        self.ws_gu = self.ws_d = None
        if hs:
            self.ws_gu = torch.empty((2 * hs, d), dtype=torch.bfloat16, device=device)
            self.ws_d = torch.empty((d, hs), dtype=torch.bfloat16, device=device)
            moegen.fill_shared_device(cfg, layer, self.ws_gu.data_ptr(), self.ws_d.data_ptr(), stream_ptr())

    def buffers(self, T=None):
        c = self.cfg
        return moe.LayerBuffers.allocate(c.T if T is None else T, c.d, c.E, c.k, c.h, c.hs)

    def forward(self, buf, shared="fused", shared_stream=None, diag_groups=None):
        return buf.forward(self.x, self.wr, self.b, self.c, self.w_gu, self.w_d, self.ws_gu, self.ws_d,
                           self.cfg.routed_scale, shared=shared, shared_stream=shared_stream,
                           diag_groups=diag_groups)


def pool_size():
    return moegen.threads()


def oracle_route_all(dl: DeviceLayer, tokens=None):
    """Oracle routing of the listed rows (all if None), in parallel chunks."""
    c = dl.cfg
    idx = np.arange(c.T) if tokens is None else np.asarray(tokens)
    chunks = [a for a in np.array_split(idx, pool_size() * 2) if a.size]
    with ThreadPoolExecutor(pool_size()) as pool:
        parts = list(pool.map(lambda a: oracle.route(dl.x_h[a], dl.wr_h, dl.b_h, c.k, logit_bias=dl.c_h), chunks))
    ids = np.concatenate([p[0] for p in parts])
    w = np.concatenate([p[1] for p in parts])
    gap = np.concatenate([p[2] for p in parts])
    return ids, w, gap


def oracle_layer_tokens(dl: DeviceLayer, tokens, ids_of_tokens):
    """Oracle forward of the listed tokens; expert weights generated on the
    host for exactly the experts those tokens select."""
    c = dl.cfg
    needed = sorted(set(int(e) for e in np.asarray(ids_of_tokens).ravel()))
    ew = moegen.expert_weights_host(c, dl.layer, needed)
    gu = [ew[e][0] if e in ew else None for e in range(c.E)]
    wd = [ew[e][1] if e in ew else None for e in range(c.E)]
    sgu, swd = moegen.shared_weights_host(c, dl.layer)
    tokens = np.asarray(tokens, np.int32)
    chunks = [a for a in np.array_split(tokens, min(len(tokens), pool_size() * 2)) if a.size]
    with ThreadPoolExecutor(pool_size()) as pool:
        parts = list(pool.map(lambda a: oracle.layer(dl.x_h, dl.wr_h, dl.b_h, c.k, gu, wd, sgu, swd,
                                                     c.routed_scale, logit_bias=dl.c_h, tokens=a), chunks))
    ids = np.concatenate([p[0] for p in parts])
    y = np.concatenate([p[3] for p in parts])
    return ids, y


def check_routing(gpu_ids, gpu_w, gpu_gap, gpu_counts, or_ids, or_w, or_gap, E):
    """Routing ids bit-exact except near-tie tokens (which must still pick a
    valid set); counts exact against the GPU's own ids and against the oracle
    where no token differs.  Returns (mask of tokens that match, near count)."""
    T, k = or_ids.shape
    same = np.all(gpu_ids == or_ids, axis=1)
    near = or_gap < NEAR_TIE
    bad = ~same & ~near
    assert not bad.any(), f"{bad.sum()} tokens routed differently with gap >= {NEAR_TIE}: {np.where(bad)[0][:8]}"
    # Every row: k distinct ascending ids in range.
    assert np.all((gpu_ids >= 0) & (gpu_ids < E))
    assert np.all(np.diff(gpu_ids, axis=1) > 0)
    np.testing.assert_array_equal(gpu_counts, np.bincount(gpu_ids.ravel(), minlength=E))
    if same.all():
        np.testing.assert_array_equal(gpu_counts, np.bincount(or_ids.ravel(), minlength=E))
    np.testing.assert_allclose(gpu_w[same], or_w[same], rtol=2e-5, atol=2e-6)
    np.testing.assert_allclose(gpu_w.astype(np.float64).sum(1), 1.0, atol=2e-5)
    finite = np.isfinite(or_gap) & same
    np.testing.assert_allclose(gpu_gap[finite], or_gap[finite], rtol=0, atol=2e-5)
    return same, int(near.sum())


def assert_same_up_to_order(a, b, what=""):
    """Two device results of the same layer computed with different reduction
    splits (the standalone shared call may pick another kernel).  Beyond f32
    summation order, a bf16 hidden activation can round one ulp apart, which
    moves its whole row of outputs; each side is held to the oracle at the
    full tolerance elsewhere, and to the other here at a fifth of it."""
    if a.dtype == np.uint16:
        a, b = moegen.bf16_to_f32(a), moegen.bf16_to_f32(b)
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    err = a - b
    scale = np.sqrt(np.mean(b ** 2)) if b.size else 0.0
    rel = np.linalg.norm(err) / max(np.linalg.norm(b), 1e-300)
    mx = np.abs(err).max() if err.size else 0.0
    log(f"  {what}: rel_l2={rel:.3e} max_abs={mx:.3e} (rms {scale:.3e})")
    assert rel <= REL_L2_TOL / 5, f"{what}: relative L2 {rel:.3e}"
    # Per element: one bf16 ulp of the value (the output's own rounding can
    # land either side) on top of a third of the oracle's max-error bound.
    bound = 2.0 ** -7 * np.maximum(np.abs(a), np.abs(b)) + MAX_ABS_TOL / 3 * scale
    assert np.all(np.abs(err) <= bound), f"{what}: max abs {mx:.3e}"


def check_output(y_gpu, y_ref, what=""):
    """Relative L2 <= 5e-3 and max |err| <= 3e-2 * RMS(ref)."""
    y_gpu = np.asarray(y_gpu, np.float64)
    y_ref = np.asarray(y_ref, np.float64)
    err = y_gpu - y_ref
    rel = np.linalg.norm(err) / max(np.linalg.norm(y_ref), 1e-300)
    rms = np.sqrt(np.mean(y_ref ** 2))
    mx = np.abs(err).max() if err.size else 0.0
    log(f"  {what}: rel_l2={rel:.3e} max_abs={mx:.3e} (rms {rms:.3e})")
    assert rel <= REL_L2_TOL, f"{what}: relative L2 {rel:.3e} > {REL_L2_TOL}"
    assert mx <= MAX_ABS_TOL * rms, f"{what}: max abs {mx:.3e} > {MAX_ABS_TOL} * rms {rms:.3e}"
    return rel, mx / max(rms, 1e-300)
