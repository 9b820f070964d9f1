"""Shared pieces of the GPU parity tests: device setup of a workload from the
seeded generator, threaded calls of the CPU oracle, and the acceptance checks.

Inputs for both sides come from moegen only.  The oracle never receives a
value the GPU computed: parity of each call is checked on generator or
oracle-made inputs, and whole-layer parity compares the GPU's output with the
oracle's forward pass of the same generator inputs.  Where a near tie makes
two chosen sets both correct, the oracle enumerates its acceptable sets from
its own scores and the GPU's pick only selects which of them the output is
compared under ("given the same routing").
"""
import itertools
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


def oracle_route_rows(x_rows, wr_h, b_h, k, c_h=None):
    """Oracle routing of token rows, in parallel chunks.  Returns (ids, w,
    gap, beta) with beta = fl32(s + b) [n, E], the biased scores the
    selection compares."""
    n = x_rows.shape[0]
    chunks = [a for a in np.array_split(np.arange(n), pool_size() * 2) if a.size]
    with ThreadPoolExecutor(pool_size()) as pool:
        parts = list(pool.map(lambda a: oracle.route(x_rows[a], wr_h, b_h, k, logit_bias=c_h, want_scores=True),
                              chunks))
    ids = np.concatenate([p[0] for p in parts])
    w = np.concatenate([p[1] for p in parts])
    gap = np.concatenate([p[2] for p in parts])
    scores = np.concatenate([p[3] for p in parts])
    beta = (scores + b_h.astype(np.float32)[None, :]).astype(np.float32)
    return ids, w, gap, beta


def oracle_route_all(dl: DeviceLayer, tokens=None, with_beta=False):
    """Oracle routing of the listed rows (all if None): (ids, w, gap) and,
    with_beta, the biased scores too."""
    c = dl.cfg
    idx = np.arange(c.T) if tokens is None else np.asarray(tokens)
    ids, w, gap, beta = oracle_route_rows(dl.x_h[idx], dl.wr_h, dl.b_h, c.k, dl.c_h)
    return (ids, w, gap, beta) if with_beta else (ids, w, gap)


def acceptable_sets(beta_row, k, tol=NEAR_TIE):
    """Every k-set of experts that a selection within `tol` of the oracle's
    biased scores may pick: S is acceptable iff min_S beta >= max_{not S}
    beta - tol.  Such a set holds every expert more than tol above the k-th
    largest score and fills the rest from those within tol of it, so the
    candidates are enumerated from that window (sets ascending)."""
    beta_row = np.asarray(beta_row, np.float64)
    E = beta_row.shape[0]
    if k >= E:
        return [tuple(range(E))]
    bk = np.sort(beta_row)[::-1][k - 1]
    sure = [e for e in range(E) if beta_row[e] > bk + tol]
    window = [e for e in range(E) if abs(beta_row[e] - bk) <= tol]
    m = k - len(sure)
    assert 0 < m <= len(window) and len(window) <= 12, f"tie window of {len(window)} experts"
    out = []
    for extra in itertools.combinations(window, m):
        S = sorted(sure + list(extra))
        rest = np.delete(beta_row, S)
        if beta_row[S].min() >= rest.max() - tol:
            out.append(tuple(S))
    return out


def check_routing(gpu_ids, gpu_w, gpu_gap, gpu_counts, or_ids, or_w, or_gap, E, beta=None, exact=False):
    """Routing ids bit-exact except near-tie tokens, whose GPU set must be one
    of the oracle's acceptable sets when the oracle's biased scores are given
    (and a valid top-k set in any case); exact=True allows no exception.
    Counts exact against the GPU's own ids and against the oracle where no
    token differs.  Returns (mask of tokens that match, near count)."""
    T, k = or_ids.shape
    same = np.all(gpu_ids == or_ids, axis=1)
    near = or_gap < NEAR_TIE
    if exact:
        bad = np.where(~same)[0]
        assert bad.size == 0, (f"{bad.size} tokens differ from the oracle's tie-broken routing: tokens {bad[:8]}, "
                               f"gpu {gpu_ids[bad[:2]]}, oracle {or_ids[bad[:2]]}")
    bad = ~same & ~near
    assert not bad.any(), f"{bad.sum()} tokens routed differently with gap >= {NEAR_TIE}: {np.where(bad)[0][:8]}"
    if beta is not None:
        for t in np.where(~same)[0]:
            assert tuple(int(e) for e in gpu_ids[t]) in acceptable_sets(beta[t], k), f"token {t}: not a top-k set"
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


def expected_ids(gpu_ids, or_ids, beta):
    """The chosen set the oracle's output is computed for, per token: its own
    where the GPU agrees; where a near tie makes several sets correct, the
    one among the oracle's acceptable sets (from its own scores) that the GPU
    picked -- "given the same routing"."""
    ids = or_ids.copy()
    k = or_ids.shape[1]
    for t in np.where(np.any(gpu_ids != or_ids, axis=1))[0]:
        g = tuple(int(e) for e in gpu_ids[t])
        match = [c for c in acceptable_sets(beta[t], k) if c == g]
        assert match, f"token {t}: the GPU's set is none of the oracle's acceptable sets"
        ids[t] = match[0]
    return ids


def oracle_given_routing_rows(cfg, layer, x_rows, wr_h, c_h, ids, what=""):
    """Oracle forward of token rows under the given chosen sets ids [n,k];
    expert weights generated on the host for exactly the experts named."""
    needed = sorted(set(int(e) for e in np.asarray(ids).ravel()))
    ew = moegen.expert_weights_host(cfg, layer, needed)
    gu = [ew[e][0] if e in ew else None for e in range(cfg.E)]
    wd = [ew[e][1] if e in ew else None for e in range(cfg.E)]
    sgu, swd = moegen.shared_weights_host(cfg, layer)
    n = x_rows.shape[0]
    nchunks = min(n, max(pool_size() * 2, n // 64))
    chunks = [a for a in np.array_split(np.arange(n), nchunks) if a.size]
    done = [0]

    def run(a):
        r = oracle.forward_given_routing(x_rows[a], wr_h, ids[a], gu, wd, sgu, swd, cfg.routed_scale, logit_bias=c_h)
        done[0] += a.size
        if n >= 1024 and len(chunks) > 4 and done[0] * 8 // n != (done[0] - a.size) * 8 // n:
            log(f"  oracle {what}: {done[0]}/{n} tokens")
        return r

    with ThreadPoolExecutor(pool_size()) as pool:
        parts = list(pool.map(run, chunks))
    return np.concatenate([p[1] for p in parts])


def oracle_layer_tokens(dl: DeviceLayer, tokens, ids_of_tokens):
    """Oracle forward of the listed tokens of dl under the given chosen sets."""
    tokens = np.asarray(tokens, np.int64)
    c = dl.cfg
    return None, oracle_given_routing_rows(c, dl.layer, dl.x_h[tokens], dl.wr_h, dl.c_h,
                                           np.asarray(ids_of_tokens, np.int32), f"config {c.index}")


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


def check_output(y_gpu, y_ref, what="", own_rounding=False):
    """Relative L2 <= 5e-3 and max |err| <= 3e-2 * RMS(ref).  own_rounding:
    each element's bound also takes the bf16 half-ulp of its own value
    (2^-8 |ref|), which the stored bf16 output can be off by on its own --
    for shapes whose outputs reach several times their RMS (the shape sweep),
    not for the workloads, which meet the plain bar."""
    y_gpu = np.asarray(y_gpu, np.float64)
    y_ref = np.asarray(y_ref, np.float64)
    err = y_gpu - y_ref
    rel = np.linalg.norm(err) / max(np.linalg.norm(y_ref), 1e-300)
    rms = np.sqrt(np.mean(y_ref ** 2))
    mx = np.abs(err).max() if err.size else 0.0
    log(f"  {what}: rel_l2={rel:.3e} max_abs={mx:.3e} (rms {rms:.3e})")
    assert rel <= REL_L2_TOL, f"{what}: relative L2 {rel:.3e} > {REL_L2_TOL}"
    if own_rounding:
        bound = MAX_ABS_TOL * rms + 2.0 ** -8 * np.abs(y_ref)
        worst = int(np.argmax(np.abs(err) - bound)) if err.size else 0
        assert np.all(np.abs(err) <= bound), (f"{what}: |err| {np.abs(err).flat[worst]:.3e} > "
                                              f"{MAX_ABS_TOL} * rms {rms:.3e} + 2^-8 * |ref| {np.abs(y_ref).flat[worst]:.3e}")
    else:
        assert mx <= MAX_ABS_TOL * rms, f"{what}: max abs {mx:.3e} > {MAX_ABS_TOL} * rms {rms:.3e}"
    return rel, mx / max(rms, 1e-300)
