#!/usr/bin/env python3
"""Throughput of the sparse MoE FFN layer forward (libmoe) on one MI355X.

A step is one forward pass of the layer over one batch, enqueued on one
stream: moe_route -> moe_permute -> moe_expert_gate_up -> moe_expert_down ->
moe_combine, with the shared expert running as one more group inside the two
grouped expert launches.  Inputs and weights are resident in HBM before timing starts;
they come from the seeded generator (synthetic values with the shapes and
distributions of the model's layer; no trained weights exist here).

Default workload: the decode batch (T=64 tokens, d_model 4096, 288 experts,
top-8, expert and shared hidden 1280).  The prefill batch (T=8192) is timed
after it and reported in the "prefill" object; the skewed-load batch
(T=4096) and the 12-layer stack (T=256) follow as supplementary "skew" and
"stack" objects.  Prints one JSON line.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-prefill]
                       [--no-cpu-baseline] [--cpu-sample N] [--cpu-sample-large N]
                       [--cpu-sample-stack N]
       python bench.py --write-traffic PMC_DIR   (HBM bytes from counter runs)
"""
import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "MoE layer tok/s; % HBM BW at T=64, % bf16 MFMA peak at T=8192"
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, published
BF16_PEAK_TFLOPS = 2500.0      # MI355X dense bf16 MFMA, published
DIAG_GROUPS = 8                # expert groups of the load-balance statistic: EP8, 36 experts per rank
PROFILES = os.path.join(ROOT, "profiles")


# Sources of the two grouped expert kernels: counter readings are valid for
# the build they were taken on only.
EXPERT_SOURCES = ("expert.hip", "expert_tiled.hip", "grouped.h", "common.h")
# Kernel-name patterns of each phase: the streaming kernels (decode) and the
# LDS-tiled kernels (prefill).
PHASE_KERNELS = {"gate_up": ("k_gate_up<", "k_expert_tiled<0"), "down": ("k_down<", "k_expert_tiled<1")}
COPY_KERNEL = "__amd_rocclr_copyBuffer"
COPY_BYTES = 1 << 30            # the --copy-probe copy: bytes read, and bytes written, per copy


def kernel_source_hash() -> str:
    """Hash of the expert kernel sources with // comments and blank lines
    removed: an edit of the prose alone keeps the counter figures valid."""
    import re
    h = hashlib.sha256()
    for name in EXPERT_SOURCES:
        with open(os.path.join(ROOT, "sparse_moe_transformer_ffn_amd", "csrc", name)) as f:
            for line in f:
                code = re.sub(r"//.*", "", line).rstrip()
                if code:
                    h.update(code.encode() + b"\n")
    return h.hexdigest()[:16]


def load_traffic(workload: str, kernel: str):
    """HBM bytes per launch from committed rocprofv3 counter runs, if they
    were taken on the current kernel source (else None)."""
    path = os.path.join(PROFILES, f"traffic_{kernel}_{workload}.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    if rec.get("source_hash") != kernel_source_hash():
        return None
    return rec.get("hbm_bytes_per_launch")


def _counter_means(pmc_dir, run, counter, patterns):
    """Mean counter value (KiB) per dispatch of the kernels matching any of
    `patterns` in one rocprofv3 --pmc run, and the number of dispatches."""
    import csv
    path = os.path.join(pmc_dir, run, f"{run}_counter_collection.csv")
    with open(path) as f:
        vals = [float(r["Counter_Value"]) for r in csv.DictReader(f)
                if r["Counter_Name"] == counter and any(p in r["Kernel_Name"] for p in patterns)]
    if not vals:
        raise SystemExit(f"{path}: no {counter} rows for {patterns}")
    return sum(vals) / len(vals), len(vals)


def write_traffic(pmc_dir):
    """Turn rocprofv3 counter runs into per-launch HBM bytes of the expert
    kernels: FETCH_SIZE and WRITE_SIZE (KiB per dispatch), each scaled by the
    ratio of known bytes to what the same counter reads for a plain device
    copy of COPY_BYTES.  Expects runs named copy_fetch, copy_write (this
    script with --copy-probe) and {dec,pre}_{fetch,write} (the decode and
    prefill workloads), each made with one counter:

      rocprofv3 --pmc FETCH_SIZE -f csv -d <pmc_dir>/copy_fetch -o copy_fetch -- python3 bench.py --copy-probe
      rocprofv3 --pmc FETCH_SIZE -f csv -d <pmc_dir>/dec_fetch -o dec_fetch -- \
          python3 bench.py --steps 2 --warmup 1 --no-cpu-baseline --no-prefill --no-extras
      rocprofv3 --pmc FETCH_SIZE -f csv -d <pmc_dir>/pre_fetch -o pre_fetch -- \
          python3 bench.py --steps 2 --warmup 1 --only-prefill
      rocprofv3 --pmc FETCH_SIZE -f csv -d <pmc_dir>/skw_fetch -o skw_fetch -- \
          python3 bench.py --steps 2 --warmup 1 --only-skew
      rocprofv3 --pmc FETCH_SIZE -f csv -d <pmc_dir>/stk_fetch -o stk_fetch -- \
          python3 bench.py --steps 2 --warmup 1 --only-stack
      (and the same five with WRITE_SIZE into *_write; a workload whose runs
      are missing is skipped).  The stack's figure is the mean over its twelve
      layers' launches.
    """
    copy_fetch, _ = _counter_means(pmc_dir, "copy_fetch", "FETCH_SIZE", (COPY_KERNEL,))
    copy_write, _ = _counter_means(pmc_dir, "copy_write", "WRITE_SIZE", (COPY_KERNEL,))
    f_fetch = COPY_BYTES / (copy_fetch * 1024)
    f_write = COPY_BYTES / (copy_write * 1024)
    src = kernel_source_hash()
    for workload, run in (("decode", "dec"), ("prefill", "pre"), ("skew", "skw"), ("stack", "stk")):
        if not os.path.exists(os.path.join(pmc_dir, f"{run}_fetch")):
            print(f"{workload}: no {run}_fetch run in {pmc_dir}, skipped")
            continue
        for kernel, patterns in PHASE_KERNELS.items():
            fetch, n = _counter_means(pmc_dir, f"{run}_fetch", "FETCH_SIZE", patterns)
            write, _ = _counter_means(pmc_dir, f"{run}_write", "WRITE_SIZE", patterns)
            rec = {"workload": workload, "kernel": kernel, "source_hash": src,
                   "hbm_bytes_per_launch": fetch * 1024 * f_fetch + write * 1024 * f_write,
                   "fetch_kib_per_dispatch": fetch, "write_kib_per_dispatch": write, "dispatches": n,
                   "fetch_factor": f_fetch, "write_factor": f_write,
                   "copy_probe": {"bytes": COPY_BYTES, "fetch_kib": copy_fetch, "write_kib": copy_write},
                   "made_by": "python bench.py --write-traffic <pmc_dir> over the rocprofv3 runs listed in "
                              "bench.write_traffic's docstring"}
            with open(os.path.join(PROFILES, f"traffic_{kernel}_{workload}.json"), "w") as f:
                json.dump(rec, f, indent=1)
                f.write("\n")
            print(f"{workload:8s} {kernel:8s} {rec['hbm_bytes_per_launch'] / 1e9:8.3f} GB per launch "
                  f"(fetch {fetch:.0f} KiB x {f_fetch:.3f}, write {write:.0f} KiB x {f_write:.3f}, {n} dispatches)")


class Workload:
    """Device tensors of one recipe, filled by the generator."""

    def __init__(self, cfg, dev, layer=0):
        import numpy as np
        import torch
        import moegen
        import sparse_moe_transformer_ffn_amd as moe
        self.cfg = cfg
        self.x_h = moegen.x(cfg, layer)
        self.wr_h = moegen.router(cfg, layer)
        self.b_h = moegen.sel_bias(cfg, layer)
        self.c_h = moegen.logit_bias(cfg, layer)

        def bf16(a):
            return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(dev)

        self.x, self.wr = bf16(self.x_h), bf16(self.wr_h)
        self.b = torch.from_numpy(self.b_h).to(dev)
        self.c = None if self.c_h is None else torch.from_numpy(self.c_h).to(dev)
        E, d, h, hs = cfg.E, cfg.d, cfg.h, cfg.hs
        self.w_gu = torch.empty((E, 2 * h, d), dtype=torch.bfloat16, device=dev)
        self.w_d = torch.empty((E, d, h), dtype=torch.bfloat16, device=dev)
        self.ws_gu = torch.empty((2 * hs, d), dtype=torch.bfloat16, device=dev)
        self.ws_d = torch.empty((d, hs), dtype=torch.bfloat16, device=dev)
        s = torch.cuda.current_stream().cuda_stream
        moegen.fill_experts_device(cfg, layer, self.w_gu.data_ptr(), self.w_d.data_ptr(), s)
        moegen.fill_shared_device(cfg, layer, self.ws_gu.data_ptr(), self.ws_d.data_ptr(), s)
        self.buf = moe.LayerBuffers.allocate(cfg.T, d, E, cfg.k, h, hs, device=dev)
        self.hid = torch.empty((cfg.T * cfg.k, h), dtype=torch.bfloat16, device=dev)
        self.hid_shared = torch.empty((cfg.T, hs), dtype=torch.bfloat16, device=dev)
        # Diagnostics outputs (routing statistics over DIAG_GROUPS expert
        # groups, per-expert activation RMS and its spread).
        self.p_e = torch.empty((E,), dtype=torch.float32, device=dev)
        self.f_e = torch.empty((E,), dtype=torch.float32, device=dev)
        self.route_summary = torch.empty((2,), dtype=torch.float32, device=dev)
        self.expert_rms = torch.empty((E + 1,), dtype=torch.float32, device=dev)
        self.rms_ratio = torch.empty((2,), dtype=torch.float32, device=dev)
        self.x_norm = torch.empty_like(self.x)
        torch.cuda.synchronize()

    def step(self, main, ev=None, diag=False, prenorm=False):
        """One forward; ev = (step start, before gate_up, after gate_up,
        after down, step end) events; diag: the routing and combine calls
        with their diagnostic side outputs; prenorm: the pre-norm block, with
        x taken as the residual stream, normalised inside the router call
        into x_norm, and added back inside the combine."""
        import sparse_moe_transformer_ffn_amd as moe
        b, sh, c = self.buf, self.buf.shape, self.cfg
        x = self.x_norm if prenorm else self.x
        if ev:
            ev[0].record(main)
        if prenorm:
            moe.moe_rmsnorm_route(sh, self.x, None, 1e-6, self.wr, self.b, self.c, self.x_norm, b.topk_ids,
                                  b.topk_weights, b.expert_counts, b.topk_gap, b.workspace, main)
        elif diag:
            moe.moe_route_diag(sh, self.x, self.wr, self.b, self.c, b.topk_ids, b.topk_weights, b.expert_counts,
                               b.topk_gap, DIAG_GROUPS, self.p_e, self.f_e, self.route_summary, b.workspace, main)
        else:
            moe.moe_route(sh, self.x, self.wr, self.b, self.c, b.topk_ids, b.topk_weights, b.expert_counts,
                          b.topk_gap, b.workspace, main)
        moe.moe_permute(sh, b.topk_ids, b.expert_offsets, b.perm_pairs, b.pair_pos, b.workspace, main)
        if ev:
            ev[1].record(main)
        moe.moe_expert_gate_up(sh, x, b.expert_offsets, b.perm_pairs, self.w_gu, self.hid, b.workspace, main,
                               ws_gate_up=self.ws_gu, hid_shared=self.hid_shared)
        if ev:
            ev[2].record(main)
        moe.moe_expert_down(sh, b.expert_offsets, self.hid, self.w_d, b.y_perm, b.workspace, main,
                            hid_shared=self.hid_shared, ws_down=self.ws_d, y_shared=b.y_shared)
        if ev:
            ev[3].record(main)
        if prenorm:
            moe.moe_combine_residual(sh, b.y_perm, b.pair_pos, b.topk_weights, b.y_shared, c.routed_scale, self.x,
                                     b.y, main)
        elif diag:
            moe.moe_combine_diag(sh, b.y_perm, b.pair_pos, b.topk_weights, b.y_shared, c.routed_scale, b.y,
                                 b.expert_offsets, self.expert_rms, self.rms_ratio, b.workspace, main)
        else:
            moe.moe_combine(sh, b.y_perm, b.pair_pos, b.topk_weights, b.y_shared, c.routed_scale, b.y, main)
        if ev:
            ev[4].record(main)


def algorithmic(cfg, n_touched):
    """Bytes and flops the method itself must move / compute (not the dense
    E-expert work it avoids; intermediates excluded)."""
    T, d, E, k, h, hs = cfg.T, cfg.d, cfg.E, cfg.k, cfg.h, cfg.hs
    w_expert = 3 * d * h * 2
    step_bytes = n_touched * w_expert + 3 * d * hs * 2 + E * d * 2 + T * d * 2 * 2 + T * k * 4 * 4
    step_flops = 2 * T * k * 3 * d * h + 2 * T * 3 * d * hs + 2 * T * d * E
    # The grouped launches include the shared expert (one more group).
    gate_up_bytes = (n_touched * 2 * h + 2 * hs) * d * 2 + T * d * 2 + T * (k * h + hs) * 2
    gate_up_flops = 2 * T * (k * 2 * h + 2 * hs) * d
    down_bytes = (n_touched * h + hs) * d * 2 + T * (k * h + hs) * 2 + T * k * d * 2 + T * d * 4
    down_flops = 2 * T * (k * h + hs) * d
    return dict(step_bytes=step_bytes, step_flops=step_flops, gate_up_bytes=gate_up_bytes,
                gate_up_flops=gate_up_flops, down_bytes=down_bytes, down_flops=down_flops)


def time_workload(cfg, steps, warmup, dev, extras=True):
    import numpy as np
    import torch
    wl = Workload(cfg, dev)
    main = torch.cuda.current_stream()
    for _ in range(warmup):
        wl.step(main)
    torch.cuda.synchronize()
    # The timed steps: nothing recorded between them.  Each event record on
    # the stream leaves the GPU idle for about 5 us before the next kernel,
    # so the per-kernel times come from a second, instrumented pass.
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    t0.record(main)
    for _ in range(steps):
        wl.step(main)
    t1.record(main)
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    ms = t0.elapsed_time(t1) / steps
    # The same number of steps with events at the step ends and around the
    # two expert launches (five records per step).
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(5)] for _ in range(steps)]
    for i in range(steps):
        wl.step(main, evs[i])
    torch.cuda.synchronize()
    gate_up_ms = float(np.mean([e[1].elapsed_time(e[2]) for e in evs]))
    down_ms = float(np.mean([e[2].elapsed_time(e[3]) for e in evs]))
    per_step = np.array([e[0].elapsed_time(e[4]) for e in evs])
    counts = wl.buf.expert_counts.cpu().numpy()
    n_touched = int((counts > 0).sum())
    alg = algorithmic(cfg, n_touched)
    res = dict(ms_per_step=ms, wall_ms_per_step=wall * 1e3 / steps, gate_up_ms=gate_up_ms, down_ms=down_ms,
               ms_per_step_median=float(np.median(per_step)), ms_per_step_min=float(per_step.min()),
               ms_per_step_instrumented=float(per_step.mean()),
               n_touched=n_touched, max_load=int(counts.max()), idle_experts=int((counts == 0).sum()), alg=alg)
    if not extras:
        return wl, res
    # The same steps with the diagnostic side outputs, timed separately (not
    # part of the headline figure).
    wl.step(main, diag=True)
    dev_ev = [[torch.cuda.Event(enable_timing=True) for _ in range(5)] for _ in range(steps)]
    for i in range(steps):
        wl.step(main, dev_ev[i], diag=True)
    torch.cuda.synchronize()
    diag_step = np.array([e[0].elapsed_time(e[4]) for e in dev_ev])
    # The pre-norm block (RMSNorm fused into the router, residual into the
    # combine), timed the same way.
    wl.step(main, prenorm=True)
    pre_ev = [[torch.cuda.Event(enable_timing=True) for _ in range(5)] for _ in range(steps)]
    for i in range(steps):
        wl.step(main, pre_ev[i], prenorm=True)
    torch.cuda.synchronize()
    pre_step = np.array([e[0].elapsed_time(e[4]) for e in pre_ev])
    # The step captured once into a HIP graph and replayed (launch costs off
    # the host; the same kernels).
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        wl.step(torch.cuda.current_stream())
    graph.replay()
    g_ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    torch.cuda.synchronize()
    for a, z in g_ev:
        a.record(main)
        graph.replay()
        z.record(main)
    torch.cuda.synchronize()
    graph_step = np.array([a.elapsed_time(z) for a, z in g_ev])
    del graph
    diag = dict(ep_groups=DIAG_GROUPS, ms_per_step_median=float(np.median(diag_step)),
                l_ep=float(wl.route_summary[0]), confidence=float(wl.route_summary[1]),
                rms_min_to_median=float(wl.rms_ratio[0]), rms_max_to_median=float(wl.rms_ratio[1]))
    diag["overhead_ms"] = diag["ms_per_step_median"] - res["ms_per_step_median"]
    res["diagnostics"] = diag
    res["prenorm_block"] = {"ms_per_step_median": float(np.median(pre_step)),
                            "overhead_ms": float(np.median(pre_step)) - res["ms_per_step_median"]}
    res["graph_replay"] = {"ms_per_step_median": float(np.median(graph_step)),
                           "ms_per_step_min": float(graph_step.min())}
    return wl, res


def time_skew(steps, warmup, dev, cpu_sample=0):
    """The skewed-load workload (T = 4096, Zipf(1.1) logit offset: the
    busiest expert gets about ten times the mean load) timed like the others;
    a supplementary figure, not the bench line.  Its dominant kernel (the
    grouped gate/up launch) is HBM-bound: the roofline objects give its
    algorithmic bytes and flops over its time."""
    import moegen
    cfg = moegen.CONFIGS[3]
    wl, r = time_workload(cfg, steps, warmup, dev, extras=False)
    alg = r["alg"]
    sec = r["ms_per_step"] * 1e-3
    gu_sec = r["gate_up_ms"] * 1e-3
    out = {"workload": cfg.workload, "tok_s": cfg.T / sec, "ms_per_step": r["ms_per_step"],
           "instrumented": instrumented(r), "steps": steps,
           "step_hbm_gbs": alg["step_bytes"] / sec / 1e9, "step_hbm_frac": alg["step_bytes"] / sec / 1e9 / HBM_PEAK_GBS,
           "step_tflops": alg["step_flops"] / sec / 1e12,
           "step_mfma_frac": alg["step_flops"] / sec / 1e12 / BF16_PEAK_TFLOPS,
           "roofline": roofline("hbm", alg["gate_up_bytes"] / gu_sec / 1e9, load_traffic("skew", "gate_up")),
           "roofline_mfma": roofline("mfma", alg["gate_up_flops"] / gu_sec / 1e12, None),
           "kernels": {"gate_up_ms": r["gate_up_ms"], "down_ms": r["down_ms"],
                       "gate_up_gbs": alg["gate_up_bytes"] / gu_sec / 1e9,
                       "down_gbs": alg["down_bytes"] / (r["down_ms"] * 1e-3) / 1e9},
           "touched_experts": r["n_touched"], "max_load": r["max_load"], "idle_experts": r["idle_experts"]}
    if cpu_sample:
        out["cpu_baseline"] = cpu_baseline(wl, cpu_sample)
    del wl
    return out


def time_stack(steps, warmup, dev, cpu_sample=0):
    """The 12-layer stack (T = 256, distinct weights per layer, 109 GB
    resident): layer l + 1 takes the unit-gain RMSNorm of layer l's output.
    One pass = 12 layer steps and 11 normalisations; supplementary figure.
    Its dominant kernel (each layer's grouped gate/up launch) is HBM-bound:
    the roofline object gives its algorithmic bytes over its time, summed
    over the layers, and its counted traffic as the mean per launch."""
    import numpy as np
    import torch
    import moegen
    import sparse_moe_transformer_ffn_amd as moe
    cfg = moegen.CONFIGS[4]
    layers = [Workload(cfg, dev, layer=l) for l in range(cfg.layers)]
    main = torch.cuda.current_stream()

    def chain(ev=None):
        for l, wl in enumerate(layers):
            wl.step(main, ev[l] if ev else None)
            if l + 1 < cfg.layers:
                moe.moe_rmsnorm(cfg.T, cfg.d, wl.buf.y, None, 1e-6, layers[l + 1].x, main)

    for _ in range(warmup):
        chain()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    torch.cuda.synchronize()
    for a, z in ev:
        a.record(main)
        chain()
        z.record(main)
    torch.cuda.synchronize()
    per = np.array([a.elapsed_time(z) for a, z in ev])
    # The same passes with events around each layer's two expert launches
    # (records idle the GPU between kernels, so these are not the timed
    # passes): the dominant kernel's time.
    lev = [[[torch.cuda.Event(enable_timing=True) for _ in range(5)] for _ in layers] for _ in range(steps)]
    for p in lev:
        chain(p)
    torch.cuda.synchronize()
    gu_ms = np.array([[e[1].elapsed_time(e[2]) for e in p] for p in lev]).mean(0)   # per layer
    dn_ms = np.array([[e[2].elapsed_time(e[3]) for e in p] for p in lev]).mean(0)
    touched = [int((wl.buf.expert_counts.cpu().numpy() > 0).sum()) for wl in layers]
    algs = [algorithmic(cfg, n) for n in touched]
    nbytes = sum(a["step_bytes"] for a in algs)
    gu_gbs = sum(a["gate_up_bytes"] for a in algs) / (gu_ms.sum() * 1e-3) / 1e9
    dn_gbs = sum(a["down_bytes"] for a in algs) / (dn_ms.sum() * 1e-3) / 1e9
    ms = float(np.median(per))
    x0 = layers[0].x_h
    del layers
    out = {"workload": cfg.workload, "layers": cfg.layers, "tok_s": cfg.T / (ms * 1e-3), "ms_per_pass_median": ms,
           "ms_per_pass_min": float(per.min()), "passes": steps, "hbm_gbs": nbytes / (ms * 1e-3) / 1e9,
           "hbm_frac": nbytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS,
           "roofline": roofline("hbm", gu_gbs, load_traffic("stack", "gate_up")),
           "kernels": {"gate_up_ms_per_layer": float(gu_ms.mean()), "down_ms_per_layer": float(dn_ms.mean()),
                       "gate_up_gbs": gu_gbs, "down_gbs": dn_gbs},
           "touched_experts_per_layer": touched}
    if cpu_sample:
        out["cpu_baseline"] = cpu_baseline_stack(cfg, x0, cpu_sample)
    return out


def mean_ms(call, n, stream):
    """Mean time of n back-to-back calls on `stream`, events only around the
    whole loop."""
    import torch
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0.record(stream)
    for _ in range(n):
        call()
    t1.record(stream)
    torch.cuda.synchronize()
    return t0.elapsed_time(t1) / n


DENSE_HIDDEN = 11264   # dense FFN hidden size of the first blocks and the MTP heads


def time_dense(T, steps, dev):
    """The dense SwiGLU FFN (d = 4096, hidden 11,264) on T tokens through the
    grouped kernels: median launch time, algorithmic bytes and flops."""
    import numpy as np
    import torch
    import moegen
    import sparse_moe_transformer_ffn_amd as moe
    cfg = moegen.custom(1, T=T, hs=DENSE_HIDDEN)
    d, H = cfg.d, DENSE_HIDDEN
    x = torch.from_numpy(moegen.x(cfg).view(np.int16)).view(torch.bfloat16).to(dev)
    w_gu = torch.empty((2 * H, d), dtype=torch.bfloat16, device=dev)
    w_d = torch.empty((d, H), dtype=torch.bfloat16, device=dev)
    moegen.fill_shared_device(cfg, 0, w_gu.data_ptr(), w_d.data_ptr(), torch.cuda.current_stream().cuda_stream)
    y = torch.empty((T, d), dtype=torch.float32, device=dev)
    ws = torch.empty(moe.moe_dense_workspace_bytes(T, d, H), dtype=torch.uint8, device=dev)
    main = torch.cuda.current_stream()
    for _ in range(2):
        moe.moe_dense_swiglu(T, d, H, x, w_gu, w_d, y, ws, main)
    ms = mean_ms(lambda: moe.moe_dense_swiglu(T, d, H, x, w_gu, w_d, y, ws, main), steps, main)
    nbytes = 3 * d * H * 2 + T * d * 2 + T * d * 4
    flops = 2 * T * 3 * d * H
    return {"tokens": T, "ms": ms, "tok_s": T / (ms * 1e-3),
            "hbm_gbs": nbytes / (ms * 1e-3) / 1e9, "hbm_frac": nbytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS,
            "tflops": flops / (ms * 1e-3) / 1e12, "mfma_frac": flops / (ms * 1e-3) / 1e12 / BF16_PEAK_TFLOPS}


EP_SHARES = 8   # expert-parallel group size the pages deploy: 36 of 288 experts per GPU


def time_share(wl, steps):
    """One GPU's share of an 8-way expert-parallel layer: the grouped expert
    kernels on experts [0, E/8) with their weights only, on the routing the
    timed steps produced.  Median launch time next to the whole call's."""
    import numpy as np
    import torch
    import sparse_moe_transformer_ffn_amd as moe
    b, sh, c = wl.buf, wl.buf.shape, wl.cfg
    e1 = c.E // EP_SHARES
    main = torch.cuda.current_stream()

    def share():
        moe.moe_expert_swiglu_range(sh, 0, e1, wl.x, b.expert_offsets, b.perm_pairs, wl.w_gu[:e1], wl.w_d[:e1],
                                    b.y_perm, b.workspace, main)

    for _ in range(2):
        share()
    ms = mean_ms(share, steps, main)
    counts = b.expert_counts.cpu().numpy()[:e1]
    rows = int(counts.sum())
    touched = int((counts > 0).sum())
    nbytes = touched * 3 * c.d * c.h * 2 + rows * c.d * 2 * 2
    flops = 2 * rows * 3 * c.d * c.h
    return {"experts": [0, e1], "rows": rows, "touched_experts": touched, "ms": ms,
            "hbm_gbs": nbytes / (ms * 1e-3) / 1e9, "tflops": flops / (ms * 1e-3) / 1e12}


def cpu_baseline(wl, n_sample):
    """The CPU oracle, single-threaded, on a bounded sample of the same
    workload's tokens (whole layer per token).  Weight generation is not
    timed."""
    import numpy as np
    import moegen
    import oracle
    cfg = wl.cfg
    tokens = np.linspace(0, cfg.T - 1, n_sample).astype(np.int32)
    ids, _, _, _ = oracle.route(wl.x_h[tokens], wl.wr_h, wl.b_h, cfg.k, logit_bias=wl.c_h)
    needed = sorted(set(ids.ravel().tolist()))
    ew = moegen.expert_weights_host(cfg, 0, needed)
    gu = [ew[e][0] if e in ew else None for e in range(cfg.E)]
    wd = [ew[e][1] if e in ew else None for e in range(cfg.E)]
    sgu, swd = moegen.shared_weights_host(cfg)
    # One thread, pinned to one core for the timed call.
    saved = os.sched_getaffinity(0)
    core = min(saved)
    os.sched_setaffinity(0, {core})
    try:
        t = time.perf_counter()
        oracle.layer(wl.x_h, wl.wr_h, wl.b_h, cfg.k, gu, wd, sgu, swd, cfg.routed_scale, logit_bias=wl.c_h,
                     tokens=tokens)
        dt = time.perf_counter() - t
    finally:
        os.sched_setaffinity(0, saved)
    flops_per_token = 2 * cfg.d * cfg.E + 2 * 3 * cfg.d * (cfg.k * cfg.h + cfg.hs)
    return {"value": n_sample / dt, "unit": "tok/s", "cores": 1, "kind": "oracle",
            "gflops": n_sample * flops_per_token / dt / 1e9,
            "host": {"cpu": host_cpu_model(), "online_cores": os.cpu_count(), "affinity_cores": len(saved),
                     "pinned_to": core},
            "sample": f"{n_sample} of the {cfg.T} tokens of the {cfg.name} workload, whole layer per token "
                      f"(route over {cfg.E} experts, {cfg.k} routed + 1 shared SwiGLU expert, combine); "
                      f"{dt:.1f} s on one host thread pinned to one core"}


def _to_bf16(a):
    """float32 -> bf16 bit patterns, round to nearest even (the layer output
    as the stack stores it)."""
    import numpy as np
    b = np.ascontiguousarray(a, np.float32).view(np.uint32).astype(np.uint64)
    return ((b + 0x7FFF + ((b >> 16) & 1)) >> 16).astype(np.uint16)


def cpu_baseline_stack(cfg, x0, n_sample):
    """The CPU oracle on the 12-layer stack: n_sample tokens carried through
    all layers (each layer's output rounded to bf16 and normalised, as the
    chained run does), single-threaded; weight generation is not timed."""
    import numpy as np
    import moegen
    import oracle
    tokens = np.linspace(0, cfg.T - 1, n_sample).astype(np.int64)
    x = np.ascontiguousarray(x0[tokens])
    saved = os.sched_getaffinity(0)
    core = min(saved)
    dt = 0.0
    for l in range(cfg.layers):
        wr, b = moegen.router(cfg, l), moegen.sel_bias(cfg, l)
        ids, _, _, _ = oracle.route(x, wr, b, cfg.k)
        ew = moegen.expert_weights_host(cfg, l, sorted(set(ids.ravel().tolist())))
        gu = [ew[e][0] if e in ew else None for e in range(cfg.E)]
        wd = [ew[e][1] if e in ew else None for e in range(cfg.E)]
        sgu, swd = moegen.shared_weights_host(cfg, l)
        os.sched_setaffinity(0, {core})
        try:
            t = time.perf_counter()
            _, _, _, y = oracle.layer(x, wr, b, cfg.k, gu, wd, sgu, swd, cfg.routed_scale)
            if l + 1 < cfg.layers:
                x = oracle.rmsnorm(_to_bf16(y), None, 1e-6)
            dt += time.perf_counter() - t
        finally:
            os.sched_setaffinity(0, saved)
    n = n_sample * cfg.layers
    flops_per_token = 2 * cfg.d * cfg.E + 2 * 3 * cfg.d * (cfg.k * cfg.h + cfg.hs)
    return {"value": n_sample / dt, "unit": "tok/s (through all 12 layers)", "cores": 1, "kind": "oracle",
            "gflops": n * flops_per_token / dt / 1e9,
            "host": {"cpu": host_cpu_model(), "online_cores": os.cpu_count(), "affinity_cores": len(saved),
                     "pinned_to": core},
            "sample": f"{n_sample} of the {cfg.T} tokens of the {cfg.name} workload carried through all "
                      f"{cfg.layers} layers ({n} token-layers: route, {cfg.k} routed + 1 shared SwiGLU expert, "
                      f"combine, RMSNorm between layers); {dt:.1f} s on one host thread pinned to one core"}


def host_cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def instrumented(r):
    """Step times of the instrumented pass (five event records per step)."""
    return {"ms_per_step": r["ms_per_step_instrumented"], "ms_per_step_median": r["ms_per_step_median"],
            "ms_per_step_min": r["ms_per_step_min"], "event_records_per_step": 5}


def roofline(kind, achieved, traffic):
    if kind == "hbm":
        return {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": achieved / HBM_PEAK_GBS, "traffic": traffic}
    return {"bound": "mfma", "achieved": achieved, "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
            "frac": achieved / BF16_PEAK_TFLOPS, "traffic": traffic}


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--no-prefill", action="store_true")
    ap.add_argument("--only-prefill", action="store_true", help="time only the prefill workload (profiling)")
    ap.add_argument("--only-skew", action="store_true", help="time only the skewed-load workload (profiling)")
    ap.add_argument("--only-stack", action="store_true", help="time only the 12-layer stack (profiling)")
    ap.add_argument("--copy-probe", action="store_true",
                    help="run only a plain 1 GiB device copy (the known-size reference for HBM byte counters)")
    ap.add_argument("--prefill-steps", type=int, default=10)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-dense", action="store_true", help="skip the dense SwiGLU FFN lines")
    ap.add_argument("--no-extras", action="store_true",
                    help="time the layer step only: no diagnostics, pre-norm block, expert share or dense FFN "
                         "(profiling runs)")
    ap.add_argument("--no-supplementary", action="store_true",
                    help="skip the skewed-load workload and the 12-layer stack")
    ap.add_argument("--cpu-sample", type=int, default=64, help="tokens of the decode batch the oracle runs")
    ap.add_argument("--cpu-sample-large", type=int, default=32,
                    help="tokens of the prefill and skewed batches the oracle runs")
    ap.add_argument("--cpu-sample-stack", type=int, default=2,
                    help="tokens the oracle carries through the 12-layer stack")
    ap.add_argument("--write-traffic", metavar="PMC_DIR",
                    help="no GPU work: write profiles/traffic_*.json from rocprofv3 counter runs in PMC_DIR")
    args = ap.parse_args()
    if args.write_traffic:
        write_traffic(args.write_traffic)
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: the layer's hot path is built and timed on a single MI355X "
              "(no expert parallelism across GPUs in this library). Run with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import torch
    import moegen
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    if args.copy_probe:
        src = torch.ones(1 << 29, dtype=torch.int16, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes": src.numel() * 2, "copies": 3}), flush=True)
        return
    if args.only_prefill or args.only_skew:
        pcfg = moegen.CONFIGS[2 if args.only_prefill else 3]
        _, p = time_workload(pcfg, args.steps, args.warmup, dev, extras=False)
        print(json.dumps({"workload": pcfg.workload, "ms_per_step": p["ms_per_step"],
                          "gate_up_ms": p["gate_up_ms"], "down_ms": p["down_ms"]}), flush=True)
        return
    if args.only_stack:
        print(json.dumps(time_stack(args.steps, args.warmup, dev)), flush=True)
        return
    cfg = moegen.CONFIGS[1]
    extras = not args.no_extras
    wl, r = time_workload(cfg, args.steps, args.warmup, dev, extras)
    alg = r["alg"]
    tok_s = cfg.T / (r["ms_per_step"] * 1e-3)
    gate_up_gbs = alg["gate_up_bytes"] / (r["gate_up_ms"] * 1e-3) / 1e9
    out = {
        "metric": METRIC, "value": tok_s, "unit": "tok/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": r["ms_per_step"], "instrumented": instrumented(r),
        "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": cfg.workload, "tokens": cfg.T, "d_model": cfg.d, "experts": cfg.E, "top_k": cfg.k,
                   "expert_hidden": cfg.h, "shared_hidden": cfg.hs, "seed": cfg.seed},
        "roofline": roofline("hbm", gate_up_gbs, load_traffic("decode", "gate_up")),
        "step": {"algorithmic_bytes": alg["step_bytes"], "algorithmic_flops": alg["step_flops"],
                 "hbm_gbs": alg["step_bytes"] / (r["ms_per_step"] * 1e-3) / 1e9,
                 "hbm_frac": alg["step_bytes"] / (r["ms_per_step"] * 1e-3) / 1e9 / HBM_PEAK_GBS,
                 "touched_experts": r["n_touched"], "max_load": r["max_load"], "idle_experts": r["idle_experts"]},
        "kernels": {"gate_up_ms": r["gate_up_ms"], "down_ms": r["down_ms"],
                    "gate_up_gbs": gate_up_gbs,
                    "down_gbs": alg["down_bytes"] / (r["down_ms"] * 1e-3) / 1e9},
    }
    if extras:
        out["diagnostics"] = r["diagnostics"]
        out["prenorm_block"] = r["prenorm_block"]
        out["graph_replay"] = r["graph_replay"]
        out["ep_share"] = time_share(wl, args.steps)
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(wl, args.cpu_sample)
    del wl
    torch.cuda.empty_cache()
    if extras and not args.no_dense:
        out["dense_ffn"] = {"d_model": cfg.d, "hidden": DENSE_HIDDEN,
                            "decode": time_dense(cfg.T, args.steps, dev),
                            "prefill": None if args.no_prefill else time_dense(moegen.CONFIGS[2].T, 10, dev)}
        torch.cuda.empty_cache()

    if not args.no_prefill:
        pcfg = moegen.CONFIGS[2]
        pwl, p = time_workload(pcfg, args.prefill_steps, args.warmup, dev, extras)
        palg = p["alg"]
        gate_up_tf = palg["gate_up_flops"] / (p["gate_up_ms"] * 1e-3) / 1e12
        step_tf = palg["step_flops"] / (p["ms_per_step"] * 1e-3) / 1e12
        out["prefill"] = {
            "workload": pcfg.workload, "tok_s": pcfg.T / (p["ms_per_step"] * 1e-3), "ms_per_step": p["ms_per_step"],
            "instrumented": instrumented(p),
            "steps": args.prefill_steps, "step_tflops": step_tf, "step_mfma_frac": step_tf / BF16_PEAK_TFLOPS,
            "roofline": roofline("mfma", gate_up_tf, load_traffic("prefill", "gate_up")),
            "kernels": {"gate_up_ms": p["gate_up_ms"], "down_ms": p["down_ms"],
                        "down_tflops": palg["down_flops"] / (p["down_ms"] * 1e-3) / 1e12},
            "touched_experts": p["n_touched"], "max_load": p["max_load"], "idle_experts": p["idle_experts"],
        }
        if extras:
            # Supplementary, not one of the workloads: the same batch with a
            # selection bias of U[-0.005, 0.005], which spreads the loads
            # nearly evenly over the experts.
            bcfg = moegen.custom(2, bias=0.005)
            bwl, bp = time_workload(bcfg, args.prefill_steps, args.warmup, dev, extras=False)
            del bwl
            btf = bp["alg"]["step_flops"] / (bp["ms_per_step"] * 1e-3) / 1e12
            out["prefill"]["balanced_bias_0.005"] = {
                "ms_per_step": bp["ms_per_step"], "tok_s": bcfg.T / (bp["ms_per_step"] * 1e-3),
                "step_tflops": btf, "step_mfma_frac": btf / BF16_PEAK_TFLOPS,
                "gate_up_tflops": bp["alg"]["gate_up_flops"] / (bp["gate_up_ms"] * 1e-3) / 1e12,
                "touched_experts": bp["n_touched"], "max_load": bp["max_load"], "idle_experts": bp["idle_experts"]}
            out["prefill"].update(diagnostics=p["diagnostics"], prenorm_block=p["prenorm_block"],
                                  graph_replay=p["graph_replay"],
                                  ep_share=time_share(pwl, args.prefill_steps))
        if not args.no_cpu_baseline:
            out["prefill"]["cpu_baseline"] = cpu_baseline(pwl, args.cpu_sample_large)
        del pwl
    if extras and not args.no_supplementary:
        torch.cuda.empty_cache()
        no_cpu = args.no_cpu_baseline
        out["skew"] = time_skew(args.prefill_steps, args.warmup, dev, 0 if no_cpu else args.cpu_sample_large)
        torch.cuda.empty_cache()
        out["stack"] = time_stack(args.prefill_steps, args.warmup, dev, 0 if no_cpu else args.cpu_sample_stack)
        torch.cuda.empty_cache()
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
