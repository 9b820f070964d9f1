"""sparse_moe_transformer_ffn_amd: forward pass of one fine-grained sparse MoE
FFN layer (Step 3.5 Flash shape: 288 routed SwiGLU experts of hidden 1,280,
top-8 sigmoid routing with a selection-only balancing bias, one shared
expert) on an AMD Instinct MI355X.

The compute is the C-ABI library libmoe (include/moe.h, HIP kernels for
gfx950).  This package is its Python binding (``_lib``: one function per
C entry point, same names) plus ``LayerBuffers``, which allocates the device
tensors one forward pass needs with torch and calls the entry points in order.
"""
from dataclasses import dataclass
from typing import Optional

from ._lib import (EXPORTS, LIB_PATH, MoeError, lib, make_shape, moe_check_shape, moe_combine, moe_combine_diag,
                   moe_combine_residual, moe_dense_swiglu, moe_dense_workspace_bytes, moe_expert_down,
                   moe_expert_gate_up, moe_expert_swiglu, moe_expert_swiglu_clamped, moe_expert_swiglu_noalloc,
                   moe_expert_swiglu_range, moe_permute, moe_rmsnorm,
                   moe_rmsnorm_route, moe_route, moe_route_diag, moe_shape, moe_shared_swiglu, moe_status_str,
                   moe_workspace_bytes)

__all__ = [
    "EXPORTS", "LIB_PATH", "MoeError", "lib", "make_shape", "moe_check_shape", "moe_combine", "moe_combine_diag",
    "moe_combine_residual", "moe_dense_swiglu", "moe_dense_workspace_bytes", "moe_expert_down", "moe_expert_gate_up",
    "moe_expert_swiglu", "moe_expert_swiglu_clamped", "moe_expert_swiglu_noalloc", "moe_expert_swiglu_range", "moe_permute", "moe_rmsnorm", "moe_rmsnorm_route", "moe_route",
    "moe_route_diag", "moe_shape", "moe_shared_swiglu", "moe_status_str", "moe_workspace_bytes", "LayerBuffers",
]


@dataclass
class LayerBuffers:
    """Device outputs and workspaces of one layer forward for a fixed shape.

    Two workspaces so the shared expert may run on its own stream, concurrently
    with the routed experts."""
    shape: moe_shape
    topk_ids: "object"
    topk_weights: "object"
    topk_gap: "object"
    expert_counts: "object"
    expert_offsets: "object"
    perm_pairs: "object"
    pair_pos: "object"
    y_perm: "object"
    y_shared: Optional["object"]
    y: "object"
    workspace: "object"
    workspace_shared: "object"
    p_e: "object" = None            # diagnostics (forward with diag_groups)
    f_e: "object" = None
    route_summary: "object" = None  # (L_EP, routing confidence)
    expert_rms: "object" = None     # [E+1], entry E the shared expert
    rms_ratio: "object" = None      # (min, max) / median expert RMS

    @staticmethod
    def allocate(T, d, E, k, h, hs, device="cuda"):
        import torch
        shape = make_shape(T, d, E, k, h, hs)
        nb = moe_workspace_bytes(shape)
        i32, f32, bf16 = torch.int32, torch.float32, torch.bfloat16
        dev = torch.device(device)
        return LayerBuffers(
            shape=shape,
            topk_ids=torch.empty((T, k), dtype=i32, device=dev),
            topk_weights=torch.empty((T, k), dtype=f32, device=dev),
            topk_gap=torch.empty((T,), dtype=f32, device=dev),
            expert_counts=torch.empty((E,), dtype=i32, device=dev),
            expert_offsets=torch.empty((E + 1,), dtype=i32, device=dev),
            perm_pairs=torch.empty((T * k,), dtype=i32, device=dev),
            pair_pos=torch.empty((T * k,), dtype=i32, device=dev),
            y_perm=torch.empty((T * k, d), dtype=bf16, device=dev),
            y_shared=torch.empty((T, d), dtype=f32, device=dev) if hs else None,
            y=torch.empty((T, d), dtype=bf16, device=dev),
            workspace=torch.empty((nb,), dtype=torch.uint8, device=dev),
            workspace_shared=torch.empty((nb,), dtype=torch.uint8, device=dev),
            p_e=torch.empty((E,), dtype=f32, device=dev),
            f_e=torch.empty((E,), dtype=f32, device=dev),
            route_summary=torch.empty((2,), dtype=f32, device=dev),
            expert_rms=torch.empty((E + 1,), dtype=f32, device=dev),
            rms_ratio=torch.empty((2,), dtype=f32, device=dev),
        )

    def forward(self, x, w_router, sel_bias, logit_bias, w_gate_up, w_down, ws_gate_up=None, ws_down=None,
                routed_scale=1.0, stream=None, shared="fused", shared_stream=None, diag_groups=None):
        """route -> permute -> experts -> combine, enqueued on `stream`
        (default: current).  The shared expert runs
          "fused":  as one more group inside the grouped expert launches;
          "stream": as moe_shared_swiglu on `shared_stream`, concurrently,
                    joined before the combine;
          "serial": as moe_shared_swiglu on `stream` after the experts.
        diag_groups = G: route and combine through moe_route_diag and
        moe_combine_diag, filling p_e, f_e, route_summary (L_EP over G
        contiguous expert groups, routing confidence), expert_rms and
        rms_ratio; y is the same either way."""
        import torch
        s = stream if stream is not None else torch.cuda.current_stream()
        sh = self.shape
        use_shared = sh.d_shared > 0 and ws_gate_up is not None
        if use_shared and shared == "stream":
            shared_stream.wait_stream(s)
            moe_shared_swiglu(sh, x, ws_gate_up, ws_down, self.y_shared, self.workspace_shared, shared_stream)
        if diag_groups is not None:
            moe_route_diag(sh, x, w_router, sel_bias, logit_bias, self.topk_ids, self.topk_weights,
                           self.expert_counts, self.topk_gap, diag_groups, self.p_e, self.f_e, self.route_summary,
                           self.workspace, s)
        else:
            moe_route(sh, x, w_router, sel_bias, logit_bias, self.topk_ids, self.topk_weights, self.expert_counts,
                      self.topk_gap, self.workspace, s)
        moe_permute(sh, self.topk_ids, self.expert_offsets, self.perm_pairs, self.pair_pos, self.workspace, s)
        fused = use_shared and shared == "fused"
        moe_expert_swiglu(sh, x, self.expert_offsets, self.perm_pairs, w_gate_up, w_down, self.y_perm,
                          self.workspace, s, ws_gate_up=ws_gate_up if fused else None,
                          ws_down=ws_down if fused else None, y_shared=self.y_shared if fused else None)
        if use_shared and shared == "serial":
            moe_shared_swiglu(sh, x, ws_gate_up, ws_down, self.y_shared, self.workspace, s)
        if use_shared and shared == "stream":
            s.wait_stream(shared_stream)
        y_shared = self.y_shared if use_shared else None
        if diag_groups is not None:
            moe_combine_diag(sh, self.y_perm, self.pair_pos, self.topk_weights, y_shared, routed_scale, self.y,
                             self.expert_offsets, self.expert_rms, self.rms_ratio, self.workspace, s)
        else:
            moe_combine(sh, self.y_perm, self.pair_pos, self.topk_weights, y_shared, routed_scale, self.y, s)
        return self.y
