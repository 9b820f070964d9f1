"""ctypes binding of libmoe (include/moe.h).

Argument marshalling only: every function forwards torch tensors' device
pointers and the current HIP stream to the C ABI and raises MoeError on a
non-OK status.  All arithmetic runs in libmoe's HIP kernels; there is no
fallback.  Tensors must be contiguous and on the GPU (a host pointer handed to
a kernel would fault the device, so that is checked here).
"""
import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libmoe.so")

STATUS = {
    0: "MOE_OK",
    1: "MOE_ERR_INVALID_ARGUMENT",
    2: "MOE_ERR_UNSUPPORTED_SHAPE",
    3: "MOE_ERR_MISALIGNED",
    4: "MOE_ERR_WORKSPACE_TOO_SMALL",
    5: "MOE_ERR_HIP",
}

EXPORTS = (
    "moe_status_str", "moe_check_shape", "moe_workspace_bytes", "moe_route", "moe_permute", "moe_expert_swiglu",
    "moe_expert_gate_up", "moe_expert_down", "moe_shared_swiglu", "moe_combine", "moe_rmsnorm", "moe_route_diag",
    "moe_combine_diag", "moe_dense_workspace_bytes", "moe_dense_swiglu", "moe_expert_swiglu_range",
    "moe_rmsnorm_route", "moe_combine_residual", "moe_expert_swiglu_clamped", "moe_expert_swiglu_noalloc",
)


class MoeError(RuntimeError):
    def __init__(self, fn, code):
        super().__init__(f"{fn} failed: {STATUS.get(code, code)}")
        self.code = code


class moe_shape(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in
                ("num_tokens", "d_model", "num_experts", "top_k", "d_expert", "d_shared")]


_P = ctypes.c_void_p
_SP = ctypes.POINTER(moe_shape)
_lib = None


def lib():
    """The loaded libmoe.so.  Raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"libmoe is not built ({LIB_PATH} missing); run __graft_entry__.build()")
        L = ctypes.CDLL(LIB_PATH)
        L.moe_status_str.restype = ctypes.c_char_p
        L.moe_status_str.argtypes = [ctypes.c_int]
        L.moe_check_shape.argtypes = [_SP]
        L.moe_workspace_bytes.argtypes = [_SP, ctypes.POINTER(ctypes.c_size_t)]
        L.moe_route.argtypes = [_SP, _P, _P, _P, _P, _P, _P, _P, _P, _P, ctypes.c_size_t, _P]
        L.moe_permute.argtypes = [_SP, _P, _P, _P, _P, _P, ctypes.c_size_t, _P]
        L.moe_expert_swiglu.argtypes = [_SP, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, ctypes.c_size_t, _P]
        L.moe_expert_gate_up.argtypes = [_SP, _P, _P, _P, _P, _P, _P, _P, _P, ctypes.c_size_t, _P]
        L.moe_expert_down.argtypes = [_SP, _P, _P, _P, _P, _P, _P, _P, _P, ctypes.c_size_t, _P]
        L.moe_shared_swiglu.argtypes = [_SP, _P, _P, _P, _P, _P, ctypes.c_size_t, _P]
        L.moe_combine.argtypes = [_SP, _P, _P, _P, _P, ctypes.c_float, _P, _P]
        L.moe_rmsnorm.argtypes = [ctypes.c_int32, ctypes.c_int32, _P, _P, ctypes.c_float, _P, _P]
        L.moe_route_diag.argtypes = [_SP, _P, _P, _P, _P, _P, _P, _P, _P, ctypes.c_int32, _P, _P, _P, _P,
                                     ctypes.c_size_t, _P]
        L.moe_dense_workspace_bytes.argtypes = [ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
                                                 ctypes.POINTER(ctypes.c_size_t)]
        L.moe_dense_swiglu.argtypes = [ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, _P, _P, _P, _P, _P,
                                       ctypes.c_size_t, _P]
        L.moe_expert_swiglu_range.argtypes = [_SP, ctypes.c_int32, ctypes.c_int32, _P, _P, _P, _P, _P, _P, _P,
                                              ctypes.c_size_t, _P]
        L.moe_rmsnorm_route.argtypes = [_SP, _P, _P, ctypes.c_float, _P, _P, _P, _P, _P, _P, _P, _P, _P,
                                         ctypes.c_size_t, _P]
        L.moe_combine_residual.argtypes = [_SP, _P, _P, _P, _P, ctypes.c_float, _P, _P, _P]
        L.moe_expert_swiglu_clamped.argtypes = [_SP, _P, _P, _P, _P, _P, _P, _P, _P, _P, ctypes.c_float, _P,
                                                ctypes.c_size_t, _P]
        L.moe_expert_swiglu_noalloc.argtypes = [_SP, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P]
        L.moe_combine_diag.argtypes = [_SP, _P, _P, _P, _P, ctypes.c_float, _P, _P, _P, _P, _P, ctypes.c_size_t,
                                       _P]
        for name in EXPORTS[1:]:
            getattr(L, name).restype = ctypes.c_int
        _lib = L
    return _lib


def make_shape(T, d, E, k, h, hs) -> moe_shape:
    return moe_shape(int(T), int(d), int(E), int(k), int(h), int(hs))


def _ptr(t):
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError("libmoe takes device tensors only")
    if not t.is_contiguous():
        raise ValueError("libmoe takes contiguous tensors only")
    return t.data_ptr()


def _stream(stream):
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    return getattr(stream, "cuda_stream", stream)


def _ws(workspace):
    return (None, 0) if workspace is None else (_ptr(workspace), workspace.numel() * workspace.element_size())


def _check(name, rc):
    if rc != 0:
        raise MoeError(name, rc)


def moe_status_str(code: int) -> str:
    return lib().moe_status_str(code).decode()


def moe_check_shape(shape: moe_shape) -> int:
    return lib().moe_check_shape(ctypes.byref(shape))


def moe_workspace_bytes(shape: moe_shape) -> int:
    n = ctypes.c_size_t(0)
    _check("moe_workspace_bytes", lib().moe_workspace_bytes(ctypes.byref(shape), ctypes.byref(n)))
    return n.value


def moe_route(shape, x, w_router, sel_bias, logit_bias, topk_ids, topk_weights, expert_counts, topk_gap, workspace,
              stream=None):
    ws, nb = _ws(workspace)
    _check("moe_route", lib().moe_route(ctypes.byref(shape), _ptr(x), _ptr(w_router), _ptr(sel_bias),
                                        _ptr(logit_bias), _ptr(topk_ids), _ptr(topk_weights), _ptr(expert_counts),
                                        _ptr(topk_gap), ws, nb, _stream(stream)))


def moe_permute(shape, topk_ids, expert_offsets, perm_pairs, pair_pos, workspace, stream=None):
    ws, nb = _ws(workspace)
    _check("moe_permute", lib().moe_permute(ctypes.byref(shape), _ptr(topk_ids), _ptr(expert_offsets),
                                            _ptr(perm_pairs), _ptr(pair_pos), ws, nb, _stream(stream)))


def moe_expert_swiglu(shape, x, expert_offsets, perm_pairs, w_gate_up, w_down, y_perm, workspace, stream=None,
                      ws_gate_up=None, ws_down=None, y_shared=None):
    ws, nb = _ws(workspace)
    _check("moe_expert_swiglu", lib().moe_expert_swiglu(ctypes.byref(shape), _ptr(x), _ptr(expert_offsets),
                                                        _ptr(perm_pairs), _ptr(w_gate_up), _ptr(w_down),
                                                        _ptr(ws_gate_up), _ptr(ws_down), _ptr(y_perm),
                                                        _ptr(y_shared), ws, nb, _stream(stream)))


def moe_expert_gate_up(shape, x, expert_offsets, perm_pairs, w_gate_up, hid, workspace, stream=None,
                       ws_gate_up=None, hid_shared=None):
    ws, nb = _ws(workspace)
    _check("moe_expert_gate_up", lib().moe_expert_gate_up(ctypes.byref(shape), _ptr(x), _ptr(expert_offsets),
                                                          _ptr(perm_pairs), _ptr(w_gate_up), _ptr(ws_gate_up),
                                                          _ptr(hid), _ptr(hid_shared), ws, nb, _stream(stream)))


def moe_expert_down(shape, expert_offsets, hid, w_down, y_perm, workspace, stream=None, hid_shared=None,
                    ws_down=None, y_shared=None):
    ws, nb = _ws(workspace)
    _check("moe_expert_down", lib().moe_expert_down(ctypes.byref(shape), _ptr(expert_offsets), _ptr(hid),
                                                    _ptr(hid_shared), _ptr(w_down), _ptr(ws_down), _ptr(y_perm),
                                                    _ptr(y_shared), ws, nb, _stream(stream)))


def moe_shared_swiglu(shape, x, ws_gate_up, ws_down, y_shared, workspace, stream=None):
    ws, nb = _ws(workspace)
    _check("moe_shared_swiglu", lib().moe_shared_swiglu(ctypes.byref(shape), _ptr(x), _ptr(ws_gate_up),
                                                        _ptr(ws_down), _ptr(y_shared), ws, nb, _stream(stream)))


def moe_combine(shape, y_perm, pair_pos, topk_weights, y_shared, routed_scale, y, stream=None):
    _check("moe_combine", lib().moe_combine(ctypes.byref(shape), _ptr(y_perm), _ptr(pair_pos), _ptr(topk_weights),
                                            _ptr(y_shared), float(routed_scale), _ptr(y), _stream(stream)))


def moe_rmsnorm(rows, cols, inp, gamma, eps, out, stream=None):
    _check("moe_rmsnorm", lib().moe_rmsnorm(int(rows), int(cols), _ptr(inp), _ptr(gamma), float(eps), _ptr(out),
                                            _stream(stream)))


def moe_route_diag(shape, x, w_router, sel_bias, logit_bias, topk_ids, topk_weights, expert_counts, topk_gap,
                   ep_groups, p_e, f_e, summary, workspace, stream=None):
    ws, nb = _ws(workspace)
    _check("moe_route_diag", lib().moe_route_diag(ctypes.byref(shape), _ptr(x), _ptr(w_router), _ptr(sel_bias),
                                                  _ptr(logit_bias), _ptr(topk_ids), _ptr(topk_weights),
                                                  _ptr(expert_counts), _ptr(topk_gap), int(ep_groups), _ptr(p_e),
                                                  _ptr(f_e), _ptr(summary), ws, nb, _stream(stream)))


def moe_combine_diag(shape, y_perm, pair_pos, topk_weights, y_shared, routed_scale, y, expert_offsets, expert_rms,
                     rms_ratio, workspace, stream=None):
    ws, nb = _ws(workspace)
    _check("moe_combine_diag", lib().moe_combine_diag(ctypes.byref(shape), _ptr(y_perm), _ptr(pair_pos),
                                                      _ptr(topk_weights), _ptr(y_shared), float(routed_scale),
                                                      _ptr(y), _ptr(expert_offsets), _ptr(expert_rms),
                                                      _ptr(rms_ratio), ws, nb, _stream(stream)))


def moe_dense_workspace_bytes(num_tokens, d_model, d_hidden) -> int:
    n = ctypes.c_size_t(0)
    _check("moe_dense_workspace_bytes", lib().moe_dense_workspace_bytes(int(num_tokens), int(d_model), int(d_hidden),
                                                                        ctypes.byref(n)))
    return n.value


def moe_dense_swiglu(num_tokens, d_model, d_hidden, x, w_gate_up, w_down, y, workspace, stream=None):
    ws, nb = _ws(workspace)
    _check("moe_dense_swiglu", lib().moe_dense_swiglu(int(num_tokens), int(d_model), int(d_hidden), _ptr(x),
                                                      _ptr(w_gate_up), _ptr(w_down), _ptr(y), ws, nb,
                                                      _stream(stream)))


def moe_expert_swiglu_range(shape, expert_begin, expert_end, x, expert_offsets, perm_pairs, w_gate_up, w_down,
                            y_perm, workspace, stream=None):
    ws, nb = _ws(workspace)
    _check("moe_expert_swiglu_range", lib().moe_expert_swiglu_range(
        ctypes.byref(shape), int(expert_begin), int(expert_end), _ptr(x), _ptr(expert_offsets), _ptr(perm_pairs),
        _ptr(w_gate_up), _ptr(w_down), _ptr(y_perm), ws, nb, _stream(stream)))


def moe_rmsnorm_route(shape, h, gamma, eps, w_router, sel_bias, logit_bias, x_out, topk_ids, topk_weights,
                      expert_counts, topk_gap, workspace, stream=None):
    ws, nb = _ws(workspace)
    _check("moe_rmsnorm_route", lib().moe_rmsnorm_route(
        ctypes.byref(shape), _ptr(h), _ptr(gamma), float(eps), _ptr(w_router), _ptr(sel_bias), _ptr(logit_bias),
        _ptr(x_out), _ptr(topk_ids), _ptr(topk_weights), _ptr(expert_counts), _ptr(topk_gap), ws, nb,
        _stream(stream)))


def moe_combine_residual(shape, y_perm, pair_pos, topk_weights, y_shared, routed_scale, residual, y, stream=None):
    _check("moe_combine_residual", lib().moe_combine_residual(
        ctypes.byref(shape), _ptr(y_perm), _ptr(pair_pos), _ptr(topk_weights), _ptr(y_shared),
        float(routed_scale), _ptr(residual), _ptr(y), _stream(stream)))


def moe_expert_swiglu_clamped(shape, x, expert_offsets, perm_pairs, w_gate_up, w_down, y_perm, act_clamp, workspace,
                              stream=None, ws_gate_up=None, ws_down=None, y_shared=None):
    ws, nb = _ws(workspace)
    _check("moe_expert_swiglu_clamped", lib().moe_expert_swiglu_clamped(
        ctypes.byref(shape), _ptr(x), _ptr(expert_offsets), _ptr(perm_pairs), _ptr(w_gate_up), _ptr(w_down),
        _ptr(ws_gate_up), _ptr(ws_down), _ptr(y_perm), _ptr(y_shared), float(act_clamp), ws, nb, _stream(stream)))


def moe_expert_swiglu_noalloc(shape, x, expert_offsets, perm_pairs, w_gate_up, w_down, y_perm, stream=None,
                              ws_gate_up=None, ws_down=None, y_shared=None):
    _check("moe_expert_swiglu_noalloc", lib().moe_expert_swiglu_noalloc(
        ctypes.byref(shape), _ptr(x), _ptr(expert_offsets), _ptr(perm_pairs), _ptr(w_gate_up), _ptr(w_down),
        _ptr(ws_gate_up), _ptr(ws_down), _ptr(y_perm), _ptr(y_shared), _stream(stream)))
