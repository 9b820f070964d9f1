"""CPU oracle for the sparse MoE FFN layer -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  The GPU library and its Python binding
never import it.  The arithmetic lives in ``moe_oracle.cc`` (plain
single-threaded C++); this module is argument marshalling over ctypes.

Functions take and return numpy arrays.  bf16 tensors are ``np.uint16`` bit
patterns.
"""
import ctypes
import os

import numpy as np

from . import build as _build

_lib = None

_P = ctypes.c_void_p
_I = ctypes.c_int


def lib():
    global _lib
    if _lib is None:
        path = os.environ.get("MOE_ORACLE_LIB", _build.LIB)
        if path == _build.LIB and not os.path.exists(path):
            _build.build()
        L = ctypes.CDLL(path)
        L.oracle_route.argtypes = [_I, _I, _I, _I, _P, _P, _P, _P, _P, _P, _P, _P]
        L.oracle_permute.argtypes = [_I, _I, _I, _P, _P, _P, _P, _P]
        L.oracle_expert.argtypes = [_I, _I, _P, _P, _P, _P]
        L.oracle_layer.argtypes = [_I, _I, _I, _I, _I, _I, _P, _P, _P, _P, _P, _P, _P, _P, ctypes.c_float,
                                   _I, _P, _P, _P, _P, _P]
        L.oracle_forward_given_routing.argtypes = [_I, _I, _I, _I, _I, _I, _P, _P, _P, _P, _P, _P, _P,
                                                   ctypes.c_float, _I, _P, _P, _P, _P]
        L.oracle_rmsnorm.argtypes = [_I, _I, _P, _P, ctypes.c_float, _P]
        L.oracle_combine.argtypes = [_I, _I, _I, _P, _P, _P, _P, ctypes.c_float, _P, _P]
        L.oracle_route_diag.argtypes = [_I, _I, _I, _I, _P, _P, _P, _P, _P, _P]
        L.oracle_activation_rms.argtypes = [_I, _I, _P, _P]
        L.oracle_expert_clamped.argtypes = [_I, _I, _P, _P, _P, ctypes.c_double, _P]
        for f in (L.oracle_route, L.oracle_permute, L.oracle_expert, L.oracle_layer,
                  L.oracle_forward_given_routing, L.oracle_rmsnorm,
                  L.oracle_combine, L.oracle_route_diag, L.oracle_activation_rms, L.oracle_expert_clamped):
            f.restype = ctypes.c_int
        _lib = L
    return _lib


def _ptr(a):
    return None if a is None else a.ctypes.data


def _c(a, dtype):
    return None if a is None else np.ascontiguousarray(a, dtype=dtype)


def _check(rc, name):
    if rc != 0:
        raise ValueError(f"{name} returned {rc}")


def route(x, w_router, sel_bias, k, logit_bias=None, want_scores=False):
    """Routing for every row of x.  Returns (ids [T,k] int32 ascending,
    weights [T,k] f32, gap [T] f32, scores [T,E] f32 or None)."""
    x = _c(x, np.uint16)
    w_router = _c(w_router, np.uint16)
    sel_bias = _c(sel_bias, np.float32)
    logit_bias = _c(logit_bias, np.float32)
    T, d = x.shape
    E = w_router.shape[0]
    ids = np.zeros((T, k), np.int32)
    wts = np.zeros((T, k), np.float32)
    gap = np.zeros(T, np.float32)
    scores = np.zeros((T, E), np.float32) if want_scores else None
    rc = lib().oracle_route(T, d, E, k, _ptr(x), _ptr(w_router), _ptr(sel_bias), _ptr(logit_bias), _ptr(ids),
                            _ptr(wts), _ptr(gap), _ptr(scores))
    _check(rc, "oracle_route")
    return ids, wts, gap, scores


def permute(topk_ids, num_experts):
    """Stable (expert, token) permutation.  Returns (counts [E], offsets [E+1],
    perm_pairs [T*k], pair_pos [T*k]), all int32."""
    ids = _c(topk_ids, np.int32)
    T, k = ids.shape
    E = num_experts
    counts = np.zeros(E, np.int32)
    offsets = np.zeros(E + 1, np.int32)
    perm = np.zeros(T * k, np.int32)
    pos = np.zeros(T * k, np.int32)
    rc = lib().oracle_permute(T, E, k, _ptr(ids), _ptr(counts), _ptr(offsets), _ptr(perm), _ptr(pos))
    _check(rc, "oracle_permute")
    return counts, offsets, perm, pos


def expert(x_row, w_gu, w_d):
    """One SwiGLU expert on one bf16 row: W_d (SiLU(W_g x) * W_u x), f32 [d]."""
    x_row = _c(x_row, np.uint16)
    w_gu = _c(w_gu, np.uint16)
    w_d = _c(w_d, np.uint16)
    d = x_row.shape[0]
    h = w_gu.shape[0] // 2
    out = np.zeros(d, np.float32)
    _check(lib().oracle_expert(d, h, _ptr(x_row), _ptr(w_gu), _ptr(w_d), _ptr(out)), "oracle_expert")
    return out


def expert_clamped(x_row, w_gu, w_d, clamp):
    """oracle expert with every hidden activation clipped to [-clamp, clamp]."""
    x_row = _c(x_row, np.uint16)
    w_gu = _c(w_gu, np.uint16)
    w_d = _c(w_d, np.uint16)
    d = x_row.shape[0]
    h = w_gu.shape[0] // 2
    out = np.zeros(d, np.float32)
    _check(lib().oracle_expert_clamped(d, h, _ptr(x_row), _ptr(w_gu), _ptr(w_d), float(clamp), _ptr(out)),
           "oracle_expert_clamped")
    return out


def _expert_ptrs(w_gu, w_d, E):
    """ctypes arrays of expert weight pointers (NULL where None) and the
    contiguous copies that keep them alive."""
    keep = []
    gu_ptrs = (ctypes.c_void_p * E)()
    d_ptrs = (ctypes.c_void_p * E)()
    for e in range(E):
        if w_gu[e] is not None:
            a = _c(w_gu[e], np.uint16)
            b = _c(w_d[e], np.uint16)
            keep += [a, b]
            gu_ptrs[e] = a.ctypes.data
            d_ptrs[e] = b.ctypes.data
    return gu_ptrs, d_ptrs, keep


def layer(x, w_router, sel_bias, k, w_gu, w_d, ws_gu=None, ws_d=None, routed_scale=1.0, logit_bias=None,
          tokens=None):
    """Whole layer on the listed token rows (all rows if tokens is None).

    w_gu / w_d: sequences of length E whose entries are [2h,d] / [d,h] uint16
    arrays, or None for experts no listed token selects.
    Returns (ids [n,k], weights [n,k], gap [n], y [n,d] f32)."""
    x = _c(x, np.uint16)
    w_router = _c(w_router, np.uint16)
    sel_bias = _c(sel_bias, np.float32)
    logit_bias = _c(logit_bias, np.float32)
    T, d = x.shape
    E = w_router.shape[0]
    assert len(w_gu) == E and len(w_d) == E
    h = next(w.shape[0] // 2 for w in w_gu if w is not None)
    gu_ptrs, d_ptrs, keep = _expert_ptrs(w_gu, w_d, E)
    hs = 0
    if ws_gu is not None:
        ws_gu = _c(ws_gu, np.uint16)
        ws_d = _c(ws_d, np.uint16)
        hs = ws_gu.shape[0] // 2
    tok = None if tokens is None else np.ascontiguousarray(tokens, np.int32)
    n = T if tok is None else tok.shape[0]
    ids = np.zeros((n, k), np.int32)
    wts = np.zeros((n, k), np.float32)
    gap = np.zeros(n, np.float32)
    y = np.zeros((n, d), np.float32)
    rc = lib().oracle_layer(T, d, E, k, h, hs, _ptr(x), _ptr(w_router), _ptr(sel_bias), _ptr(logit_bias), gu_ptrs,
                            d_ptrs, _ptr(ws_gu), _ptr(ws_d), float(routed_scale), n, _ptr(tok), _ptr(ids),
                            _ptr(wts), _ptr(gap), _ptr(y))
    del keep
    _check(rc, "oracle_layer")
    return ids, wts, gap, y


def forward_given_routing(x, w_router, ids, w_gu, w_d, ws_gu=None, ws_d=None, routed_scale=1.0, logit_bias=None,
                          tokens=None):
    """The layer on the listed token rows under the given chosen sets ids
    [n,k] (each row ascending and distinct): weights from the unbiased scores
    of those experts, the experts, the shared expert and the scaled combine.
    Returns (weights [n,k] f32, y [n,d] f32)."""
    x = _c(x, np.uint16)
    w_router = _c(w_router, np.uint16)
    logit_bias = _c(logit_bias, np.float32)
    ids = _c(ids, np.int32)
    T, d = x.shape
    E = w_router.shape[0]
    n, k = ids.shape
    assert len(w_gu) == E and len(w_d) == E
    h = next(w.shape[0] // 2 for w in w_gu if w is not None)
    gu_ptrs, d_ptrs, keep = _expert_ptrs(w_gu, w_d, E)
    hs = 0
    if ws_gu is not None:
        ws_gu = _c(ws_gu, np.uint16)
        ws_d = _c(ws_d, np.uint16)
        hs = ws_gu.shape[0] // 2
    tok = None if tokens is None else np.ascontiguousarray(tokens, np.int32)
    assert (T if tok is None else tok.shape[0]) == n
    wts = np.zeros((n, k), np.float32)
    y = np.zeros((n, d), np.float32)
    rc = lib().oracle_forward_given_routing(T, d, E, k, h, hs, _ptr(x), _ptr(w_router), _ptr(logit_bias), gu_ptrs,
                                            d_ptrs, _ptr(ws_gu), _ptr(ws_d), float(routed_scale), n, _ptr(tok),
                                            _ptr(ids), _ptr(wts), _ptr(y))
    del keep
    _check(rc, "oracle_forward_given_routing")
    return wts, y


def combine(y_perm, pair_pos, weights, y_shared=None, routed_scale=1.0, residual=None):
    """y = residual + (y_shared + routed_scale * sum_j w[t,j] y_perm[pos[t*k+j]]);
    f32 [T,d].  residual: bf16 bits [T,d] or None."""
    y_perm = _c(y_perm, np.uint16)
    weights = _c(weights, np.float32)
    pair_pos = _c(pair_pos, np.int32)
    y_shared = _c(y_shared, np.float32)
    residual = _c(residual, np.uint16)
    T, k = weights.shape
    d = y_perm.shape[1]
    y = np.zeros((T, d), np.float32)
    rc = lib().oracle_combine(T, d, k, _ptr(y_perm), _ptr(pair_pos), _ptr(weights), _ptr(y_shared),
                              float(routed_scale), _ptr(residual), _ptr(y))
    _check(rc, "oracle_combine")
    return y


def rmsnorm(v, gamma=None, eps=1e-6):
    """Zero-centred RMSNorm of bf16 rows; bf16 out (uint16)."""
    v = _c(v, np.uint16)
    gamma = _c(gamma, np.float32)
    T, d = v.shape
    out = np.zeros((T, d), np.uint16)
    _check(lib().oracle_rmsnorm(T, d, _ptr(v), _ptr(gamma), float(eps), _ptr(out)), "oracle_rmsnorm")
    return out


def route_diag(scores, topk_ids, groups=1):
    """Routing diagnostics from the unbiased scores [T,E] and chosen ids [T,k].
    Returns (p_e [E], f_e [E], l_ep, confidence), all float64."""
    scores = _c(scores, np.float32)
    ids = _c(topk_ids, np.int32)
    T, E = scores.shape
    k = ids.shape[1]
    p_e = np.zeros(E)
    f_e = np.zeros(E)
    l_ep = ctypes.c_double()
    conf = ctypes.c_double()
    rc = lib().oracle_route_diag(T, E, k, int(groups), _ptr(scores), _ptr(ids), _ptr(p_e), _ptr(f_e),
                                 ctypes.addressof(l_ep), ctypes.addressof(conf))
    _check(rc, "oracle_route_diag")
    return p_e, f_e, l_ep.value, conf.value


def activation_rms(rows):
    """RMS over every element of one expert's output rows [n,d] (0 if n = 0)."""
    rows = _c(rows, np.float32)
    n, d = rows.shape
    out = ctypes.c_double()
    _check(lib().oracle_activation_rms(n, d, _ptr(rows), ctypes.addressof(out)), "oracle_activation_rms")
    return out.value


def expert_rms(y_perm, offsets, y_shared=None):
    """Per-expert activation RMS of the permuted expert outputs y_perm [T*k,d]
    (bf16 bits) grouped by offsets [E+1], plus the shared expert's y_shared
    [T,d] f32 (entry E; 0 if None), and the spread (min, max) / median over
    the experts with at least one row ([Blog] §4.1.3, Figure 4: maximum against
    median expert output norm; [Digest] expert collapse: min-to-median).  An
    even count's median is the mean of the two middle values (numpy's).
    Returns (rms [E+1] float64, ratio [2] float64; (0, 0) without a row)."""
    offsets = np.asarray(offsets, np.int64)
    E = offsets.shape[0] - 1
    rows = (np.asarray(y_perm, np.uint16).astype(np.uint32) << 16).view(np.float32)
    rms = np.zeros(E + 1)
    for e in range(E):
        rms[e] = activation_rms(rows[offsets[e]:offsets[e + 1]].reshape(-1, rows.shape[1]))
    if y_shared is not None:
        rms[E] = activation_rms(y_shared)
    used = rms[:E][offsets[1:] > offsets[:-1]]
    ratio = np.zeros(2)
    if used.size:
        med = float(np.median(used))
        if med > 0:
            ratio[:] = used.min() / med, used.max() / med
    return rms, ratio
