"""Seeded synthetic inputs for the sparse MoE FFN layer.

This package draws numbers and nothing else: it holds none of the layer's
arithmetic.  Tests, the benchmark and the oracle's harness all take their
inputs from here, so the CPU oracle and the GPU library see identical bf16
tensors.  The stream definition (SplitMix64 + Box-Muller, bf16 round to
nearest even) is in ``moegen.h``; tensors are regenerable per
(seed, layer, tensor kind, expert), element by element, on the host or the
device with bit-identical results.

Workload recipes (shapes and value distributions of the model the pages
describe: 288 routed SwiGLU experts of hidden 1,280 with top-8 routing plus one
shared expert; d_model = 4096 is a chosen value the pages do not state):

  0  tiny:    T=64,   d=256,  E=16,  k=2, h=hs=128; x ~ N(0,1); bias U[-.05,.05]
  1  decode:  T=64,   d=4096, E=288, k=8, h=hs=1280; x rows N(0,1) scaled to
              RMS 1; bias U[-.1,.1]
  2  prefill: T=8192, otherwise as 1
  3  skew:    T=4096, as 1 plus a per-expert logit offset A * r^-1.1 over a
              seeded ranking r of the experts (Zipf, s = 1.1)
  4  stack:   12 layers of 1 with distinct weights, T=256 (64 sequences x 4
              positions), x_{l+1} = unit-gain RMSNorm(y_l)
All weights ~ N(0, 0.02^2); seed = recipe index.
"""
import ctypes
import os
from dataclasses import dataclass, replace

import numpy as np

from . import build as _build

# Tensor kinds (part of each stream's key).
KIND_X = 1
KIND_ROUTER = 2
KIND_SEL_BIAS = 3
KIND_ZIPF_RANK = 4
KIND_W_GATE_UP = 5
KIND_W_DOWN = 6
KIND_SHARED_GATE_UP = 7
KIND_SHARED_DOWN = 8

WEIGHT_STD = 0.02

# Logit-offset amplitude of the skewed recipe, found by bisection with the
# oracle's router so that the busiest expert receives about ten times the mean
# load (oracle/calibrate_skew.py).
SKEW_AMPLITUDE = 3.29


@dataclass(frozen=True)
class Config:
    index: int
    name: str
    T: int
    d: int
    E: int
    k: int
    h: int
    hs: int
    bias: float          # selection bias ~ U[-bias, bias]
    x_rms: bool          # scale each x row to unit RMS
    seed: int
    layers: int = 1
    zipf_s: float = 0.0  # 0: no logit offset
    zipf_amp: float = 0.0
    routed_scale: float = 1.0

    @property
    def workload(self) -> str:
        s = (f"{self.name}: T={self.T}, d_model={self.d}, E={self.E}, top-{self.k}, expert hidden {self.h}, "
             f"shared hidden {self.hs}")
        if self.layers > 1:
            s += f", {self.layers} layers"
        if self.zipf_s:
            s += f", Zipf({self.zipf_s}) logit offset A={self.zipf_amp}"
        return s


CONFIGS = {
    0: Config(0, "tiny", 64, 256, 16, 2, 128, 128, 0.05, False, 0),
    1: Config(1, "decode", 64, 4096, 288, 8, 1280, 1280, 0.1, True, 1),
    2: Config(2, "prefill", 8192, 4096, 288, 8, 1280, 1280, 0.1, True, 2),
    3: Config(3, "skew", 4096, 4096, 288, 8, 1280, 1280, 0.1, True, 3, zipf_s=1.1, zipf_amp=SKEW_AMPLITUDE),
    4: Config(4, "stack", 256, 4096, 288, 8, 1280, 1280, 0.1, True, 4, layers=12),
}


def custom(base: int = 0, **kw) -> Config:
    """A recipe derived from one of the above with some fields replaced."""
    return replace(CONFIGS[base], **kw)


_lib = None
_U64 = ctypes.c_uint64
_P = ctypes.c_void_p


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_build.LIB):
            _build.build()
        L = ctypes.CDLL(_build.LIB)
        L.moegen_splitmix.restype = _U64
        L.moegen_splitmix.argtypes = [_U64, _U64]
        L.moegen_stream_key.restype = _U64
        L.moegen_stream_key.argtypes = [_U64] * 4
        L.moegen_normal_f64_host.argtypes = [_U64, _U64, _U64, _P, ctypes.c_int]
        L.moegen_uniform_f64_host.argtypes = [_U64, _U64, _U64, _P]
        L.moegen_normal_bf16_host.argtypes = [_U64, _U64, _U64, ctypes.c_double, _P, ctypes.c_int]
        L.moegen_experts_bf16_host.argtypes = [_U64] * 6 + [ctypes.c_double, _P, ctypes.c_int]
        L.moegen_rows_bf16_host.argtypes = [_U64, _U64, _U64, ctypes.c_int, _P, ctypes.c_int]
        L.moegen_normal_bf16_device.argtypes = [_U64, _U64, _U64, ctypes.c_double, _P, _P]
        L.moegen_normal_bf16_device.restype = ctypes.c_int
        L.moegen_experts_bf16_device.argtypes = [_U64] * 6 + [ctypes.c_double, _P, _P]
        L.moegen_experts_bf16_device.restype = ctypes.c_int
        _lib = L
    return _lib


def threads() -> int:
    n = os.cpu_count() or 1
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        pass
    return max(1, min(n, 16))


def key(cfg: Config, layer: int, kind: int, expert: int = 0) -> int:
    return lib().moegen_stream_key(cfg.seed, layer, kind, expert)


def x(cfg: Config, layer: int = 0) -> np.ndarray:
    """Token rows [T, d] bf16 (uint16)."""
    out = np.empty((cfg.T, cfg.d), np.uint16)
    lib().moegen_rows_bf16_host(key(cfg, layer, KIND_X), cfg.T, cfg.d, int(cfg.x_rms), out.ctypes.data, threads())
    return out


def router(cfg: Config, layer: int = 0) -> np.ndarray:
    """Router weights [E, d] bf16 (uint16), N(0, 0.02^2)."""
    out = np.empty((cfg.E, cfg.d), np.uint16)
    lib().moegen_normal_bf16_host(key(cfg, layer, KIND_ROUTER), 0, out.size, WEIGHT_STD, out.ctypes.data, threads())
    return out


def sel_bias(cfg: Config, layer: int = 0) -> np.ndarray:
    """Selection bias [E] f32 ~ U[-bias, bias]."""
    u = np.empty(cfg.E, np.float64)
    lib().moegen_uniform_f64_host(key(cfg, layer, KIND_SEL_BIAS), 0, cfg.E, u.ctypes.data)
    return (-cfg.bias + 2.0 * cfg.bias * u).astype(np.float32)


def zipf_ranks(cfg: Config, layer: int = 0) -> np.ndarray:
    """A seeded permutation of the ranks 1..E (Fisher-Yates on the stream)."""
    E = cfg.E
    u = np.empty(E, np.float64)
    lib().moegen_uniform_f64_host(key(cfg, layer, KIND_ZIPF_RANK), 0, E, u.ctypes.data)
    r = np.arange(1, E + 1, dtype=np.int64)
    for i in range(E - 1, 0, -1):
        j = min(int(u[i] * (i + 1)), i)
        r[i], r[j] = r[j], r[i]
    return r


def logit_bias(cfg: Config, layer: int = 0, amplitude: float = None):
    """Per-expert logit offset [E] f32 (Zipf over a seeded ranking), or None."""
    if not cfg.zipf_s:
        return None
    a = cfg.zipf_amp if amplitude is None else amplitude
    r = zipf_ranks(cfg, layer).astype(np.float64)
    return (a * r ** (-cfg.zipf_s)).astype(np.float32)


def expert_weights_host(cfg: Config, layer: int, experts):
    """Host copies of the listed experts' weights: dict e -> (w_gu [2h,d], w_d [d,h])."""
    L = lib()
    out = {}
    for e in experts:
        gu = np.empty((2 * cfg.h, cfg.d), np.uint16)
        dn = np.empty((cfg.d, cfg.h), np.uint16)
        L.moegen_experts_bf16_host(cfg.seed, layer, KIND_W_GATE_UP, int(e), 1, gu.size, WEIGHT_STD, gu.ctypes.data,
                                   threads())
        L.moegen_experts_bf16_host(cfg.seed, layer, KIND_W_DOWN, int(e), 1, dn.size, WEIGHT_STD, dn.ctypes.data,
                                   threads())
        out[int(e)] = (gu, dn)
    return out


def shared_weights_host(cfg: Config, layer: int = 0):
    """Shared expert (w_gu [2hs,d], w_d [d,hs]) on the host, or (None, None)."""
    if cfg.hs == 0:
        return None, None
    L = lib()
    gu = np.empty((2 * cfg.hs, cfg.d), np.uint16)
    dn = np.empty((cfg.d, cfg.hs), np.uint16)
    L.moegen_normal_bf16_host(key(cfg, layer, KIND_SHARED_GATE_UP), 0, gu.size, WEIGHT_STD, gu.ctypes.data,
                              threads())
    L.moegen_normal_bf16_host(key(cfg, layer, KIND_SHARED_DOWN), 0, dn.size, WEIGHT_STD, dn.ctypes.data, threads())
    return gu, dn


def fill_experts_device(cfg: Config, layer: int, w_gu_ptr: int, w_d_ptr: int, stream: int) -> None:
    """Fill all E experts' weights of one layer in device memory:
    w_gu [E, 2h, d] and w_d [E, d, h] bf16, contiguous per expert."""
    L = lib()
    rc = L.moegen_experts_bf16_device(cfg.seed, layer, KIND_W_GATE_UP, 0, cfg.E, 2 * cfg.h * cfg.d, WEIGHT_STD,
                                      w_gu_ptr, stream)
    rc = rc or L.moegen_experts_bf16_device(cfg.seed, layer, KIND_W_DOWN, 0, cfg.E, cfg.d * cfg.h, WEIGHT_STD,
                                            w_d_ptr, stream)
    if rc:
        raise RuntimeError(f"moegen device fill failed: hipError {rc}")


def fill_shared_device(cfg: Config, layer: int, ws_gu_ptr: int, ws_d_ptr: int, stream: int) -> None:
    """Fill the shared expert's weights in device memory."""
    L = lib()
    rc = L.moegen_normal_bf16_device(key(cfg, layer, KIND_SHARED_GATE_UP), 0, 2 * cfg.hs * cfg.d, WEIGHT_STD,
                                     ws_gu_ptr, stream)
    rc = rc or L.moegen_normal_bf16_device(key(cfg, layer, KIND_SHARED_DOWN), 0, cfg.d * cfg.hs, WEIGHT_STD,
                                           ws_d_ptr, stream)
    if rc:
        raise RuntimeError(f"moegen device fill failed: hipError {rc}")


def bf16_to_f32(a: np.ndarray) -> np.ndarray:
    """Decode bf16 bit patterns (uint16) to float32 exactly."""
    return (np.asarray(a, np.uint16).astype(np.uint32) << 16).view(np.float32)


def normal_bf16(seed: int, kind: int, shape, std: float = 1.0) -> np.ndarray:
    """A free-standing N(0, std^2) bf16 tensor (test inputs for single calls)."""
    out = np.empty(shape, np.uint16)
    k = lib().moegen_stream_key(seed, 0, kind, 0)
    lib().moegen_normal_bf16_host(k, 0, out.size, std, out.ctypes.data, threads())
    return out


def uniform(seed: int, kind: int, n: int) -> np.ndarray:
    """n uniform [0,1) doubles from a free-standing stream."""
    u = np.empty(n, np.float64)
    lib().moegen_uniform_f64_host(lib().moegen_stream_key(seed, 0, kind, 0), 0, n, u.ctypes.data)
    return u


def random_ids(seed: int, T: int, E: int, k: int) -> np.ndarray:
    """[T, k] int32: k distinct experts per token, ascending (partial
    Fisher-Yates on a uniform stream) -- synthetic routing for the
    permutation and expert calls."""
    u = uniform(seed, 101, T * k).reshape(T, k) if T else np.zeros((0, k))
    out = np.empty((T, k), np.int32)
    for t in range(T):
        pool = list(range(E))
        for j in range(k):
            i = j + min(int(u[t, j] * (E - j)), E - j - 1)
            pool[j], pool[i] = pool[i], pool[j]
        out[t] = np.sort(pool[:k])
    return out
