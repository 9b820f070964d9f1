// moegen.hip -- host and device fills for the seeded input generator defined
// in moegen.h.  Exposed with a C ABI for the Python harness (tests, bench).
//
// Host fills run on std::thread workers; device fills are grid-stride HIP
// kernels.  Both evaluate the same moegen.h functions, so a tensor filled on
// the device is bit-identical to the same tensor filled on the host.
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <cmath>
#include <thread>
#include <vector>
#include "moegen.h"

using namespace moegen;

namespace {

template <class F>
void parallel_for(uint64_t n, int nthreads, F&& fn) {
  if (nthreads < 1) nthreads = 1;
  if ((uint64_t)nthreads > n / 4096 + 1) nthreads = (int)(n / 4096 + 1);
  if (nthreads == 1) { fn(0, n); return; }
  std::vector<std::thread> ws;
  const uint64_t per = (n + nthreads - 1) / nthreads;
  for (int w = 0; w < nthreads; ++w) {
    const uint64_t b = per * w, e = b + per < n ? b + per : n;
    if (b >= e) break;
    ws.emplace_back([=, &fn] { fn(b, e); });
  }
  for (auto& t : ws) t.join();
}

__global__ void k_normal_bf16(uint64_t key, uint64_t start, uint64_t n, double stdev, uint16_t* out) {
  const uint64_t stride = (uint64_t)gridDim.x * blockDim.x;
  for (uint64_t i = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride)
    out[i] = normal_bf16(key, start + i, stdev);
}

// One key per expert: expert e's tensor of `per` elements lands at out + e*per.
__global__ void k_experts_bf16(uint64_t seed, uint64_t layer, uint64_t kind, uint64_t e0, uint64_t per,
                               uint64_t n_total, double stdev, uint16_t* out) {
  const uint64_t stride = (uint64_t)gridDim.x * blockDim.x;
  for (uint64_t i = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n_total; i += stride) {
    const uint64_t e = i / per, j = i - e * per;
    out[i] = normal_bf16(stream_key(seed, layer, kind, e0 + e), j, stdev);
  }
}

int launch_blocks(uint64_t n) {
  uint64_t b = (n + 255) / 256;
  if (b > 65536) b = 65536;
  if (b < 1) b = 1;
  return (int)b;
}

}  // namespace

extern "C" {

uint64_t moegen_splitmix(uint64_t state, uint64_t i) { return splitmix(state, i); }

uint64_t moegen_stream_key(uint64_t seed, uint64_t layer, uint64_t kind, uint64_t expert) {
  return stream_key(seed, layer, kind, expert);
}

// Raw standard normals (double) for elements [start, start+n) of a stream.
void moegen_normal_f64_host(uint64_t key, uint64_t start, uint64_t n, double* out, int nthreads) {
  parallel_for(n, nthreads, [&](uint64_t b, uint64_t e) {
    for (uint64_t i = b; i < e; ++i) out[i] = normal_from_u64(splitmix(key, start + i));
  });
}

// Uniform [0,1) doubles for elements [start, start+n) of a stream.
void moegen_uniform_f64_host(uint64_t key, uint64_t start, uint64_t n, double* out) {
  for (uint64_t i = 0; i < n; ++i) out[i] = uniform_from_u64(splitmix(key, start + i));
}

// N(0, stdev^2) as bf16, elements [start, start+n) of a stream.
void moegen_normal_bf16_host(uint64_t key, uint64_t start, uint64_t n, double stdev, uint16_t* out,
                             int nthreads) {
  parallel_for(n, nthreads, [&](uint64_t b, uint64_t e) {
    for (uint64_t i = b; i < e; ++i) out[i] = normal_bf16(key, start + i, stdev);
  });
}

// Experts [e0, e0 + ne) of a per-expert tensor kind, `per` elements each.
void moegen_experts_bf16_host(uint64_t seed, uint64_t layer, uint64_t kind, uint64_t e0, uint64_t ne,
                              uint64_t per, double stdev, uint16_t* out, int nthreads) {
  parallel_for(ne * per, nthreads, [&](uint64_t b, uint64_t e) {
    uint64_t cur_e = ~0ull, key = 0;
    for (uint64_t i = b; i < e; ++i) {
      const uint64_t ex = i / per;
      if (ex != cur_e) { cur_e = ex; key = stream_key(seed, layer, kind, e0 + ex); }
      out[i] = normal_bf16(key, i - ex * per, stdev);
    }
  });
}

// Token rows of N(0,1) values, each row scaled to unit RMS, stored as bf16.
// rms_normalize = 0 keeps the raw N(0,1) draw.
void moegen_rows_bf16_host(uint64_t key, uint64_t rows, uint64_t cols, int rms_normalize, uint16_t* out,
                           int nthreads) {
  parallel_for(rows, nthreads, [&](uint64_t b, uint64_t e) {
    std::vector<double> z(cols);
    for (uint64_t r = b; r < e; ++r) {
      double ss = 0.0;
      for (uint64_t c = 0; c < cols; ++c) {
        z[c] = normal_from_u64(splitmix(key, r * cols + c));
        ss += z[c] * z[c];
      }
      const double scale = rms_normalize ? 1.0 / std::sqrt(ss / (double)cols) : 1.0;
      for (uint64_t c = 0; c < cols; ++c) out[r * cols + c] = f32_to_bf16_rne((float)(z[c] * scale));
    }
  });
}

// Device fills.  Return 0 on success, else the hipError_t of the launch.
int moegen_normal_bf16_device(uint64_t key, uint64_t start, uint64_t n, double stdev, uint16_t* out,
                              void* stream) {
  if (n == 0) return 0;
  hipLaunchKernelGGL(k_normal_bf16, dim3(launch_blocks(n)), dim3(256), 0, (hipStream_t)stream, key, start, n,
                     stdev, out);
  return (int)hipGetLastError();
}

int moegen_experts_bf16_device(uint64_t seed, uint64_t layer, uint64_t kind, uint64_t e0, uint64_t ne,
                               uint64_t per, double stdev, uint16_t* out, void* stream) {
  const uint64_t n = ne * per;
  if (n == 0) return 0;
  hipLaunchKernelGGL(k_experts_bf16, dim3(launch_blocks(n)), dim3(256), 0, (hipStream_t)stream, seed, layer,
                     kind, e0, per, n, stdev, out);
  return (int)hipGetLastError();
}

}  // extern "C"
