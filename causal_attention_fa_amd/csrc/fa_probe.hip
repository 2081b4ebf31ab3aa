// Measurement behind the choice of the dQ strategy (the backward accumulates
// dQ either in a separate query-parallel pass or with float atomics from the
// key-parallel dK/dV pass, chosen by measurement).  This kernel issues exactly
// the global traffic the atomic variant needs and nothing else: one workgroup
// per (batch, KV head, key block) in the dK/dV pass's order (XCD-contiguous,
// as decode_work), walking the G query heads and the query tiles its keys can
// see, and per tile adding a [tile rows x d] block of fp32 values into a
// [B, H, T, d] fp32 accumulator with one global atomic add per element (the
// reduction over the block's keys already done).  Its time is a lower bound
// on the atomic variant's cost beyond the dK/dV pass itself.
#include <hip/hip_runtime.h>

#include "device_common.h"
#include "internal.h"

namespace fa {

__global__ __launch_bounds__(256) void dq_atomic_probe_kernel(float* acc, int B, int H, int Hkv,
                                                              int T, int d, int W, int bkvb,
                                                              int bqb) {
  const int nkb = (T + bkvb - 1) / bkvb;
  const WorkItem w = decode_work(blockIdx.x, nkb, B, Hkv, 1, false);
  const int G = H / Hkv;
  const int k0 = w.blk * bkvb;
  const int qt_lo = k0 / bqb;
  const int q_hi = W > 0 ? min(T, k0 + bkvb - 1 + W) : T;
  const int nqt = (q_hi + bqb - 1) / bqb - qt_lo;
  const float v = 1e-3f * (threadIdx.x + 1);
  const int n = bqb * d;   // elements per tile
  for (int hi = 0; hi < G; ++hi) {
    float* base = acc + ((size_t)w.b * H + w.hkv * G + hi) * T * d;
    for (int t = 0; t < nqt; ++t) {
      const int q0 = (qt_lo + t) * bqb;
      for (int lin = threadIdx.x; lin < n; lin += 256) {
        const int r = q0 + lin / d;
        if (r < T) atomicAdd(base + (size_t)r * d + lin % d, v);
      }
    }
  }
}

hipError_t launch_dq_atomic_probe(float* acc, int B, int H, int Hkv, int T, int d, int W,
                                  int bkvb, int bqb, hipStream_t stream) {
  const int nkb = (T + bkvb - 1) / bkvb;
  hipLaunchKernelGGL(dq_atomic_probe_kernel, dim3((unsigned)nkb * B * Hkv), dim3(256), 0, stream,
                     acc, B, H, Hkv, T, d, W, bkvb, bqb);
  return hipGetLastError();
}

}  // namespace fa
