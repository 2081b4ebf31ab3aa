// float32 twins of the attention forward and backward.
//
// Same mathematics as the bf16 kernels (Forge ARCHITECTURES.md, plan wave 2,
// items 8-9; Forge attention.h commit log, "Wave 2"), computed entirely in
// fp32 on the vector ALUs: nothing is rounded through bf16, so results match
// a float64 evaluation to ~1e-6.  These serve the fp32 parity tier, where
// the workload is latency-bound; they favour simplicity over throughput.
//
// Layout of every kernel: a workgroup of 256 threads = 16 rows x 16 lanes.
// Each row is one query (forward, dq) or one key (dk/dv); its 16 lanes
// split the score columns of a tile and own every 16th output column.
// Row reductions are xor-shuffles within the 16 lanes.  The same tile
// bounds as the bf16 path skip key (or query) tiles outside the window.
#include <hip/hip_runtime.h>
#include <math.h>

#include "internal.h"

namespace fa {
namespace {

constexpr int kRows = 16;
constexpr int kLanes = 16;
constexpr int kTile = 32;      // keys (forward, dq) or queries (dk/dv) per tile
constexpr float kInit = -1.0e30f;

__device__ __forceinline__ float row_max(float x) {
#pragma unroll
  for (int o = 1; o < kLanes; o <<= 1) x = fmaxf(x, __shfl_xor(x, o));
  return x;
}
__device__ __forceinline__ float row_sum(float x) {
#pragma unroll
  for (int o = 1; o < kLanes; o <<= 1) x += __shfl_xor(x, o);
  return x;
}

__device__ __forceinline__ bool visible(int q, int kv, int W, int T) {
  return q < T && kv <= q && (W == 0 || kv > q - W);
}

// Capped score and tanh (for the backward chain).
__device__ __forceinline__ float capped(float s, float cap, float& th) {
  if (cap > 0.f) {
    th = tanhf(s / cap);
    return cap * th;
  }
  th = 0.f;
  return s;
}

// Copy rows [row0, row0+nrows) of a [*, D] fp32 matrix into LDS with row
// stride ld; rows at or past T are zero.
template <int D>
__device__ __forceinline__ void load_rows(float* dst, int ld, const float* src, int row0,
                                          int nrows, int T) {
  for (int e = threadIdx.x; e < nrows * D; e += blockDim.x) {
    const int r = e / D, c = e % D;
    const int gr = row0 + r;
    dst[r * ld + c] = gr < T ? src[(size_t)gr * D + c] : 0.f;
  }
}

template <int D>
__global__ __launch_bounds__(256) void fwd_f32_kernel(F32Args a) {
  constexpr int LDK = D + 1;
  constexpr int NC = D / kLanes;
  __shared__ float Qs[kRows * D];
  __shared__ float Ks[kTile * LDK];
  __shared__ float Vs[kTile * D];
  __shared__ float Ps[kRows * kTile];
  const int r = threadIdx.x / kLanes, t = threadIdx.x % kLanes;
  const int T = a.T, W = a.window, G = a.H / a.Hkv;
  const int q0 = blockIdx.x * kRows;
  const int h = blockIdx.y, b = blockIdx.z;
  const size_t bh = (size_t)b * a.H + h, bkv = (size_t)b * a.Hkv + h / G;
  const int q = q0 + r;
  load_rows<D>(Qs, D, a.q + bh * T * D, q0, kRows, T);
  float acc[NC];
#pragma unroll
  for (int k = 0; k < NC; ++k) acc[k] = 0.f;
  float m = kInit, l = 0.f;
  const int kv_lo = W > 0 ? max(0, q0 - W + 1) : 0;
  const int kv_hi = min(T, q0 + kRows);
  for (int kv0 = (kv_lo / kTile) * kTile; kv0 < kv_hi; kv0 += kTile) {
    __syncthreads();
    load_rows<D>(Ks, LDK, a.k + bkv * T * D, kv0, kTile, T);
    load_rows<D>(Vs, D, a.v + bkv * T * D, kv0, kTile, T);
    __syncthreads();
    float s[2];
    float mx = -INFINITY;
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int kk = t + u * kLanes;
      float dot = 0.f;
      for (int c = 0; c < D; ++c) dot += Qs[r * D + c] * Ks[kk * LDK + c];
      float th;
      const float sc = capped(dot * a.scale, a.softcap, th);
      s[u] = visible(q, kv0 + kk, W, T) ? sc : -INFINITY;
      mx = fmaxf(mx, s[u]);
    }
    const float mnew = fmaxf(m, row_max(mx));
    const float alpha = expf(m - mnew);
    float ps = 0.f;
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const float p = expf(s[u] - mnew);
      Ps[r * kTile + t + u * kLanes] = p;
      ps += p;
    }
    l = l * alpha + row_sum(ps);
    m = mnew;
    __syncthreads();
#pragma unroll
    for (int k = 0; k < NC; ++k) {
      const int c = t + k * kLanes;
      float v = acc[k] * alpha;
      for (int kk = 0; kk < kTile; ++kk) v += Ps[r * kTile + kk] * Vs[kk * D + c];
      acc[k] = v;
    }
  }
  if (q < T) {
    float* o = a.out + (bh * T + q) * D;
#pragma unroll
    for (int k = 0; k < NC; ++k) o[t + k * kLanes] = acc[k] / l;
    if (t == 0) a.lse_out[bh * T + q] = m + logf(l);
  }
}

template <int D>
__global__ __launch_bounds__(256) void dq_f32_kernel(F32Args a) {
  constexpr int LDK = D + 1;
  constexpr int NC = D / kLanes;
  __shared__ float Qs[kRows * D];
  __shared__ float dOs[kRows * D];
  __shared__ float Ks[kTile * LDK];
  __shared__ float Vs[kTile * LDK];
  __shared__ float Ps[kRows * kTile];
  const int r = threadIdx.x / kLanes, t = threadIdx.x % kLanes;
  const int T = a.T, W = a.window, G = a.H / a.Hkv;
  const int q0 = blockIdx.x * kRows;
  const int h = blockIdx.y, b = blockIdx.z;
  const size_t bh = (size_t)b * a.H + h, bkv = (size_t)b * a.Hkv + h / G;
  const int q = q0 + r;
  load_rows<D>(Qs, D, a.q + bh * T * D, q0, kRows, T);
  load_rows<D>(dOs, D, a.dO + bh * T * D, q0, kRows, T);
  __syncthreads();
  // D_q = <dO_q, o_q>
  float part = 0.f;
  const int qc = q < T ? q : T - 1;
#pragma unroll
  for (int k = 0; k < NC; ++k) {
    const int c = t + k * kLanes;
    part += dOs[r * D + c] * a.o[(bh * T + qc) * D + c];
  }
  const float Dq = row_sum(part);
  if (q < T && t == 0) a.Dst[bh * T + q] = Dq;
  const float lse = a.lse[bh * T + qc];
  float acc[NC];
#pragma unroll
  for (int k = 0; k < NC; ++k) acc[k] = 0.f;
  const int kv_lo = W > 0 ? max(0, q0 - W + 1) : 0;
  const int kv_hi = min(T, q0 + kRows);
  for (int kv0 = (kv_lo / kTile) * kTile; kv0 < kv_hi; kv0 += kTile) {
    __syncthreads();
    load_rows<D>(Ks, LDK, a.k + bkv * T * D, kv0, kTile, T);
    load_rows<D>(Vs, LDK, a.v + bkv * T * D, kv0, kTile, T);
    __syncthreads();
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int kk = t + u * kLanes;
      float qk = 0.f, dp = 0.f;
      for (int c = 0; c < D; ++c) {
        qk += Qs[r * D + c] * Ks[kk * LDK + c];
        dp += dOs[r * D + c] * Vs[kk * LDK + c];
      }
      float th;
      const float sc = capped(qk * a.scale, a.softcap, th);
      const float p = visible(q, kv0 + kk, W, T) ? expf(sc - lse) : 0.f;
      float ds = p * (dp - Dq);
      if (a.softcap > 0.f) ds *= 1.f - th * th;
      Ps[r * kTile + kk] = ds;
    }
    __syncthreads();
#pragma unroll
    for (int k = 0; k < NC; ++k) {
      const int c = t + k * kLanes;
      float v = acc[k];
      for (int kk = 0; kk < kTile; ++kk) v += Ps[r * kTile + kk] * Ks[kk * LDK + c];
      acc[k] = v;
    }
  }
  if (q < T) {
    float* dq = a.dq + (bh * T + q) * D;
#pragma unroll
    for (int k = 0; k < NC; ++k) dq[t + k * kLanes] = acc[k] * a.scale;
  }
}

template <int D>
__global__ __launch_bounds__(256) void dkdv_f32_kernel(F32Args a) {
  constexpr int LD = D + 1;
  constexpr int NC = D / kLanes;
  __shared__ float Ks[kRows * LD];
  __shared__ float Vs[kRows * LD];
  __shared__ float Qs[kTile * LD];
  __shared__ float dOs[kTile * LD];
  __shared__ float Ps[kTile * kRows];
  __shared__ float dSs[kTile * kRows];
  __shared__ float Ls[kTile];
  __shared__ float Ds[kTile];
  const int r = threadIdx.x / kLanes, t = threadIdx.x % kLanes;
  const int T = a.T, W = a.window, G = a.H / a.Hkv;
  const int k0 = blockIdx.x * kRows;
  const int hkv = blockIdx.y, b = blockIdx.z;
  const size_t bkv = (size_t)b * a.Hkv + hkv;
  const int kv = k0 + r;
  load_rows<D>(Ks, LD, a.k + bkv * T * D, k0, kRows, T);
  load_rows<D>(Vs, LD, a.v + bkv * T * D, k0, kRows, T);
  float dk[NC], dv[NC];
#pragma unroll
  for (int k = 0; k < NC; ++k) dk[k] = dv[k] = 0.f;
  const int q_hi = W > 0 ? min(T, k0 + kRows - 1 + W) : T;
  for (int hh = hkv * G; hh < (hkv + 1) * G; ++hh) {
    const size_t bh = (size_t)b * a.H + hh;
    for (int q0 = (k0 / kTile) * kTile; q0 < q_hi; q0 += kTile) {
      __syncthreads();
      load_rows<D>(Qs, LD, a.q + bh * T * D, q0, kTile, T);
      load_rows<D>(dOs, LD, a.dO + bh * T * D, q0, kTile, T);
      if (threadIdx.x < kTile) {
        const int qq = min(q0 + (int)threadIdx.x, T - 1);
        Ls[threadIdx.x] = a.lse[bh * T + qq];
        Ds[threadIdx.x] = a.Dst[bh * T + qq];
      }
      __syncthreads();
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const int qq = t + u * kLanes;
        float qk = 0.f, dp = 0.f;
        for (int c = 0; c < D; ++c) {
          qk += Qs[qq * LD + c] * Ks[r * LD + c];
          dp += dOs[qq * LD + c] * Vs[r * LD + c];
        }
        float th;
        const float sc = capped(qk * a.scale, a.softcap, th);
        const float p = visible(q0 + qq, kv, W, T) ? expf(sc - Ls[qq]) : 0.f;
        float ds = p * (dp - Ds[qq]);
        if (a.softcap > 0.f) ds *= 1.f - th * th;
        Ps[qq * kRows + r] = p;
        dSs[qq * kRows + r] = ds;
      }
      __syncthreads();
#pragma unroll
      for (int k = 0; k < NC; ++k) {
        const int c = t + k * kLanes;
        float vv = dv[k], kk2 = dk[k];
        for (int qq = 0; qq < kTile; ++qq) {
          vv += Ps[qq * kRows + r] * dOs[qq * LD + c];
          kk2 += dSs[qq * kRows + r] * Qs[qq * LD + c];
        }
        dv[k] = vv;
        dk[k] = kk2;
      }
    }
  }
  if (kv < T) {
    float* dkp = a.dk + (bkv * T + kv) * D;
    float* dvp = a.dv + (bkv * T + kv) * D;
#pragma unroll
    for (int k = 0; k < NC; ++k) {
      dkp[t + k * kLanes] = dk[k] * a.scale;
      dvp[t + k * kLanes] = dv[k];
    }
  }
}

template <int D>
hipError_t fwd_d(const F32Args& a, hipStream_t s) {
  const dim3 grid((unsigned)((a.T + kRows - 1) / kRows), (unsigned)a.H, (unsigned)a.B);
  hipLaunchKernelGGL((fwd_f32_kernel<D>), grid, dim3(256), 0, s, a);
  stage_mark(s);
  return hipGetLastError();
}

template <int D>
hipError_t bwd_d(const F32Args& a, hipStream_t s) {
  const dim3 gq((unsigned)((a.T + kRows - 1) / kRows), (unsigned)a.H, (unsigned)a.B);
  hipLaunchKernelGGL((dq_f32_kernel<D>), gq, dim3(256), 0, s, a);
  stage_mark(s);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const dim3 gk((unsigned)((a.T + kRows - 1) / kRows), (unsigned)a.Hkv, (unsigned)a.B);
  hipLaunchKernelGGL((dkdv_f32_kernel<D>), gk, dim3(256), 0, s, a);
  stage_mark(s);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_fwd_f32(const F32Args& a, hipStream_t s) {
  switch (a.d) {
    case 64: return fwd_d<64>(a, s);
    case 128: return fwd_d<128>(a, s);
    case 256: return fwd_d<256>(a, s);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_bwd_f32(const F32Args& a, hipStream_t s) {
  switch (a.d) {
    case 64: return bwd_d<64>(a, s);
    case 128: return bwd_d<128>(a, s);
    case 256: return bwd_d<256>(a, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace fa
