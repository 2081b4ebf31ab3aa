// Rotary position embedding on interleaved pairs, bf16 and fp32 I/O.
//
// y[2i]   = x[2i] cos(t f_i) - x[2i+1] sin(t f_i)
// y[2i+1] = x[2i] sin(t f_i) + x[2i+1] cos(t f_i)
// with f the host-computed inverse-frequency table and the angle the fp32
// product t * f_i (Forge README: interleaved pairs; Forge attention.h commit
// log, "Wave 1": kernels read a host-precomputed inv-freq table).  The
// backward is the transpose (rotation by -angle).
//
// HBM-bound elementwise work.  The angle depends only on (t, i), not on the
// (b, h) row, so each thread fixes one 16-byte group of a [T, d] slice,
// evaluates its cos/sin once (accurate sincosf: angles reach ~8e3 rad) and
// then handles that group in BH_PER (b, h) slices: all BH_PER 16-byte loads
// are issued before the first store (each thread touches only its own
// addresses, so this order is safe in place), trigonometry amortised over
// the slices.  The launcher picks BH_PER (1, 2, 4 or 8) as the largest
// value that still gives the grid at least 2 workgroups per CU: the
// accurate sincosf costs more than the occupancy it buys back (measured on
// MI355X: 25 MB calls 3.6 -> 4.7 TB/s against 8 workgroups per CU).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "device_common.h"
#include "internal.h"

namespace fa {

namespace {

constexpr int kThreads = 256;
constexpr int kBhPer = 8;

template <typename T>
struct Vec;
template <>
struct Vec<__bf16> {
  static constexpr int N = 8;  // elements per 16 bytes
  typedef __bf16 V __attribute__((ext_vector_type(8)));
};
template <>
struct Vec<float> {
  static constexpr int N = 4;
  typedef float V __attribute__((ext_vector_type(4)));
};

template <typename T, bool BWD, int BH_PER>
__global__ __launch_bounds__(kThreads) void rope_vec_kernel(RopeArgs a) {
  constexpr int N = Vec<T>::N;
  typedef typename Vec<T>::V V;
  const long slice = (long)a.T * a.d;             // elements per (b, h)
  const long e0 = ((long)blockIdx.x * kThreads + threadIdx.x) * N;
  if (e0 >= slice) return;
  const int t = (int)(e0 / a.d);
  const int c0 = (int)(e0 % a.d);                 // even: N and d are even
  const int bh0 = blockIdx.y * BH_PER;
  const int nb = min(a.BH - bh0, BH_PER);        // ragged last row of the grid
  const T* x = (const T*)a.x;
  T* y = (T*)a.y;
  V v[BH_PER];
#pragma unroll
  for (int j = 0; j < BH_PER; ++j)
    if (j < nb) v[j] = *(const V*)(x + (long)(bh0 + j) * slice + e0);
  float cs[N / 2], sn[N / 2];
#pragma unroll
  for (int p = 0; p < N / 2; ++p) rope_sincos((float)t, a.inv_freq[c0 / 2 + p], BWD, cs[p], sn[p]);
#pragma unroll
  for (int j = 0; j < BH_PER; ++j) {
    if (j < nb) {
      V r;
#pragma unroll
      for (int p = 0; p < N / 2; ++p) {
        float xe = (float)v[j][2 * p], xo = (float)v[j][2 * p + 1];
        rope_pair(cs[p], sn[p], xe, xo);
        r[2 * p] = (T)xe;
        r[2 * p + 1] = (T)xo;
      }
      *(V*)(y + (long)(bh0 + j) * slice + e0) = r;
    }
  }
}

// Any even d: one pair per thread.
template <typename T, bool BWD>
__global__ __launch_bounds__(kThreads) void rope_pair_kernel(RopeArgs a) {
  const long slice = (long)a.T * a.d;
  const long e0 = ((long)blockIdx.x * kThreads + threadIdx.x) * 2;
  if (e0 >= slice) return;
  const int t = (int)(e0 / a.d);
  const int c0 = (int)(e0 % a.d);
  float sn, cs;
  rope_sincos((float)t, a.inv_freq[c0 / 2], BWD, cs, sn);
  const int bh0 = blockIdx.y * kBhPer;
  const int bh1 = min(a.BH, bh0 + kBhPer);
  const T* x = (const T*)a.x;
  T* y = (T*)a.y;
  for (int bh = bh0; bh < bh1; ++bh) {
    const long off = (long)bh * slice + e0;
    float xe = (float)x[off], xo = (float)x[off + 1];
    rope_pair(cs, sn, xe, xo);
    y[off] = (T)xe;
    y[off + 1] = (T)xo;
  }
}

template <typename T, bool BWD, int BH_PER>
void launch_vec(const RopeArgs& a, unsigned gx, hipStream_t stream) {
  const dim3 grid(gx, (unsigned)((a.BH + BH_PER - 1) / BH_PER));
  hipLaunchKernelGGL((rope_vec_kernel<T, BWD, BH_PER>), grid, dim3(kThreads), 0, stream, a);
}

template <typename T, bool BWD>
void launch_vec_bh(const RopeArgs& a, unsigned gx, hipStream_t stream) {
  // largest slices-per-thread count that keeps at least 2 workgroups per CU
  constexpr long kMinGroups = 2 * 256;
  const long per1 = (long)gx * a.BH;               // workgroups at one slice per thread
  if (per1 >= 8 * kMinGroups)
    launch_vec<T, BWD, 8>(a, gx, stream);
  else if (per1 >= 4 * kMinGroups)
    launch_vec<T, BWD, 4>(a, gx, stream);
  else if (per1 >= 2 * kMinGroups)
    launch_vec<T, BWD, 2>(a, gx, stream);
  else
    launch_vec<T, BWD, 1>(a, gx, stream);
}

template <typename T>
hipError_t launch_rope(const RopeArgs& a, bool bwd, hipStream_t stream) {
  const long slice = (long)a.T * a.d;
  const int N = Vec<T>::N;
  if (a.d % N == 0) {
    const unsigned gx = (unsigned)((slice / N + kThreads - 1) / kThreads);
    if (bwd)
      launch_vec_bh<T, true>(a, gx, stream);
    else
      launch_vec_bh<T, false>(a, gx, stream);
    stage_mark(stream);
  } else {
    const unsigned gy = (unsigned)((a.BH + kBhPer - 1) / kBhPer);
    const dim3 grid((unsigned)((slice / 2 + kThreads - 1) / kThreads), gy);
    if (bwd)
      hipLaunchKernelGGL((rope_pair_kernel<T, true>), grid, dim3(kThreads), 0, stream, a);
    else
      hipLaunchKernelGGL((rope_pair_kernel<T, false>), grid, dim3(kThreads), 0, stream, a);
    stage_mark(stream);
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_rope_bf16(const RopeArgs& a, bool bwd, hipStream_t stream) {
  return launch_rope<__bf16>(a, bwd, stream);
}
hipError_t launch_rope_f32(const RopeArgs& a, bool bwd, hipStream_t stream) {
  return launch_rope<float>(a, bwd, stream);
}

__global__ __launch_bounds__(256) void rope_table_kernel(const float* inv_freq, float2* cs, int T,
                                                        int half) {
  const long e = (long)blockIdx.x * 256 + threadIdx.x;
  if (e >= (long)T * half) return;
  const int t = (int)(e / half);
  const int i = (int)(e % half);
  float c, sn;
  rope_sincos((float)t, inv_freq[i], false, c, sn);
  cs[e] = make_float2(c, sn);
}

hipError_t launch_rope_table(const float* inv_freq, float* cs, int T, int half, hipStream_t stream) {
  const long n = (long)T * half;
  hipLaunchKernelGGL(rope_table_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, stream,
                     inv_freq, (float2*)cs, T, half);
  return hipGetLastError();
}

}  // namespace fa
