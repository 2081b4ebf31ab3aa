// d = 256 dQ pass of the causal flash-attention backward for gfx950
// (bf16 in, fp32 accumulate): the same gradient as fa_bwd_dq_kernel in
// fa_bwd.hip (dq = scale dS K with dS = P (dP - D) and, under a softcap, the
// factor 1 - tanh^2), software-pipelined for one wave per SIMD.  It lives in
// a file of its own because it is compiled with the VGPR form of the MFMA
// (its dQ accumulator is pinned to the AGPRs, so the score and dP products
// must not follow it there), which the dK/dV pass in fa_bwd.hip must not get.
#include <type_traits>

#include "device_common.h"
#include "internal.h"

namespace fa {

// Head size 256, dQ pass, software-pipelined like the d = 256 forward: one
// wave per 32 query rows holds the whole q and dO rows (128 VGPRs), dQ lives
// in the accumulation registers, and per 32-key unit i three MFMA blocks run,
// each carrying the VALU of another unit:
//   S(i+1)  = K(i+1) Q^T        carrying  dS(i) = f(i) (dP(i) - D), bf16 pack
//   dQ^T   += K(i)^T dS(i)^T    carrying  the cap's tanh and the mask of S(i+1)
//   dP(i+1) = V(i+1) dO^T - D   carrying  f(i+1) = P (1 - tanh^2) (P without a cap)
// The dP accumulators start from -D_i, so they end as dP - D.  Iteration i
// reads K(i) (transposed, for dQ), K(i+1) and V(i+1) while K(i+2) and V(i+2)
// load, so both tiles are triple-buffered (loop unrolled by three); one
// barrier per unit.  Units of the workgroup's key range outside a wave's band
// are computed fully masked (exact zeros), so every wave runs the same
// straight-line schedule.  Also writes D_i for the dK/dV pass.
template <bool CAP>
__global__ __launch_bounds__(256, 1) void fa_bwd_dq_pipe_kernel(BwdArgs a) {
  constexpr int D = 256, NW = 4, BQ = 32 * NW, BKV = 32;
  // a tile image, rounded up to whole rounds of the loaders' 1 KB pieces
  constexpr int TILE = TileDma<D, BKV, NW>::IMG;
  constexpr int NC = D / 16;     // chunks of the S and dP contractions
  constexpr int NDB = D / 32;    // 32-wide blocks of dq
  constexpr int NQ = 2 * NDB;    // MFMAs of the dQ block
  constexpr int PD = 2;
  __shared__ __attribute__((aligned(1024))) char kt0[TILE];
  __shared__ __attribute__((aligned(1024))) char kt1[TILE];
  __shared__ __attribute__((aligned(1024))) char kt2[TILE];
  __shared__ __attribute__((aligned(1024))) char vt0[TILE];
  __shared__ __attribute__((aligned(1024))) char vt1[TILE];
  __shared__ __attribute__((aligned(1024))) char vt2[TILE];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = lane >> 5;
  const int l32 = lane & 31;
  const int T = a.T;
  const int W = a.window;
  const int G = a.H / a.Hkv;
  const int nqb = (T + BQ - 1) / BQ;
  const WorkItem w = decode_work(blockIdx.x, nqb, a.B, a.Hkv, G, true);
  const int h = w.hkv * G + w.r;
  const int q0 = w.blk * BQ;
  const int qw0 = q0 + 32 * wave;
  const int qrow = qw0 + l32;
  const int qr = qrow < T ? qrow : T - 1;
  const size_t bh = (size_t)w.b * a.H + h;
  const size_t bkv = (size_t)w.b * a.Hkv + w.hkv;
  const bf16* Kp = a.k + bkv * T * D;
  const bf16* Vp = a.v + bkv * T * D;

  // q and dO rows as B operands (lane = query row); D_i; lse in log2 units
  bf16x8 qreg[NC], doreg[NC];
  float Di;
  {
    const size_t roff = (bh * T + qr) * D + 8 * g;
    const bf16x8* qs = (const bf16x8*)(a.q + roff);
    const bf16x8* ds = (const bf16x8*)(a.dO + roff);
    const bf16x8* os = (const bf16x8*)(a.o + roff);
    float part = 0.f;
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      qreg[c] = qs[2 * c];
      doreg[c] = ds[2 * c];
      const bf16x8 ov = os[2 * c];
#pragma unroll
      for (int j = 0; j < 8; ++j) part += (float)doreg[c][j] * (float)ov[j];
    }
    Di = xor32_sum(part);
    if (g == 0 && qrow < T) a.Dst[bh * T + qrow] = Di;
  }
  const float lse2 = a.lse[bh * T + qr] * kLog2e;
  if (a.sinks) {
    float c = (g == 0 && qrow < T) ? fast_exp2(a.sinks[h] * kLog2e - lse2) * Di : 0.f;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) c += __shfl_xor(c, off);
    if (lane == 0) atomicAdd(a.dsinks + h, -c);
  }

  int kv_lo = 0;
  if (W > 0) kv_lo = max(0, q0 - W + 1);
  const int t_lo = kv_lo / BKV;
  const int kv_hi = min(T, q0 + BQ);
  const int nu = (kv_hi + BKV - 1) / BKV - t_lo;
  const unsigned span = W > 0 ? (unsigned)W : 0x7fffffffu;
  const float cexp = CAP ? a.cap_log2e : a.scale_log2e;

  f32x16 dqacc[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db)
#pragma unroll
    for (int i = 0; i < 16; ++i) dqacc[db][i] = 0.f;

  TileDma<D, BKV, NW> dm;
  dm.init(wave, lane);
  LaneOffs<D> lo;
  lo.init(lane);
  using I0 = std::integral_constant<int, 0>;
  using I1 = std::integral_constant<int, 1>;
  using I2 = std::integral_constant<int, 2>;
  auto kbuf = [&](auto b_c) -> LDS_AS char* {
    constexpr int b = decltype(b_c)::value;
    return b == 0 ? (LDS_AS char*)kt0 : b == 1 ? (LDS_AS char*)kt1 : (LDS_AS char*)kt2;
  };
  auto vbuf = [&](auto b_c) -> LDS_AS char* {
    constexpr int b = decltype(b_c)::value;
    return b == 0 ? (LDS_AS char*)vt0 : b == 1 ? (LDS_AS char*)vt1 : (LDS_AS char*)vt2;
  };

  // per-unit tiles, indexed by unit parity: sx holds S, then the masked
  // capped score, then f; dpx holds dP - D; tt the factor 1 - tanh^2 of the
  // unit being prepared (cap only)
  f32x16 sx[2], dpx[2];
  f32x16 tt;
  bf16x8 dsb[2];

  // S(u) into sx[X] / dP(u) - D into dpx[X], hook(k) after MFMA k
  auto s_block = [&](auto x_c, const LDS_AS char* Kt, auto&& hook) __attribute__((always_inline)) {
    constexpr int X = decltype(x_c)::value;
#pragma unroll
    for (int i = 0; i < 16; ++i) sx[X][i] = 0.f;
    auto f = [&](int k) { return lds_row_op<D>(Kt, lo, 0, k); };
    MfmaSeq<NC, PD> sq;
    sq.start(f);
    sq.run(f, [&](int k) { return qreg[k]; }, [&](int) -> f32x16& { return sx[X]; }, hook);
  };
  auto dp_block = [&](auto x_c, const LDS_AS char* Vt, auto&& hook) __attribute__((always_inline)) {
    constexpr int X = decltype(x_c)::value;
#pragma unroll
    for (int i = 0; i < 16; ++i) dpx[X][i] = -Di;
    auto f = [&](int k) { return lds_row_op<D>(Vt, lo, 0, k); };
    MfmaSeq<NC, PD> pq;
    pq.start(f);
    pq.run(f, [&](int k) { return doreg[k]; }, [&](int) -> f32x16& { return dpx[X]; }, hook);
  };
  // dQ^T += K^T dS^T for the unit whose dS is in dsb (K tile read transposed),
  // accumulator pinned to the AGPRs
  auto q_block = [&](const LDS_AS char* Kt, auto&& hook) __attribute__((always_inline)) {
    auto f = [&](int k) { return lds_tr_op<D>(Kt, lo, k / NDB, k % NDB); };
    constexpr int R = PD + 1;
    bf16x8 op[R];
#pragma unroll
    for (int k = 0; k < PD; ++k) op[k] = f(k);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int k = 0; k < NQ; ++k) {
      if (k + PD < NQ) op[(k + PD) % R] = f(k + PD);
      mfma32_agpr(dqacc[k % NDB], op[k % R], dsb[k / NDB]);
      hook(k);
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  // cap and mask of unit u's scores, elements [e0, e1) (factor 1 - tanh^2
  // into tt, zero where masked; masked scores -inf so that P = 0)
  // (MASK false: every row of the wave sees the whole unit)
  auto part_a = [&](auto x_c, auto mask_c, int u, int e0, int e1) __attribute__((always_inline)) {
    constexpr int X = decltype(x_c)::value;
    constexpr bool MASK = decltype(mask_c)::value;
    const int base = qrow - (t_lo + u) * BKV - 4 * g;
#pragma unroll
    for (int i = e0; i < e1; ++i) {
      const bool vis = !MASK || (unsigned)(base - (8 * (i >> 2) + (i & 3))) < span;
      float x = sx[X][i];
      if (CAP) {
        const float e = fast_exp2(x * a.two_scale_over_cap_log2e);
        x = 1.f - 2.f * __builtin_amdgcn_rcpf(e + 1.f);   // tanh
        tt[i] = vis ? fmaf(-x, x, 1.f) : 0.f;
      }
      sx[X][i] = vis ? x : -INFINITY;
    }
  };
  // f = P (1 - tanh^2), P = 2^(S' c - lse), elements [e0, e1)
  auto part_b = [&](auto x_c, int e0, int e1) __attribute__((always_inline)) {
    constexpr int X = decltype(x_c)::value;
#pragma unroll
    for (int i = e0; i < e1; ++i) {
      const float p = fast_exp2(fmaf(sx[X][i], cexp, -lse2));
      sx[X][i] = CAP ? p * tt[i] : p;
    }
  };
  // dS = f (dP - D), elements [e0, e1), bf16 packs per 16-key chunk
  auto part_c = [&](auto x_c, int e0, int e1) __attribute__((always_inline)) {
    constexpr int X = decltype(x_c)::value;
#pragma unroll
    for (int i = e0; i < e1; ++i) {
      sx[X][i] *= dpx[X][i];
      if (i == 7 || i == 15) {
        float tmp[8];
#pragma unroll
        for (int jj = 0; jj < 8; ++jj) tmp[jj] = sx[X][i - 7 + jj];
        dsb[i >> 3] = pack_bf16(tmp);
      }
    }
  };

  // prologue: K(0), V(0), K(1), V(1) resident; S(0), its cap and mask, dP(0)
  // with f(0)
  dm.load(Kp, T * D * 2, kbuf(I0{}), t_lo * BKV, wave);
  dm.load(Vp, T * D * 2, vbuf(I0{}), t_lo * BKV, wave);
  if (nu > 1) {
    dm.load(Kp, T * D * 2, kbuf(I1{}), (t_lo + 1) * BKV, wave);
    dm.load(Vp, T * D * 2, vbuf(I1{}), (t_lo + 1) * BKV, wave);
  }
  wait_vmem();
  __syncthreads();
  using MT = std::true_type;
  using MF = std::false_type;
  s_block(I0{}, kbuf(I0{}), [&](int) {});
  part_a(I0{}, MT{}, 0, 0, 16);
  dp_block(I0{}, vbuf(I0{}), [&](int k) __attribute__((always_inline)) { part_b(I0{}, k, k + 1); });

  // iteration i (buffer slots: K(i) in B0, K(i+1) and V(i+1) in B1, loads
  // into B2; unit parities X for unit i, 1 - X for unit i + 1).  The unit
  // count is padded to a multiple of three: units past the workgroup's key
  // range hold only keys later than all its query rows (or past T, where the
  // buffer range reads zeros), so they are fully masked and add exact zeros;
  // every step then computes a next unit, and after each group of three the
  // next unit's tiles move back to parity 0.
  // K(i+2) and V(i+2) load one piece after each of the S block's first
  // MFMAs (whose hooks carry little VALU), branch-free: a wave with no piece
  // k left loads zeros into the image's partial last round
  constexpr int PER = TileDma<D, BKV, NW>::PER;
  static_assert(2 * PER <= NC, "one load per S MFMA");
  auto step = [&](auto b0, auto b1, auto b2, auto x_c, auto mask_c, const int i)
                  __attribute__((always_inline)) {
    using XN = std::integral_constant<int, 1 - decltype(x_c)::value>;
    lo.refresh();
    s_block(XN{}, kbuf(b1), [&](int k) __attribute__((always_inline)) {
      part_c(x_c, k, k + 1);
      if (k < PER)
        dm.load_piece(k, Kp, T * D * 2, kbuf(b2), (t_lo + i + 2) * BKV, wave);
      else if (k < 2 * PER)
        dm.load_piece(k - PER, Vp, T * D * 2, vbuf(b2), (t_lo + i + 2) * BKV, wave);
    });
    q_block(kbuf(b0), [&](int k) __attribute__((always_inline)) {
      part_a(XN{}, mask_c, i + 1, k, k + 1);
    });
    dp_block(XN{}, vbuf(b1), [&](int k) __attribute__((always_inline)) { part_b(XN{}, k, k + 1); });
    wait_vmem();
    __syncthreads();
  };
  auto group = [&](auto mask_c, const int i) __attribute__((always_inline)) {
    step(I0{}, I1{}, I2{}, I0{}, mask_c, i);
    step(I1{}, I2{}, I0{}, I1{}, mask_c, i + 1);
    step(I2{}, I0{}, I1{}, I0{}, mask_c, i + 2);
    sx[0] = sx[1];
    dpx[0] = dpx[1];
  };
  // Groups of three steps whose units (i + 1 .. i + 3) every row of the wave
  // sees whole form one range [ga, gb): the units in [mlo, mhi).  The groups
  // before and after it evaluate the mask; those in it carry none.
  const int ng = (nu + 2) / 3;
  const int mhi = qw0 / BKV - t_lo;   // first unit holding a key past row qw0
  const int wlo = qw0 + 31 - W;       // keys above it are in every row's window
  const int mlo = (W > 0 && wlo >= 0) ? max(0, wlo / BKV + 1 - t_lo) : 0;
  const int ga = min(ng, max(0, (mlo + 1) / 3));          // first group with 3 gi + 1 >= mlo
  const int gb = min(ng, max(ga, mhi >= 4 ? (mhi - 4) / 3 + 1 : 0));   // 3 gi + 3 < mhi
  int gi = 0;
  for (; gi < ga; ++gi) group(MT{}, 3 * gi);
  for (; gi < gb; ++gi) group(MF{}, 3 * gi);
  for (; gi < ng; ++gi) group(MT{}, 3 * gi);

  agpr_acc_fence(dqacc);
  if (qrow < T) {
    bf16* Qd = a.dq + (bh * T + qrow) * D;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int i4 = 0; i4 < 4; ++i4) {
        float x[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) x[e] = dqacc[db][4 * i4 + e] * a.scale;
        if (a.rope_cs) {
          // RoPE backward fused into the store (pairs 16 db + 4 i4 + 2 g + {0, 1})
          const float4 r = *(const float4*)(a.rope_cs + (size_t)qrow * D +
                                            2 * (16 * db + 4 * i4 + 2 * g));
          rope_pair(r.x, -r.y, x[0], x[1]);
          rope_pair(r.z, -r.w, x[2], x[3]);
        }
        bf16x4 v;
#pragma unroll
        for (int e = 0; e < 4; ++e) v[e] = (bf16)x[e];
        *(bf16x4*)(Qd + 32 * db + 8 * i4 + 4 * g) = v;
      }
  }
}

hipError_t launch_bwd_dq_pipe(const BwdArgs& a, bool cap, hipStream_t stream) {
  const int nqb = (a.T + 127) / 128;
  const dim3 grid((unsigned)nqb * a.B * a.H);
  if (cap)
    hipLaunchKernelGGL(fa_bwd_dq_pipe_kernel<true>, grid, dim3(256), 0, stream, a);
  else
    hipLaunchKernelGGL(fa_bwd_dq_pipe_kernel<false>, grid, dim3(256), 0, stream, a);
  return hipGetLastError();
}

}  // namespace fa
