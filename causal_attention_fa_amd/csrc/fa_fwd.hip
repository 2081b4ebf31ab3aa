// Fused causal flash-attention forward for gfx950 (bf16 in, fp32 accumulate).
//
// Computes o = softmax(mask(capped(scale * q k^T))) v and the natural-log
// row log-sum-exp (lse), with GQA, a sliding window whose out-of-window key
// tiles are never loaded, and the optional softcap cap*tanh(s/cap) on the
// scaled scores (Forge ARCHITECTURES.md, implementation plan wave 2, items 8
// and 9; Forge attention.h commit log, "Wave 2").
//
// Structure (one workgroup = 4 waves = 128 query rows of one (b, h)):
//   * each wave owns 32 query rows; its Q rows stay in registers as the B
//     operand of S^T = K Q^T, so every lane owns one query row (column of
//     S^T) and the online-softmax max/sum are per-lane values combined with
//     the partner lane l^32 -- no cross-lane row reductions inside a tile;
//   * K and V tiles (BKV keys) stream through LDS, double-buffered: the next
//     tile goes straight from HBM into the idle padded LDS buffer (direct
//     buffer loads, no staging registers), issued at the top of an
//     iteration and waited for before its closing barrier;
//   * P^T leaves the S^T accumulators as bf16 and is directly the B operand
//     of O^T += V^T P^T; V^T comes from the natural V tile through the
//     gfx950 LDS transpose read, so nothing is transposed in registers;
//   * tiles entirely outside a wave's causal/window band are skipped, tiles
//     entirely inside are not masked; only diagonal and window-edge tiles
//     evaluate the mask.
// Head size 128 runs fa_fwd_sp_kernel, the same structure software-pipelined
// across tiles (the next tile's scores computed under this tile's softmax);
// head size 256 runs fa_fwd_pipe_kernel.
#include <type_traits>

#include "device_common.h"
#include "internal.h"

namespace fa {


// LDS operand reads run this many MFMAs ahead of their use (the one-tile
// kernel, the software-pipelined kernel).
constexpr int kFwdPD = 3;       // one-tile kernel: LDS operands this many MFMAs ahead
constexpr int kFwdPipePD = 2;   // pipelined d = 256 kernel: the same

// One wave owns 32 query rows.  DK is the head size of q and k, DV that of
// v and o (equal except for MLA-style heads).  NSTG (2..4) K/V tiles are in
// LDS or in flight at once: the load of tile j + NSTG - 1 is issued when
// tile j's compute starts, so an HBM load has NSTG - 1 tiles of compute to
// arrive in.  MINWG > 0 asks for that many resident workgroups per CU (the
// compiler then caps the registers to fit them); 0 keeps two waves per SIMD.
template <int DK, int DV, int BKV, int NW, bool CAP, int NSTG = 2, int MINWG = 0>
__global__ __launch_bounds__(64 * NW, (MINWG > 0 ? MINWG : DK >= 256 ? 1 : 8 / NW)) void fa_fwd_kernel(
    FwdArgs a) {
  static_assert(NSTG >= 2 && NSTG <= 4, "2 to 4 tile buffers");
  constexpr int BQ = 32 * NW;         // query rows per workgroup
  constexpr int TILE_K = Lay<DK>::template bytes<BKV>();  // one K tile
  constexpr int TILE_V = Lay<DV>::template bytes<BKV>();  // one V tile
  constexpr int NDB = DV / 32;        // 32-wide blocks of the output
  constexpr int NS = BKV / 32;        // 32-key sub-tiles
  constexpr int NC = DK / 16;         // 16-wide chunks of the q.k contraction
  constexpr int NP = BKV / 16;        // 16-key chunks of P (B operands of O^T += V^T P^T)
  // one LDS object per buffer: the compiler can then tell the buffer being
  // filled by direct loads from the one being read, and does not make the
  // reads wait for the loads
  __shared__ __attribute__((aligned(1024))) char kb0[TILE_K];
  __shared__ __attribute__((aligned(1024))) char kb1[TILE_K];
  __shared__ __attribute__((aligned(1024))) char kb2[NSTG > 2 ? TILE_K : 4];
  __shared__ __attribute__((aligned(1024))) char kb3[NSTG > 3 ? TILE_K : 4];
  __shared__ __attribute__((aligned(1024))) char vb0[TILE_V];
  __shared__ __attribute__((aligned(1024))) char vb1[TILE_V];
  __shared__ __attribute__((aligned(1024))) char vb2[NSTG > 2 ? TILE_V : 4];
  __shared__ __attribute__((aligned(1024))) char vb3[NSTG > 3 ? TILE_V : 4];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  __builtin_assume(wave < NW);
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
  const size_t bh = (size_t)w.b * a.H + h;
  const size_t bkv = (size_t)w.b * a.Hkv + w.hkv;
  const bf16* Kp = a.k + bkv * T * DK;
  const bf16* Vp = a.v + bkv * T * DV;

  // Q as the B operand of S^T = K Q^T: lane holds Q[qrow][16c + 8g .. +7].
  bf16x8 qreg[NC];
  {
    const bf16x8* src = (const bf16x8*)(a.q + (bh * T + min(qrow, T - 1)) * DK + 8 * g);
#pragma unroll
    for (int c = 0; c < NC; ++c) qreg[c] = src[2 * c];
  }
  // RoPE fused into the Q load: this lane's 8-element chunks hold the pairs
  // 8c + 4g + p of its row (position = row index), whose (cos, sin) come from
  // the call's table; the rotated row is optionally written out once for the
  // backward.
  if (a.rope_cs) {
    const float4* cs4 = (const float4*)(a.rope_cs + (size_t)min(qrow, T - 1) * DK);
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      bf16x8 x = qreg[c];
      // pairs 8c + 4g .. +3: 4 (cos, sin) = two float4
      const float4 r0 = cs4[(8 * c + 4 * g) / 2], r1 = cs4[(8 * c + 4 * g) / 2 + 1];
      const float cv[4] = {r0.x, r0.z, r1.x, r1.z}, sv[4] = {r0.y, r0.w, r1.y, r1.w};
#pragma unroll
      for (int p = 0; p < 4; ++p) {
        float xe = (float)x[2 * p], xo = (float)x[2 * p + 1];
        rope_pair(cv[p], sv[p], xe, xo);
        x[2 * p] = (bf16)xe;
        x[2 * p + 1] = (bf16)xo;
      }
      qreg[c] = x;
    }
    if (a.q_rot && qrow < T) {
      bf16x8* dst = (bf16x8*)(a.q_rot + (bh * T + qrow) * DK + 8 * g);
#pragma unroll
      for (int c = 0; c < NC; ++c) dst[2 * c] = qreg[c];
    }
  }

  int kv_lo = 0;
  if (W > 0) kv_lo = max(0, q0 - W + 1);
  const int t_lo = kv_lo / BKV;
  const int kv_hi = min(T, q0 + BQ);
  const int ntiles = (kv_hi + BKV - 1) / BKV - t_lo;

  // Attention sink (ARCHITECTURES.md plan wave 2 item 10): the online
  // softmax starts from the sink logit, whose exp(0) = 1 enters the sum once
  // (lane half 0) and whose value contribution is zero.
  const bool has_sink = a.sinks != nullptr;
  const float sink2 = has_sink ? a.sinks[h] * kLog2e : 0.f;
  f32x16 oacc[NDB];
  float m = has_sink ? sink2 : kMaxInit;
  float lsum = (has_sink && g == 0) ? 1.f : 0.f;
  float mxl = -INFINITY;
#pragma unroll
  for (int db = 0; db < NDB; ++db)
#pragma unroll
    for (int i = 0; i < 16; ++i) oacc[db][i] = 0.f;

  // K, V tiles go straight from HBM to the idle LDS buffers (no staging
  // registers)
  using KDma = TileDma<DK, BKV, NW>;
  using VDma = TileDma<DV, BKV, NW>;
  KDma kdm;
  VDma vdm;
  kdm.init(wave, lane);
  vdm.init(wave, lane);
  auto kbuf = [&](auto p_c) -> LDS_AS char* {
    constexpr int P = decltype(p_c)::value;
    return P == 0 ? (LDS_AS char*)kb0 : P == 1 ? (LDS_AS char*)kb1 : P == 2 ? (LDS_AS char*)kb2 : (LDS_AS char*)kb3;
  };
  auto vbuf = [&](auto p_c) -> LDS_AS char* {
    constexpr int P = decltype(p_c)::value;
    return P == 0 ? (LDS_AS char*)vb0 : P == 1 ? (LDS_AS char*)vb1 : P == 2 ? (LDS_AS char*)vb2 : (LDS_AS char*)vb3;
  };
  using I0 = std::integral_constant<int, 0>;
  using I1 = std::integral_constant<int, 1>;
  using I2 = std::integral_constant<int, 2>;
  using I3 = std::integral_constant<int, 3>;
  // tile j (counted from t_lo) into buffer P
  auto issue = [&](auto p_c, int j) __attribute__((always_inline)) {
    kdm.load(Kp, T * DK * 2, kbuf(p_c), (t_lo + j) * BKV, wave);
    vdm.load(Vp, T * DV * 2, vbuf(p_c), (t_lo + j) * BKV, wave);
  };
  // Waits until this wave's share of the oldest tile in flight is in LDS,
  // while the `newer` tiles issued after it (0 .. NSTG - 2) may stay in
  // flight.  Loads finish in issue order, and a wave issues at least LMIN
  // loads per tile (when a tile's 1 KB pieces do not divide evenly among the
  // waves, some issue one more), so allowing newer * LMIN outstanding never
  // lets part of the oldest tile through.
  constexpr int LMIN = KDma::NI / NW + VDma::NI / NW;
  auto wait_tile = [&](int newer) __attribute__((always_inline)) {
    if constexpr (NSTG >= 4) {
      if (newer >= 2) {
        wait_vmem<2 * LMIN>();
        return;
      }
    }
    if constexpr (NSTG >= 3) {
      if (newer >= 1) {
        wait_vmem<LMIN>();
        return;
      }
    }
    wait_vmem<0>();
  };
  issue(I0{}, 0);
  if constexpr (NSTG >= 3)
    if (1 < ntiles) issue(I1{}, 1);
  if constexpr (NSTG >= 4)
    if (2 < ntiles) issue(I2{}, 2);
  wait_tile(min(NSTG - 2, ntiles - 1));
  lds_barrier();

  // The exponent's FMA carries the constant: scale*log2(e) on raw scores
  // without a cap, cap*log2(e) on tanh(scale*x/cap) with one (the max
  // scales with it either way).
  const float cexp = CAP ? a.cap_log2e : a.scale_log2e;
  const int qa = qw0, qb = qw0 + 31;
  // one iteration on the tile in buffer P (the loop is unrolled by NSTG so
  // that the buffers are compile-time choices)
  auto step = [&](auto p_c, const int j) __attribute__((always_inline)) {
    constexpr int P = decltype(p_c)::value;
    using PN = std::integral_constant<int, (P + NSTG - 1) % NSTG>;
    const LDS_AS char* Kt = kbuf(p_c);
    const LDS_AS char* Vt = vbuf(p_c);
    // tile j + NSTG - 1 into the buffer that tile j - 1 used (every wave has
    // passed the barrier that ended tile j - 1): its latency hides behind
    // NSTG - 1 tiles of compute
    if (j + NSTG - 1 < ntiles) issue(PN{}, j + NSTG - 1);
    const int kv0 = (t_lo + j) * BKV;
    const bool empty = qa >= T || kv0 > qb || (W > 0 && kv0 + BKV - 1 <= qa - W);
    const bool full = kv0 + BKV - 1 <= qa && (W == 0 || kv0 > qb - W);
    if (!empty) {
      // S^T = K Q^T as a pinned MFMA sequence whose K operands are read
      // kFwdPD MFMAs ahead: left to itself the compiler sinks each read down
      // to its MFMA, and the LDS latency stalls the matrix unit.
      f32x16 s[NS];
#pragma unroll
      for (int t = 0; t < NS; ++t)
#pragma unroll
        for (int i = 0; i < 16; ++i) s[t][i] = 0.f;
      {
        MfmaSeq<NC * NS, kFwdPD> sq;
        auto fK = [&](int k) __attribute__((always_inline)) {
          return lds_row_operand<DK>(Kt, 32 * (k % NS), k / NS, lane);
        };
        sq.start(fK);
        sq.run(fK, [&](int k) __attribute__((always_inline)) { return qreg[k / NS]; },
               [&](int k) __attribute__((always_inline)) -> f32x16& { return s[k % NS]; },
               [](int) {});
      }
      // the transposed V operands of O^T += V^T P^T are requested now, their
      // latency hidden behind the softmax
      MfmaSeq<NP * NDB, kFwdPD> vq;
      auto fV = [&](int k) __attribute__((always_inline)) {
        return lds_tr_operand<DV>(Vt, 0, k / NDB, 32 * (k % NDB), lane);
      };
      vq.start(fV);
      if (CAP) {
#pragma unroll
        for (int t = 0; t < NS; ++t)
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            // cap * tanh(scale*x / cap) * log2(e)
            const float e = fast_exp2(s[t][i] * a.two_scale_over_cap_log2e);
            s[t][i] = 1.f - 2.f * __builtin_amdgcn_rcpf(e + 1.f);  // tanh
          }
      }
      if (!full) {
#pragma unroll
        for (int t = 0; t < NS; ++t)
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const int kv = kv0 + 32 * t + acc_row(i, g);
            const bool vis = (kv <= qrow) & ((W == 0) | (kv > qrow - W));
            s[t][i] = vis ? s[t][i] : -INFINITY;
          }
      }
      float mt = -INFINITY;
#pragma unroll
      for (int t = 0; t < NS; ++t)
#pragma unroll
        for (int i = 0; i < 16; ++i) mt = fmaxf(mt, s[t][i]);
      mt = xor32_max(mt) * cexp;
      if (a.max_logit) mxl = fmaxf(mxl, qrow < T ? mt : -INFINITY);
      // Lazy rescaling: the running max only moves (and O, l are rescaled)
      // when some row's tile max exceeds it by more than kRescaleSlack, so
      // p = 2^(s - m) stays below 2^kRescaleSlack; the branch is uniform.
      if (__any(mt > m + kRescaleSlack)) {
        const float mnew = fmaxf(m, mt);
        const float alpha = fast_exp2(m - mnew);
        m = mnew;
        lsum *= alpha;
#pragma unroll
        for (int db = 0; db < NDB; ++db)
#pragma unroll
          for (int i = 0; i < 16; ++i) oacc[db][i] *= alpha;
      }
      // P^T in bf16, 16 keys (one B operand) at a time: chunk c + 1 is
      // computed under the MFMAs that consume chunk c.
      bf16x8 pb[NP];
      float ps = 0.f;
      auto pchunk = [&](int c, int e0, int e1) __attribute__((always_inline)) {
#pragma unroll
        for (int e = e0; e < e1; ++e) {
          const float p = fast_exp2(fmaf(s[c >> 1][8 * (c & 1) + e], cexp, -m));
          s[c >> 1][8 * (c & 1) + e] = p;
          ps += p;
        }
        if (e1 == 8) {
          float tmp[8];
#pragma unroll
          for (int e = 0; e < 8; ++e) tmp[e] = s[c >> 1][8 * (c & 1) + e];
          pb[c] = pack_bf16(tmp);
        }
      };
      pchunk(0, 0, 8);
      constexpr int EPM = 8 / NDB > 0 ? 8 / NDB : 1;   // exponentials per MFMA
      vq.run(fV, [&](int k) __attribute__((always_inline)) { return pb[k / NDB]; },
             [&](int k) __attribute__((always_inline)) -> f32x16& { return oacc[k % NDB]; },
             [&](int k) __attribute__((always_inline)) {
               const int c = k / NDB + 1, part = k % NDB;
               if (c < NP && part * EPM < 8) pchunk(c, part * EPM, min(8, part * EPM + EPM));
             });
      lsum += ps;
    }
    // tile j + 1 complete before the barrier that publishes it.  The wait
    // is unconditional (a no-op when nothing is in flight): behind a branch
    // the compiler sees a path with a load still pending into the buffer
    // the next step reads, and stalls that step's first read on it.
    wait_tile(min(NSTG - 2, ntiles - j - 2));
    lds_barrier();
  };
  int j = 0;
  for (; j + NSTG <= ntiles; j += NSTG) {
    step(I0{}, j);
    step(I1{}, j + 1);
    if constexpr (NSTG >= 3) step(I2{}, j + 2);
    if constexpr (NSTG >= 4) step(I3{}, j + 3);
  }
  if (j < ntiles) step(I0{}, j);
  if constexpr (NSTG >= 3)
    if (j + 1 < ntiles) step(I1{}, j + 1);
  if constexpr (NSTG >= 4)
    if (j + 2 < ntiles) step(I2{}, j + 2);

  if (a.max_logit) {
    // largest logit of the wave's rows (natural log units), one atomic per wave
    float v = mxl;
#pragma unroll
    for (int off = 1; off < 32; off <<= 1) v = fmaxf(v, __shfl_xor(v, off));
    if (lane == 0 && v > -INFINITY) atomic_max_f32(a.max_logit + bh, v * kLn2);
  }
  const float ltot = xor32_sum(lsum);
  if (qrow < T) {
    const float inv = 1.f / ltot;
    bf16* Op = a.o + (bh * T + qrow) * DV;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int i4 = 0; i4 < 4; ++i4) {
        bf16x4 v;
#pragma unroll
        for (int e = 0; e < 4; ++e) v[e] = (bf16)(oacc[db][4 * i4 + e] * inv);
        *(bf16x4*)(Op + 32 * db + 8 * i4 + 4 * g) = v;
      }
    if (g == 0) a.lse[bh * T + qrow] = (m + __log2f(ltot)) * kLn2;
  }
}

// Head size 128, software-pipelined across 64-key tiles at two waves per
// SIMD.  Each wave owns 32 query rows as in fa_fwd_kernel; per tile j it
// issues the score block of the next tile before the O block of this one,
// and puts under each the softmax VALU that does not wait for it:
//   S(j+1) = K(j+1) Q^T (16 MFMAs)    carrying  exp2, row sum and bf16 packs of
//                                              P(j)'s keys 32..63, and the tile
//                                              loads of K(j+2) and V(j+1)
//   O^T += V(j)^T P(j)^T (16 MFMAs)   carrying  cap, mask and row max of S(j+1),
//                                              the rescale decision, and P(j+1)
//                                              of its keys 0..31
// The O rescale that tile j+1's max may need waits until the O block is done
// (rare: the running max moves only past the slack).  K(j+1) and V(j) are read
// in step j while K(j+2) and V(j+1) load, so both tiles are double-buffered,
// one barrier per step.  Every wave walks the workgroup's whole key range:
// tiles outside a wave's band are computed fully masked (exact zeros).
// Tiles every row of the wave sees whole run in a mask-free segment.
template <bool CAP>
__global__ __launch_bounds__(256, 2) void fa_fwd_sp_kernel(FwdArgs a) {
  constexpr int D = 128, NW = 4, BQ = 32 * NW, BKV = 64;
  using Dma = TileDma<D, BKV, NW>;
  constexpr int TILE = Dma::IMG;
  constexpr int PER = Dma::PER;
  constexpr int NC = D / 16;       // 16-wide chunks of the q.k contraction
  constexpr int NDB = D / 32;      // 32-wide blocks of the output
  constexpr int NSQ = 2 * NC;      // MFMAs of the score block (two 32-key halves)
  constexpr int NPV = 4 * NDB;     // MFMAs of the O block (four 16-key chunks)
  constexpr int PD = 2;      // operand reads this many MFMAs ahead (3: no faster)
  // the first O-block MFMA whose hook starts the next tile's exponentials
  // (the hooks before it take the next tile's cap, mask and max; 6: no faster)
  constexpr int KE0 = 8;
  static_assert(2 * PER <= NSQ, "one tile load per score MFMA");
  __shared__ __attribute__((aligned(1024))) char kb0[TILE];
  __shared__ __attribute__((aligned(1024))) char kb1[TILE];
  __shared__ __attribute__((aligned(1024))) char vb0[TILE];
  __shared__ __attribute__((aligned(1024))) char vb1[TILE];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = lane >> 5;
  const int T = a.T;
  const int W = a.window;
  const int G = a.H / a.Hkv;
  const int nqb = (T + BQ - 1) / BQ;
  const WorkItem w = decode_work(blockIdx.x, nqb, a.B, a.Hkv, G, true);
  const int h = w.hkv * G + w.r;
  const int q0 = w.blk * BQ;
  const int qw0 = q0 + 32 * wave;
  const int qrow = qw0 + (lane & 31);
  const size_t bh = (size_t)w.b * a.H + h;
  const size_t bkv = (size_t)w.b * a.Hkv + w.hkv;
  const bf16* Kp = a.k + bkv * T * D;
  const bf16* Vp = a.v + bkv * T * D;

  // q as the B operand of S^T = K Q^T (RoPE fused into the load as in
  // fa_fwd_kernel)
  bf16x8 qreg[NC];
  {
    const int qr = min(qrow, T - 1);
    const bf16x8* src = (const bf16x8*)(a.q + (bh * T + qr) * D + 8 * g);
#pragma unroll
    for (int c = 0; c < NC; ++c) qreg[c] = src[2 * c];
    if (a.rope_cs) {
      const float4* cs4 = (const float4*)(a.rope_cs + (size_t)qr * D);
#pragma unroll
      for (int c = 0; c < NC; ++c) {
        bf16x8 x = qreg[c];
        const float4 r0 = cs4[(8 * c + 4 * g) / 2], r1 = cs4[(8 * c + 4 * g) / 2 + 1];
        const float cv[4] = {r0.x, r0.z, r1.x, r1.z}, sv[4] = {r0.y, r0.w, r1.y, r1.w};
#pragma unroll
        for (int p = 0; p < 4; ++p) {
          float xe = (float)x[2 * p], xo = (float)x[2 * p + 1];
          rope_pair(cv[p], sv[p], xe, xo);
          x[2 * p] = (bf16)xe;
          x[2 * p + 1] = (bf16)xo;
        }
        qreg[c] = x;
      }
      if (a.q_rot && qrow < T) {
        bf16x8* dst = (bf16x8*)(a.q_rot + (bh * T + qrow) * D + 8 * g);
#pragma unroll
        for (int c = 0; c < NC; ++c) dst[2 * c] = qreg[c];
      }
    }
  }

  int kv_lo = 0;
  if (W > 0) kv_lo = max(0, q0 - W + 1);
  const int t_lo = kv_lo / BKV;
  const int kv_hi = min(T, q0 + BQ);
  const int ntiles = (kv_hi + BKV - 1) / BKV - t_lo;

  const bool has_sink = a.sinks != nullptr;
  const float sink2 = has_sink ? a.sinks[h] * kLog2e : 0.f;
  f32x16 oacc[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db)
#pragma unroll
    for (int i = 0; i < 16; ++i) oacc[db][i] = 0.f;
  float m = has_sink ? sink2 : kMaxInit;
  float lsum = (has_sink && g == 0) ? 1.f : 0.f;
  float mxl = -INFINITY;
  const float cexp = CAP ? a.cap_log2e : a.scale_log2e;
  const bool want_max = a.max_logit != nullptr;

  Dma dm;
  dm.init(wave, lane);
  using I0 = std::integral_constant<int, 0>;
  using I1 = std::integral_constant<int, 1>;
  auto kbuf = [&](auto p_c) -> LDS_AS char* {
    return decltype(p_c)::value == 0 ? (LDS_AS char*)kb0 : (LDS_AS char*)kb1;
  };
  auto vbuf = [&](auto p_c) -> LDS_AS char* {
    return decltype(p_c)::value == 0 ? (LDS_AS char*)vb0 : (LDS_AS char*)vb1;
  };

  f32x16 sn[2];   // S of the tile being prepared (two 32-key halves)
  float mt;       // its row max (log2 units), mnew the running max it leads to
  auto zero_s = [&]() __attribute__((always_inline)) {
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int i = 0; i < 16; ++i) sn[t][i] = 0.f;
  };
  LaneOffs<D> lo;
  lo.init(lane);
  auto fK = [&](auto p_c) {
    const LDS_AS char* kt = kbuf(p_c);
    return [=, &lo](int k) { return lds_row_op<D>(kt, lo, k & 1, k >> 1); };
  };
  // cap and mask of the prepared tile's elements [e0, e1) of 32 (e = 16 t
  // + i: half t, accumulator i), folded into its running max mt
  // (key kv is visible to row qrow iff 0 <= qrow - kv < span)
  const unsigned span = W > 0 ? (unsigned)W : 0x7fffffffu;
  auto prep = [&](auto mask_c, int kv0, int e0, int e1) __attribute__((always_inline)) {
    constexpr bool MASK = decltype(mask_c)::value;
    const int base = qrow - kv0 - 4 * g;   // qrow - kv = base - (32 t + 8 (i / 4) + i % 4)
#pragma unroll
    for (int e = e0; e < e1; ++e) {
      const int t = e >> 4, i = e & 15;
      float x = sn[t][i];
      if (CAP) {
        const float ex = fast_exp2(x * a.two_scale_over_cap_log2e);
        x = 1.f - 2.f * __builtin_amdgcn_rcpf(ex + 1.f);
      }
      if (MASK) {
        const bool vis = (unsigned)(base - (32 * t + 8 * (i >> 2) + (i & 3))) < span;
        x = vis ? x : -INFINITY;
      }
      sn[t][i] = x;
      mt = fmaxf(mt, x);
    }
  };
  // the rescale decision for the prepared tile: the running max moves only
  // when some row's tile max passes it by more than the slack
  float mnew, alpha;
  bool resc;
  auto decide = [&]() __attribute__((always_inline)) {
    mt = xor32_max(mt) * cexp;
    if (want_max) mxl = fmaxf(mxl, qrow < T ? mt : -INFINITY);
    resc = __any(mt > m + kRescaleSlack);
    mnew = resc ? fmaxf(m, mt) : m;
    alpha = fast_exp2(m - mnew);
  };
  // P = 2^(x c - mref) of one element, summed into ps
  auto pexp = [&](float x, float mref, float& ps) __attribute__((always_inline)) {
    const float p = fast_exp2(fmaf(x, cexp, -mref));
    ps += p;
    return p;
  };
  // element e (0 .. 15) of a 16-key chunk pair, packed to bf16 as each pair
  // of elements completes (two bf16 per register: no eight-float staging);
  // the chunk's operand is out[e / 8] once element 8 k + 7 is in
  struct Packer {
    float prev;
    uint32_t wd[4];
    __device__ __forceinline__ void put(int e, float p, bf16x8 (&out)[2]) {
      if ((e & 1) == 0) {
        prev = p;
        return;
      }
      typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
      const bf16x2 v = {(bf16)prev, (bf16)p};
      wd[(e & 7) >> 1] = __builtin_bit_cast(uint32_t, v);
      if ((e & 7) == 7) {
        const u32x4 u = {wd[0], wd[1], wd[2], wd[3]};
        out[e >> 3] = __builtin_bit_cast(bf16x8, u);
      }
    }
  };

  // prologue: K(0), V(0), K(1) resident; tile 0's scores, max and the P of
  // its keys 0..31
  dm.load(Kp, T * D * 2, kbuf(I0{}), t_lo * BKV, wave);
  dm.load(Vp, T * D * 2, vbuf(I0{}), t_lo * BKV, wave);
  dm.load(Kp, ntiles > 1 ? T * D * 2 : 0, kbuf(I1{}), (t_lo + 1) * BKV, wave);
  wait_vmem();
  __syncthreads();
  bf16x8 pa[2];          // P of the current tile's keys 0..31 (chunks 0, 1)
  f32x16 sc;             // raw scores of its keys 32..63
  float ps = 0.f;        // row sum of its P so far
  {
    zero_s();
    auto f = fK(I0{});
    MfmaSeq<NSQ, PD> sq;
    sq.start(f);
    sq.run(f, [&](int k) { return qreg[k >> 1]; }, [&](int k) -> f32x16& { return sn[k & 1]; },
           [](int) {});
    mt = -INFINITY;
    prep(std::true_type{}, t_lo * BKV, 0, 32);
    decide();
    if (resc) lsum *= alpha;   // O is still zero
    m = mnew;
    Packer pk;
#pragma unroll
    for (int e = 0; e < 16; ++e) pk.put(e, pexp(sn[0][e], m, ps), pa);
    sc = sn[1];
  }
  lds_barrier();   // every wave is done with K(0) before K(2) loads into its buffer

  // step j (buffers by parity P = j % 2: K(j+1) in kbuf(1-P), V(j) in
  // vbuf(P); K(j+2) loads into kbuf(P), V(j+1) into vbuf(1-P)).  LAST: the
  // final tile (no next tile: its keys 32..63 go under the O block's first
  // half instead).
  auto step = [&](auto p_c, auto mask_c, auto last_c, const int j) __attribute__((always_inline)) {
    constexpr int P = decltype(p_c)::value;
    constexpr bool LAST = decltype(last_c)::value;
    using PN = std::integral_constant<int, 1 - P>;
    lo.refresh();
    bf16x8 pb2[2];   // P of keys 32..63
    Packer pk2;
    auto pchunk_hi = [&](int e) __attribute__((always_inline)) {   // element e of 16
      pk2.put(e, pexp(sc[e], m, ps), pb2);
    };
    auto fV = [&](int k) { return lds_tr_op<D>(vbuf(p_c), lo, k / NDB, k % NDB); };
    MfmaSeq<NPV, PD> vq;
    if constexpr (!LAST) {
      const int n2 = j + 2 < ntiles ? T * D * 2 : 0;
      const int row2 = (t_lo + j + 2) * BKV, row1 = (t_lo + j + 1) * BKV;
      zero_s();
      auto f = fK(PN{});
      MfmaSeq<NSQ, PD> sq;
      sq.start(f);
      sq.run(f, [&](int k) { return qreg[k >> 1]; }, [&](int k) -> f32x16& { return sn[k & 1]; },
             [&](int k) __attribute__((always_inline)) {
               pchunk_hi(k);
               if (k < PER)
                 dm.load_piece(k, Kp, n2, kbuf(p_c), row2, wave);
               else if (k < 2 * PER)
                 dm.load_piece(k - PER, Vp, T * D * 2, vbuf(PN{}), row1, wave);
               if (k == NSQ - PD) vq.start(fV);
             });
    } else {
      vq.start(fV);
    }
    // O^T += V(j)^T P(j)^T; under it, tile j+1's cap, mask, max and the P of
    // its keys 0..31 (or, on the last tile, this tile's keys 32..63)
    const int kv1 = (t_lo + j + 1) * BKV;
    bf16x8 pn[2];
    float psn = 0.f;
    Packer pkn;
    mt = -INFINITY;
    vq.run(fV,
           [&](int k) { return k < 8 ? pa[k >> 2] : pb2[(k >> 2) - 2]; },
           [&](int k) -> f32x16& { return oacc[k % NDB]; },
           [&](int k) __attribute__((always_inline)) {
             if constexpr (LAST) {
               if (k < 8) {
                 pchunk_hi(2 * k);
                 pchunk_hi(2 * k + 1);
               }
             } else {
               if (k >= 1 && k <= 4) prep(mask_c, kv1, 8 * (k - 1), 8 * k);
               if (k == 5) decide();
               if (k >= KE0) {
                 // keys 0..31 (half 0), elements spread over hooks KE0 .. 15
                 constexpr int NH = 16 - KE0;
#pragma unroll
                 for (int e = 16 * (k - KE0) / NH; e < 16 * (k - KE0 + 1) / NH; ++e)
                   pkn.put(e, pexp(sn[0][e], mnew, psn), pn);
               }
             }
           });
    lsum += ps;
    if constexpr (!LAST) {
      if (resc) {
        lsum *= alpha;
#pragma unroll
        for (int db = 0; db < NDB; ++db)
#pragma unroll
          for (int i = 0; i < 16; ++i) oacc[db][i] *= alpha;
      }
      m = mnew;
      ps = psn;
      pa[0] = pn[0];
      pa[1] = pn[1];
      sc = sn[1];
      wait_vmem();
      lds_barrier();
    }
  };
  // per-wave range of tiles every row sees whole: [tb, ta]
  const int qa = qw0, qb = qw0 + 31;
  const int ta = qa >= BKV - 1 ? (qa - (BKV - 1)) / BKV - t_lo : -1;
  const int tb = (W > 0 && qb - W >= 0) ? (qb - W) / BKV + 1 - t_lo : 0;
  // step j prepares tile j + 1: steps [ja, jb) carry no mask
  const int jl = ntiles - 1;
  const int ja = min(jl, max(0, tb - 1));
  const int jb = min(jl, max(ja, ta));
  using MT = std::true_type;
  using MF = std::false_type;
  int j = 0;
  // a segment of steps [j, jend): unrolled by two so that every buffer is a
  // compile-time choice (a run-time parity branch around the steps makes the
  // compiler hold two copies of the state, and it spills), an odd first step
  // peeled
  auto run = [&](auto mask_c, const int jend) __attribute__((always_inline)) {
    if ((j & 1) && j < jend) {
      step(I1{}, mask_c, MF{}, j);
      ++j;
    }
    for (; j + 1 < jend; j += 2) {
      step(I0{}, mask_c, MF{}, j);
      step(I1{}, mask_c, MF{}, j + 1);
    }
    if (j < jend) {
      step(I0{}, mask_c, MF{}, j);
      ++j;
    }
  };
  run(MT{}, ja);
  run(MF{}, jb);
  run(MT{}, jl);
  if (jl & 1)
    step(I1{}, MT{}, MT{}, jl);
  else
    step(I0{}, MT{}, MT{}, jl);

  if (want_max) {
    float v = mxl;
#pragma unroll
    for (int off = 1; off < 32; off <<= 1) v = fmaxf(v, __shfl_xor(v, off));
    if (lane == 0 && v > -INFINITY) atomic_max_f32(a.max_logit + bh, v * kLn2);
  }
  const float ltot = xor32_sum(lsum);
  if (qrow < T) {
    const float inv = 1.f / ltot;
    bf16* Op = a.o + (bh * T + qrow) * D;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int i4 = 0; i4 < 4; ++i4) {
        bf16x4 v;
#pragma unroll
        for (int e = 0; e < 4; ++e) v[e] = (bf16)(oacc[db][4 * i4 + e] * inv);
        *(bf16x4*)(Op + 32 * db + 8 * i4 + 4 * g) = v;
      }
    if (g == 0) a.lse[bh * T + qrow] = (m + __log2f(ltot)) * kLn2;
  }
}

// Software-pipelined forward (one wave per 32 query rows holding the whole
// head, the key range walked in 32-key units).  Per unit i the wave issues
// two MFMA blocks and puts the softmax VALU of the *other* unit under each:
//   S(i+1) = K(i+1) Q^T  (D/16 MFMAs)  carrying  exp2, row sum, bf16 pack of P(i)
//   O^T += V(i)^T P(i)^T (2 D/32 MFMAs) carrying  cap tanh, mask, row max of S(i+1)
// so the matrix core always has the next product while the VALU works on a
// unit that no MFMA in flight touches.  The online-softmax rescale of O
// that unit i+1's max may require is applied after the O^T block (O is not
// being accumulated then); the running sum is rescaled with it.  Unit i+1's
// K tile and unit i's V tile are read in iteration i, so K(i+2) and V(i+1)
// are loaded during it into the buffers that K(i) and V(i-1) left: both are
// double-buffered, one barrier per unit.  Head size 256 runs one wave per
// SIMD (the 32 x 256 accumulator lives in the accumulation registers, q in
// 64 VGPRs); head size 128 fits two.
//
// With the cap every logit lies in [-cap, cap], so the softmax needs no
// running max: the reference m = cap log2(e) - 64 keeps every p = 2^(s - m)
// in [2^-80, 2^64], inside the normal range of fp32 and bf16 (a sink above
// that reference becomes the reference).  The cap path therefore never
// rescales, and tracks the max only for the max-logit output (MAXL).
template <int D, bool CAP, bool MAXL>
__global__ __launch_bounds__(256, D >= 256 ? 1 : 2) void fa_fwd_pipe_kernel(FwdArgs a) {
  constexpr bool TRACK = !CAP || MAXL;   // the unit max is computed
  constexpr int NW = 4, BQ = 32 * NW, BKV = 32;
  // a tile image, rounded up to whole rounds of the loaders' 1 KB pieces
  constexpr int TILE = TileDma<D, BKV, NW>::IMG;
  constexpr int NC = D / 16;     // 16-wide chunks of the q.k contraction
  constexpr int NDB = D / 32;    // 32-wide blocks of the output
  constexpr int NO = 2 * NDB;    // MFMAs of the O^T block
  constexpr int PD = kFwdPipePD; // LDS operands issued this many MFMAs ahead
  // head size 256: O (32 x 256 fp32 = 128 registers per lane) stays in the
  // AGPRs, beside q (64 VGPRs) and the working set in the VGPRs
  constexpr bool AGPR_O = D >= 256;
  __shared__ __attribute__((aligned(1024))) char kb0[TILE];
  __shared__ __attribute__((aligned(1024))) char kb1[TILE];
  __shared__ __attribute__((aligned(1024))) char vb0[TILE];
  __shared__ __attribute__((aligned(1024))) char vb1[TILE];

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
  const size_t bh = (size_t)w.b * a.H + h;
  const size_t bkv = (size_t)w.b * a.Hkv + w.hkv;
  const bf16* Kp = a.k + bkv * T * D;
  const bf16* Vp = a.v + bkv * T * D;

  // q as the B operand of S^T = K Q^T: lane holds q[qrow][16c + 8g .. +7]
  bf16x8 qreg[NC];
  {
    const int qr = min(qrow, T - 1);
    const bf16x8* src = (const bf16x8*)(a.q + (bh * T + qr) * D + 8 * g);
#pragma unroll
    for (int c = 0; c < NC; ++c) qreg[c] = src[2 * c];
    if (a.rope_cs) {
      // RoPE fused into the load: chunk c holds the pairs 8c + 4g + p
      const float4* cs4 = (const float4*)(a.rope_cs + (size_t)qr * D);
#pragma unroll
      for (int c = 0; c < NC; ++c) {
        bf16x8 x = qreg[c];
        const float4 r0 = cs4[(8 * c + 4 * g) / 2], r1 = cs4[(8 * c + 4 * g) / 2 + 1];
        const float cv[4] = {r0.x, r0.z, r1.x, r1.z}, sv[4] = {r0.y, r0.w, r1.y, r1.w};
#pragma unroll
        for (int p = 0; p < 4; ++p) {
          float xe = (float)x[2 * p], xo = (float)x[2 * p + 1];
          rope_pair(cv[p], sv[p], xe, xo);
          x[2 * p] = (bf16)xe;
          x[2 * p + 1] = (bf16)xo;
        }
        qreg[c] = x;
      }
      if (a.q_rot && qrow < T) {
        bf16x8* dst = (bf16x8*)(a.q_rot + (bh * T + qrow) * D + 8 * g);
#pragma unroll
        for (int c = 0; c < NC; ++c) dst[2 * c] = qreg[c];
      }
    }
  }

  int kv_lo = 0;
  if (W > 0) kv_lo = max(0, q0 - W + 1);
  const int t_lo = kv_lo / BKV;
  const int kv_hi = min(T, q0 + BQ);
  const int nu = (kv_hi + BKV - 1) / BKV - t_lo;   // units of the workgroup

  const bool has_sink = a.sinks != nullptr;
  const float sink2 = has_sink ? a.sinks[h] * kLog2e : 0.f;
  f32x16 oacc[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db)
#pragma unroll
    for (int i = 0; i < 16; ++i) oacc[db][i] = 0.f;
  const float cexp = CAP ? a.cap_log2e : a.scale_log2e;
  float m, lsum;
  if (CAP) {
    m = has_sink ? fmaxf(cexp - 64.f, sink2) : cexp - 64.f;
    lsum = (has_sink && g == 0) ? fast_exp2(sink2 - m) : 0.f;
  } else {
    m = has_sink ? sink2 : kMaxInit;
    lsum = (has_sink && g == 0) ? 1.f : 0.f;
  }
  float mxl = -INFINITY;

  TileDma<D, BKV, NW> dm;
  dm.init(wave, lane);
  using I0 = std::integral_constant<int, 0>;
  using I1 = std::integral_constant<int, 1>;
  auto kbuf = [&](auto p_c) -> LDS_AS char* {
    return decltype(p_c)::value ? (LDS_AS char*)kb1 : (LDS_AS char*)kb0;
  };
  auto vbuf = [&](auto p_c) -> LDS_AS char* {
    return decltype(p_c)::value ? (LDS_AS char*)vb1 : (LDS_AS char*)vb0;
  };
  // per-lane parts of the LDS operand addresses (the rest are immediates)
  LaneOffs<D> lo;
  lo.init(lane);
  // keys visible to this lane's row: qrow - span < key <= qrow.  Units of
  // the workgroup's range that hold none of a wave's keys (at most a few
  // per wave: near the diagonal, at the window's start) are computed
  // anyway, fully masked: they add exact zeros, and every wave runs the
  // same straight-line schedule.
  const unsigned span = W > 0 ? (unsigned)W : 0x7fffffffu;

  // the two score tiles (unit parity)
  f32x16 sa[2];
  float mt = CAP ? INFINITY : -INFINITY;   // running max (cap: min r) of the unit being prepared
  float ps = 0.f;              // row sum of the unit being exponentiated
  bf16x8 pb[2];                // P of the current unit, bf16, per 16-key chunk

  // S(u) into sa[X] (+ sb[X]), hook(k) after MFMA k
  auto s_block = [&](auto x_c, const LDS_AS char* Kt, auto&& hook) __attribute__((always_inline)) {
    constexpr int X = decltype(x_c)::value;
#pragma unroll
    for (int i = 0; i < 16; ++i) sa[X][i] = 0.f;
    auto fS = [&](int k) { return lds_row_op<D>(Kt, lo, 0, k); };
    MfmaSeq<NC, PD> sq;
    sq.start(fS);
    sq.run(fS, [&](int k) { return qreg[k]; }, [&](int) -> f32x16& { return sa[X]; }, hook);
  };
  // softmax part A of the unit in tile X: score elements [e0, e1) -- the
  // partial sums added, cap, mask -- and their running max
  // softmax part A of the unit in tile X: score elements [e0, e1) -- cap,
  // visibility mask (branch-free, every unit) -- and their running max.
  // Element i of the tile is key kv0 + acc_row(i, g); it is visible iff
  // 0 <= qrow - key < span (span = W, or everything for a causal layer)
  // With the cap the tile keeps r = 1 / (e^(2y) + 1) instead of tanh(y) =
  // 1 - 2r: the "1 - 2r" folds into part B's exponent FMA, and the running
  // max of tanh is the running min of r (masked keys: r = +inf).  Units that
  // no row of the wave sees partially (MASK false) skip the mask.
  auto part_a = [&](auto x_c, auto mask_c, int u, int e0, int e1) __attribute__((always_inline)) {
    constexpr int X = decltype(x_c)::value;
    constexpr bool MASK = decltype(mask_c)::value;
    const int base = qrow - (t_lo + u) * BKV - 4 * g;   // qrow - key for acc_row(i, g) = 4g
#pragma unroll
    for (int i = e0; i < e1; ++i) {
      float x = sa[X][i];
      if (CAP) x = __builtin_amdgcn_rcpf(fast_exp2(x * a.two_scale_over_cap_log2e) + 1.f);
      if (MASK) {
        const bool vis = (unsigned)(base - (8 * (i >> 2) + (i & 3))) < span;
        x = vis ? x : (CAP ? INFINITY : -INFINITY);
      }
      sa[X][i] = x;
      if (TRACK) mt = CAP ? fminf(mt, x) : fmaxf(mt, x);
    }
  };
  // the unit's max across the lane pair, then (after the O^T block that
  // precedes it) the lazy rescale of O and l
  auto a_tail = [&]() __attribute__((always_inline)) {
    if (!TRACK) return;
    if (CAP)
      mt = cexp - 2.f * cexp * xor32_min(mt);   // cexp * tanh at the row's min r
    else
      mt = xor32_max(mt) * cexp;
    if (a.max_logit) mxl = fmaxf(mxl, qrow < T ? mt : -INFINITY);
  };
  auto rescale = [&]() __attribute__((always_inline)) {
    if (CAP) {   // fixed reference: nothing to rescale
      mt = INFINITY;
      return;
    }
    if (__any(mt > m + kRescaleSlack)) {
      if constexpr (AGPR_O) agpr_acc_fence(oacc);
      const float mnew = fmaxf(m, mt);
      const float alpha = fast_exp2(m - mnew);
      m = mnew;
      lsum *= alpha;
#pragma unroll
      for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int i = 0; i < 16; ++i) oacc[db][i] *= alpha;
    }
    mt = CAP ? INFINITY : -INFINITY;
  };
  // softmax part B of the unit in tile X: p = 2^(s c - m) for elements
  // [e0, e1), row sum, bf16 packs of the 16-key chunks as they complete
  auto part_b = [&](auto x_c, int e0, int e1) __attribute__((always_inline)) {
    constexpr int X = decltype(x_c)::value;
    // cap: c tanh - m = c (1 - 2r) - m
    const float f_mul = CAP ? -2.f * cexp : cexp, f_add = CAP ? cexp - m : -m;
#pragma unroll
    for (int i = e0; i < e1; ++i) {
      const float p = fast_exp2(fmaf(sa[X][i], f_mul, f_add));
      sa[X][i] = p;
      ps += p;
      if (i == 7 || i == 15) {
        float tmp[8];
#pragma unroll
        for (int jj = 0; jj < 8; ++jj) tmp[jj] = sa[X][i - 7 + jj];
        pb[i >> 3] = pack_bf16(tmp);
      }
    }
  };
  auto b_tail = [&]() __attribute__((always_inline)) {
    lsum += ps;
    ps = 0.f;
  };
  // O^T += V^T P^T for the unit whose P is in pb, hook(k) after MFMA k
  auto o_block = [&](const LDS_AS char* Vt, auto&& hook) __attribute__((always_inline)) {
    auto fV = [&](int k) { return lds_tr_op<D>(Vt, lo, k / NDB, k % NDB); };
    if constexpr (AGPR_O) {
      // the ring of MfmaSeq, with the accumulator pinned to the AGPRs
      constexpr int R = PD + 1;
      bf16x8 op[R];
#pragma unroll
      for (int k = 0; k < PD; ++k) op[k] = fV(k);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int k = 0; k < NO; ++k) {
        if (k + PD < NO) op[(k + PD) % R] = fV(k + PD);
        mfma32_agpr(oacc[k % NDB], op[k % R], pb[k / NDB]);
        hook(k);
        __builtin_amdgcn_sched_barrier(0);
      }
    } else {
      MfmaSeq<NO, PD> vq;
      vq.start(fV);
      vq.run(fV, [&](int k) { return pb[k / NDB]; },
             [&](int k) -> f32x16& { return oacc[k % NDB]; }, hook);
    }
  };

  // prologue: K(0), V(0), K(1) resident; S(0) and its part A
  dm.load(Kp, T * D * 2, kbuf(I0{}), t_lo * BKV, wave);
  dm.load(Vp, T * D * 2, vbuf(I0{}), t_lo * BKV, wave);
  if (nu > 1) dm.load(Kp, T * D * 2, kbuf(I1{}), (t_lo + 1) * BKV, wave);
  wait_vmem();
  __syncthreads();
  using MT = std::true_type;
  using MF = std::false_type;
  s_block(I0{}, kbuf(I0{}), [&](int) {});
  part_a(I0{}, MT{}, 0, 0, 16);
  a_tail();
  rescale();
  __syncthreads();   // every wave is done with K(0) before K(2) replaces it

  // iteration i: tiles K(i+1) in kbuf[(i+1)&1], V(i) in vbuf[i&1]; score
  // tile of unit i in sa[i&1], of unit i+1 in sa[(i+1)&1]
  // MASK: some row of the wave sees only part of unit i + 1 (its part A
  // evaluates the mask)
  auto step = [&](auto p_c, auto more_c, auto mask_c, const int i) __attribute__((always_inline)) {
    constexpr int P = decltype(p_c)::value;
    constexpr bool more = decltype(more_c)::value;   // a unit i + 1 exists
    using PN = std::integral_constant<int, 1 - P>;
    lo.refresh();   // addresses formed per step, not hoisted for every buffer
    constexpr int EP = 16 / NC > 0 ? 16 / NC : 1;   // elements per S MFMA
    constexpr int EA = 16 / NO > 0 ? 16 / NO : 1;   // elements per O MFMA
    constexpr int PER = TileDma<D, BKV, NW>::PER;
    static_assert(2 * PER <= NC, "one load per S MFMA");
    if constexpr (more) {
      // S(i+1) with P(i)'s exponentials under its MFMAs, and one load of
      // K(i+2) or V(i+1) after each of the first 2 PER.  K(i+2) is loaded
      // even past the last unit (rows past the end read as zeros): its
      // buffer is then never read again.
      s_block(PN{}, kbuf(PN{}), [&](int k) __attribute__((always_inline)) {
        if (k * EP < 16) part_b(p_c, k * EP, k * EP + EP);
        if (k < PER)
          dm.load_piece(k, Kp, T * D * 2, kbuf(p_c), (t_lo + i + 2) * BKV, wave);
        else if (k < 2 * PER)
          dm.load_piece(k - PER, Vp, T * D * 2, vbuf(PN{}), (t_lo + i + 1) * BKV, wave);
      });
      if (16 / NC == 0) part_b(p_c, 0, 16);
      b_tail();
      // O^T += V(i)^T P(i)^T with S(i+1)'s cap, mask and max under its MFMAs
      o_block(vbuf(p_c), [&](int k) __attribute__((always_inline)) {
        if (k * EA < 16) part_a(PN{}, mask_c, i + 1, k * EA, k * EA + EA);
      });
      if (16 / NO == 0) part_a(PN{}, mask_c, i + 1, 0, 16);
      a_tail();
      rescale();
      wait_vmem();
      __syncthreads();
    } else {
      part_b(p_c, 0, 16);
      b_tail();
      o_block(vbuf(p_c), [&](int) {});
      // The last step runs in one of two parity branches, and their join
      // may copy the accumulator between AGPRs: copies the compiler places
      // right after the last MFMA, whose latency it does not see.  The wait
      // comes first, inside the branch.
      if constexpr (AGPR_O) agpr_acc_fence(oacc);
    }
  };
  using T1 = std::true_type;
  using F1 = std::false_type;
  // The units every row of the wave sees whole form one range [mlo, mhi):
  // below it the window's first keys, above it the diagonal and the units
  // past it.  Steps 0 .. nu-2 run in three segments -- mask, no mask, mask --
  // so that the straight-line steps of the long middle segment carry no mask
  // arithmetic; every wave still passes one barrier per step.
  const int mhi = qw0 / BKV - t_lo;   // first unit holding a key past row qw0
  // first unit whose keys are all above qw0 + 31 - W (every key counts when
  // that bound is negative)
  const int wlo = qw0 + 31 - W;
  const int mlo = (W > 0 && wlo >= 0) ? max(0, wlo / BKV + 1 - t_lo) : 0;
  const int ia = min(max(mlo - 1, 0), nu - 1);
  const int ib = min(max(mhi - 1, ia), nu - 1);
  // steps [i, iend) with the buffer parity of each step index
  auto run = [&](auto mask_c, int& i, const int iend) __attribute__((always_inline)) {
    if (i < iend && (i & 1)) {
      step(I1{}, T1{}, mask_c, i);
      ++i;
    }
    for (; i + 2 <= iend; i += 2) {
      step(I0{}, T1{}, mask_c, i);
      step(I1{}, T1{}, mask_c, i + 1);
    }
    if (i < iend) {
      step(I0{}, T1{}, mask_c, i);
      ++i;
    }
  };
  int i = 0;
  for (int seg = 0; seg < 3; ++seg) {
    const int iend = seg == 0 ? ia : seg == 1 ? ib : nu - 1;
    if (seg == 1)
      run(MF{}, i, iend);
    else
      run(MT{}, i, iend);
  }
  if ((nu - 1) & 1)
    step(I1{}, F1{}, MT{}, nu - 1);
  else
    step(I0{}, F1{}, MT{}, nu - 1);

  if (a.max_logit) {
    float v = mxl;
#pragma unroll
    for (int off = 1; off < 32; off <<= 1) v = fmaxf(v, __shfl_xor(v, off));
    if (lane == 0 && v > -INFINITY) atomic_max_f32(a.max_logit + bh, v * kLn2);
  }
  const float ltot = xor32_sum(lsum);
  // (the last step has waited for the accumulator's last MFMAs)
  if (qrow < T) {
    const float inv = 1.f / ltot;
    bf16* Op = a.o + (bh * T + qrow) * D;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int i4 = 0; i4 < 4; ++i4) {
        bf16x4 v;
#pragma unroll
        for (int e = 0; e < 4; ++e) v[e] = (bf16)(oacc[db][4 * i4 + e] * inv);
        *(bf16x4*)(Op + 32 * db + 8 * i4 + 4 * g) = v;
      }
    if (g == 0) a.lse[bh * T + qrow] = (m + __log2f(ltot)) * kLn2;
  }
}

// Tile shape of the one-tile kernel at d = 192/128 (keys per tile, waves),
// chosen by measurement on MI355X.

template <int DK, int DV, int BKV, int NW, int NSTG = 2, int MINWG = 0>
static hipError_t launch_fwd_d(const FwdArgs& a, hipStream_t stream) {
  const int nqb = (a.T + 32 * NW - 1) / (32 * NW);
  const dim3 grid((unsigned)nqb * a.B * a.H);
  if (a.cap_log2e > 0.f)
    hipLaunchKernelGGL((fa_fwd_kernel<DK, DV, BKV, NW, true, NSTG, MINWG>), grid, dim3(64 * NW), 0, stream,
                       a);
  else
    hipLaunchKernelGGL((fa_fwd_kernel<DK, DV, BKV, NW, false, NSTG, MINWG>), grid, dim3(64 * NW), 0, stream,
                       a);
  stage_mark(stream);
  return hipGetLastError();
}

template <int D>
static hipError_t launch_fwd_pipe(const FwdArgs& a, hipStream_t stream) {
  const int nqb = (a.T + 127) / 128;
  const dim3 grid((unsigned)nqb * a.B * a.H);
  if (a.cap_log2e > 0.f) {
    if (a.max_logit)
      hipLaunchKernelGGL((fa_fwd_pipe_kernel<D, true, true>), grid, dim3(256), 0, stream, a);
    else
      hipLaunchKernelGGL((fa_fwd_pipe_kernel<D, true, false>), grid, dim3(256), 0, stream, a);
  } else {
    hipLaunchKernelGGL((fa_fwd_pipe_kernel<D, false, true>), grid, dim3(256), 0, stream, a);
  }
  stage_mark(stream);
  return hipGetLastError();
}

__global__ void fill_f32_kernel(float* p, int n, float v) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = v;
}

hipError_t launch_fill_f32(float* p, int n, float v, hipStream_t stream) {
  hipLaunchKernelGGL(fill_f32_kernel, dim3((n + 255) / 256), dim3(256), 0, stream, p, n, v);
  return hipGetLastError();
}

static hipError_t launch_fwd_sp(const FwdArgs& a, hipStream_t stream) {
  const int nqb = (a.T + 127) / 128;
  const dim3 grid((unsigned)nqb * a.B * a.H);
  if (a.cap_log2e > 0.f)
    hipLaunchKernelGGL(fa_fwd_sp_kernel<true>, grid, dim3(256), 0, stream, a);
  else
    hipLaunchKernelGGL(fa_fwd_sp_kernel<false>, grid, dim3(256), 0, stream, a);
  stage_mark(stream);
  return hipGetLastError();
}


hipError_t launch_fwd_bf16(const FwdArgs& a, int d, int d_v, hipStream_t stream) {
  if (d == d_v) {
    switch (d) {
      case 64: return launch_fwd_d<64, 64, 64, 4>(a, stream);
      // the software-pipelined two-wave kernel (mistral forward 1.64 -> 1.59
      // ms, qwen25 0.329 -> 0.314 ms against fa_fwd_kernel at 64-key tiles)
      case 128: return launch_fwd_sp(a, stream);
      // one wave cannot hold q, the 256-wide O accumulator and a tile of
      // scores at two waves per SIMD: the software-pipelined kernel keeps
      // the matrix unit busy at one
      case 256: return launch_fwd_pipe<256>(a, stream);
    }
  } else if (d == 192 && d_v == 128) {
    return launch_fwd_d<192, 128, 32, 4>(a, stream);
  }
  return hipErrorInvalidValue;
}

}  // namespace fa
