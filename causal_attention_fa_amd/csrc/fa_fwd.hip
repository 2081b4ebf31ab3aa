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
#include <type_traits>

#include "device_common.h"
#include "internal.h"

namespace fa {


// QW query blocks of 32 rows per wave: each K or V operand read from LDS
// feeds QW MFMAs, dividing the LDS traffic per flop by QW.  DK is the head
// size of q and k, DV that of v and o (equal except for MLA-style heads).
template <int DK, int DV, int BKV, int NW, int QW, bool CAP>
__global__ __launch_bounds__(64 * NW, (DK >= 256 || QW > 1 ? 1 : 8 / NW)) void fa_fwd_kernel(
    FwdArgs a) {
  constexpr int NT = 64 * NW;         // threads per workgroup
  constexpr int RW = 32 * QW;         // query rows per wave
  constexpr int BQ = RW * NW;         // query rows per workgroup
  constexpr int TILE_K = Lay<DK>::template bytes<BKV>();  // one K tile
  constexpr int TILE_V = Lay<DV>::template bytes<BKV>();  // one V tile
  constexpr int NDB = DV / 32;        // 32-wide blocks of the output
  constexpr int NS = BKV / 32;        // 32-key sub-tiles
  constexpr int NC = DK / 16;         // 16-wide chunks of the q.k contraction
  // one LDS object per buffer: the compiler can then tell the buffer being
  // filled by direct loads from the one being read, and does not make the
  // reads wait for the loads
  __shared__ __attribute__((aligned(1024))) char kb0[TILE_K];
  __shared__ __attribute__((aligned(1024))) char kb1[TILE_K];
  __shared__ __attribute__((aligned(1024))) char vb0[TILE_V];
  __shared__ __attribute__((aligned(1024))) char vb1[TILE_V];

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
  const int qw0 = q0 + RW * wave;
  const size_t bh = (size_t)w.b * a.H + h;
  const size_t bkv = (size_t)w.b * a.Hkv + w.hkv;
  const bf16* Kp = a.k + bkv * T * DK;
  const bf16* Vp = a.v + bkv * T * DV;

  // Q as the B operand of S^T = K Q^T: lane holds Q[qrow][16c + 8g .. +7]
  // of its row in each of the wave's QW blocks.
  bf16x8 qreg[QW][NC];
#pragma unroll
  for (int u = 0; u < QW; ++u) {
    const int qr = min(qw0 + 32 * u + l32, T - 1);
    const bf16x8* src = (const bf16x8*)(a.q + (bh * T + qr) * DK + 8 * g);
#pragma unroll
    for (int c = 0; c < NC; ++c) qreg[u][c] = src[2 * c];
  }
  // RoPE fused into the Q load: this lane's 8-element chunks hold the pairs
  // 8c + 4g + p of its row (position = row index), whose (cos, sin) come from
  // the call's table; the rotated row is optionally written out once for the
  // backward.
  if (a.rope_cs) {
#pragma unroll
    for (int u = 0; u < QW; ++u) {
      const int qrow = qw0 + 32 * u + l32;
      const float4* cs4 = (const float4*)(a.rope_cs + (size_t)min(qrow, T - 1) * DK);
#pragma unroll
      for (int c = 0; c < NC; ++c) {
        bf16x8 x = qreg[u][c];
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
        qreg[u][c] = x;
      }
      if (a.q_rot && qrow < T) {
        bf16x8* dst = (bf16x8*)(a.q_rot + (bh * T + qrow) * DK + 8 * g);
#pragma unroll
        for (int c = 0; c < NC; ++c) dst[2 * c] = qreg[u][c];
      }
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
  f32x16 oacc[QW][NDB];
  float m[QW], lsum[QW], mxl[QW];
#pragma unroll
  for (int u = 0; u < QW; ++u) {
    m[u] = has_sink ? sink2 : kMaxInit;
    lsum[u] = (has_sink && g == 0) ? 1.f : 0.f;
    mxl[u] = -INFINITY;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int i = 0; i < 16; ++i) oacc[u][db][i] = 0.f;
  }

  // K, V tiles go straight from HBM to the idle LDS buffers (no staging
  // registers): issued at the top of an iteration, waited for before its
  // closing barrier
  TileDma<DK, BKV, NW> kdm;
  TileDma<DV, BKV, NW> vdm;
  kdm.init(wave, lane);
  vdm.init(wave, lane);
  auto kbuf = [&](auto p_c) -> LDS_AS char* {
    return decltype(p_c)::value ? (LDS_AS char*)kb1 : (LDS_AS char*)kb0;
  };
  auto vbuf = [&](auto p_c) -> LDS_AS char* {
    return decltype(p_c)::value ? (LDS_AS char*)vb1 : (LDS_AS char*)vb0;
  };
  using I0 = std::integral_constant<int, 0>;
  using I1 = std::integral_constant<int, 1>;
  kdm.load(Kp, T * DK * 2, kbuf(I0{}), t_lo * BKV, wave);
  vdm.load(Vp, T * DV * 2, vbuf(I0{}), t_lo * BKV, wave);
  wait_vmem();
  __syncthreads();

  const int qa = qw0, qb = qw0 + RW - 1;
  // one iteration on the tile in buffer P (the loop is unrolled by two so
  // that the buffers are compile-time choices)
  auto step = [&](auto p_c, const int j) __attribute__((always_inline)) {
    constexpr int P = decltype(p_c)::value;
    using PN = std::integral_constant<int, 1 - P>;
    const LDS_AS char* Kt = kbuf(p_c);
    const LDS_AS char* Vt = vbuf(p_c);
    const bool more = j + 1 < ntiles;
    // next K and V tiles into the idle buffers: their latency hides behind
    // this iteration
    if (more) {
      kdm.load(Kp, T * DK * 2, kbuf(PN{}), (t_lo + j + 1) * BKV, wave);
      vdm.load(Vp, T * DV * 2, vbuf(PN{}), (t_lo + j + 1) * BKV, wave);
    }
    const int kv0 = (t_lo + j) * BKV;
    const bool empty = qa >= T || kv0 > qb || (W > 0 && kv0 + BKV - 1 <= qa - W);
    const bool full = kv0 + BKV - 1 <= qa && (W == 0 || kv0 > qb - W);
    if (!empty) {
      // S^T = K Q^T for every query block; each K operand feeds QW MFMAs and
      // the next chunk's operands are requested before this chunk's MFMAs.
      f32x16 s[QW][NS];
      {
        bf16x8 op[2][NS];
#pragma unroll
        for (int t = 0; t < NS; ++t) {
          op[0][t] = lds_row_operand<DK>(Kt, 32 * t, 0, lane);
#pragma unroll
          for (int u = 0; u < QW; ++u)
#pragma unroll
            for (int i = 0; i < 16; ++i) s[u][t][i] = 0.f;
        }
#pragma unroll
        for (int c = 0; c < NC; ++c) {
          if (c + 1 < NC) {
#pragma unroll
            for (int t = 0; t < NS; ++t) op[(c + 1) & 1][t] = lds_row_operand<DK>(Kt, 32 * t, c + 1, lane);
          }
#pragma unroll
          for (int t = 0; t < NS; ++t)
#pragma unroll
            for (int u = 0; u < QW; ++u) s[u][t] = mfma32(op[c & 1][t], qreg[u][c], s[u][t]);
        }
      }
      // The exponent's FMA carries the constant: scale*log2(e) on raw scores
      // without a cap, cap*log2(e) on tanh(scale*x/cap) with one (the max
      // scales with it either way).
      const float cexp = CAP ? a.cap_log2e : a.scale_log2e;
      bf16x8 pb[QW][BKV / 16];
#pragma unroll
      for (int u = 0; u < QW; ++u) {
        const int qrow = qw0 + 32 * u + l32;
        if (CAP) {
#pragma unroll
          for (int t = 0; t < NS; ++t)
#pragma unroll
            for (int i = 0; i < 16; ++i) {
              // cap * tanh(scale*x / cap) * log2(e)
              const float e = fast_exp2(s[u][t][i] * a.two_scale_over_cap_log2e);
              s[u][t][i] = 1.f - 2.f * __builtin_amdgcn_rcpf(e + 1.f);  // tanh
            }
        }
        if (!full) {
#pragma unroll
          for (int t = 0; t < NS; ++t)
#pragma unroll
            for (int i = 0; i < 16; ++i) {
              const int kv = kv0 + 32 * t + acc_row(i, g);
              const bool vis = (kv <= qrow) & ((W == 0) | (kv > qrow - W));
              s[u][t][i] = vis ? s[u][t][i] : -INFINITY;
            }
        }
        float mt = -INFINITY;
#pragma unroll
        for (int t = 0; t < NS; ++t)
#pragma unroll
          for (int i = 0; i < 16; ++i) mt = fmaxf(mt, s[u][t][i]);
        mt = xor32_max(mt) * cexp;
        if (a.max_logit) mxl[u] = fmaxf(mxl[u], qrow < T ? mt : -INFINITY);
        // Lazy rescaling: the running max only moves (and O, l are rescaled)
        // when some row's tile max exceeds it by more than kRescaleSlack, so
        // p = 2^(s - m) stays below 2^kRescaleSlack; the branch is uniform.
        if (__any(mt > m[u] + kRescaleSlack)) {
          const float mnew = fmaxf(m[u], mt);
          const float alpha = fast_exp2(m[u] - mnew);
          m[u] = mnew;
          lsum[u] *= alpha;
#pragma unroll
          for (int db = 0; db < NDB; ++db)
#pragma unroll
            for (int i = 0; i < 16; ++i) oacc[u][db][i] *= alpha;
        }
        float ps = 0.f;
#pragma unroll
        for (int t = 0; t < NS; ++t)
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const float p = fast_exp2(fmaf(s[u][t][i], cexp, -m[u]));
            s[u][t][i] = p;
            ps += p;
          }
        lsum[u] += ps;
#pragma unroll
        for (int c16 = 0; c16 < BKV / 16; ++c16) {
          float tmp[8];
#pragma unroll
          for (int jj = 0; jj < 8; ++jj) tmp[jj] = s[u][c16 >> 1][8 * (c16 & 1) + jj];
          pb[u][c16] = pack_bf16(tmp);
        }
      }
      // O^T += V^T P^T: each transposed V operand feeds QW MFMAs.
#pragma unroll
      for (int c16 = 0; c16 < BKV / 16; ++c16)
#pragma unroll
        for (int db = 0; db < NDB; ++db) {
          const bf16x8 vop = lds_tr_operand<DV>(Vt, 0, c16, 32 * db, lane);
#pragma unroll
          for (int u = 0; u < QW; ++u) oacc[u][db] = mfma32(vop, pb[u][c16], oacc[u][db]);
        }
    }
    if (more) wait_vmem();
    __syncthreads();
  };
  int j = 0;
  for (; j + 1 < ntiles; j += 2) {
    step(I0{}, j);
    step(I1{}, j + 1);
  }
  if (j < ntiles) step(I0{}, j);

  if (a.max_logit) {
    // largest logit of the wave's rows (natural log units), one atomic per wave
    float v = -INFINITY;
#pragma unroll
    for (int u = 0; u < QW; ++u) v = fmaxf(v, mxl[u]);
#pragma unroll
    for (int off = 1; off < 32; off <<= 1) v = fmaxf(v, __shfl_xor(v, off));
    if (lane == 0 && v > -INFINITY) atomic_max_f32(a.max_logit + bh, v * kLn2);
  }
#pragma unroll
  for (int u = 0; u < QW; ++u) {
    const int qrow = qw0 + 32 * u + l32;
    const float ltot = xor32_sum(lsum[u]);
    if (qrow < T) {
      const float inv = 1.f / ltot;
      bf16* Op = a.o + (bh * T + qrow) * DV;
#pragma unroll
      for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int i4 = 0; i4 < 4; ++i4) {
          bf16x4 v;
#pragma unroll
          for (int e = 0; e < 4; ++e) v[e] = (bf16)(oacc[u][db][4 * i4 + e] * inv);
          *(bf16x4*)(Op + 32 * db + 8 * i4 + 4 * g) = v;
        }
      if (g == 0) a.lse[bh * T + qrow] = (m[u] + __log2f(ltot)) * kLn2;
    }
  }
}

// Head size 256: one wave cannot hold q and the 256-wide O accumulator at
// two waves per SIMD, and one wave per SIMD leaves
// the matrix pipe idle.  So waves work in pairs on the same 32 query rows:
// wave half hf holds q[:, 128 hf .. +127], computes the partial scores over
// its half of d, and owns output columns 128 hf .. +127.  The pair swaps
// partial scores through LDS (one extra barrier per tile); both then add
// them in the same order, so their scores, softmax state and P are
// identical, and each accumulates its half of O^T += V^T P^T.
template <int D, int BKV, bool CAP>
__global__ __launch_bounds__(512, 1) void fa_fwd_pair_kernel(FwdArgs a) {
  constexpr int NW = 8, NT = 64 * NW;
  constexpr int HD = D / 2;             // columns per wave
  constexpr int BQ = 32 * NW / 2;       // query rows per workgroup
  constexpr int TILE = Lay<D>::template bytes<BKV>();
  constexpr int NDB = HD / 32;          // output blocks per wave
  constexpr int NS = BKV / 32;
  constexpr int NC = HD / 16;           // chunks of the half contraction
  constexpr int XS = NS * 16 * 64 * 4;  // one wave's partial scores (bytes)
  // K, V buffers as separate LDS objects (direct loads into one, reads from
  // the other, without the compiler making the reads wait), the partial
  // score exchange area
  __shared__ __attribute__((aligned(1024))) char kb0[TILE];
  __shared__ __attribute__((aligned(1024))) char kb1[TILE];
  __shared__ __attribute__((aligned(1024))) char vb0[TILE];
  __shared__ __attribute__((aligned(1024))) char vb1[TILE];
  __shared__ __attribute__((aligned(1024))) char xsm[NW * XS];
  LDS_AS float* xsb = (LDS_AS float*)xsm;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int pair = wave >> 1;
  const int hf = wave & 1;
  const int g = lane >> 5;
  const int l32 = lane & 31;
  const int T = a.T;
  const int W = a.window;
  const int G = a.H / a.Hkv;
  const int nqb = (T + BQ - 1) / BQ;
  const WorkItem w = decode_work(blockIdx.x, nqb, a.B, a.Hkv, G, true);
  const int h = w.hkv * G + w.r;
  const int q0 = w.blk * BQ;
  const int qw0 = q0 + 32 * pair;
  const int qrow = qw0 + l32;
  const size_t bh = (size_t)w.b * a.H + h;
  const size_t bkv = (size_t)w.b * a.Hkv + w.hkv;
  const bf16* Kp = a.k + bkv * T * D;
  const bf16* Vp = a.v + bkv * T * D;

  // this wave's half of the q row: chunk c holds columns HD hf + 16c + 8g ..
  bf16x8 qreg[NC];
  {
    const int qr = min(qrow, T - 1);
    const bf16x8* src = (const bf16x8*)(a.q + (bh * T + qr) * D + HD * hf + 8 * g);
#pragma unroll
    for (int c = 0; c < NC; ++c) qreg[c] = src[2 * c];
    if (a.rope_cs) {
      // fused RoPE on this half: chunk c holds pairs HD/2 hf + 8c + 4g + p
      const float4* cs4 = (const float4*)(a.rope_cs + (size_t)qr * D);
#pragma unroll
      for (int c = 0; c < NC; ++c) {
        bf16x8 x = qreg[c];
        const int p0 = HD / 2 * hf + 8 * c + 4 * g;
        const float4 r0 = cs4[p0 / 2], r1 = cs4[p0 / 2 + 1];
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
        bf16x8* dst = (bf16x8*)(a.q_rot + (bh * T + qrow) * D + HD * hf + 8 * g);
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

  TileDma<D, BKV, NW> kdm, vdm;
  kdm.init(wave, lane);
  vdm.init(wave, lane);
  auto kbuf = [&](auto p_c) -> LDS_AS char* {
    return decltype(p_c)::value ? (LDS_AS char*)kb1 : (LDS_AS char*)kb0;
  };
  auto vbuf = [&](auto p_c) -> LDS_AS char* {
    return decltype(p_c)::value ? (LDS_AS char*)vb1 : (LDS_AS char*)vb0;
  };
  using I0 = std::integral_constant<int, 0>;
  using I1 = std::integral_constant<int, 1>;
  kdm.load(Kp, T * D * 2, kbuf(I0{}), t_lo * BKV, wave);
  vdm.load(Vp, T * D * 2, vbuf(I0{}), t_lo * BKV, wave);
  wait_vmem();
  __syncthreads();

  LDS_AS float* const xs_mine = xsb + wave * (XS / 4);
  const LDS_AS float* const xs_peer = xsb + (wave ^ 1) * (XS / 4);
  const int qa = qw0, qb = qw0 + 31;
  // one iteration on the tile in buffer P (unrolled by two)
  auto step = [&](auto p_c, const int j) __attribute__((always_inline)) {
    constexpr int P = decltype(p_c)::value;
    using PN = std::integral_constant<int, 1 - P>;
    const LDS_AS char* Kt = kbuf(p_c);
    const LDS_AS char* Vt = vbuf(p_c);
    const bool more = j + 1 < ntiles;
    if (more) {
      kdm.load(Kp, T * D * 2, kbuf(PN{}), (t_lo + j + 1) * BKV, wave);
      vdm.load(Vp, T * D * 2, vbuf(PN{}), (t_lo + j + 1) * BKV, wave);
    }
    const int kv0 = (t_lo + j) * BKV;
    // the same for both waves of a pair (same rows)
    const bool empty = qa >= T || kv0 > qb || (W > 0 && kv0 + BKV - 1 <= qa - W);
    const bool full = kv0 + BKV - 1 <= qa && (W == 0 || kv0 > qb - W);
    f32x16 s[NS];
    if (!empty) {
      // partial S^T over this wave's half of d (chunks NC*hf .. of the row)
      bf16x8 op[2][NS];
#pragma unroll
      for (int t = 0; t < NS; ++t) {
#pragma unroll
        for (int i = 0; i < 16; ++i) s[t][i] = 0.f;
        op[0][t] = lds_row_operand<D>(Kt, 32 * t, NC * hf, lane);
      }
#pragma unroll
      for (int c = 0; c < NC; ++c) {
        if (c + 1 < NC) {
#pragma unroll
          for (int t = 0; t < NS; ++t)
            op[(c + 1) & 1][t] = lds_row_operand<D>(Kt, 32 * t, NC * hf + c + 1, lane);
        }
#pragma unroll
        for (int t = 0; t < NS; ++t) s[t] = mfma32(op[c & 1][t], qreg[c], s[t]);
      }
#pragma unroll
      for (int t = 0; t < NS; ++t)
#pragma unroll
        for (int i4 = 0; i4 < 4; ++i4)   // lane-major 16-byte groups
          *(LDS_AS f32x4*)(xs_mine + ((t * 4 + i4) * 64 + lane) * 4) =
              f32x4{s[t][4 * i4], s[t][4 * i4 + 1], s[t][4 * i4 + 2], s[t][4 * i4 + 3]};
    }
    __syncthreads();
    if (!empty) {
      // full scores: lower half + upper half, the same order in both waves
#pragma unroll
      for (int t = 0; t < NS; ++t)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const float peer = xs_peer[((t * 4 + i / 4) * 64 + lane) * 4 + i % 4];
          s[t][i] = hf == 0 ? s[t][i] + peer : peer + s[t][i];
        }
      if (CAP) {
#pragma unroll
        for (int t = 0; t < NS; ++t)
#pragma unroll
          for (int i = 0; i < 16; ++i) {
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
      float ps = 0.f;
#pragma unroll
      for (int t = 0; t < NS; ++t)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const float p = fast_exp2(fmaf(s[t][i], cexp, -m));
          s[t][i] = p;
          ps += p;
        }
      lsum += ps;
      bf16x8 pb[BKV / 16];
#pragma unroll
      for (int c16 = 0; c16 < BKV / 16; ++c16) {
        float tmp[8];
#pragma unroll
        for (int jj = 0; jj < 8; ++jj) tmp[jj] = s[c16 >> 1][8 * (c16 & 1) + jj];
        pb[c16] = pack_bf16(tmp);
      }
#pragma unroll
      for (int c16 = 0; c16 < BKV / 16; ++c16)
#pragma unroll
        for (int db = 0; db < NDB; ++db)
          oacc[db] = mfma32(lds_tr_operand<D>(Vt, 0, c16, HD * hf + 32 * db, lane), pb[c16],
                            oacc[db]);
    }
    if (more) wait_vmem();
    __syncthreads();
  };
  int j = 0;
  for (; j + 1 < ntiles; j += 2) {
    step(I0{}, j);
    step(I1{}, j + 1);
  }
  if (j < ntiles) step(I0{}, j);

  if (a.max_logit && hf == 0) {
    float v = mxl;
#pragma unroll
    for (int off = 1; off < 32; off <<= 1) v = fmaxf(v, __shfl_xor(v, off));
    if (lane == 0 && v > -INFINITY) atomic_max_f32(a.max_logit + bh, v * kLn2);
  }
  const float ltot = xor32_sum(lsum);
  if (qrow < T) {
    const float inv = 1.f / ltot;
    bf16* Op = a.o + (bh * T + qrow) * D + HD * hf;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int i4 = 0; i4 < 4; ++i4) {
        bf16x4 v;
#pragma unroll
        for (int e = 0; e < 4; ++e) v[e] = (bf16)(oacc[db][4 * i4 + e] * inv);
        *(bf16x4*)(Op + 32 * db + 8 * i4 + 4 * g) = v;
      }
    if (g == 0 && hf == 0) a.lse[bh * T + qrow] = (m + __log2f(ltot)) * kLn2;
  }
}

// Tile shapes per head size (keys per tile, waves, query blocks per wave),
// chosen by measurement on MI355X.
#ifndef FWD128_CFG
#define FWD128_CFG 64, 4, 1
#endif

#ifndef FWD192_CFG
#define FWD192_CFG 32, 4, 1
#endif

template <int DK, int DV, int BKV, int NW, int QW>
static hipError_t launch_fwd_d(const FwdArgs& a, hipStream_t stream) {
  const int nqb = (a.T + 32 * NW * QW - 1) / (32 * NW * QW);
  const dim3 grid((unsigned)nqb * a.B * a.H);
  if (a.cap_log2e > 0.f)
    hipLaunchKernelGGL((fa_fwd_kernel<DK, DV, BKV, NW, QW, true>), grid, dim3(64 * NW), 0, stream, a);
  else
    hipLaunchKernelGGL((fa_fwd_kernel<DK, DV, BKV, NW, QW, false>), grid, dim3(64 * NW), 0, stream, a);
  stage_mark(stream);
  return hipGetLastError();
}

#ifndef FWD256_BKV
#define FWD256_BKV 32
#endif
// d = 256 forward: paired waves (two per SIMD, each holding half of d), or
// the one-wave-per-row kernel at one wave per SIMD (FWD256_CFG shape)
#ifndef FWD256_PAIR
#define FWD256_PAIR 1
#endif
#ifndef FWD256_CFG
#define FWD256_CFG 64, 4, 1
#endif

template <int D, int BKV>
static hipError_t launch_fwd_pair(const FwdArgs& a, hipStream_t stream) {
  constexpr int BQ = 128;   // 4 pairs x 32 query rows
  const int nqb = (a.T + BQ - 1) / BQ;
  const dim3 grid((unsigned)nqb * a.B * a.H);
  if (a.cap_log2e > 0.f)
    hipLaunchKernelGGL((fa_fwd_pair_kernel<D, BKV, true>), grid, dim3(512), 0, stream, a);
  else
    hipLaunchKernelGGL((fa_fwd_pair_kernel<D, BKV, false>), grid, dim3(512), 0, stream, a);
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

hipError_t launch_fwd_bf16(const FwdArgs& a, int d, int d_v, hipStream_t stream) {
  if (d == d_v) {
    switch (d) {
      case 64: return launch_fwd_d<64, 64, 64, 4, 1>(a, stream);
      case 128: return launch_fwd_d<128, 128, FWD128_CFG>(a, stream);
      case 256:
#if FWD256_PAIR
        return launch_fwd_pair<256, FWD256_BKV>(a, stream);
#else
        return launch_fwd_d<256, 256, FWD256_CFG>(a, stream);
#endif
    }
  } else if (d == 192 && d_v == 128) {
    return launch_fwd_d<192, 128, FWD192_CFG>(a, stream);
  }
  return hipErrorInvalidValue;
}

}  // namespace fa
