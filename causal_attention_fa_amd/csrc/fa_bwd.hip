// Fused causal flash-attention backward for gfx950 (bf16 in, fp32 accumulate).
//
// Gradients of L = sum(o * dO) by recomputation of the probabilities from
// the forward's lse, with the exact softcap derivative 1 - tanh^2 (Forge
// attention.h commit log, "Wave 2"; ARCHITECTURES.md plan wave 2, items 8-9).
//
//   dP = dO V^T,  D_i = <dO_i, o_i>,  dS' = P * (dP - D),
//   dS = dS' * (1 - tanh^2) (softcap),  dq = scale dS K,
//   dk = scale dS^T Q,  dv = P^T dO  (dk, dv summed over the GQA group).
//
// Two launches, deterministic (the only atomics accumulate the attention
// sinks' gradient).  Every pass streams its tiles straight from HBM into
// multi-buffered LDS (direct buffer loads, one tile ahead):
//   1. fa_bwd_dq_kernel -- query-parallel, the forward's structure: each
//      lane owns one query row; S^T = K Q^T and dP^T = V dO^T come out with
//      the query along the lane, so lse, D and the softcap chain are
//      per-lane scalars; dQ^T += K^T dS^T reads K^T through the LDS
//      transpose read.  It also computes D_i for its rows (the backward
//      prologue) and writes it to a [B, H, T] fp32 scratch for the dK/dV
//      pass.  At d = 128 and 256 fa_bwd_dq_pipe_kernel (fa_bwd_pipe.hip)
//      runs one software-pipelined wave per 32 rows.
//   2. fa_bwd_dkdv_pair_kernel -- key-parallel: a workgroup owns 128 key
//      rows (64 at d = 256) of one (b, kv head) and loops over the query
//      heads of the GQA group and over the query tiles that can see its
//      keys (the window bounds the loop).  Each lane owns one key row, and
//      two waves share each 32 rows: one keeps K in registers and computes
//      S, P and dV, the other keeps V and computes dP, dS and dK one tile
//      later from the factor the first leaves in LDS.  dV^T += dO^T P and
//      dK^T += Q^T dS take dO^T and Q^T from the natural tiles through the
//      LDS transpose read.  At d = 128 fa_bwd_kv_pipe_kernel
//      (fa_bwd_pipe.hip) runs instead: one software-pipelined wave per 32
//      keys does both sides' work, with no exchange through LDS.
#include <type_traits>

#include "device_common.h"
#include "internal.h"

namespace fa {

// dQ pass: the K and V tiles of both buffers live in one LDS array (the
// compiler then makes the transposed LDS reads wait for every outstanding
// direct load; that costs overlap but also bounds how far it moves work,
// and so its register use -- chosen by measurement).  Its loop is unrolled
// by two (buffers chosen at compile time), or at d = 192 the buffer is
// picked at run time (fewer registers).
// per head size: K, V tiles double-buffered in one array with the loop
// unrolled by two (not at 192: spills), and how many MFMAs ahead the LDS
// operands are read (192: as needed)
constexpr bool bwd_unroll(int dk) { return dk != 192; }
constexpr int bwd_lds_pd(int dk) { return dk == 192 ? 0 : 2; }

// exp2 argument of P: capped score in the log2 domain minus the row's lse
// (log2), with the constant folded into one FMA -- cap*log2(e)*tanh(scale*x/
// cap) with a cap (th = the tanh, for the chain rule), scale*log2(e)*x
// without.
template <bool CAP>
__device__ __forceinline__ float p_arg(float x, const BwdArgs& a, float lse2, float& th) {
  if (CAP) {
    const float e = fast_exp2(x * a.two_scale_over_cap_log2e);
    th = 1.f - 2.f * __builtin_amdgcn_rcpf(e + 1.f);
    return fmaf(th, a.cap_log2e, -lse2);
  }
  th = 0.f;
  return fmaf(x, a.scale_log2e, -lse2);
}

// ------------------------------------------------------------------ dQ pass
template <int DK, int DV, int BKV, int NW, bool CAP>
__global__ __launch_bounds__(64 * NW, (DK >= 192 ? 1 : 8 / NW)) void fa_bwd_dq_kernel(BwdArgs a) {
  constexpr int NT = 64 * NW;
  constexpr int BQ = 32 * NW;
  constexpr int TILE_K = Lay<DK>::template bytes<BKV>();
  constexpr int TILE_V = Lay<DV>::template bytes<BKV>();
  constexpr int NDB = DK / 32;   // 32-wide blocks of dq
  constexpr int NS = BKV / 32;
  // K, V tiles double-buffered in one array (see bwd_unroll)
  constexpr bool UNROLL = bwd_unroll(DK);
  __shared__ __attribute__((aligned(1024))) char one[2 * (TILE_K + TILE_V)];

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
  const bf16* Kp = a.k + bkv * T * DK;
  const bf16* Vp = a.v + bkv * T * DV;

  // Q and dO rows as B operands (lane = query row), D_i, lse in log2.
  bf16x8 qreg[DK / 16], doreg[DV / 16];
  float Di;
  {
    const bf16x8* qs = (const bf16x8*)(a.q + (bh * T + qr) * DK + 8 * g);
    const size_t voff = (bh * T + qr) * DV + 8 * g;
    const bf16x8* ds = (const bf16x8*)(a.dO + voff);
    const bf16x8* os = (const bf16x8*)(a.o + voff);
    float part = 0.f;
#pragma unroll
    for (int c = 0; c < DK / 16; ++c) qreg[c] = qs[2 * c];
#pragma unroll
    for (int c = 0; c < DV / 16; ++c) {
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
    // d sink_h = -sum_i exp(sink_h - lse_i) D_i over this head's rows (all
    // batches accumulate into the same [H] entry).
    float c = (g == 0 && qrow < T) ? fast_exp2(a.sinks[h] * kLog2e - lse2) * Di : 0.f;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) c += __shfl_xor(c, off);
    if (lane == 0) atomicAdd(a.dsinks + h, -c);
  }

  int kv_lo = 0;
  if (W > 0) kv_lo = max(0, q0 - W + 1);
  const int t_lo = kv_lo / BKV;
  const int kv_hi = min(T, q0 + BQ);
  const int ntiles = (kv_hi + BKV - 1) / BKV - t_lo;

  f32x16 dqacc[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db)
#pragma unroll
    for (int i = 0; i < 16; ++i) dqacc[db][i] = 0.f;

  // K, V tiles go straight from HBM into the idle LDS buffer (no staging
  // registers): issued at the top of an iteration, waited for before its
  // closing barrier.
  TileDma<DK, BKV, NW> kdm;
  TileDma<DV, BKV, NW> vdm;
  kdm.init(wave, lane);
  vdm.init(wave, lane);
  auto kbuf = [&](auto b_c) -> LDS_AS char* {
    return (LDS_AS char*)one + decltype(b_c)::value * TILE_K;
  };
  auto vbuf = [&](auto b_c) -> LDS_AS char* {
    return (LDS_AS char*)one + 2 * TILE_K + decltype(b_c)::value * TILE_V;
  };
  using I0 = std::integral_constant<int, 0>;
  using I1 = std::integral_constant<int, 1>;
  kdm.load(Kp, T * DK * 2, kbuf(I0{}), t_lo * BKV, wave);
  vdm.load(Vp, T * DV * 2, vbuf(I0{}), t_lo * BKV, wave);
  wait_vmem();
  __syncthreads();

  const int qa = qw0, qb = qw0 + 31;
  // one key tile: S, dP, dS, then dQ^T += K^T dS^T
  auto compute = [&](const LDS_AS char* Kt, const LDS_AS char* Vt, const int kv0)
                     __attribute__((always_inline)) {
      const bool empty = qa >= T || kv0 > qb || (W > 0 && kv0 + BKV - 1 <= qa - W);
      const bool full = kv0 + BKV - 1 <= qa && (W == 0 || kv0 > qb - W);
      f32x16 s[NS], dp[NS];
      TrPipe<DK, NDB, BKV / 16, bwd_lds_pd(DK)> ktp;
      constexpr int NC16 = BKV / 16;
      auto pack_chunk = [&](int c16) __attribute__((always_inline)) {
        float tmp[8];
  #pragma unroll
        for (int jj = 0; jj < 8; ++jj) tmp[jj] = s[c16 >> 1][8 * (c16 & 1) + jj];
        return pack_bf16(tmp);
      };
      if constexpr (NS == 1 && bwd_lds_pd(DK) > 0 && 16 % (DV / 16) == 0) {
        // S first, then dP with P = 2^(...) computed under its MFMAs; dS =
        // P (dP - D) chunk by chunk under the dQ product's MFMAs.
        if (empty) return;
        constexpr int PD = bwd_lds_pd(DK), NK = DK / 16, NV = DV / 16, EP = 16 / NV;
  #pragma unroll
        for (int i = 0; i < 16; ++i) {
          s[0][i] = 0.f;
          dp[0][i] = 0.f;
        }
        auto fS = [&](int k) { return lds_row_operand<DK>(Kt, 0, k, lane); };
        auto fV = [&](int k) { return lds_row_operand<DV>(Vt, 0, k, lane); };
        MfmaSeq<NK, PD> sq;
        MfmaSeq<NV, PD> vq;
        sq.start(fS);
        sq.run(fS, [&](int k) { return qreg[k]; }, [&](int) -> f32x16& { return s[0]; },
               [&](int) {});
        vq.start(fV);
        if (!full) {
          // invisible pairs: S = -inf gives P = 0, and under a cap
          // tanh = -1, so that the factor 1 - tanh^2 is 0
  #pragma unroll
          for (int i = 0; i < 16; ++i) {
            const int kv = kv0 + acc_row(i, g);
            const bool vis = (kv <= qrow) & ((W == 0) | (kv > qrow - W));
            s[0][i] = vis ? s[0][i] : -INFINITY;
          }
        }
        float thv[CAP ? 16 : 1];
        vq.run(fV, [&](int k) { return doreg[k]; }, [&](int) -> f32x16& { return dp[0]; },
               [&](int k) __attribute__((always_inline)) {
  #pragma unroll
                 for (int e = 0; e < EP; ++e) {
                   const int i = k * EP + e;
                   float th;
                   s[0][i] = fast_exp2(p_arg<CAP>(s[0][i], a, lse2, th));
                   if (CAP) thv[i] = th;
                 }
               });
        ktp.start(Kt, 0, lane);
        auto fin = [&](int i) __attribute__((always_inline)) {
          float ds = s[0][i] * (dp[0][i] - Di);
          if (CAP) ds *= 1.f - thv[i] * thv[i];
          s[0][i] = ds;
        };
        bf16x8 dsb[NC16];
  #pragma unroll
        for (int jj = 0; jj < 8; ++jj) fin(jj);
        dsb[0] = pack_chunk(0);
        ktp.run(dqacc, Kt, 0, dsb, lane, [&](int k) __attribute__((always_inline)) {
          const int c = k / NDB, r = k % NDB;
          if (c + 1 < NC16) {
  #pragma unroll
            for (int e = r * 8 / NDB; e < (r + 1) * 8 / NDB; ++e) fin(8 * (c + 1) + e);
            if (r == NDB - 1) dsb[c + 1] = pack_chunk(c + 1);
          }
        });
        return;
      }
      if (!empty) {
        mma_rows2<DK, DV, NS, bwd_lds_pd(DK)>(s, Kt, qreg, dp, Vt, doreg, lane);
        ktp.start(Kt, 0, lane);   // first K^T operands of dQ, read during the softmax
      }
      auto elem = [&](int t, int i) __attribute__((always_inline)) {
        float th;
        const float p = fast_exp2(p_arg<CAP>(s[t][i], a, lse2, th));
        float ds = p * (dp[t][i] - Di);
        if (CAP) ds *= 1.f - th * th;
        s[t][i] = ds;
      };
      if constexpr (bwd_lds_pd(DK) > 0 && 8 % NDB == 0) {
        if (!empty) {
          if (!full) {
            // invisible pairs: S = -inf gives p = 0 without a cap; with one,
            // p <= 1 stays finite and dP = D_i makes dS exactly 0
  #pragma unroll
            for (int t = 0; t < NS; ++t)
  #pragma unroll
              for (int i = 0; i < 16; ++i) {
                const int kv = kv0 + 32 * t + acc_row(i, g);
                const bool vis = (kv <= qrow) & ((W == 0) | (kv > qrow - W));
                s[t][i] = vis ? s[t][i] : -INFINITY;
                if (CAP) dp[t][i] = vis ? dp[t][i] : Di;
              }
          }
          // chunk 0's dS first, then the dQ MFMAs of chunk c carry the dS
          // VALU of chunk c + 1 (8 / NDB elements after each MFMA)
          bf16x8 dsb[NC16];
  #pragma unroll
          for (int jj = 0; jj < 8; ++jj) elem(0, jj);
          dsb[0] = pack_chunk(0);
          ktp.run(dqacc, Kt, 0, dsb, lane, [&](int k) __attribute__((always_inline)) {
            constexpr int EPH = 8 / NDB;
            const int c = k / NDB, r = k % NDB;
            if (c + 1 < NC16) {
  #pragma unroll
              for (int e = 0; e < EPH; ++e) {
                const int jj = r * EPH + e;
                elem((c + 1) >> 1, 8 * ((c + 1) & 1) + jj);
              }
              if (r == NDB - 1) dsb[c + 1] = pack_chunk(c + 1);
            }
          });
          return;
        }
      }
      if (!empty) {
        // dS^T in s[] (fp32), then bf16 operands.  Every element is computed
        // branch-free; partial tiles then zero the invisible ones in one block
        // (ds = 0 exactly where p = 0).
  #pragma unroll
        for (int t = 0; t < NS; ++t)
  #pragma unroll
          for (int i = 0; i < 16; ++i) elem(t, i);
        if (!full) {
  #pragma unroll
          for (int t = 0; t < NS; ++t)
  #pragma unroll
            for (int i = 0; i < 16; ++i) {
              const int kv = kv0 + 32 * t + acc_row(i, g);
              const bool vis = (kv <= qrow) & ((W == 0) | (kv > qrow - W));
              s[t][i] = vis ? s[t][i] : 0.f;
            }
        }
        bf16x8 dsb[NC16];
  #pragma unroll
        for (int c16 = 0; c16 < NC16; ++c16) dsb[c16] = pack_chunk(c16);
        ktp.run(dqacc, Kt, 0, dsb, lane);
      }
  };

  // one iteration on the tile in buffer B (loop unrolled by two so that the
  // buffers are compile-time choices)
  auto step = [&](auto b_c, const int j) __attribute__((always_inline)) {
    using BN = std::integral_constant<int, 1 - decltype(b_c)::value>;
    const bool more = j + 1 < ntiles;
    if (more) {
      kdm.load(Kp, T * DK * 2, kbuf(BN{}), (t_lo + j + 1) * BKV, wave);
      vdm.load(Vp, T * DV * 2, vbuf(BN{}), (t_lo + j + 1) * BKV, wave);
    }
    compute(kbuf(b_c), vbuf(b_c), (t_lo + j) * BKV);
    if (more) wait_vmem();
    __syncthreads();
  };
  if constexpr (UNROLL) {
    int j = 0;
    for (; j + 1 < ntiles; j += 2) {
      step(I0{}, j);
      step(I1{}, j + 1);
    }
    if (j < ntiles) step(I0{}, j);
  } else {
    // the buffer picked at run time in the one array
    for (int j = 0; j < ntiles; ++j) {
      const int cur = j & 1;
      const bool more = j + 1 < ntiles;
      if (more) {
        kdm.load(Kp, T * DK * 2, (LDS_AS char*)one + (cur ^ 1) * TILE_K, (t_lo + j + 1) * BKV, wave);
        vdm.load(Vp, T * DV * 2, (LDS_AS char*)one + 2 * TILE_K + (cur ^ 1) * TILE_V,
                 (t_lo + j + 1) * BKV, wave);
      }
      compute((LDS_AS char*)one + cur * TILE_K, (LDS_AS char*)one + 2 * TILE_K + cur * TILE_V,
              (t_lo + j) * BKV);
      if (more) wait_vmem();
      __syncthreads();
    }
  }

  if (qrow < T) {
    bf16* Qd = a.dq + (bh * T + qrow) * DK;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int i4 = 0; i4 < 4; ++i4) {
        float x[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) x[e] = dqacc[db][4 * i4 + e] * a.scale;
        if (a.rope_cs) {
          // RoPE backward fused into the store: elements d = 32 db + 8 i4
          // + 4 g + e hold the pairs 16 db + 4 i4 + 2 g + {0, 1}; rotate by
          // the negative angle
          const float4 r = *(const float4*)(a.rope_cs + (size_t)qrow * DK +
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

// ----------------------------------------------------------------- dK/dV pass
// ------------------------------------------------------ fused dK/dV pass
constexpr int kPairPD = 3;     // LDS operands read this many MFMAs ahead
constexpr int kPairBQB = 64;   // query tile of the paired pass (d = 256: 32)
// One launch for dK and dV, with paired waves: waves p and p + NP own the
// same 32 key rows (NP = 4 pairs, 128 keys per workgroup; at d = 256 NP = 2
// and one wave per SIMD, see PairShape).  Wave p (the P side) keeps K in
// registers; per query tile it computes S = Q K^T and P, accumulates
// dV^T += dO^T P, and leaves the factor that multiplies (dP - D) in dS --
// P, or with the cap P (1 - tanh^2) -- to its partner in LDS as bf16.
// Wave p + NP (the dS side) keeps V in registers; per tile it computes
// dP = dO V^T, and one tile later, once the barrier has published the P
// side's factor, dS = factor (dP - D) and dK^T += Q^T dS.  S and the exp
// chain are computed once per tile (the two-launch scheme computes them in
// both passes), and each wave holds one gradient accumulator, so two waves
// per SIMD still fit below d = 256.  Because the dS side lags one tile, Q
// tiles and the row statistics are triple-buffered (the tile being loaded,
// the current one, and the previous one the dS side still reads); dO tiles
// are triple- or, where LDS is short (d_k = 192), double-buffered.  Each buffer is its
// own LDS object and the loop is unrolled by three (or six), so every
// buffer is a compile-time choice.  Within a tile, each side's VALU work
// runs under the MFMAs of its next product (MfmaSeq hooks).
template <int DK, int DV, int BQB>
struct PairShape {
  // 64-query tiles: 8 waves (4 pairs, 128 keys), two waves per SIMD;
  // 32-query tiles (d = 256): 4 waves (2 pairs, 64 keys), one wave per SIMD
  // (a wave's K rows and 32 x 256 accumulator need more than 256 registers)
  static constexpr int NW = BQB == 32 ? 4 : 8;
  static constexpr int NP = NW / 2;
  static constexpr int TILE_Q = Lay<DK>::template bytes<BQB>();
  static constexpr int TILE_O = Lay<DV>::template bytes<BQB>();
  static constexpr int XB = NP * (BQB / 16) * 1024;   // exchange: pairs x chunks x 64 lanes x 16 B
  static constexpr int STAT = BQB * 4;
  static constexpr int LDS_MAX = 160 * 1024;
  static constexpr int fixed = 3 * TILE_Q + 2 * XB + 3 * 2 * STAT;
  static constexpr int OSL = fixed + 3 * TILE_O <= LDS_MAX ? 3 : 2;   // dO slots
  static_assert(fixed + OSL * TILE_O <= LDS_MAX, "tiles exceed the LDS");
};

// DS (d = 256): the dS side also writes each tile's dS (bf16, as packed for
// the dK product) to the workspace a.dsw for the dQ pass that reads it
// (fa_bwd_ds.hip): its 32 keys x 32 queries tile at slot (b, query head,
// query tile, key tile - query tile + nkt_ws - 1), lane L's two packs at
// byte 64 (L % 32) + 32 (L / 32) -- the layout of fa_bwd_kv_pipe_kernel's
// stores.  Tiles outside the band (or past the range) are sent past the
// store's buffer range, which drops them: no branch.
template <int DK, int DV, int BQB, bool CAP, bool DS = false>
__global__ __launch_bounds__(BQB == 32 ? 256 : 512, 1) void fa_bwd_dkdv_pair_kernel(BwdArgs a) {
  using SH = PairShape<DK, DV, BQB>;
  constexpr int NW = SH::NW;
  constexpr int NP = SH::NP;                // wave pairs
  constexpr int BKVB = 32 * NP;             // key rows per workgroup
  constexpr int TILE_Q = SH::TILE_Q, TILE_O = SH::TILE_O, OSL = SH::OSL;
  constexpr int NDBK = DK / 32, NDBV = DV / 32;   // 32-wide blocks of dk, dv
  constexpr int NCK = DK / 16, NCV = DV / 16;     // 16-wide chunks (k steps of S, dP)
  constexpr int NS = BQB / 32;              // 32-query halves
  constexpr int NC16 = BQB / 16;            // 16-query chunks (k steps of dV, dK)
  constexpr int STAT = SH::STAT;            // bytes of one lse or D tile
  constexpr int XB = SH::XB;
  constexpr int PD = kPairPD;
  constexpr int NKV = NCK > NCV ? NCK : NCV;
  constexpr int NACC = NDBK > NDBV ? NDBK : NDBV;
  static_assert(NS == 1 || NS == 2, "32 or 64 queries per tile");
  // At d = 256 (one wave per SIMD) the gradient accumulator is pinned to the
  // AGPRs: the score and dP products then stay in the VGPRs, where the VALU
  // reads them while the matrix unit works on the accumulator (with them in
  // the AGPRs VALU and MFMA co-executed 3 % of the time; gemma-global dK/dV
  // 1.37 -> 1.24 ms).  Its P side also skips the mask on tiles every pair of
  // which its keys see by running segments of mask-free and masked tile
  // groups (nothing hides a per-tile branch at one wave per SIMD; with two
  // waves per SIMD a per-tile branch costs little: mistral -3.5 % against
  // masking every tile).
  constexpr bool AG = DK == 256;
  static_assert(!DS || (AG && BQB == 32), "dS stores: d = 256, 32-query tiles");
  __shared__ __attribute__((aligned(1024))) char qs0[TILE_Q];
  __shared__ __attribute__((aligned(1024))) char qs1[TILE_Q];
  __shared__ __attribute__((aligned(1024))) char qs2[TILE_Q];
  __shared__ __attribute__((aligned(1024))) char os0[TILE_O];
  __shared__ __attribute__((aligned(1024))) char os1[TILE_O];
  __shared__ __attribute__((aligned(1024))) char os2[OSL == 3 ? TILE_O : 16];
  __shared__ __attribute__((aligned(1024))) char xsa[2 * XB];
  __shared__ __attribute__((aligned(16))) char sbuf[3 * 2 * STAT];
  LDS_AS char* stat = (LDS_AS char*)sbuf;  // [slot][lse2 | D][BQB] fp32

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const bool pside = wave < NP;
  const int pr = wave & (NP - 1);
  const int g = lane >> 5;
  const int l32 = lane & 31;
  const int T = a.T;
  const int W = a.window;
  const int G = a.H / a.Hkv;
  const int nkb = (T + BKVB - 1) / BKVB;
  const WorkItem w = decode_work(blockIdx.x, nkb, a.B, a.Hkv, 1, false);
  const int k0 = w.blk * BKVB;
  const int kw0 = k0 + 32 * pr;
  const int krow = kw0 + l32;
  const int kr = krow < T ? krow : T - 1;
  const size_t bkv = (size_t)w.b * a.Hkv + w.hkv;

  // K (P side) or V (dS side) rows: the B operand of S = Q K^T or dP = dO V^T
  bf16x8 kv[NKV];
  if (pside) {
    const bf16x8* src = (const bf16x8*)(a.k + (bkv * T + kr) * DK + 8 * g);
#pragma unroll
    for (int c = 0; c < NCK; ++c) kv[c] = src[2 * c];
  } else {
    const bf16x8* src = (const bf16x8*)(a.v + (bkv * T + kr) * DV + 8 * g);
#pragma unroll
    for (int c = 0; c < NCV; ++c) kv[c] = src[2 * c];
  }
  f32x16 acc[NACC];   // dV (P side, NDBV blocks) or dK (dS side, NDBK blocks)

  // Query tiles that can see keys [k0, k0 + BKVB).
  const int qt_lo = k0 / BQB;
  const int q_hi = W > 0 ? min(T, k0 + BKVB - 1 + W) : T;
  const int nqt = (q_hi + BQB - 1) / BQB - qt_lo;
  const int niter = G * nqt;
  // query q sees this lane's key iff 0 <= q - krow < span
  const unsigned span = (unsigned)max(0, min(T, W > 0 ? krow + W : T) - krow);

  // iteration it visits query head (hkv*G + hi) and tile ti, it = hi*nqt + ti
  auto stage_stats = [&](int hi, int ti) -> float {
    const int hh = w.hkv * G + hi;
    const int q0 = (qt_lo + ti) * BQB;
    const size_t bhh = (size_t)w.b * a.H + hh;
    float v = 0.f;
    if (wave < 2 * BQB / 64) {   // the waves holding threads 0 .. 2 BQB - 1 (wave-uniform)
      // one load, raw (the lse is scaled when it is stored to LDS): a use
      // here would make these waves wait for the load at once
      int qq = q0 + (tid % BQB);
      qq = qq < T ? qq : T - 1;
      v = (tid < BQB ? a.lse : a.Dst)[bhh * T + qq];
    }
    return v;
  };
  // lse (log2 units) or -D, as stored in the LDS statistics tile (the dS
  // side starts its dP accumulators from -D, so they finish as dP - D)
  auto stat_val = [&](float v) { return tid < BQB ? v * kLog2e : -v; };
  auto tile_src = [&](int hi, const bf16* base, int dd) {
    return base + ((size_t)w.b * a.H + w.hkv * G + hi) * T * dd;
  };
  auto tile_q0 = [&](int ti) { return (qt_lo + ti) * BQB; };
  auto advance = [&](int& hi, int& ti) {
    if (++ti == nqt) {
      ti = 0;
      ++hi;
    }
  };
  TileDma<DK, BQB, NW> qdm;
  TileDma<DV, BQB, NW> odm;
  qdm.init(wave, lane);
  odm.init(wave, lane);
  // tile it uses Q and statistics slot it % 3 and dO slot it % OSL
  auto qbuf = [&](auto b_c) -> LDS_AS char* {
    constexpr int b = decltype(b_c)::value;
    return b == 0 ? (LDS_AS char*)qs0 : b == 1 ? (LDS_AS char*)qs1 : (LDS_AS char*)qs2;
  };
  auto obuf = [&](auto b_c) -> LDS_AS char* {
    constexpr int b = decltype(b_c)::value;
    return b == 0 ? (LDS_AS char*)os0 : b == 1 ? (LDS_AS char*)os1 : (LDS_AS char*)os2;
  };
  auto sbufp = [&](auto b_c) -> LDS_AS float* {
    constexpr int b = decltype(b_c)::value;
    return (LDS_AS float*)(stat + b * 2 * STAT);
  };
  // exchange slot b (written with ordinary LDS stores: a run-time choice)
  auto xbuf = [&](int b, int xo) -> LDS_AS char* { return (LDS_AS char*)xsa + b * XB + xo; };
  auto issue = [&](LDS_AS char* qdst, LDS_AS char* odst, int hi, int ti)
                   __attribute__((always_inline)) -> float {
    const float v = stage_stats(hi, ti);
    qdm.load(tile_src(hi, a.q, DK), T * DK * 2, qdst, tile_q0(ti), wave);
    odm.load(tile_src(hi, a.dO, DV), T * DV * 2, odst, tile_q0(ti), wave);
    return v;
  };
  using I0 = std::integral_constant<int, 0>;
  using I1 = std::integral_constant<int, 1>;
  using I2 = std::integral_constant<int, 2>;
  {
    const float v = issue(qbuf(I0{}), obuf(I0{}), 0, 0);
    if (wave < 2 * BQB / 64) sbufp(I0{})[tid] = stat_val(v);
    wait_vmem();
  }
  int h1 = 0, t1 = 0;
  advance(h1, t1);   // tile 1
  __syncthreads();

  const int ka = kw0, kb = kw0 + 31;
  auto empty_tile = [&](int q0) {
    return ka >= T || q0 + BQB - 1 < ka || (W > 0 && q0 - kb >= W);
  };

  // Element (t, i) of a 32x32 accumulator pair held by this lane: query
  // 32t + 8(i/4) + 4g + i%4 of the tile; chunk c16 = 2t + i/8 of the
  // 16-query k steps holds elements i%8 of that half.  VALU work of M
  // elements spread over the N MFMAs of a sequence: hook k takes elements
  // [M k / N, M (k + 1) / N).
  auto span_of = [](int M, int N, int k, int& e0, int& e1) {
    e0 = M * k / N;
    e1 = M * (k + 1) / N;
  };

  // P side, one query tile: S of the two halves in turn (exp of half 0 under
  // the MFMAs of half 1), then dV^T += dO^T P over the 16-query chunks (exp of
  // half 1 under the MFMAs of chunks 0-1); P and the exchange factor are
  // packed per chunk as soon as its eight elements exist.
  // mask_c: 1 evaluate the mask, 0 none (a tile every pair of which the
  // wave's keys see), 2 decide per tile
  auto p_tile = [&](const LDS_AS char* Qt, const LDS_AS char* dOt, LDS_AS char* X,
                    const LDS_AS float* lse2t, const int q0, const LaneOffs<DK>& lq,
                    const LaneOffs<DV>& lv_, auto mask_c, auto&& ld) __attribute__((always_inline)) {
    constexpr int MSK = decltype(mask_c)::value;
    const int vb = q0 + 4 * g - krow;   // q - krow = vb + 32t + 8(i/4) + i%4
    // every pair of the tile visible to every key of the wave: no mask
    const bool full = q0 >= kb && q0 + BQB <= T && (W == 0 || q0 + BQB - 1 - ka < W);
    f32x16 s[NS];
    f32x16 cx[CAP ? NS : 1];
#pragma unroll
    for (int t = 0; t < NS; ++t)
#pragma unroll
      for (int i = 0; i < 16; ++i) s[t][i] = 0.f;
    bf16x8 pb[NC16];
    f32x4 lv[NS][4];   // lse (log2) of the lane's rows
    auto fS = [&](int k) { return lds_row_op<DK>(Qt, lq, k / NCK, k % NCK); };
    auto fV = [&](int k) { return lds_tr_op<DV>(dOt, lv_, k / NDBV, k % NDBV); };
    constexpr int NSQ = NS * NCK, NVQ = NC16 * NDBV;
    MfmaSeq<NSQ, PD> sq;
    std::conditional_t<AG, AgprSeq<NVQ, PD>, MfmaSeq<NVQ, PD>> vq;
    sq.start(fS);
#pragma unroll
    for (int i4 = 0; i4 < 4; ++i4) lv[0][i4] = *(const LDS_AS f32x4*)(lse2t + 8 * i4 + 4 * g);
    auto elem = [&](int t, int i) __attribute__((always_inline)) {
      float th;
      float p = fast_exp2(p_arg<CAP>(s[t][i], a, lv[t][i >> 2][i & 3], th));
      if (MSK == 1 || (MSK == 2 && !full)) {
        const bool vis = (unsigned)(vb + 32 * t + 8 * (i >> 2) + (i & 3)) < span;
        p = vis ? p : 0.f;
      }
      s[t][i] = p;
      if (CAP) cx[t][i] = p * (1.f - th * th);
    };
    auto pack_chunk = [&](int c16) __attribute__((always_inline)) {
      float tp[8], tc[8];
#pragma unroll
      for (int jj = 0; jj < 8; ++jj) {
        tp[jj] = s[c16 >> 1][8 * (c16 & 1) + jj];
        if (CAP) tc[jj] = cx[c16 >> 1][8 * (c16 & 1) + jj];
      }
      pb[c16] = pack_bf16(tp);
      *(LDS_AS bf16x8*)(X + c16 * 1024) = CAP ? pack_bf16(tc) : pb[c16];
    };
    // half t's 16 elements [e0, e1), packing each chunk when it completes
    auto elems = [&](int t, int e0, int e1) __attribute__((always_inline)) {
#pragma unroll
      for (int e = e0; e < e1; ++e) {
        elem(t, e);
        if (e == 7) pack_chunk(2 * t);
        if (e == 15) pack_chunk(2 * t + 1);
      }
    };
    // (with one half, S is one chain of dependent MFMAs: a 32x32x16
    // product issues back to back on its own accumulator at full rate)
    sq.run(fS, [&](int k) { return kv[k % NCK]; },
           [&](int k) -> f32x16& { return s[k / NCK]; },
           [&](int k) __attribute__((always_inline)) {
             if (NS == 2 && k == 0) {
#pragma unroll
               for (int i4 = 0; i4 < 4; ++i4)
                 lv[NS - 1][i4] = *(const LDS_AS f32x4*)(lse2t + 32 + 8 * i4 + 4 * g);
             }
             if (NS == 2 && k >= NCK) {
               int e0, e1;
               span_of(16, NCK, k - NCK, e0, e1);
               elems(0, e0, e1);
             }
             ld(k);
             if (k == NSQ - PD) vq.start(fV);
           });
    // the last half: with one half, its first chunk before the dV product
    // and the second under the MFMAs of the first
    // (with the accumulator in the AGPRs the compiler does not separate a
    // VALU write from the MFMA that reads it: the last chunk is packed two
    // MFMAs before its first use, and a wait follows the first pack)
    constexpr int TL = NS - 1;
    constexpr int NH = (NS == 2 ? 2 * NDBV : NDBV) - (AG ? 2 : 0);   // dV MFMAs that carry exp work
    constexpr int EH = NS == 2 ? 16 : 8;            // elements placed in them
    if constexpr (NS == 1) elems(0, 0, 8);
    if constexpr (AG) {
      // the packs stay above this point, two wait states before the MFMA
      __builtin_amdgcn_sched_barrier(0);
      asm volatile("s_nop 1");
    }
    vq.run(fV, [&](int k) { return pb[k / NDBV]; }, [&](int k) -> f32x16& { return acc[k % NDBV]; },
           [&](int k) __attribute__((always_inline)) {
             if (k < NH) {
               int e0, e1;
               span_of(EH, NH, k, e0, e1);
               elems(TL, 16 - EH + e0, 16 - EH + e1);
             }
           });
  };

  // dS side, the previous tile: dS = factor * (dP - D) per chunk, each
  // chunk computed under the MFMAs of the one before, dK^T += Q^T dS;
  // tail() runs a few MFMAs before the end (it starts the next product)
  auto ds_prev = [&](f32x16 (&dp)[NS], const LDS_AS char* Qt, const LDS_AS char* X,
                     const LDS_AS float* Dt, const LaneOffs<DK>& lq, auto&& tail, auto&& ld,
                     auto&& sto) __attribute__((always_inline)) {
    (void)Dt;
    bf16x8 xf[NC16];
    // the exchange factor of chunk c16, read a chunk before its use
    auto load_chunk = [&](int c16) __attribute__((always_inline)) {
      xf[c16] = *(const LDS_AS bf16x8*)(X + c16 * 1024);
    };
    load_chunk(0);
    load_chunk(1);
    auto fK = [&](int k) { return lds_tr_op<DK>(Qt, lq, k / NDBK, k % NDBK); };
    constexpr int NKQ = NC16 * NDBK;
    std::conditional_t<AG, AgprSeq<NKQ, PD>, MfmaSeq<NKQ, PD>> kq;
    kq.start(fK);
    float td[NC16][8];
    bf16x8 dsb[NC16];
    auto dsel = [&](int c16, int jj) __attribute__((always_inline)) {
      const int t = c16 >> 1, i = 8 * (c16 & 1) + jj;
      td[c16][jj] = (float)xf[c16][jj] * dp[t][i];   // dp holds dP - D
      if (jj == 7) dsb[c16] = pack_bf16(td[c16]);
    };
#pragma unroll
    for (int jj = 0; jj < 8; ++jj) dsel(0, jj);
    if constexpr (AG) {
      __builtin_amdgcn_sched_barrier(0);
      asm volatile("s_nop 1");
    }
    // chunk c + 1 under chunk c's MFMAs (with AGPR accumulators, finished two
    // MFMAs before its first use)
    constexpr int NDS = NDBK - (AG ? 2 : 0);
    kq.run(fK, [&](int k) { return dsb[k / NDBK]; }, [&](int k) -> f32x16& { return acc[k % NDBK]; },
           [&](int k) __attribute__((always_inline)) {
             const int c = k / NDBK + 1;   // the chunk after this MFMA's
             if (k % NDBK == 0 && c + 1 < NC16) load_chunk(c + 1);
             if (c < NC16 && k % NDBK < NDS) {
               int j0, j1;
               span_of(8, NDS, k % NDBK, j0, j1);
#pragma unroll
               for (int jj = j0; jj < j1; ++jj) dsel(c, jj);
             }
             ld(k);
             sto(k, dsb);
             if (k == NKQ - PD) tail();
           });
  };
  // dS side, the current tile: dP - D, the accumulators starting from -D
  // (the statistics tile holds -D); the two halves' accumulations alternate
  // (independent MFMAs back to back)
  auto dp_cur = [&](f32x16 (&dp)[NS], MfmaSeq<NS * NCV, PD>& pq, auto&& fP, const bool started,
                    const LDS_AS float* Dn, auto&& ld) __attribute__((always_inline)) {
#pragma unroll
    for (int t = 0; t < NS; ++t)
#pragma unroll
      for (int i4 = 0; i4 < 4; ++i4) {
        const f32x4 d4 = *(const LDS_AS f32x4*)(Dn + 32 * t + 8 * i4 + 4 * g);
#pragma unroll
        for (int e = 0; e < 4; ++e) dp[t][4 * i4 + e] = d4[e];
      }
    if (!started) pq.start(fP);
    pq.run(fP, [&](int k) { return kv[k / NS]; }, [&](int k) -> f32x16& { return dp[k % NS]; }, ld);
  };

  // Iteration it (0 .. niter; the last one only finishes the dS side's
  // lag): load tile it+1, P side on tile it, dS side on tiles it-1 and it.
  // The two sides run separate copies of the loop (the same loads and
  // barriers), so that neither holds the other's registers.
  int tc = 0, tp = 0;   // tile index (within the head) of tiles it and it-1
  int hc = 0, hp = 0;   // their query heads (within the group)
  LaneOffs<DK> lq0;
  LaneOffs<DV> lv0;
  lq0.init(lane);
  lv0.init(lane);
  int xo0 = pr * NC16 * 1024 + lane * 16;   // this lane's exchange slot
  f32x16 dp[NS];        // dS side: dP of the previous tile
  // qc, qn, qp: Q / statistics slots of tiles it, it+1, it-1; oc, on: dO
  // slots of tiles it, it+1
  // first_c: the first step (it = 0; the dS side has no previous tile)
  auto step = [&](auto side_c, auto mask_c, auto first_c, const int it, auto qc, auto qn, auto qp,
                  auto oc, auto on) __attribute__((always_inline)) {
    constexpr bool PS = decltype(side_c)::value;
    constexpr bool FIRST = decltype(first_c)::value;
    const int xs = it & 1;   // exchange slot of tile it
    const bool more = it + 1 < niter;
    float sv = 0.f;
    if (more) sv = stage_stats(h1, t1);
    // with AGPR accumulators every step runs both products (a branch around
    // them makes the compiler copy the accumulator at the join): the tile
    // past the range (zero Q and dO) gets lse = +inf and D = 0, so its P is 0
    if (AG && !more) sv = tid < BQB ? INFINITY : 0.f;
    // Tile it+1's Q and dO loads go out one after each MFMA of this step's
    // first product (a burst of them stalls the wave until the memory
    // pipeline has taken them), branch-free: with no tile it+1 they read an
    // empty range (zeros, no memory touched) into a slot no one reads.
    // Every wave of a side issues the same number of 1 KB pieces.
    constexpr int W0 = PS ? 0 : NP, W1 = PS ? NP - 1 : NW - 1;   // the side's waves
    constexpr int NQI = TileDma<DK, BQB, NW>::NI, NOI = TileDma<DV, BQB, NW>::NI;
    constexpr int NLQ = (NQI - W0 + NW - 1) / NW, NLO = (NOI - W0 + NW - 1) / NW;
    static_assert(NLQ == (NQI - W1 + NW - 1) / NW && NLO == (NOI - W1 + NW - 1) / NW,
                  "every wave of a side loads as many pieces");
    static_assert(NLQ + NLO <= 16, "one load per MFMA of a 16-MFMA product");
    const bf16* qsrc = tile_src(h1, a.q, DK);
    const bf16* osrc = tile_src(h1, a.dO, DV);
    const int nq = more ? T * DK * 2 : 0, no = more ? T * DV * 2 : 0, row1 = tile_q0(t1);
    auto ld = [&](int k) __attribute__((always_inline)) {
      if (k < NLQ)
        qdm.load_piece(k, qsrc, nq, qbuf(qn), row1, wave);
      else if (k < NLQ + NLO)
        odm.load_piece(k - NLQ, osrc, no, obuf(on), row1, wave);
    };
    auto ld_all = [&]() __attribute__((always_inline)) {
#pragma unroll
      for (int k = 0; k < NLQ + NLO; ++k) ld(k);
    };
    auto no_ld = [](int) {};
    // dS of tile it-1 to the workspace (DS): both packs after the step's
    // last tile load (and after the second pack exists), so that the wait at
    // the step's end can leave them in flight
    auto no_sto = [](int, const bf16x8*) {};
    auto sto = [&](int k, const bf16x8* dsb) __attribute__((always_inline)) {
      if constexpr (DS) {
        constexpr int KS = NLQ + NLO > NDBK - 2 ? NLQ + NLO : NDBK - 2;
        static_assert(KS < NC16 * NDBK, "stores inside the dK product");
        if (k == KS) {
          const int qt = qt_lo + tp;
          const int hh = w.hkv * G + (hp < G ? hp : G - 1);
          const int row = __builtin_amdgcn_readfirstlane(
              ((w.b * a.H + hh) * a.nqt_ws + (qt < a.nqt_ws ? qt : 0)) * a.nkt_ws);
          const int nrec = hp < G && qt < a.nqt_ws ? a.nkt_ws * 2048 : 0;
          const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
              a.dsw + (size_t)row * 1024, 0, __builtin_amdgcn_readfirstlane(nrec), 0x00020000);
          // slot of the key tile in the query tile's row; outside the band a
          // slot far past any row's range (the lane offset cannot wrap it)
          const unsigned j0 = (unsigned)(kw0 / 32 - qt + a.nkt_ws - 1);
          const unsigned j = j0 < (unsigned)a.nkt_ws ? j0 : 0x40000u;
          const unsigned vo = j * 2048u + 64u * l32 + 32u * g;
#if defined(__HIP_DEVICE_COMPILE__)
          __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, dsb[0]), rs, vo, 0, 2);
          __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, dsb[1]), rs, vo + 16, 0,
                                                 2);
#endif
        }
      }
    };
    // where spreading them keeps the side spill-free (measured per shape);
    // elsewhere all at the top of the step
    constexpr bool SPREAD = PS ? (DK <= 128 || AG) : DK != 192;
    // lane offsets refreshed per step (in place): the buffer addresses
    // derived from them are formed here (one add per buffer) instead of
    // hoisted out of the loop, where those of all the buffers would stay live
    lq0.refresh();
    lv0.refresh();
    asm volatile("" : "+v"(xo0));
    const LaneOffs<DK>& lq = lq0;
    const LaneOffs<DV>& lv = lv0;
    const int xo = xo0;
    if constexpr (PS && AG) {
      // tiles outside the band are computed fully masked (they are in the
      // masked segments): exact zeros
      if constexpr (SPREAD) {
        p_tile(qbuf(qc), obuf(oc), xbuf(xs, xo), sbufp(qc), tile_q0(tc), lq, lv, mask_c, ld);
      } else {
        ld_all();
        p_tile(qbuf(qc), obuf(oc), xbuf(xs, xo), sbufp(qc), tile_q0(tc), lq, lv, mask_c, no_ld);
      }
    } else if constexpr (!PS && AG) {
      auto fP = [&](int k) { return lds_row_op<DV>(obuf(oc), lv, k % NS, k / NS); };
      MfmaSeq<NS * NCV, PD> pq;
      if constexpr (!SPREAD) ld_all();
      if constexpr (!FIRST) {
        if constexpr (SPREAD)
          ds_prev(dp, qbuf(qp), xbuf(xs ^ 1, xo), sbufp(qp) + BQB, lq, [&]() { pq.start(fP); }, ld,
                  sto);
        else
          ds_prev(dp, qbuf(qp), xbuf(xs ^ 1, xo), sbufp(qp) + BQB, lq, [&]() { pq.start(fP); }, no_ld,
                  sto);
      } else if constexpr (SPREAD) {
        ld_all();
      }
      dp_cur(dp, pq, fP, !FIRST, sbufp(qc) + BQB, no_ld);
    } else if constexpr (PS) {
      const bool cur = it < niter && !empty_tile(tile_q0(tc));
      if constexpr (SPREAD) {
        if (cur)
          p_tile(qbuf(qc), obuf(oc), xbuf(xs, xo), sbufp(qc), tile_q0(tc), lq, lv, mask_c, ld);
        else
          ld_all();
      } else {
        ld_all();
        if (cur)
          p_tile(qbuf(qc), obuf(oc), xbuf(xs, xo), sbufp(qc), tile_q0(tc), lq, lv, mask_c, no_ld);
      }
    } else {
      const bool cur = it < niter && !empty_tile(tile_q0(tc));
      auto fP = [&](int k) { return lds_row_op<DV>(obuf(oc), lv, k % NS, k / NS); };
      MfmaSeq<NS * NCV, PD> pq;   // dP of the current tile, its first reads issued early
      // spread, the loads go under the previous tile's dK product; without
      // one (the first step, an empty previous tile) all at once
      if constexpr (!SPREAD) ld_all();
      bool started = false;
      if (it > 0 && !empty_tile(tile_q0(tp))) {
        if constexpr (SPREAD)
          ds_prev(dp, qbuf(qp), xbuf(xs ^ 1, xo), sbufp(qp) + BQB, lq, [&]() {
            if (cur) pq.start(fP);
          }, ld, no_sto);
        else
          ds_prev(dp, qbuf(qp), xbuf(xs ^ 1, xo), sbufp(qp) + BQB, lq, [&]() {
            if (cur) pq.start(fP);
          }, no_ld, no_sto);
        started = true;
      } else if constexpr (SPREAD) {
        ld_all();
      }
      if (cur) dp_cur(dp, pq, fP, started, sbufp(qc) + BQB, no_ld);
    }
    if ((AG || more) && wave < 2 * BQB / 64) sbufp(qn)[tid] = stat_val(sv);
    if constexpr (DS) {
      // this step's tile loads (and everything older: vector-memory
      // operations report completion in issue order) are done; the dS
      // side's two stores, issued last, may stay in flight until the next
      // step's wait.  An LDS-only barrier: __syncthreads would wait for them.
      wait_vmem<(!PS && !FIRST) ? 2 : 0>();
      lds_barrier();
    } else {
      wait_vmem();
      __syncthreads();
    }
    tp = tc;
    tc = t1;
    hp = hc;
    hc = h1;
    advance(h1, t1);
  };
  auto run = [&](auto side_c) __attribute__((always_inline)) {
    constexpr int NDB_ = decltype(side_c)::value ? NDBV : NDBK;
#pragma unroll
    for (int db = 0; db < NDB_; ++db)
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[db][i] = 0.f;
    if constexpr (OSL == 3) {
      // iterations it .. it+2 (false: the last one, niter, was among them);
      // first_c marks the group of iteration 0
      using TF = std::true_type;
      using FF = std::false_type;
      auto group = [&](auto mask_c, auto first_c, const int it) __attribute__((always_inline)) -> bool {
        step(side_c, mask_c, first_c, it, I0{}, I1{}, I2{}, I0{}, I1{});
        if (it + 1 > niter) return false;
        step(side_c, mask_c, FF{}, it + 1, I1{}, I2{}, I0{}, I1{}, I2{});
        if (it + 2 > niter) return false;
        step(side_c, mask_c, FF{}, it + 2, I2{}, I0{}, I1{}, I2{}, I0{});
        return it + 2 < niter;
      };
      using M0 = std::integral_constant<int, 0>;
      using M1 = std::integral_constant<int, 1>;
      using M2 = std::integral_constant<int, 2>;
      if constexpr (AG) {
        // whole groups of three, no exit inside one (each exit is a point
        // where the accumulator would have to sit in its final registers):
        // the iterations past niter see tiles past the range, zero tiles
        // with P = 0, and add exact zeros
        auto group3 = [&](auto mask_c, auto first_c, const int it) __attribute__((always_inline)) {
          step(side_c, mask_c, first_c, it, I0{}, I1{}, I2{}, I0{}, I1{});
          step(side_c, mask_c, FF{}, it + 1, I1{}, I2{}, I0{}, I1{}, I2{});
          step(side_c, mask_c, FF{}, it + 2, I2{}, I0{}, I1{}, I2{}, I0{});
        };
        const int ng = niter / 3 + 1;   // groups covering iterations 0 .. niter
        group3(M1{}, TF{}, 0);          // holds the wave's diagonal tile: masked
        int gi = 1;
        if constexpr (decltype(side_c)::value) {
          // P side: groups of three tiles that every key of the wave sees
          // whole (tiles [fl, fh) of each head) carry no mask; the rest
          // evaluate it
          const int fl = min(nqt, pr + 1);
          const int t_end = T >= BQB ? (T - BQB) / BQB + 1 - qt_lo : 0;   // q0 + BQB <= T
          const int fw = W > 0 ? (W >= BQB ? pr + (W - BQB) / BQB + 1 : fl) : nqt;
          const int fh = max(fl, min(nqt, min(t_end, fw)));
          for (int hi = 0; hi < G; ++hi) {
            const int u0 = hi * nqt + fl, u1 = hi * nqt + fh;   // mask-free tiles [u0, u1)
            const int ga = min(ng, max(gi, (u0 + 2) / 3));        // 3 g >= u0
            const int gb = min(ng, max(ga, u1 >= 3 ? (u1 - 3) / 3 + 1 : 0));   // 3 g + 2 < u1
            for (; gi < ga; ++gi) group3(M1{}, FF{}, 3 * gi);
            for (; gi < gb; ++gi) group3(M0{}, FF{}, 3 * gi);
          }
        }
        for (; gi < ng; ++gi) group3(M1{}, FF{}, 3 * gi);
      } else {
        if (group(M2{}, TF{}, 0))
          for (int it = 3; it <= niter; it += 3)
            if (!group(M2{}, FF{}, it)) break;
      }
    } else {
      using M2 = std::integral_constant<int, 2>;
      for (int it = 0; it <= niter; it += 6) {
        step(side_c, M2{}, std::false_type{}, it, I0{}, I1{}, I2{}, I0{}, I1{});
        if (it + 1 > niter) break;
        step(side_c, M2{}, std::false_type{}, it + 1, I1{}, I2{}, I0{}, I1{}, I0{});
        if (it + 2 > niter) break;
        step(side_c, M2{}, std::false_type{}, it + 2, I2{}, I0{}, I1{}, I0{}, I1{});
        if (it + 3 > niter) break;
        step(side_c, M2{}, std::false_type{}, it + 3, I0{}, I1{}, I2{}, I1{}, I0{});
        if (it + 4 > niter) break;
        step(side_c, M2{}, std::false_type{}, it + 4, I1{}, I2{}, I0{}, I0{}, I1{});
        if (it + 5 > niter) break;
        step(side_c, M2{}, std::false_type{}, it + 5, I2{}, I0{}, I1{}, I1{}, I0{});
      }
    }
    // this side's gradient rows: dV (P side) or scale * dK (dS side)
    if constexpr (AG) agpr_acc_fence(acc);
    if (krow < T) {
      constexpr bool PS = decltype(side_c)::value;
      constexpr int DD = PS ? DV : DK;
      bf16* dst = (PS ? a.dv : a.dk) + (bkv * T + krow) * DD;
      const float f = PS ? 1.f : a.scale;
#pragma unroll
      for (int db = 0; db < NDB_; ++db)
#pragma unroll
        for (int i4 = 0; i4 < 4; ++i4) {
          bf16x4 v4;
#pragma unroll
          for (int e = 0; e < 4; ++e) v4[e] = (bf16)(acc[db][4 * i4 + e] * f);
          *(bf16x4*)(dst + 32 * db + 8 * i4 + 4 * g) = v4;
        }
    }
  };
  if (pside)
    run(std::true_type{});
  else
    run(std::false_type{});
}

// dQ pass tile shape per head size (keys per tile, waves), chosen by
// measurement on MI355X; d = 128 and 256 run the software-pipelined kernel.

// d = 128 runs the software-pipelined kernels of fa_bwd_pipe.hip: the dK/dV
// pass at one wave per SIMD (against the paired-wave kernel: mistral 3.24 ->
// 3.05 ms) and the dQ pass at two (against fa_bwd_dq_kernel: 2.15 -> 2.08 ms;
// at one wave per SIMD 2.31); d = 256 its dQ pass.
constexpr bool pipe_dq(int dk, int dv) { return dk == dv && (dk == 128 || dk == 256); }
constexpr bool pipe_kv(int dk, int dv) { return dk == 128 && dv == 128; }

// the dQ pass, then the fused dK/dV pass; with a dS workspace (a.dsw) the
// row statistics D, the dK/dV pass storing dS, then dQ from the stored dS
template <int DK, int DV, bool CAP, int DQ_BKV, int DQ_NW>
static hipError_t launch_bwd_t(const BwdArgs& a, hipStream_t stream) {
  hipError_t e;
  if constexpr (ds_workspace_sizes(DK, DV)) {
    if (a.dsw) {
      e = launch_bwd_rowdot(a, DK, stream);   // fa_bwd_ds.hip
      stage_mark(stream);
      if (e != hipSuccess) return e;
      if constexpr (pipe_kv(DK, DV)) {
        e = launch_bwd_kv_pipe(a, CAP, stream);
      } else {
        using SH = PairShape<DK, DV, 32>;
        const dim3 grid((unsigned)((a.T + 32 * SH::NP - 1) / (32 * SH::NP)) * a.B * a.Hkv);
        hipLaunchKernelGGL((fa_bwd_dkdv_pair_kernel<DK, DV, 32, CAP, true>), grid,
                           dim3(64 * SH::NW), 0, stream, a);
        e = hipGetLastError();
      }
      stage_mark(stream);
      if (e != hipSuccess) return e;
      e = launch_bwd_dq_ds(a, DK, stream);
      stage_mark(stream);
      return e;
    }
  }
  if constexpr (pipe_dq(DK, DV)) {
    e = launch_bwd_dq_pipe(a, DK, CAP, stream);   // fa_bwd_pipe.hip
  } else {
    const int nqb = (a.T + 32 * DQ_NW - 1) / (32 * DQ_NW);
    hipLaunchKernelGGL((fa_bwd_dq_kernel<DK, DV, DQ_BKV, DQ_NW, CAP>), dim3((unsigned)nqb * a.B * a.H),
                       dim3(64 * DQ_NW), 0, stream, a);
    e = hipGetLastError();
  }
  stage_mark(stream);
  if (e != hipSuccess) return e;
  if constexpr (pipe_kv(DK, DV)) {
    e = launch_bwd_kv_pipe(a, CAP, stream);   // fa_bwd_pipe.hip
  } else {
    constexpr int BQB = DK == 256 ? 32 : kPairBQB;
    using SH = PairShape<DK, DV, BQB>;
    constexpr int BKVB = 32 * SH::NP;
    const dim3 grid((unsigned)((a.T + BKVB - 1) / BKVB) * a.B * a.Hkv);
    hipLaunchKernelGGL((fa_bwd_dkdv_pair_kernel<DK, DV, BQB, CAP>), grid, dim3(64 * SH::NW), 0, stream,
                       a);
    e = hipGetLastError();
  }
  stage_mark(stream);
  return e;
}

template <int DK, int DV, int DQ_BKV = 32, int DQ_NW = 4>
static hipError_t launch_bwd_d(const BwdArgs& a, hipStream_t stream) {
  if (a.cap_log2e > 0.f) return launch_bwd_t<DK, DV, true, DQ_BKV, DQ_NW>(a, stream);
  return launch_bwd_t<DK, DV, false, DQ_BKV, DQ_NW>(a, stream);
}

const char* bwd_kernel_plan(int d, int d_v, int mode) {
  if (ds_mode_applies(mode, d, d_v)) return "rowdot,dkdv,dq_ds";
  if ((d == d_v && (d == 64 || d == 128 || d == 256)) || (d == 192 && d_v == 128)) return "dq,dkdv";
  return nullptr;
}

hipError_t launch_bwd_bf16(const BwdArgs& a, int d, int d_v, hipStream_t stream) {
  if (d == d_v) {
    switch (d) {
      case 64: return launch_bwd_d<64, 64, 64, 4>(a, stream);
      case 128: return launch_bwd_d<128, 128>(a, stream);
      case 256: return launch_bwd_d<256, 256>(a, stream);
    }
  } else if (d == 192 && d_v == 128) {
    return launch_bwd_d<192, 128, 32, 8>(a, stream);
  }
  return hipErrorInvalidValue;
}

}  // namespace fa
