// Software-pipelined passes of the causal flash-attention backward for
// gfx950 (bf16 in, fp32 accumulate), one wave per SIMD, with the same
// gradients as the kernels in fa_bwd.hip (dS = P (dP - D) and, under a
// softcap, the factor 1 - tanh^2):
//   fa_bwd_dq_pipe_kernel -- the dQ pass (dq = scale dS K) at d = 256 (one
//                            wave per SIMD) and d = 128 (two);
//   fa_bwd_kv_pipe_kernel -- the d = 128 dK/dV pass (dk = scale dS^T Q,
//                            dv = P^T dO), in place of the paired-wave one.
// They live in a file of their own because it is compiled with the VGPR form
// of the MFMA (their gradient accumulators are pinned to the AGPRs, so the
// score and dP products must not follow them there), which the paired-wave
// dK/dV kernel in fa_bwd.hip must not get.
#include <type_traits>

#include "device_common.h"
#include "internal.h"

namespace fa {

// dQ pass (head size 128 or 256), software-pipelined like the d = 256
// forward: one wave per 32 query rows holds the whole q and dO rows (D / 2
// VGPRs), dQ lives in the accumulation registers, and per 32-key unit i three
// MFMA blocks run, each carrying the VALU of another unit (a unit's 16 score
// elements spread over a block's MFMAs):
//   S(i+1)  = K(i+1) Q^T        carrying  dS(i) = f(i) (dP(i) - D), bf16 pack
//   dQ^T   += K(i)^T dS(i)^T    carrying  the cap's tanh and the mask of S(i+1)
//   dP(i+1) = V(i+1) dO^T - D   carrying  f(i+1) = P (1 - tanh^2) (P without a cap)
// The dP accumulators start from -D_i, so they end as dP - D.  Iteration i
// reads K(i) (transposed, for dQ), K(i+1) and V(i+1) while K(i+2) and V(i+2)
// load, so both tiles are triple-buffered (loop unrolled by three); one
// barrier per unit.  Units of the workgroup's key range outside a wave's band
// are computed fully masked (exact zeros), so every wave runs the same
// straight-line schedule.  Also writes D_i for the dK/dV pass.
// At d = 128 the working set fits two waves per SIMD (one is slower,
// measured).
template <int D, bool CAP>
__global__ __launch_bounds__(256, D >= 256 ? 1 : 2) void fa_bwd_dq_pipe_kernel(BwdArgs a) {
  constexpr int NW = 4, BQ = 32 * NW, BKV = 32;
  // a tile image, rounded up to whole rounds of the loaders' 1 KB pieces
  constexpr int TILE = TileDma<D, BKV, NW>::IMG;
  constexpr int NC = D / 16;     // chunks of the S and dP contractions
  constexpr int NDB = D / 32;    // 32-wide blocks of dq
  constexpr int NQ = 2 * NDB;    // MFMAs of the dQ block
  constexpr int PD = 2;
  // each block has NC = NQ MFMAs; the hooks of a block cover a unit's 16
  // score elements, EPB after each MFMA
  constexpr int EPB = 16 / NC;
  static_assert(NC == NQ && EPB * NC == 16, "16 elements over the MFMAs of a block");
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
    // D's fixed summation order (the stored-dS path's prologue computes the
    // same bits): an 8-term chain per 8-column chunk t = 2 c + g, then a
    // balanced tree over t with the pairs (t, t ^ 1) at its leaves
    float u[NC];
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      qreg[c] = qs[2 * c];
      doreg[c] = ds[2 * c];
      const bf16x8 ov = os[2 * c];
      float part = 0.f;
#pragma unroll
      for (int j = 0; j < 8; ++j) part += (float)doreg[c][j] * (float)ov[j];
      u[c] = xor32_sum(part);
    }
#pragma unroll
    for (int st = 1; st < NC; st <<= 1)
#pragma unroll
      for (int c = 0; c < NC; c += 2 * st) u[c] = u[c] + u[c + st];
    Di = u[0];
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
  // K(1) and V(1) load even past the last unit: the first step computes
  // S(1) and dP(1) whatever nu is, and a masked P of 0 times stale LDS
  // contents (possibly NaN) would not be 0; past T the range reads zeros
  dm.load(Kp, T * D * 2, kbuf(I0{}), t_lo * BKV, wave);
  dm.load(Vp, T * D * 2, vbuf(I0{}), t_lo * BKV, wave);
  dm.load(Kp, T * D * 2, kbuf(I1{}), (t_lo + 1) * BKV, wave);
  dm.load(Vp, T * D * 2, vbuf(I1{}), (t_lo + 1) * BKV, wave);
  wait_vmem();
  __syncthreads();
  using MT = std::true_type;
  using MF = std::false_type;
  s_block(I0{}, kbuf(I0{}), [&](int) {});
  part_a(I0{}, MT{}, 0, 0, 16);
  dp_block(I0{}, vbuf(I0{}), [&](int k) __attribute__((always_inline)) {
    part_b(I0{}, EPB * k, EPB * k + EPB);
  });

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
      part_c(x_c, EPB * k, EPB * k + EPB);
      if (k < PER)
        dm.load_piece(k, Kp, T * D * 2, kbuf(b2), (t_lo + i + 2) * BKV, wave);
      else if (k < 2 * PER)
        dm.load_piece(k - PER, Vp, T * D * 2, vbuf(b2), (t_lo + i + 2) * BKV, wave);
    });
    q_block(kbuf(b0), [&](int k) __attribute__((always_inline)) {
      part_a(XN{}, mask_c, i + 1, EPB * k, EPB * k + EPB);
    });
    dp_block(XN{}, vbuf(b1), [&](int k) __attribute__((always_inline)) {
      part_b(XN{}, EPB * k, EPB * k + EPB);
    });
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

// Head size 128, dK/dV pass, software-pipelined: one wave per SIMD owns 32
// key rows and does all of their work -- K and V rows in registers (the B
// operands of S = Q K^T and dP = dO V^T), dK^T and dV^T in the accumulation
// registers, P and dS never leaving the wave.  A workgroup (4 waves, 128
// keys) walks the 32-query units of the GQA group's heads that can see its
// keys; per unit i four MFMA blocks run, each carrying the VALU of a
// neighbouring unit:
//   S(i+1)   = Q(i+1) K^T          carrying  dS(i) = f(i) (dP(i) - D), bf16 pack,
//                                            and the tile loads of unit i+2
//   dK^T    += Q(i)^T dS(i)        carrying  the cap's tanh and the mask of S(i+1)
//   dP(i+1)  = dO(i+1) V^T - D     carrying  P(i+1) (bf16 pack) and f(i+1) =
//                                            P (1 - tanh^2) (P without a cap)
//   dV^T    += dO(i+1)^T P(i+1)
// (VALU under the blocks that read their operands transposed costs more
// than under those that read rows, measured.)
// Q and dO tiles and the row statistics (lse, -D) are triple-buffered in LDS,
// the buffer of each unit picked at run time; one barrier per unit.  Units of
// the workgroup's query range outside a wave's band are computed fully
// masked (exact zeros), so every wave runs the same schedule; units every
// row of which sees all 32 keys carry no mask.
// DS: each unit's dS (bf16, as packed for the dK product) is also written to
// the workspace a.dsw for the dQ pass that reads it (fa_bwd_ds.hip): the
// wave's 32 keys x 32 queries tile at slot (b, query head, query tile,
// key tile - query tile + nkt_ws - 1), lane L's 32 bytes at byte
// 64 (L % 32) + 32 (L / 32): row r of the tile is key r.  Units outside the
// band the workspace holds (fully masked ones, padding) are sent past the
// store's buffer range, which drops them: no branch.
template <bool CAP, bool DS>
__global__ __launch_bounds__(256, 1) void fa_bwd_kv_pipe_kernel(BwdArgs a) {
  constexpr int D = 128, NW = 4, BQ = 32, BKVB = 32 * NW;
  using Dma = TileDma<D, BQ, NW>;
  constexpr int TILE = Dma::IMG;   // a tile image, whole rounds of 1 KB pieces
  constexpr int PER = Dma::PER;
  constexpr int NC = D / 16;       // k steps of S and dP
  constexpr int NDB = D / 32;      // 32-wide blocks of dK and dV
  constexpr int NQ = 2 * NDB;      // MFMAs of the dK and dV blocks
  constexpr int PD = 2;   // operand reads run two MFMAs ahead (3: slower)
  constexpr int NSL = 3;   // buffers per tile kind
  static_assert(2 * PER <= NC, "one tile load per S MFMA");
  // one LDS object per buffer (the compiler then sees that a tile load
  // into one does not touch the tiles being read, and keeps it in flight)
  __shared__ __attribute__((aligned(1024))) char qs0[TILE];
  __shared__ __attribute__((aligned(1024))) char qs1[TILE];
  __shared__ __attribute__((aligned(1024))) char qs2[TILE];
  __shared__ __attribute__((aligned(1024))) char os0[TILE];
  __shared__ __attribute__((aligned(1024))) char os1[TILE];
  __shared__ __attribute__((aligned(1024))) char os2[TILE];
  __shared__ __attribute__((aligned(16))) float stat[NSL * 2 * BQ];   // [slot][lse2 | -D]

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = lane >> 5;
  const int l32 = lane & 31;
  const int T = a.T;
  const int W = a.window;
  const int G = a.H / a.Hkv;
  const int nkb = (T + BKVB - 1) / BKVB;
  const WorkItem w = decode_work(blockIdx.x, nkb, a.B, a.Hkv, 1, false);
  const int k0 = w.blk * BKVB;
  const int ka = k0 + 32 * wave;
  const int krow = ka + l32;
  const int kr = krow < T ? krow : T - 1;
  const size_t bkv = (size_t)w.b * a.Hkv + w.hkv;

  bf16x8 kreg[NC], vreg[NC];
  {
    const bf16x8* ks = (const bf16x8*)(a.k + (bkv * T + kr) * D + 8 * g);
    const bf16x8* vs = (const bf16x8*)(a.v + (bkv * T + kr) * D + 8 * g);
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      kreg[c] = ks[2 * c];
      vreg[c] = vs[2 * c];
    }
  }
  f32x16 dkacc[NDB], dvacc[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db)
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      dkacc[db][i] = 0.f;
      dvacc[db][i] = 0.f;
    }

  // query tiles that can see keys [k0, k0 + BKVB), for every head of the group
  const int qt_lo = k0 / BQ;
  const int q_hi = W > 0 ? min(T, k0 + BKVB - 1 + W) : T;
  const int nqt = (q_hi + BQ - 1) / BQ - qt_lo;
  const int niter = G * nqt;   // unit u: head u / nqt, tile u % nqt
  // query q sees this lane's key iff (unsigned)(q - krow) < span
  const unsigned span = W > 0 ? (unsigned)W : 0x7fffffffu;
  const float cexp = CAP ? a.cap_log2e : a.scale_log2e;

  Dma dm;
  dm.init(wave, lane);
  LaneOffs<D> lo;
  lo.init(lane);
  auto head_base = [&](int hi, const bf16* base) {
    const int hh = w.hkv * G + (hi < G ? hi : G - 1);
    return base + ((size_t)w.b * a.H + hh) * T * D;
  };
  // the statistics of a unit (lane < 32: lse, else D of row q0 + lane % 32),
  // fetched into a register and stored to LDS by wave 0 once the step's
  // loads are waited for.  Rows past T and units past the range get lse =
  // +inf and D = 0, so that their P is exactly 0 whatever the (zero) tiles
  // hold: no mask is needed for them.
  auto stat_load = [&](int hi, int ti) -> float {
    const int hh = w.hkv * G + (hi < G ? hi : G - 1);
    const int q = (qt_lo + ti) * BQ + l32;
    const float v = (g == 0 ? a.lse : a.Dst)[((size_t)w.b * a.H + hh) * T + (q < T ? q : T - 1)];
    return hi < G && q < T ? v : (g == 0 ? INFINITY : 0.f);
  };
  auto stat_store = [&](LDS_AS float* st, float v) {
    if (wave == 0) st[lane] = g == 0 ? v * kLog2e : -v;
  };
  // the dS store of unit (hi, ti): its workspace row (query tile) as a
  // buffer of nkt_ws slots, empty for units past the range
  const int kt_w = ka / 32;
  auto ds_rsrc = [&](int hi, int ti) {
    const int qt = qt_lo + ti;
    const int hh = w.hkv * G + (hi < G ? hi : G - 1);
    const int row = __builtin_amdgcn_readfirstlane(
        ((w.b * a.H + hh) * a.nqt_ws + (qt < a.nqt_ws ? qt : 0)) * a.nkt_ws);
    const int nrec = hi < G && qt < a.nqt_ws ? a.nkt_ws * 2048 : 0;
    return __builtin_amdgcn_make_buffer_rsrc(a.dsw + (size_t)row * 1024, 0,
                                             __builtin_amdgcn_readfirstlane(nrec), 0x00020000);
  };
  // slot of the unit's key tile in its query tile's row; outside the band a
  // slot far past any row's range (adding the lane offset cannot wrap it)
  auto ds_voff = [&](int ti) -> unsigned {
    const unsigned j0 = (unsigned)(kt_w - (qt_lo + ti) + a.nkt_ws - 1);
    const unsigned j = j0 < (unsigned)a.nkt_ws ? j0 : 0x40000u;
    return j * 2048u + 64u * l32 + 32u * g;
  };
  auto ds_store = [&](const __amdgpu_buffer_rsrc_t& rs, unsigned voff, int c, bf16x8 v) {
#if defined(__HIP_DEVICE_COMPILE__)
    __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, v), rs, voff + 16 * c, 0, 2);
#endif
  };

  f32x16 sacc;   // S of the unit being prepared, then its capped, masked score
  f32x16 fx;     // f of the unit whose dS is due: P (1 - tanh^2), or P
  f32x16 dp;     // dP - D of that unit
  f32x16 tt;     // cap: 1 - tanh^2 of the unit being prepared (0 where masked)
  bf16x8 pb[2], dsb[2];
  f32x4 lsev[4];

  // operands of the four products read from the LDS tiles: rows of Q or dO
  // (S, dP), or the tile read transposed (dK, dV)
  auto rows = [&](const LDS_AS char* X) {
    return [=, &lo](int k) { return lds_row_op<D>(X, lo, 0, k); };
  };
  auto cols = [&](const LDS_AS char* X) {
    return [=, &lo](int k) { return lds_tr_op<D>(X, lo, k / NDB, k % NDB); };
  };
  // cap and mask of the prepared unit's scores (tile at query q0), elements
  // [e0, e1); masked scores become -inf so that P = 0 (MASK false: every row
  // sees all of the wave's keys)
  auto part_a = [&](auto mask_c, int q0, int e0, int e1) __attribute__((always_inline)) {
    constexpr bool MASK = decltype(mask_c)::value;
    const int base = q0 + 4 * g - krow;
#pragma unroll
    for (int i = e0; i < e1; ++i) {
      const bool vis = !MASK || (unsigned)(base + 8 * (i >> 2) + (i & 3)) < span;
      float x = sacc[i];
      if (CAP) {
        const float e = fast_exp2(x * a.two_scale_over_cap_log2e);
        x = 1.f - 2.f * __builtin_amdgcn_rcpf(e + 1.f);   // tanh
        tt[i] = vis ? fmaf(-x, x, 1.f) : 0.f;
      }
      sacc[i] = vis ? x : -INFINITY;
    }
  };
  // P = 2^(S' c - lse) of the prepared unit, elements [e0, e1): bf16 packs of
  // P per 16-query chunk, f into fx
  auto part_b = [&](int e0, int e1) __attribute__((always_inline)) {
#pragma unroll
    for (int i = e0; i < e1; ++i) {
      const float p = fast_exp2(fmaf(sacc[i], cexp, -lsev[i >> 2][i & 3]));
      sacc[i] = p;
      fx[i] = CAP ? p * tt[i] : p;
      if (i == 7 || i == 15) {
        float tmp[8];
#pragma unroll
        for (int jj = 0; jj < 8; ++jj) tmp[jj] = sacc[i - 7 + jj];
        pb[i >> 3] = pack_bf16(tmp);
      }
    }
  };
  // dS = f (dP - D), elements [e0, e1), bf16 packs per chunk
  auto part_c = [&](int e0, int e1) __attribute__((always_inline)) {
#pragma unroll
    for (int i = e0; i < e1; ++i) {
      fx[i] *= dp[i];
      if (i == 7 || i == 15) {
        float tmp[8];
#pragma unroll
        for (int jj = 0; jj < 8; ++jj) tmp[jj] = fx[i - 7 + jj];
        dsb[i >> 3] = pack_bf16(tmp);
      }
    }
  };
  // statistics of the prepared unit: lse (log2) of the lane's rows, and -D
  // as the dP accumulator's start
  auto read_lse = [&](const LDS_AS float* st, int i4) __attribute__((always_inline)) {
    lsev[i4] = *(const LDS_AS f32x4*)(st + 8 * i4 + 4 * g);
  };
  auto read_negd = [&](const LDS_AS float* st, int i4) __attribute__((always_inline)) {
    const f32x4 d4 = *(const LDS_AS f32x4*)(st + BQ + 8 * i4 + 4 * g);
#pragma unroll
    for (int e = 0; e < 4; ++e) dp[4 * i4 + e] = d4[e];
  };
  using MT = std::true_type;
  using MF = std::false_type;
  using I0 = std::integral_constant<int, 0>;
  using I1 = std::integral_constant<int, 1>;
  using I2 = std::integral_constant<int, 2>;
  auto qbuf = [&](auto b_c) -> LDS_AS char* {
    constexpr int b = decltype(b_c)::value;
    return b == 0 ? (LDS_AS char*)qs0 : b == 1 ? (LDS_AS char*)qs1 : (LDS_AS char*)qs2;
  };
  auto obuf = [&](auto b_c) -> LDS_AS char* {
    constexpr int b = decltype(b_c)::value;
    return b == 0 ? (LDS_AS char*)os0 : b == 1 ? (LDS_AS char*)os1 : (LDS_AS char*)os2;
  };
  auto sbuf = [&](auto b_c) -> LDS_AS float* {
    return (LDS_AS float*)stat + decltype(b_c)::value * 2 * BQ;
  };

  // prologue: units 0 and 1 resident; S(0), its mask, dP(0) with P(0), dV(0)
  int h0 = 0, t0 = 0, h1 = 0, t1 = 0, h2 = 0, t2 = 0;   // units i, i+1, i+2 of iteration i
  auto advance = [&](int& hi, int& ti) {
    if (++ti == nqt) {
      ti = 0;
      ++hi;
    }
  };
  {
    dm.load(head_base(0, a.q), T * D * 2, qbuf(I0{}), qt_lo * BQ, wave);
    dm.load(head_base(0, a.dO), T * D * 2, obuf(I0{}), qt_lo * BQ, wave);
    const float v0 = stat_load(0, 0);
    advance(h1, t1);   // unit 1
    const int nb = niter > 1 ? T * D * 2 : 0;
    dm.load(head_base(h1, a.q), nb, qbuf(I1{}), (qt_lo + t1) * BQ, wave);
    dm.load(head_base(h1, a.dO), nb, obuf(I1{}), (qt_lo + t1) * BQ, wave);
    const float v1 = stat_load(h1, t1);
    wait_vmem();
    stat_store(sbuf(I0{}), v0);
    stat_store(sbuf(I1{}), v1);
    __syncthreads();
    h2 = h1;
    t2 = t1;
    advance(h2, t2);   // unit 2
  }
  {
    MfmaSeq<NC, PD> sq, pq;
    AgprSeq<NQ, PD> vq;
    const auto fS = rows(qbuf(I0{})), fP = rows(obuf(I0{}));
    const auto fV = cols(obuf(I0{}));
#pragma unroll
    for (int i = 0; i < 16; ++i) sacc[i] = 0.f;
    sq.start(fS);
    sq.run(fS, [&](int k) { return kreg[k]; }, [&](int) -> f32x16& { return sacc; }, [](int) {});
#pragma unroll
    for (int i4 = 0; i4 < 4; ++i4) {
      read_lse(sbuf(I0{}), i4);
      read_negd(sbuf(I0{}), i4);
    }
    part_a(MT{}, qt_lo * BQ, 0, 16);
    pq.start(fP);
    pq.run(fP, [&](int k) { return vreg[k]; }, [&](int) -> f32x16& { return dp; },
           [&](int k) __attribute__((always_inline)) { part_b(2 * k, 2 * k + 2); });
    vq.start(fV);
    vq.run(fV, [&](int k) { return pb[k / NDB]; }, [&](int k) -> f32x16& { return dvacc[k % NDB]; },
           [](int) {});
  }

  // iteration i: dK of unit i and units i+1 (prepared) and i+2 (loading) in
  // buffers b0, b1, b2 (compile-time: the loop is unrolled by three)
  auto step = [&](auto b0, auto b1, auto b2, auto mask_c) __attribute__((always_inline)) {
    lo.refresh();
    const bool more = h2 < G;   // unit i+2 exists
    const float sv = stat_load(h2, t2);
    const bf16* qsrc = head_base(h2, a.q);
    const bf16* osrc = head_base(h2, a.dO);
    const int nb = more ? T * D * 2 : 0;
    const int row2 = (qt_lo + t2) * BQ;
    const int q01 = (qt_lo + t1) * BQ;
    __amdgpu_buffer_rsrc_t drs;
    unsigned dvo = 0;
    if constexpr (DS) {
      drs = ds_rsrc(h0, t0);
      dvo = ds_voff(t0);
    }
    // S(i+1), carrying dS(i) and unit i+2's tile loads (one per MFMA,
    // branch-free: a wave with no piece k left loads zeros into the image's
    // partial last round).  Every block issues the next one's first operand
    // reads PD MFMAs before its end.  (Measured and not kept: the loads split
    // between the S and dP blocks, dS moved under the dV block, P split
    // between the dK and dP blocks.)
    MfmaSeq<NC, PD> sq, pq;
    AgprSeq<NQ, PD> kq, vq;
    const auto fS = rows(qbuf(b1)), fP = rows(obuf(b1));
    const auto fK = cols(qbuf(b0)), fV = cols(obuf(b1));
#pragma unroll
    for (int i = 0; i < 16; ++i) sacc[i] = 0.f;
    sq.start(fS);
    sq.run(fS, [&](int k) { return kreg[k]; }, [&](int) -> f32x16& { return sacc; },
           [&](int k) __attribute__((always_inline)) {
             part_c(2 * k, 2 * k + 2);
             if (k < PER)
               dm.load_piece(k, qsrc, nb, qbuf(b2), row2, wave);
             else if (k < 2 * PER)
               dm.load_piece(k - PER, osrc, nb, obuf(b2), row2, wave);
             // the step's two dS stores come after all of its loads, so
             // that the wait at its end can leave them in flight
             if constexpr (DS) {
               if (k == NC - 1) {
                 ds_store(drs, dvo, 0, dsb[0]);
                 ds_store(drs, dvo, 1, dsb[1]);
               }
             }
             if (k == NC - PD) kq.start(fK);
           });
    // dK(i), carrying the mask (and cap) of S(i+1) and its statistics (-D
    // as the start of dP(i+1))
    kq.run(fK, [&](int k) { return dsb[k / NDB]; }, [&](int k) -> f32x16& { return dkacc[k % NDB]; },
           [&](int k) __attribute__((always_inline)) {
             part_a(mask_c, q01, 2 * k, 2 * k + 2);
             if (k < 4)
               read_lse(sbuf(b1), k);
             else
               read_negd(sbuf(b1), k - 4);
             if (k == NQ - PD) pq.start(fP);
           });
    // dP(i+1), carrying P(i+1) and f(i+1)
    pq.run(fP, [&](int k) { return vreg[k]; }, [&](int) -> f32x16& { return dp; },
           [&](int k) __attribute__((always_inline)) {
             part_b(2 * k, 2 * k + 2);
             if (k == NC - PD) vq.start(fV);
           });
    // dV(i+1)
    vq.run(fV, [&](int k) { return pb[k / NDB]; }, [&](int k) -> f32x16& { return dvacc[k % NDB]; },
           [](int) {});
    stat_store(sbuf(b2), sv);
    // this step's loads (and everything older: vector-memory operations
    // report completion in issue order) are done; its dS stores, issued
    // last, may still be in flight until the next step's wait
    wait_vmem<DS ? 2 : 0>();
    lds_barrier();
    h0 = h1;
    t0 = t1;
    h1 = h2;
    t1 = t2;
    advance(h2, t2);
  };
  auto group = [&](auto mask_c) __attribute__((always_inline)) {
    step(I0{}, I1{}, I2{}, mask_c);
    step(I1{}, I2{}, I0{}, mask_c);
    step(I2{}, I0{}, I1{}, mask_c);
  };
  // niter iterations (the last finishes unit niter-1's dK), padded to whole
  // groups of three: the extra ones see units past the range (zero tiles,
  // P = 0) and add exact zeros.  Iteration i prepares unit i + 1; a group is
  // mask-free when all three of its units lie in a head's tiles [fl, fh),
  // those whose 32 x 32 blocks the wave sees whole.
  const int ng = (niter + 2) / 3;
  const int fl = min(nqt, wave + 1);
  const int fh = W > 0 ? (W >= 32 ? min(nqt, max(fl, wave + (W - 32) / 32 + 1)) : fl) : nqt;
  int gi = 0;
  for (int hi = 0; hi < G; ++hi) {
    const int u0 = hi * nqt + fl, u1 = hi * nqt + fh;   // its mask-free units [u0, u1)
    const int ga = min(ng, max(gi, (u0 + 1) / 3));      // first group with 3 g + 1 >= u0
    const int gb = min(ng, max(ga, u1 >= 4 ? (u1 - 4) / 3 + 1 : 0));   // 3 g + 3 < u1
    for (; gi < ga; ++gi) group(MT{});
    for (; gi < gb; ++gi) group(MF{});
  }
  for (; gi < ng; ++gi) group(MT{});

  agpr_acc_fence(dkacc);
  agpr_acc_fence(dvacc);
  if (krow < T) {
    bf16* dkp = a.dk + (bkv * T + krow) * D;
    bf16* dvp = a.dv + (bkv * T + krow) * D;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int i4 = 0; i4 < 4; ++i4) {
        bf16x4 vk, vv;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          vk[e] = (bf16)(dkacc[db][4 * i4 + e] * a.scale);
          vv[e] = (bf16)dvacc[db][4 * i4 + e];
        }
        *(bf16x4*)(dkp + 32 * db + 8 * i4 + 4 * g) = vk;
        *(bf16x4*)(dvp + 32 * db + 8 * i4 + 4 * g) = vv;
      }
  }
}

template <int D>
static hipError_t launch_dq_pipe_d(const BwdArgs& a, bool cap, hipStream_t stream) {
  const int nqb = (a.T + 127) / 128;
  const dim3 grid((unsigned)nqb * a.B * a.H);
  if (cap)
    hipLaunchKernelGGL((fa_bwd_dq_pipe_kernel<D, true>), grid, dim3(256), 0, stream, a);
  else
    hipLaunchKernelGGL((fa_bwd_dq_pipe_kernel<D, false>), grid, dim3(256), 0, stream, a);
  return hipGetLastError();
}

hipError_t launch_bwd_dq_pipe(const BwdArgs& a, int d, bool cap, hipStream_t stream) {
  if (d == 128) return launch_dq_pipe_d<128>(a, cap, stream);
  if (d == 256) return launch_dq_pipe_d<256>(a, cap, stream);
  return hipErrorInvalidValue;
}

hipError_t launch_bwd_kv_pipe(const BwdArgs& a, bool cap, hipStream_t stream) {
  const int nkb = (a.T + 127) / 128;
  const dim3 grid((unsigned)nkb * a.B * a.Hkv);
  const bool ds = a.dsw != nullptr;
  if (cap && ds)
    hipLaunchKernelGGL((fa_bwd_kv_pipe_kernel<true, true>), grid, dim3(256), 0, stream, a);
  else if (cap)
    hipLaunchKernelGGL((fa_bwd_kv_pipe_kernel<true, false>), grid, dim3(256), 0, stream, a);
  else if (ds)
    hipLaunchKernelGGL((fa_bwd_kv_pipe_kernel<false, true>), grid, dim3(256), 0, stream, a);
  else
    hipLaunchKernelGGL((fa_bwd_kv_pipe_kernel<false, false>), grid, dim3(256), 0, stream, a);
  return hipGetLastError();
}

}  // namespace fa
