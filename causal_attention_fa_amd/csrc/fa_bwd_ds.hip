// dQ of the causal flash-attention backward taken from stored dS (gfx950,
// bf16 operands, fp32 accumulate), for head sizes 128 and 256:
//   fa_bwd_rowdot_kernel -- the backward's prologue on its own: D_i =
//                           <dO_i, o_i> for every row (the dK/dV pass
//                           needs it before any dQ work has run);
//   fa_bwd_dq_ds_kernel  -- dq = scale dS K with dS read back from the
//                           workspace the dK/dV pass filled.
// The dK/dV pass forms every visible dS element anyway (dK = scale dS^T Q);
// writing it out as bf16 -- the precision the dQ product consumes it in --
// turns the dQ pass from S, dP and dQ products (6d flops per visible pair)
// into the dQ product alone (2d), at the price of 2 bytes per visible pair
// written and read once.  At d = 256 that traffic costs far less than the
// 4d of recomputation it replaces; at d = 128 the two are close and the
// recomputing pass measured faster where the dS volume is large (the dK/dV
// pass's stores cost more per byte there).  The workspace ([B, H, T/32,
// band] tiles of 2 KB) is O(T x window), which one GPU's HBM holds at the
// sizes of interest.
//
// Workspace layout: tile (b, h, qt, j) holds dS for query tile qt (queries
// 32 qt ..) and key tile kt = qt - nkt + 1 + j, as the dK/dV pass's wave
// holds it: 32 key rows of 64 bytes, row r (key 32 kt + r) = the two bf16x8
// packs of lane r, then the two of lane r + 32.  Slot s (s = 16 g + 8 c + e,
// g the lane half, c the pack, e the element) of a row holds query
//   pi(s) = 16 c + 8 (e / 4) + 4 g + e % 4
// (the query order of the MFMA accumulator the packs come from).
#include <type_traits>

#include "device_common.h"
#include "internal.h"

namespace fa {

// D_i = sum_c dO[i][c] o[i][c] (bf16 inputs, fp32 sums) in the fixed order
// the recomputing dQ pass uses too, so that both strategies hand the dK/dV
// pass the same bits: D / 8 lanes per row, lane t an 8-term chain over its
// 16-byte chunk (columns 8 t ..), then a butterfly over the row's lanes
// (xor 1, 2, 4, ...: a balanced tree whose leaves pair chunks t, t ^ 1;
// every lane ends with the same sum).  Consecutive lanes read consecutive
// chunks of a row.
template <int D>
__global__ __launch_bounds__(256) void fa_bwd_rowdot_kernel(const bf16* __restrict__ o,
                                                            const bf16* __restrict__ dO,
                                                            float* __restrict__ Dst, long rows) {
  constexpr int LPR = D / 8;
  const long row = ((long)blockIdx.x * 256 + threadIdx.x) / LPR;
  const int t = threadIdx.x % LPR;
  float part = 0.f;
  if (row < rows) {
    const bf16x8 dv = *(const bf16x8*)(dO + row * D + 8 * t);
    const bf16x8 ov = *(const bf16x8*)(o + row * D + 8 * t);
#pragma unroll
    for (int j = 0; j < 8; ++j) part += (float)dv[j] * (float)ov[j];
  }
#pragma unroll
  for (int off = 1; off < LPR; off <<= 1) part = part + __shfl_xor(part, off);
  if (row < rows && t == 0) Dst[row] = part;
}

// Transposed operand from a dS tile image in LDS (32 rows of 64 bytes, no
// padding): lane l gets tile[16 c16 + 8 (j / 4) + 4 (l / 32) + j % 4][l % 32],
// j = 0..7 -- the B operand of dQ^T += K^T dS^T for key chunk c16, in the
// key order the transposed K operand uses.  Same two ds_read_b64_tr_b16 as
// lds_tr_operand; each 32-lane half reads 4 consecutive rows = 256
// contiguous bytes, so every bank once.
__device__ __forceinline__ bf16x8 ds_tile_tr(const LDS_AS char* tile, int c16, int lane) {
  const int r = lane & 15;
  const int g = lane >> 5;
  const int half = (lane >> 4) & 1;
  const int row = 16 * c16 + 4 * g + (r >> 2);
  const int col = 16 * half + 4 * (r & 3);
  s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS_AS s16x4*)(tile + row * 64 + col * 2));
  s16x4 hi =
      __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS_AS s16x4*)(tile + (row + 8) * 64 + col * 2));
  typedef short s16x8 __attribute__((ext_vector_type(8)));
  s16x8 v = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
  return __builtin_bit_cast(bf16x8, v);
}

// dQ pass from stored dS.  A workgroup (4 waves) owns 128 query rows (query
// tiles qt_0 .. qt_0 + 3) of one (b, h) and walks the key tiles that any of
// its rows can see.  Per key tile the waves share the K tile (padded Lay<D>
// image) and the four 2 KB dS tiles (unpadded images); a key tile outside a
// query tile's band has no slot, its loads fall outside the buffer range and
// read zeros.  Wave w computes dQ^T (accumulator column = slot s) += K^T dS^T
// for query tiles 2 (w / 2) and 2 (w / 2) + 1 and the half w % 2 of d: each
// transposed K operand it reads (lds_tr_op) feeds two MFMAs, one per query
// tile; dS read transposed (ds_tile_tr).
// Loads go through registers, split by kind between the waves: waves 0 and
// 1 load the K tiles (mostly L2 hits) AK = 2 tiles ahead, waves 2 and 3 the
// dS tiles of all four query tiles (streamed from HBM, read once) AH = 4
// tiles ahead, each from a ring of register sets; at its tile's step a wave
// writes its registers into the LDS slot (where a direct load of the tile
// image would have put them) just before the barrier that publishes it.  A
// wave's vector-memory operations complete in issue order, so it waits for
// its oldest tile alone, and with one kind per wave neither kind waits
// behind the other.  (Direct HBM -> LDS loads kept in flight across a
// barrier made the compiler wait for all of them before any LDS read: the
// tiles then got one step of latency, too little for HBM; d = 256 dQ from
// dS 0.37 -> 0.34 ms at gemma-global, 0.32 -> 0.27 at gemma-local.)  The two
// kinds run separate copies of the loop (the same steps and barriers), so
// that the compiler's wait tracking of one kind never merges with the
// other's.  The loads of a tile are spread one per MFMA of the step that
// issues them and are branch-free (past the last tile they read an empty
// range, so every wave issues the same count per step and the waits are
// exact).  Two LDS slots, each an object of its own, and the loop unrolled by
// four, so slots and register sets are compile-time choices; the loop is
// padded to whole groups, and a tile past the last reads zeros and adds exact
// zeros.  The store writes slot s's row to query 32 qt + pi(s), scaled (and
// rotated back, with fused RoPE).
template <int D>
__global__ __launch_bounds__(256, 2) void fa_bwd_dq_ds_kernel(BwdArgs a) {
  constexpr int NW = 4, BQ = 32 * NW, BKV = 32;
  using Dma = TileDma<D, BKV, 2>;   // the K tiles: waves 0 and 1
  constexpr int KIMG = Dma::IMG;
  constexpr int KPER = Dma::PER;    // loads per tile of a K wave
  constexpr int SPER = 4;           // loads per tile of a dS wave (2 tiles x 2 KB)
  constexpr int NDB = D / 32;       // 32-wide blocks of dq
  constexpr int NDH = NDB / 2;      // the blocks of one half of d
  constexpr int NKO = 2 * NDH;      // K operands per tile (each feeds 2 MFMAs)
  constexpr int PD = 2;             // K operands read this many ahead
  constexpr int R = PD + 1;
  static_assert(KPER <= 2 * NKO && SPER <= 2 * NKO, "one load per MFMA");
  __shared__ __attribute__((aligned(1024))) char kt0[KIMG];
  __shared__ __attribute__((aligned(1024))) char kt1[KIMG];
  __shared__ __attribute__((aligned(1024))) char st0[NW * 2048];
  __shared__ __attribute__((aligned(1024))) char st1[NW * 2048];
  using I0 = std::integral_constant<int, 0>;
  using I1 = std::integral_constant<int, 1>;
  auto kbuf = [&](auto c) -> LDS_AS char* {
    constexpr int b = decltype(c)::value;
    return b == 0 ? (LDS_AS char*)kt0 : (LDS_AS char*)kt1;
  };
  auto sbuf = [&](auto c) -> LDS_AS char* {
    constexpr int b = decltype(c)::value;
    return b == 0 ? (LDS_AS char*)st0 : (LDS_AS char*)st1;
  };

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const bool kwave = wave < 2;
  const int g = lane >> 5;
  const int T = a.T;
  const int W = a.window;
  const int G = a.H / a.Hkv;
  const int nqb = (T + BQ - 1) / BQ;
  const WorkItem w = decode_work(blockIdx.x, nqb, a.B, a.Hkv, G, true);
  const int h = w.hkv * G + w.r;
  const int q0 = w.blk * BQ;
  const int qp = wave >> 1;   // its query tiles 2 qp, 2 qp + 1 (of the four)
  const int dh = wave & 1;    // its half of d
  const size_t bh = (size_t)w.b * a.H + h;
  const size_t bkv = (size_t)w.b * a.Hkv + w.hkv;
  const bf16* Kp = a.k + bkv * T * D;
  const int nkt = a.nkt_ws;

  // key tiles [t_lo, t_hi] of the workgroup
  const int t_lo = W > 0 ? max(0, q0 - W + 1) / BKV : 0;
  const int t_hi = min(T, q0 + BQ) - 1;
  const int nu = t_hi / BKV - t_lo + 1;

  // a dS wave loads the tiles of query tiles qt_0 + cw0 + i, i = 0, 1: each
  // one's workspace row as a buffer of nkt slots of 2 KB, empty past the
  // last query tile
  const int cw0 = kwave ? 0 : 2 * (wave - 2);
  __amdgpu_buffer_rsrc_t srs[2];
  int sq[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    sq[i] = q0 / BKV + cw0 + i;
    const int row = __builtin_amdgcn_readfirstlane((int)(bh * a.nqt_ws) +
                                                   (sq[i] < a.nqt_ws ? sq[i] : 0));
    srs[i] = __builtin_amdgcn_make_buffer_rsrc(
        a.dsw + (size_t)row * nkt * 1024, 0,
        __builtin_amdgcn_readfirstlane(sq[i] < a.nqt_ws ? nkt * 2048 : 0), 0x00020000);
  }

  Dma dm;
  dm.init(wave & 1, lane);
  LaneOffs<D> lo;
  lo.init(lane);

  // K wave: piece p of K tile v (t_lo + v) -- the 16 bytes a direct load of
  // the padded tile image would put at this lane's place in piece
  // (wave & 1) + 2 p -- into registers, AK tiles ahead; past the last tile
  // the range is empty (zeros, no traffic)
  constexpr int AK = 2;
  u32x4 stk[AK][KPER];
  auto load_kr = [&](int p, int v) __attribute__((always_inline)) -> u32x4 {
#if defined(__HIP_DEVICE_COMPILE__)
    return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(
                                         Dma::rsrc(Kp, v < nu ? T * D * 2 : 0, (t_lo + v) * BKV),
                                         dm.voff[p], 0, 0));
#else
    return u32x4{};
#endif
  };
  auto put_k = [&](const u32x4 (&r)[KPER], auto c) __attribute__((always_inline)) {
#pragma unroll
    for (int p = 0; p < KPER; ++p)
      *(LDS_AS u32x4*)(kbuf(c) + ((wave & 1) + 2 * p) * 1024 + 16 * lane) = r[p];
  };
  // dS wave: piece p (query tile cw0 + (p >> 1), half p & 1) of dS tile v
  // into registers; a slot outside the band or past the last tile is moved to
  // kNoSlot, far past any row's range, so that adding the lane offset cannot
  // wrap it back into range: zeros, no traffic
  constexpr unsigned kNoSlot = 0x40000u;
  constexpr int AH = 4;
  u32x4 stg[AH][SPER];
  auto load_s = [&](int p, int v) __attribute__((always_inline)) -> u32x4 {
    const int i = p >> 1;
    const unsigned j0 = (unsigned)(t_lo + v - sq[i] + nkt - 1);
    const unsigned j = v < nu && j0 < (unsigned)nkt ? j0 : kNoSlot;
#if defined(__HIP_DEVICE_COMPILE__)
    return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(
                                         srs[i], j * 2048u + (p & 1) * 1024 + 16 * lane, 0, 0));
#else
    return u32x4{};
#endif
  };
  // ... and its registers into LDS slot c at the places a direct load would
  // have written them (lane l at + 16 l of each 1 KB half)
  auto put_s = [&](const u32x4 (&r)[SPER], auto c) __attribute__((always_inline)) {
#pragma unroll
    for (int p = 0; p < SPER; ++p)
      *(LDS_AS u32x4*)(sbuf(c) + (cw0 + (p >> 1)) * 2048 + (p & 1) * 1024 + 16 * lane) = r[p];
  };

  f32x16 acc[2][NDH];
#pragma unroll
  for (int qi = 0; qi < 2; ++qi)
#pragma unroll
    for (int db = 0; db < NDH; ++db)
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[qi][db][i] = 0.f;

  using I2 = std::integral_constant<int, 2>;
  using I3 = std::integral_constant<int, 3>;
  // tile u: LDS slot c (K tile u + 1 loading into slot n, the one tile u - 1
  // used), dS registers x (refilled with tile u + AH once in LDS)
  auto step = [&](auto kind, const int u, auto c, auto n, auto x) __attribute__((always_inline)) {
    constexpr bool KW = decltype(kind)::value;
    constexpr int X = decltype(x)::value;
    if constexpr (KW) {
      // tile u's registers are this wave's oldest outstanding loads
      wait_vmem<(AK - 1) * KPER>();
      put_k(stk[X % AK], c);
    } else {
      // tile u's registers are this wave's oldest outstanding loads
      wait_vmem<(AH - 1) * SPER>();
      put_s(stg[X], c);
    }
    lds_barrier();
    const LDS_AS char* kb = kbuf(c);
    const LDS_AS char* sb = sbuf(c) + 2 * qp * 2048;
    bf16x8 dsop[2][2];   // [query tile][key chunk]
#pragma unroll
    for (int qi = 0; qi < 2; ++qi)
#pragma unroll
      for (int cc = 0; cc < 2; ++cc) dsop[qi][cc] = ds_tile_tr(sb + qi * 2048, cc, lane);
    // K operand k: key chunk k / NDH, block dh NDH + k % NDH of d
    auto f = [&](int k) { return lds_tr_op<D>(kb, lo, k / NDH, dh * NDH + k % NDH); };
    bf16x8 op[R];
#pragma unroll
    for (int k = 0; k < PD; ++k) op[k] = f(k);
#pragma unroll
    for (int k = 0; k < NKO; ++k) {
      if (k + PD < NKO) op[(k + PD) % R] = f(k + PD);
#pragma unroll
      for (int qi = 0; qi < 2; ++qi) {
        acc[qi][k % NDH] = mfma32(op[k % R], dsop[qi][k / NDH], acc[qi][k % NDH]);
        const int m = 2 * k + qi;
        if constexpr (KW) {
          if (m < KPER) stk[X % AK][m] = load_kr(m, u + AK);
        } else {
          if (m < SPER) stg[X][m] = load_s(m, u + AH);
        }
      }
    }
  };
  auto run = [&](auto kind) __attribute__((always_inline)) {
    // up front: K tile 0 into slot 0; dS tiles 0 .. AH - 1 into the registers
    if constexpr (decltype(kind)::value) {
#pragma unroll
      for (int v = 0; v < AK; ++v)
#pragma unroll
        for (int p = 0; p < KPER; ++p) stk[v][p] = load_kr(p, v);
    } else {
#pragma unroll
      for (int v = 0; v < AH; ++v)
#pragma unroll
        for (int p = 0; p < SPER; ++p) stg[v][p] = load_s(p, v);
    }
    for (int u = 0; u < nu; u += AH) {
      step(kind, u, I0{}, I1{}, I0{});
      step(kind, u + 1, I1{}, I0{}, I1{});
      step(kind, u + 2, I0{}, I1{}, I2{});
      step(kind, u + 3, I1{}, I0{}, I3{});
    }
  };
  if (kwave)
    run(std::true_type{});
  else
    run(std::false_type{});

  // slot s = lane % 32 of query tile qi's accumulator holds query
  // 32 (qt_0 + 2 qp + qi) + pi(s); its blocks are dh NDH .. of d
  const int s = lane & 31;
  const int ps = 16 * ((s >> 3) & 1) + 8 * ((s & 7) >> 2) + 4 * (s >> 4) + (s & 3);
#pragma unroll
  for (int qi = 0; qi < 2; ++qi) {
    const int qrow = (q0 / BKV + 2 * qp + qi) * BKV + ps;
    if (qrow < T) {
      bf16* Qd = a.dq + (bh * T + qrow) * D;
#pragma unroll
      for (int j = 0; j < NDH; ++j)
#pragma unroll
        for (int i4 = 0; i4 < 4; ++i4) {
          const int db = dh * NDH + j;
          float x[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) x[e] = acc[qi][j][4 * i4 + e] * a.scale;
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
}

hipError_t launch_bwd_rowdot(const BwdArgs& a, int d, hipStream_t stream) {
  const long rows = (long)a.B * a.H * a.T;
  const long threads = rows * (d / 8);
  const dim3 grid((unsigned)((threads + 255) / 256));
  if (d == 128)
    hipLaunchKernelGGL(fa_bwd_rowdot_kernel<128>, grid, dim3(256), 0, stream, a.o, a.dO, a.Dst, rows);
  else if (d == 256)
    hipLaunchKernelGGL(fa_bwd_rowdot_kernel<256>, grid, dim3(256), 0, stream, a.o, a.dO, a.Dst, rows);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

hipError_t launch_bwd_dq_ds(const BwdArgs& a, int d, hipStream_t stream) {
  const int nqb = (a.T + 127) / 128;
  const dim3 grid((unsigned)nqb * a.B * a.H);
  if (d == 128)
    hipLaunchKernelGGL(fa_bwd_dq_ds_kernel<128>, grid, dim3(256), 0, stream, a);
  else if (d == 256)
    hipLaunchKernelGGL(fa_bwd_dq_ds_kernel<256>, grid, dim3(256), 0, stream, a);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace fa
