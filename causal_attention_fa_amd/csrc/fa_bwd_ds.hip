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
// written and read once.  At d = 128, 256 that traffic is far cheaper than
// the recomputation; the workspace ([B, H, T/32, band] tiles of 2 KB)
// is O(T x window), which one GPU's HBM holds at the sizes of interest.
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

// dQ pass from stored dS.  A workgroup (4 waves) owns 128 query rows of one
// (b, h); wave w the 32 rows of query tile qt_w.  It walks the key tiles
// that any of its rows can see; per tile the waves share the K tile (loaded
// into LDS together, padded Lay<D> image) and each loads its own 2 KB dS
// tile (two direct 1 KB loads, no padding); a key tile outside a wave's band
// has no slot, its loads fall outside the buffer range and read zeros.
// dQ^T (D x 32 queries, accumulator column = slot s) += K^T dS^T: 2 D / 32
// MFMAs per tile, K read transposed (lds_tr_op), dS read transposed
// (ds_tile_tr).  The dS tiles stream from HBM (read once) and run NSD - 1
// tiles ahead through a ring of NSD; the K tiles, which the G heads of a
// group and neighbouring query blocks share through L2, NK - 1 ahead through
// a ring of NK (NK <= NSD).  One barrier per tile.  The store writes slot s's
// row to query 32 qt_w + pi(s), scaled (and rotated back, with fused RoPE).
template <int D, int NK, int NSD>
__global__ __launch_bounds__(256, 2) void fa_bwd_dq_ds_kernel(BwdArgs a) {
  constexpr int NW = 4, BQ = 32 * NW, BKV = 32;
  using Dma = TileDma<D, BKV, NW>;
  constexpr int KIMG = Dma::IMG;
  constexpr int PER = Dma::PER;
  constexpr int NDB = D / 32;   // 32-wide blocks of dq
  constexpr int NQ = 2 * NDB;   // MFMAs per key tile
  constexpr int PD = 2;         // K operands read this many MFMAs ahead
  constexpr int R = PD + 1;
  constexpr int AS = NSD - 1;   // dS tiles in flight ahead of the one in use
  constexpr int AK = NK - 1;    // K tiles in flight ahead of the one in use
  static_assert(AK >= 1 && AK <= AS, "rings");
  __shared__ __attribute__((aligned(1024))) char kt[NK * KIMG];
  __shared__ __attribute__((aligned(1024))) char st[NSD * NW * 2048];

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
  const int qtw = q0 / BKV + wave;
  const size_t bh = (size_t)w.b * a.H + h;
  const size_t bkv = (size_t)w.b * a.Hkv + w.hkv;
  const bf16* Kp = a.k + bkv * T * D;
  const int nkt = a.nkt_ws;

  // key tiles [t_lo, t_hi] of the workgroup
  const int t_lo = W > 0 ? max(0, q0 - W + 1) / BKV : 0;
  const int t_hi = min(T, q0 + BQ) - 1;
  const int nu = t_hi / BKV - t_lo + 1;

  // this wave's workspace row (query tile qtw): nkt slots of 2 KB, empty
  // past the last query tile
  const int wrow = __builtin_amdgcn_readfirstlane((int)(bh * a.nqt_ws) +
                                                  (qtw < a.nqt_ws ? qtw : 0));
  const __amdgpu_buffer_rsrc_t srs = __builtin_amdgcn_make_buffer_rsrc(
      a.dsw + (size_t)wrow * nkt * 1024, 0,
      __builtin_amdgcn_readfirstlane(qtw < a.nqt_ws ? nkt * 2048 : 0), 0x00020000);

  Dma dm;
  dm.init(wave, lane);
  LaneOffs<D> lo;
  lo.init(lane);

  // K tile t_lo + u into buffer u % NK: every wave issues PER loads
  // (branch-free, as TileDma::load_piece does them)
  auto load_k = [&](int u) __attribute__((always_inline)) {
    LDS_AS char* kd = (LDS_AS char*)kt + (u % NK) * KIMG;
#pragma unroll
    for (int k = 0; k < PER; ++k) dm.load_piece(k, Kp, T * D * 2, kd, (t_lo + u) * BKV, wave);
  };
  // this wave's dS tile for key tile t_lo + u into ring slot u % NSD: two
  // loads; a slot outside the band is moved to kNoSlot, far past any row's
  // range, so that adding the lane offset cannot wrap it back into range
  constexpr unsigned kNoSlot = 0x40000u;
  auto load_s = [&](int u) __attribute__((always_inline)) {
    const unsigned j0 = (unsigned)(t_lo + u - qtw + nkt - 1);
    const unsigned j = j0 < (unsigned)nkt ? j0 : kNoSlot;
    LDS_AS char* sd = (LDS_AS char*)st + ((u % NSD) * NW + wave) * 2048;
#if defined(__HIP_DEVICE_COMPILE__)
#pragma unroll
    for (int p = 0; p < 2; ++p)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(srs, (LDS_AS void*)(sd + p * 1024), 16,
                                               j * 2048u + p * 1024 + 16 * lane, 0, 0, 0);
#endif
  };

  f32x16 acc[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db)
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[db][i] = 0.f;

  // Issue order: dS(0 .. AS - AK - 1), then K(v), dS(v + AS - AK) for
  // v < AK; iteration u then issues K(u + AK), dS(u + AS).  Vector-memory
  // operations complete in issue order, so at the top of iteration u it is
  // enough that at most NWAIT operations are outstanding -- those issued
  // after the later of K(u) and dS(u): with AK < AS, dS(u + AS - AK) and
  // the AK - 1 iterations after K(u)'s; with AK = AS (dS(u) right after
  // K(u)) the AK - 1 iterations after.  Near the end fewer were issued: wait
  // for all.
  constexpr int NWAIT = (AK < AS ? 2 : 0) + (AK - 1) * (PER + 2);
  static_assert(NWAIT < 64, "vmcnt");
#pragma unroll
  for (int u = 0; u < AS - AK; ++u)
    if (u < nu) load_s(u);
#pragma unroll
  for (int v = 0; v < AK; ++v) {
    if (v < nu) load_k(v);
    if (v + AS - AK < nu) load_s(v + AS - AK);
  }

  for (int u = 0; u < nu; ++u) {
    if (u + AS - 1 < nu) wait_vmem<NWAIT>();
    else wait_vmem();
    lds_barrier();
    // the buffers unit u - 1 used are free once every wave has passed the
    // barrier
    if (u + AK < nu) load_k(u + AK);
    if (u + AS < nu) load_s(u + AS);
    const LDS_AS char* kb = (const LDS_AS char*)kt + (u % NK) * KIMG;
    const LDS_AS char* sb = (const LDS_AS char*)st + ((u % NSD) * NW + wave) * 2048;
    bf16x8 dsop[2];
    dsop[0] = ds_tile_tr(sb, 0, lane);
    dsop[1] = ds_tile_tr(sb, 1, lane);
    auto f = [&](int k) { return lds_tr_op<D>(kb, lo, k / NDB, k % NDB); };
    bf16x8 op[R];
#pragma unroll
    for (int k = 0; k < PD; ++k) op[k] = f(k);
#pragma unroll
    for (int k = 0; k < NQ; ++k) {
      if (k + PD < NQ) op[(k + PD) % R] = f(k + PD);
      acc[k % NDB] = mfma32(op[k % R], dsop[k / NDB], acc[k % NDB]);
    }
  }

  // slot s = lane % 32 of the accumulator holds query 32 qtw + pi(s)
  const int s = lane & 31;
  const int qrow = qtw * BKV + 16 * ((s >> 3) & 1) + 8 * ((s & 7) >> 2) + 4 * (s >> 4) + (s & 3);
  if (qrow < T) {
    bf16* Qd = a.dq + (bh * T + qrow) * D;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int i4 = 0; i4 < 4; ++i4) {
        float x[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) x[e] = acc[db][4 * i4 + e] * a.scale;
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
    hipLaunchKernelGGL((fa_bwd_dq_ds_kernel<128, 4, 4>), grid, dim3(256), 0, stream, a);
  else if (d == 256)
    hipLaunchKernelGGL((fa_bwd_dq_ds_kernel<256, 2, 4>), grid, dim3(256), 0, stream, a);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace fa
