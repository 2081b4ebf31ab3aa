// Device-side building blocks shared by the gfx950 attention kernels:
// vector types, the bf16 MFMA, LDS transpose reads, direct global -> LDS tile
// copies, the padded LDS tile layout and the work-item map.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fa {

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

#define LDS_AS __attribute__((address_space(3)))

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
// Running-max start value: finite, so exp2(m_old - m_new) never sees
// (-inf) - (-inf) when a row's first tiles are fully masked.
constexpr float kMaxInit = -1.0e30f;
// Headroom (log2 units) the online softmax allows before rescaling: p
// values stay below 2^20.  bf16 shares fp32's exponent range and every
// rounding is relative, so the headroom costs no precision; the fp32 sums
// of p v over up to 2^20 keys keep more than 2^80 of range.  A wide slack
// makes rescales rare: with logits of standard deviation 4 a row's max
// climbs about 10 log2 units past its first tile, and a rescale of a
// 32 x 256 accumulator costs as much VALU work as a whole tile.
constexpr float kRescaleSlack = 20.0f;

// v_mfma_f32_32x32x16_bf16.  Operand layout (measured on gfx950):
//   A: lane l holds A[row = l%32][k = 8*(l/32) + j], j = 0..7
//   B: lane l holds B[k = 8*(l/32) + j][col = l%32]
//   C: lane l, acc i holds C[row = 8*(i/4) + 4*(l/32) + i%4][col = l%32]
__device__ __forceinline__ f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// The same product with the accumulator held in the accumulation registers
// (AGPRs), for kernels whose long-lived accumulator does not fit beside
// their working set in the VGPRs.  Written as the instruction itself so that
// the accumulator's register class is fixed; the compiler's hazard tracking
// does not see it, so before any VALU access of such an accumulator (a
// rescale, the epilogue) the caller waits with agpr_acc_fence() -- the
// matrix core's write-back latency of a 32x32 product (at most 19 wait
// states for a 16-pass XDL op) -- and operands written by the VALU are
// never the instruction right before it.
__device__ __forceinline__ void mfma32_agpr(f32x16& acc, bf16x8 a, bf16x8 b) {
  asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+a"(acc) : "v"(a), "v"(b));
}
// The accumulators are operands of the wait, so no read of them can be
// scheduled ahead of it.
template <int N>
__device__ __forceinline__ void agpr_acc_fence(f32x16 (&acc)[N]) {
  static_assert(N == 4 || N == 8, "accumulator count");
  if constexpr (N == 8)
    asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7"
                 : "+a"(acc[0]), "+a"(acc[1]), "+a"(acc[2]), "+a"(acc[3]), "+a"(acc[4]),
                   "+a"(acc[5]), "+a"(acc[6]), "+a"(acc[7]));
  else
    asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7"
                 : "+a"(acc[0]), "+a"(acc[1]), "+a"(acc[2]), "+a"(acc[3]));
}

// Row index (within a 32-row MFMA output tile) held by accumulator i of a
// lane in half g = lane/32.
__device__ __forceinline__ int acc_row(int i, int g) {
  return 8 * (i >> 2) + 4 * g + (i & 3);
}

__device__ __forceinline__ float fast_exp2(float x) {
  return __builtin_amdgcn_exp2f(x);
}

// max over lanes l and l^32.
// Combine a value with the one in lane l ^ 32 through the gfx950 VGPR
// half-swap (v_permlane32_swap: lanes 32..63 of the first operand trade
// places with lanes 0..31 of the second), which stays in the VALU instead of
// a round trip through the LDS crossbar.  With both operands = x, the two
// results hold, in every lane, x[l] and x[l ^ 32] (in some order).
__device__ __forceinline__ float xor32_max(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                  false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float xor32_min(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                  false);
  return fminf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float xor32_sum(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                  false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Float atomic max through the integer order of IEEE-754 bit patterns
// (non-negative values order as signed ints, negative ones reversed as
// unsigned ints); the target must start at -inf or a real value.
__device__ __forceinline__ void atomic_max_f32(float* addr, float v) {
  // sign bit clear: larger float = larger int; set (incl. -0): smaller uint
  if (__float_as_int(v) >= 0)
    atomicMax((int*)addr, __float_as_int(v));
  else
    atomicMin((unsigned int*)addr, __float_as_uint(v));
}

// ---------------------------------------------------------------- RoPE
// Rotation of the interleaved pair (xe, xo) at position t by the angle
// fl32(t * f) (f from the host inverse-frequency table; accurate sincosf,
// angles reach ~1e4 rad); the backward rotates by -angle.  Every kernel that
// rotates uses these two definitions, so fused and standalone RoPE round
// identically.
__device__ __forceinline__ void rope_sincos(float t, float f, bool bwd, float& cs, float& sn) {
  sincosf(t * f, &sn, &cs);
  if (bwd) sn = -sn;
}
__device__ __forceinline__ void rope_pair(float cs, float sn, float& xe, float& xo) {
  const float ye = fmaf(xe, cs, -(xo * sn));
  const float yo = fmaf(xe, sn, xo * cs);
  xe = ye;
  xo = yo;
}

// ---------------------------------------------------------------- LDS tiles
// A tile of ROWS x D bf16 lives in LDS in rows of D*2 + 64 bytes (stride
// = 16 mod 64 dwords for d = 128, 256; 48 = -16 mod 64 for d = 64, 192:
// four consecutive rows start at the same four 16-dword bank offsets, in
// another order), with the 16-byte chunks of each aligned 64-byte
// group permuted by XOR with (row >> 2) & 3.  Measured on gfx950 (64 banks,
// 16 lanes per cycle for 16-byte reads, 32 lanes for the 8-byte transpose
// reads), this is conflict-free for both read patterns used here:
//   * 16-byte row reads of 16 consecutive rows, one column (row operands):
//     rows 4a+b land on dword 16b + 4*(chunk ^ a): 16 distinct groups;
//   * transpose reads, 4 consecutive rows x 64 contiguous bytes per 32
//     lanes: the rows start 16 dwords apart and the XOR stays inside each
//     row's 64-byte group.
// The XOR touches only the two low chunk bits, so every operand address is
// a per-lane base plus a compile-time immediate (no extra address
// registers in the unrolled loops).
template <int D>
struct Lay {
  static constexpr int STRIDE = D * 2 + 64;
  static constexpr int CPR = D / 8;  // 16-byte chunks per row
  template <int ROWS>
  static constexpr int bytes() { return ROWS * STRIDE; }
  // byte offset of element (r, col); col a multiple of 4
  __device__ __forceinline__ static int off(int r, int col) {
    return r * STRIDE + ((((col >> 3) ^ (r >> 2)) & 3) | ((col >> 3) & ~3)) * 16 +
           ((col & 7) << 1);
  }
};

// Direct global -> LDS tile copy (gfx950 buffer_load ... lds, 16 bytes per
// lane): each wave-level load writes 1 KB of LDS at consecutive addresses,
// lane l at +16 l, so the loader walks the padded tile image (Lay<D>) in
// 1 KB pieces and gives every lane the global chunk that belongs at its LDS
// position; lanes on row padding get an offset past the buffer, which the
// range check turns into a zero read with no memory traffic.  Rows past
// the buffer's end read as zeros as well (the buffer covers rows
// [0, nrows) of the slice), so no clamping is needed.  The data lands
// asynchronously: s_waitcnt vmcnt(0) before the barrier that publishes it.
// No staging registers: one offset per lane per 1 KB piece.

template <int D, int ROWS, int NW>
struct TileDma {
  static constexpr int STRIDE = Lay<D>::STRIDE;
  static constexpr int BYTES = ROWS * STRIDE;
  static_assert(BYTES % 1024 == 0, "tile image must be whole 1 KB pieces");
  static constexpr int NI = BYTES / 1024;          // pieces per tile
  static constexpr int PER = (NI + NW - 1) / NW;   // pieces per wave (last round ragged)
  static constexpr unsigned kOut = 0x7fffffffu;    // past any buffer: reads 0
  unsigned voff[PER];

  __device__ __forceinline__ void init(int wave, int lane) {
#pragma unroll
    for (int k = 0; k < PER; ++k) {
      const int P = (wave + k * NW) * 1024 + lane * 16;
      const int r = P / STRIDE;
      const int o = P % STRIDE;
      const int pc = o >> 4;
      const int lc = ((pc ^ (r >> 2)) & 3) | (pc & ~3);   // Lay<D>'s XOR is its own inverse
      voff[k] = (o < 2 * D && P < BYTES) ? (unsigned)(r * 2 * D + lc * 16) : kOut;
    }
  }
  // The descriptor of rows row0.. of the buffer [base, base + nbytes): its
  // base is the tile's first row and its size what is left of the buffer
  // (at least 0), so that the hardware range check -- which covers the
  // per-lane offset -- turns every byte past the buffer's end into a zero
  // read that touches no memory, whatever the tile's position.  The row
  // offset is the same in every lane; said explicitly, so that a value the
  // compiler merged through divergent code cannot turn it into a per-lane
  // loop.
  __device__ __forceinline__ static __amdgpu_buffer_rsrc_t rsrc(const void* base, int nbytes,
                                                                int row0) {
    const int off = __builtin_amdgcn_readfirstlane(row0 * 2 * D);
    const int left = nbytes - off;
    // raw buffer, 32-bit data format, no swizzle (gfx9 word 3)
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<char*>((const char*)base + off), 0,
                                             left > 0 ? left : 0, 0x00020000);
  }
  // rows row0 .. row0 + ROWS - 1 of the buffer [base, base + nbytes) into
  // the tile image at lds; AUX: the loads' cache policy (2: non-temporal,
  // for data read once)
  template <int AUX = 0>
  __device__ __forceinline__ void load(const void* base, int nbytes, LDS_AS char* lds, int row0,
                                       int wave) const {
#if defined(__HIP_DEVICE_COMPILE__)   // device-only builtins (the host pass only needs the stub)
    const __amdgpu_buffer_rsrc_t rs = rsrc(base, nbytes, row0);
#pragma unroll
    for (int k = 0; k < PER; ++k) {
      const int ins = wave + k * NW;
      if (ins < NI)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (LDS_AS void*)(lds + ins * 1024), 16, voff[k],
                                                 0, 0, AUX);
    }
#endif
  }
  // Load k (0 .. PER-1) of this wave's share of load(), alone: a caller
  // spreads the loads over its instruction stream, since a burst of them
  // stalls the wave until the memory pipeline has taken them.  Branch-free
  // (a branch per load would split the caller's instruction schedule): a
  // wave with no piece k left loads zeros (its offsets are out of range)
  // into the image's last, partial round, so the LDS buffer must hold IMG
  // bytes.
  static constexpr int IMG = PER * NW * 1024;
  __device__ __forceinline__ void load_piece(int k, const void* base, int nbytes, LDS_AS char* lds,
                                             int row0, int wave) const {
#if defined(__HIP_DEVICE_COMPILE__)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc(base, nbytes, row0),
                                             (LDS_AS void*)(lds + (wave + k * NW) * 1024), 16,
                                             voff[k], 0, 0, 0);
#endif
  }
};

// Waits until at most N of this wave's vector-memory operations (direct
// LDS loads among them) are outstanding -- vmcnt(N), the other counters left
// alone.  They complete in issue order, so N = the size of the newest batch
// waits for every older one.
template <int N = 0>
__device__ __forceinline__ void wait_vmem() {
  static_assert(N >= 0 && N < 64, "vmcnt is 6 bits");
  __builtin_amdgcn_s_waitcnt(0x0f70 | (N & 15) | ((N >> 4) << 14));
}

// Workgroup barrier between LDS tile phases.  __syncthreads() carries a
// workgroup release fence, which makes the compiler wait for every
// outstanding vector-memory operation -- every direct HBM->LDS load still in
// flight for later tiles -- before the barrier.  This barrier only finishes
// the wave's own LDS reads and writes (lgkmcnt(0)); the caller has already
// waited (wait_vmem) for the loads of the tile the barrier publishes.  The
// memory clobber keeps the compiler from moving LDS accesses across it.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// A operand for a 32-row MFMA block read along d: lane l gets
// tile[row0 + l%32][16*c + 8*(l/32) .. +7].
template <int D>
__device__ __forceinline__ bf16x8 lds_row_operand(const LDS_AS char* tile, int row0, int c,
                                                  int lane) {
  const int r = row0 + (lane & 31);
  const int col = 16 * c + 8 * (lane >> 5);
  return *(const LDS_AS bf16x8*)(tile + Lay<D>::off(r, col));
}

// Transposed operand for a contraction over tile rows: lane l gets
//   tile[row0 + 16*c16 + 8*(j/4) + 4*(l/32) + j%4][col0 + l%32], j = 0..7
// i.e. the A (or B) operand whose k index runs over rows in the order the
// 32x32 MFMA accumulator layout holds them.  Two ds_read_b64_tr_b16: within
// each 16-lane group, source lane r reads 4 elements of row (base + r/4) at
// column (col0 + 16*((l/16)%2) + 4*(r%4)); the hardware transpose hands
// lane i of the group element i of every source row.
template <int D>
__device__ __forceinline__ bf16x8 lds_tr_operand(const LDS_AS char* tile, int row0, int c16,
                                                 int col0, int lane) {
  const int r = lane & 15;
  const int g = lane >> 5;
  const int half = (lane >> 4) & 1;
  const int row = row0 + 16 * c16 + 4 * g + (r >> 2);
  const int col = col0 + 16 * half + 4 * (r & 3);
  s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (LDS_AS s16x4*)(tile + Lay<D>::off(row, col)));
  s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (LDS_AS s16x4*)(tile + Lay<D>::off(row + 8, col)));
  typedef short s16x8 __attribute__((ext_vector_type(8)));
  s16x8 v = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
  return __builtin_bit_cast(bf16x8, v);
}

// The same two read patterns with the per-lane part of the address
// computed once.  In a Lay<D> tile, moving the row operand by a 32-row
// block or by two 16-column chunks, and the transposed operand by a
// 16-row chunk or a 32-column block, moves whole rows or whole 64-byte
// groups and leaves the XOR alone, so every operand address is
//   tile + (one of four per-lane offsets) + a compile-time constant:
//   row operand (rows 32t.., chunk c):  row_e or row_o (c even / odd)
//                                       + 32t * STRIDE + 64 (c >> 1)
//   transposed (rows 16 c16.., cols 32 db..): tr_lo, tr_hi (its two
//                                       8-row reads) + 16 c16 * STRIDE + 64 db
// (the formulas are those of lds_row_operand / lds_tr_operand with the
// constant parts split off; checked against Lay<D>::off for d = 64..256).
template <int D>
struct LaneOffs {
  static constexpr int S = Lay<D>::STRIDE;
  int row_e, row_o, tr_lo, tr_hi;
  __device__ __forceinline__ void init(int lane) {
    const int l32 = lane & 31, g = lane >> 5, x = (l32 >> 2) & 3;
    const int r = lane & 15, half = (lane >> 4) & 1, b = (r & 3) >> 1;
    row_e = l32 * S + 16 * (g ^ x);
    row_o = l32 * S + 16 * ((2 + g) ^ x);
    tr_lo = (4 * g + (r >> 2)) * S + 16 * ((2 * half + b) ^ g) + 8 * (r & 1);
    tr_hi = (4 * g + (r >> 2) + 8) * S + 16 * ((2 * half + b) ^ (g + 2)) + 8 * (r & 1);
  }
  // hide the values from loop-invariant code motion: addresses derived
  // after this are recomputed where they are used instead of being hoisted
  // (one add per buffer) -- for loops that touch many LDS buffers
  __device__ __forceinline__ void refresh() {
    asm volatile("" : "+v"(row_e), "+v"(row_o), "+v"(tr_lo), "+v"(tr_hi));
  }
};

template <int D>
__device__ __forceinline__ bf16x8 lds_row_op(const LDS_AS char* tile, const LaneOffs<D>& o, int t,
                                             int c) {
  return *(const LDS_AS bf16x8*)(tile + ((c & 1) ? o.row_o : o.row_e) + 32 * t * Lay<D>::STRIDE +
                                 64 * (c >> 1));
}

template <int D>
__device__ __forceinline__ bf16x8 lds_tr_op(const LDS_AS char* tile, const LaneOffs<D>& o, int c16,
                                            int db) {
  const int imm = 16 * c16 * Lay<D>::STRIDE + 64 * db;
  s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS_AS s16x4*)(tile + o.tr_lo + imm));
  s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS_AS s16x4*)(tile + o.tr_hi + imm));
  typedef short s16x8 __attribute__((ext_vector_type(8)));
  s16x8 v = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
  return __builtin_bit_cast(bf16x8, v);
}

// A pinned sequence of N MFMAs acc(k) += A(k) B(k): A(k) from LDS through
// fetch(k), issued PD MFMAs ahead of its use (ring of PD + 1 operands), B(k)
// from registers; after MFMA k, hook(k) runs VALU work that does not wait for
// the MFMAs in flight, so the wave's own VALU fills the matrix unit's busy
// cycles.  start() issues the first PD fetches and may be called early (for
// instance from another sequence's hook) to hide their latency.
template <int N, int PD>
struct MfmaSeq {
  static_assert(PD >= 1, "reads run at least one MFMA ahead");
  static constexpr int R = PD + 1;
  bf16x8 op[R];
  template <class Fetch>
  __device__ __forceinline__ void start(Fetch&& fetch) {
#pragma unroll
    for (int k = 0; k < PD && k < N; ++k) op[k % R] = fetch(k);
    __builtin_amdgcn_sched_barrier(0);
  }
  template <class Fetch, class BOp, class Acc, class Hook>
  __device__ __forceinline__ void run(Fetch&& fetch, BOp&& bop, Acc&& acc, Hook&& hook) {
#pragma unroll
    for (int k = 0; k < N; ++k) {
      if (k + PD < N) op[(k + PD) % R] = fetch(k + PD);
      f32x16& c = acc(k);
      c = mfma32(op[k % R], bop(k), c);
      hook(k);
      __builtin_amdgcn_sched_barrier(0);
    }
  }
};

// MfmaSeq with the accumulators pinned to the AGPRs (mfma32_agpr): for
// kernels whose long-lived accumulators do not fit beside their working set
// in the VGPRs.  B operands written by the VALU must not be produced by the
// instruction right before the MFMA that reads them (the hook of an earlier
// MFMA, or earlier still, writes them).
template <int N, int PD>
struct AgprSeq {
  static constexpr int R = PD + 1;
  bf16x8 op[R];
  template <class Fetch>
  __device__ __forceinline__ void start(Fetch&& fetch) {
#pragma unroll
    for (int k = 0; k < PD && k < N; ++k) op[k % R] = fetch(k);
    __builtin_amdgcn_sched_barrier(0);
  }
  template <class Fetch, class BOp, class Acc, class Hook>
  __device__ __forceinline__ void run(Fetch&& fetch, BOp&& bop, Acc&& acc, Hook&& hook) {
#pragma unroll
    for (int k = 0; k < N; ++k) {
      if (k + PD < N) op[(k + PD) % R] = fetch(k + PD);
      mfma32_agpr(acc(k), op[k % R], bop(k));
      hook(k);
      __builtin_amdgcn_sched_barrier(0);
    }
  }
};

// acc[t] = sum_c A_t(c) B(c) over the D/16 chunks of d, where A_t(c) is
// the row operand of rows 32t.. of `tile` (read from LDS) and B(c) = breg[c]
// lives in registers: NS independent 32x32 accumulators.  The LDS operands
// of chunk c+1 are requested before the MFMAs of chunk c so their latency
// overlaps the matrix work.
template <int D, int NS>
__device__ __forceinline__ void mma_rows(f32x16 (&acc)[NS], const LDS_AS char* tile,
                                         const bf16x8 (&breg)[D / 16], int lane) {
  constexpr int NC = D / 16;
  bf16x8 op[2][NS];
#pragma unroll
  for (int t = 0; t < NS; ++t) {
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[t][i] = 0.f;
    op[0][t] = lds_row_operand<D>(tile, 32 * t, 0, lane);
  }
#pragma unroll
  for (int c = 0; c < NC; ++c) {
    if (c + 1 < NC) {
#pragma unroll
      for (int t = 0; t < NS; ++t) op[(c + 1) & 1][t] = lds_row_operand<D>(tile, 32 * t, c + 1, lane);
    }
#pragma unroll
    for (int t = 0; t < NS; ++t) acc[t] = mfma32(op[c & 1][t], breg[c], acc[t]);
  }
}

// Two independent products in one pass, their MFMAs alternating:
//   accA[t] = sum_c rows(tileA, 32t, c) bregA[c]   (DA/16 chunks)
//   accB[t] = sum_c rows(tileB, 32t, c) bregB[c]   (DB/16 chunks)
// LDS reads run PD chunks ahead through a ring of PD+1 operand sets: an LDS
// read takes about two MFMA durations to return, so reading just one chunk
// ahead stalls every MFMA.  The scheduling barrier after each chunk keeps
// the compiler from sinking the reads back next to their MFMAs.  PD = 0
// leaves the two products to the compiler's schedule (mma_rows each), which
// needs fewer registers.
template <int DA, int DB, int NS, int PD>
__device__ __forceinline__ void mma_rows2(f32x16 (&accA)[NS], const LDS_AS char* tileA,
                                          const bf16x8 (&bregA)[DA / 16], f32x16 (&accB)[NS],
                                          const LDS_AS char* tileB,
                                          const bf16x8 (&bregB)[DB / 16], int lane) {
  if constexpr (PD == 0) {
    // no pinned order: the compiler schedules (fewer live registers)
    mma_rows<DA, NS>(accA, tileA, bregA, lane);
    mma_rows<DB, NS>(accB, tileB, bregB, lane);
    return;
  }
  constexpr int NA = DA / 16, NB = DB / 16, NC = NA > NB ? NA : NB, R = PD + 1;
  bf16x8 opA[R][NS], opB[R][NS];
  auto fetch = [&](int c) __attribute__((always_inline)) {
#pragma unroll
    for (int t = 0; t < NS; ++t) {
      if (c < NA) opA[c % R][t] = lds_row_operand<DA>(tileA, 32 * t, c, lane);
      if (c < NB) opB[c % R][t] = lds_row_operand<DB>(tileB, 32 * t, c, lane);
    }
  };
#pragma unroll
  for (int t = 0; t < NS; ++t)
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      accA[t][i] = 0.f;
      accB[t][i] = 0.f;
    }
#pragma unroll
  for (int c = 0; c < PD; ++c) fetch(c);
#pragma unroll
  for (int c = 0; c < NC; ++c) {
    if (c + PD < NC) fetch(c + PD);
#pragma unroll
    for (int t = 0; t < NS; ++t) {
      if (c < NA) accA[t] = mfma32(opA[c % R][t], bregA[c], accA[t]);
      if (c < NB) accB[t] = mfma32(opB[c % R][t], bregB[c], accB[t]);
    }
    __builtin_amdgcn_sched_barrier(0);
  }
}

// One product acc[t] = sum_c rows(tile, 32t, c) breg[c], reads PD chunks
// ahead as in mma_rows2 (PD = 0: mma_rows).
template <int D, int NS, int PD>
__device__ __forceinline__ void mma_rows_pd(f32x16 (&acc)[NS], const LDS_AS char* tile,
                                            const bf16x8 (&breg)[D / 16], int lane) {
  if constexpr (PD == 0) {
    mma_rows<D, NS>(acc, tile, breg, lane);
    return;
  }
  constexpr int NC = D / 16, R = PD + 1;
  bf16x8 op[R][NS];
#pragma unroll
  for (int t = 0; t < NS; ++t)
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[t][i] = 0.f;
#pragma unroll
  for (int c = 0; c < PD; ++c)
#pragma unroll
    for (int t = 0; t < NS; ++t) op[c % R][t] = lds_row_operand<D>(tile, 32 * t, c, lane);
#pragma unroll
  for (int c = 0; c < NC; ++c) {
    if (c + PD < NC) {
#pragma unroll
      for (int t = 0; t < NS; ++t) op[(c + PD) % R][t] = lds_row_operand<D>(tile, 32 * t, c + PD, lane);
    }
#pragma unroll
    for (int t = 0; t < NS; ++t) acc[t] = mfma32(op[c % R][t], breg[c], acc[t]);
    __builtin_amdgcn_sched_barrier(0);
  }
}

// acc[db] += tr(tile, c16, col0 + 32 db) breg[c16] over c16 < NC16, db < NDB:
// a contraction over the tile's rows with the transposed LDS operand, its
// reads PD MFMAs ahead (ring of PD+1 operands), order pinned as above
// (PD = 0: plain loop, scheduled by the compiler).  start() issues the
// first PD reads; it can go before the VALU work that
// produces breg, so that their latency hides behind it.
template <int D, int NDB, int NC16, int PD>
struct TrPipe {
  static constexpr int N = NC16 * NDB, R = PD + 1;
  bf16x8 op[R];
  __device__ __forceinline__ void start(const LDS_AS char* tile, int col0, int lane) {
#pragma unroll
    for (int k = 0; k < PD && k < N; ++k)
      op[k % R] = lds_tr_operand<D>(tile, 0, k / NDB, col0 + 32 * (k % NDB), lane);
    if constexpr (PD > 0) __builtin_amdgcn_sched_barrier(0);   // keep them here
  }
  __device__ __forceinline__ void run(f32x16 (&acc)[NDB], const LDS_AS char* tile, int col0,
                                      const bf16x8 (&breg)[NC16], int lane) {
    if constexpr (PD == 0) {
#pragma unroll
      for (int k = 0; k < N; ++k)
        acc[k % NDB] = mfma32(lds_tr_operand<D>(tile, 0, k / NDB, col0 + 32 * (k % NDB), lane),
                              breg[k / NDB], acc[k % NDB]);
      return;
    }
#pragma unroll
    for (int k = 0; k < N; ++k) {
      if (k + PD < N)
        op[(k + PD) % R] =
            lds_tr_operand<D>(tile, 0, (k + PD) / NDB, col0 + 32 * ((k + PD) % NDB), lane);
      acc[k % NDB] = mfma32(op[k % R], breg[k / NDB], acc[k % NDB]);
      __builtin_amdgcn_sched_barrier(0);
    }
  }
  // as run(), with hook(k) after MFMA k: VALU work for the wave to issue
  // while the matrix unit is busy; it may fill breg[c16] for chunks whose
  // MFMAs come later (c16 > k / NDB).
  template <class Hook>
  __device__ __forceinline__ void run(f32x16 (&acc)[NDB], const LDS_AS char* tile, int col0,
                                      const bf16x8 (&breg)[NC16], int lane, Hook&& hook) {
    static_assert(PD > 0, "the hooked order is pinned");
#pragma unroll
    for (int k = 0; k < N; ++k) {
      if (k + PD < N)
        op[(k + PD) % R] =
            lds_tr_operand<D>(tile, 0, (k + PD) / NDB, col0 + 32 * ((k + PD) % NDB), lane);
      acc[k % NDB] = mfma32(op[k % R], breg[k / NDB], acc[k % NDB]);
      hook(k);
      __builtin_amdgcn_sched_barrier(0);
    }
  }
};

// Pack accumulators acc[8*h .. 8*h+7] of a 32x32 tile to 8 bf16 (RNE): the
// B operand of a contraction over the tile's rows (16 rows per chunk h).
__device__ __forceinline__ bf16x8 pack_bf16(const float* x) {
  bf16x8 r;
#pragma unroll
  for (int j = 0; j < 8; ++j) r[j] = (bf16)x[j];
  return r;
}

// ---------------------------------------------------------------- work map
// A unit is one (batch, KV head, block); a unit runs as G workgroups, one
// per query head of the GQA group (G = 1 for the key-parallel pass).  The
// dispatcher hands workgroup i to XCD i % 8.  When the (batch, KV head)
// pairs divide evenly over the 8 XCDs, XCD x is given a contiguous run of
// units -- whole heads, block after block -- so the workgroups running
// together on one XCD share their K/V (or Q/dO) windows in that XCD's
// 4 MB L2 instead of streaming them from HBM; otherwise units are dealt
// round-robin.  Within a head, blocks run heaviest first (`reverse` =
// true counts query blocks down: the last ones see the most keys).
struct WorkItem {
  int blk;   // query-block (or key-block) index
  int b;
  int hkv;
  int r;     // head within the GQA group
};

__device__ __forceinline__ WorkItem decode_work(int id, int nblk, int B, int Hkv, int G,
                                                bool reverse) {
  const int heads = B * Hkv;
  const int units = nblk * heads;
  int u, r;
  if ((heads & 7) == 0) {
    const int x = id & 7;
    const int j = id >> 3;
    r = j % G;
    u = x * (units >> 3) + j / G;
  } else {
    u = id / G;
    r = id % G;
  }
  WorkItem w;
  const int bhkv = u / nblk;
  const int bi = u % nblk;
  w.blk = reverse ? nblk - 1 - bi : bi;
  w.b = bhkv / Hkv;
  w.hkv = bhkv % Hkv;
  w.r = r;
  return w;
}

}  // namespace fa
