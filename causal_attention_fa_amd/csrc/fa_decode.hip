// Single-query decode attention over a preallocated KV cache, split along
// the cache (Forge commit "Add HF streaming data pipeline and three research
// reports", INFERENCE_RESEARCH.md, section 2: cache [layer][head][seq][d],
// a dedicated one-query kernel split-K along the cache; GQA is the largest
// saving in KV bandwidth).
//
// The work is bound by HBM: every visible K and V byte is read once and
// used by all G query heads of its KV group.  Two kernels:
//   * split: one or two waves per (batch, KV head, chunk of the cache).  K
//     and V tiles of 32 keys go straight from HBM into double-buffered LDS
//     (direct buffer loads, one tile ahead, non-temporal: the cache is read
//     once); the G query heads of the group are the columns of S^T = K Q^T, so the
//     contraction over d and P V run on the bf16 MFMA exactly as in the
//     prefill forward (columns past G are idle), and the VALU only does the
//     online softmax.  The chunk's unnormalised output O, running max m
//     (log2 units) and sum l go to a float32 scratch;
//   * combine: one wave per (batch, head) merges the chunks exactly by
//     their maxima and sums (o = sum_c 2^(m_c - M) O_c / L), adds the sink
//     to the normaliser, and writes o (bf16) and lse.
// Cache rows at or past the sequence's length are never read: the loads go
// through a buffer resource whose range ends at the sequence's last row, so
// rows past it read as zeros with no memory access, and the mask removes
// them from the softmax.
#include <type_traits>

#include "device_common.h"
#include "internal.h"

namespace fa {

// the cache is streamed once per call: non-temporal loads (cache policy 2)
constexpr int kDecAux = 2;   // cache policy bits of the direct tile loads (non-temporal)

constexpr int kDecBKV = 32;  // keys per tile

// NW waves per workgroup share the K/V tiles; each computes the (cheap,
// identical) scores and owns D/NW of the output columns (fewer accumulator
// registers per wave; at d = 256 one wave would spill).
template <int D, int NW, bool CAP>
__global__ __launch_bounds__(64 * NW, 2) void fa_decode_split_kernel(DecodeArgs a) {
  constexpr int NT = 64 * NW;
  constexpr int TILE = Lay<D>::template bytes<kDecBKV>();
  constexpr int NDB = D / 32 / NW;  // 32-wide output blocks per wave
  constexpr int NC = D / 16;
  // K, V tiles double-buffered, one LDS object per buffer (direct loads
  // into one while the other is read, without the compiler making the
  // reads wait for the loads)
  __shared__ __attribute__((aligned(1024))) char kb0[TILE];
  __shared__ __attribute__((aligned(1024))) char kb1[TILE];
  __shared__ __attribute__((aligned(1024))) char vb0[TILE];
  __shared__ __attribute__((aligned(1024))) char vb1[TILE];

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int d0 = wave * (D / NW);
  const int lane = tid & 63;
  const int g = lane >> 5;
  const int l32 = lane & 31;
  const int G = a.H / a.Hkv;
  const int unit = blockIdx.x;  // (batch, KV head, chunk), chunk fastest
  const int sp = unit % a.nsplit;
  const int bhkv = unit / a.nsplit;
  const int b = bhkv / a.Hkv;
  const int hkv = bhkv % a.Hkv;
  const int len = min(max(a.lens[b], 0), a.S);
  const int lo = a.window > 0 ? max(0, len - a.window) : 0;
  const int start = lo + sp * a.chunk;
  const int end = min(start + a.chunk, len);
  float* po = a.part_o + (size_t)unit * G * D;
  float* pml = a.part_ml + (size_t)unit * G * 2;
  if (start >= end) {
    // empty chunk: m = -inf, l = 0 and O = 0, so the combine can read every
    // chunk unconditionally (its weight is 0)
    for (int i = tid; i < G; i += NT) {
      pml[2 * i] = -INFINITY;
      pml[2 * i + 1] = 0.f;
    }
    for (int i = tid; i < G * D / 4; i += NT) ((f32x4*)po)[i] = f32x4{0.f, 0.f, 0.f, 0.f};
    return;
  }

  // The group's query heads as the B operand: lane column l32 = head
  // hkv*G + l32 (columns past G repeat the last head and are not written).
  bf16x8 qreg[NC];
  {
    const int r = min(l32, G - 1);
    const bf16x8* src = (const bf16x8*)(a.q + ((size_t)b * a.H + hkv * G + r) * D + 8 * g);
#pragma unroll
    for (int c = 0; c < NC; ++c) qreg[c] = src[2 * c];
  }

  const size_t base = (size_t)bhkv * a.S * D;
  const bf16* Kp = a.kc + base;
  const bf16* Vp = a.vc + base;
  const int ntiles = (end - start + kDecBKV - 1) / kDecBKV;
  const float cexp = CAP ? a.cap_log2e : a.scale_log2e;

  f32x16 oacc[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db)
#pragma unroll
    for (int i = 0; i < 16; ++i) oacc[db][i] = 0.f;
  float m = kMaxInit, l = 0.f;

  // the cache streams straight into LDS with non-temporal loads (read once
  // per call); rows at or past `end` read as zeros through the buffer range
  TileDma<D, kDecBKV, NW> kdm, vdm;
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
  kdm.template load<kDecAux>(Kp, end * D * 2, kbuf(I0{}), start, wave);
  vdm.template load<kDecAux>(Vp, end * D * 2, vbuf(I0{}), start, wave);
  wait_vmem();
  __syncthreads();
  auto step = [&](auto p_c, const int j) __attribute__((always_inline)) {
    using PN = std::integral_constant<int, 1 - decltype(p_c)::value>;
    const LDS_AS char* Kt = kbuf(p_c);
    const LDS_AS char* Vt = vbuf(p_c);
    const int kv0 = start + j * kDecBKV;
    if (j + 1 < ntiles) {
      kdm.template load<kDecAux>(Kp, end * D * 2, kbuf(PN{}), kv0 + kDecBKV, wave);
      vdm.template load<kDecAux>(Vp, end * D * 2, vbuf(PN{}), kv0 + kDecBKV, wave);
    }
    f32x16 sacc[1];
    mma_rows<D, 1>(sacc, Kt, qreg, lane);
    f32x16 s = sacc[0];
    if (CAP) {
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const float e = fast_exp2(s[i] * a.two_scale_over_cap_log2e);
        s[i] = 1.f - 2.f * __builtin_amdgcn_rcpf(e + 1.f);  // tanh
      }
    }
    if (kv0 + kDecBKV > end) {
#pragma unroll
      for (int i = 0; i < 16; ++i) s[i] = kv0 + acc_row(i, g) < end ? s[i] : -INFINITY;
    }
    float mt = -INFINITY;
#pragma unroll
    for (int i = 0; i < 16; ++i) mt = fmaxf(mt, s[i]);
    mt = xor32_max(mt) * cexp;
    if (__any(mt > m + kRescaleSlack)) {
      const float mnew = fmaxf(m, mt);
      const float alpha = fast_exp2(m - mnew);
      m = mnew;
      l *= alpha;
#pragma unroll
      for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int i = 0; i < 16; ++i) oacc[db][i] *= alpha;
    }
    float ps = 0.f;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const float p = fast_exp2(fmaf(s[i], cexp, -m));
      s[i] = p;
      ps += p;
    }
    l += ps;
    bf16x8 pb[2];
#pragma unroll
    for (int c16 = 0; c16 < 2; ++c16) {
      float tmp[8];
#pragma unroll
      for (int jj = 0; jj < 8; ++jj) tmp[jj] = s[8 * c16 + jj];
      pb[c16] = pack_bf16(tmp);
    }
#pragma unroll
    for (int c16 = 0; c16 < 2; ++c16)
#pragma unroll
      for (int db = 0; db < NDB; ++db)
        oacc[db] = mfma32(lds_tr_operand<D>(Vt, 0, c16, d0 + 32 * db, lane), pb[c16], oacc[db]);
    if (j + 1 < ntiles) wait_vmem();
    __syncthreads();
  };
  int j = 0;
  for (; j + 1 < ntiles; j += 2) {
    step(I0{}, j);
    step(I1{}, j + 1);
  }
  if (j < ntiles) step(I0{}, j);

  const float lt = xor32_sum(l);
  if (l32 < G) {
    // O^T accumulator: acc i of block db holds d = d0 + 32 db + acc_row(i, g)
    float* orow = po + (size_t)l32 * D + d0;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int i4 = 0; i4 < 4; ++i4) {
        f32x4 v;
#pragma unroll
        for (int e = 0; e < 4; ++e) v[e] = oacc[db][4 * i4 + e];
        *(f32x4*)(orow + 32 * db + 8 * i4 + 4 * g) = v;
      }
    if (g == 0 && wave == 0) {
      pml[2 * l32] = m;
      pml[2 * l32 + 1] = lt;
    }
  }
}

template <int D>
__global__ __launch_bounds__(64) void fa_decode_combine_kernel(DecodeArgs a) {
  constexpr int PER = D / 64;  // output elements per lane
  __shared__ float wsh[kDecMaxSplits];
  const int lane = threadIdx.x;
  const int G = a.H / a.Hkv;
  const int bh = blockIdx.x;
  const int b = bh / a.H;
  const int h = bh % a.H;
  const int hkv = h / G;
  const int r = h % G;
  const size_t unit0 = ((size_t)b * a.Hkv + hkv) * a.nsplit;
  const int ns = a.nsplit;

  float M = -INFINITY;
  for (int s = lane; s < ns; s += 64) {
    const float ms = a.part_ml[((unit0 + s) * G + r) * 2];
    M = fmaxf(M, ms);
  }
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) M = fmaxf(M, __shfl_xor(M, off));
  const bool has_sink = a.sinks != nullptr;
  const float sink2 = has_sink ? a.sinks[h] * kLog2e : -INFINITY;
  M = fmaxf(M, sink2);

  bf16* out = a.o + (size_t)bh * D + lane * PER;
  if (M == -INFINITY) {
    // no visible key and no sink: empty softmax
#pragma unroll
    for (int e = 0; e < PER; ++e) out[e] = (bf16)0.f;
    if (lane == 0 && a.lse) a.lse[bh] = -INFINITY;
    return;
  }
  float L = 0.f;
  for (int s = lane; s < ns; s += 64) {
    const float* e = a.part_ml + ((unit0 + s) * G + r) * 2;
    const float w = e[0] == -INFINITY ? 0.f : fast_exp2(e[0] - M);
    wsh[s] = w;
    L += w * e[1];
  }
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) L += __shfl_xor(L, off);
  if (has_sink) L += fast_exp2(sink2 - M);
  __syncthreads();

  // O rows of 8 chunks in flight at a time (every chunk's O is written, empty
  // ones as zeros with weight 0)
  constexpr int U = 8;
  float acc[PER];
#pragma unroll
  for (int e = 0; e < PER; ++e) acc[e] = 0.f;
  const float* base = a.part_o + (unit0 * G + r) * D + lane * PER;
  for (int s0 = 0; s0 < ns; s0 += U) {
    float wv[U], xv[U][PER];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int s = min(s0 + u, ns - 1);
      wv[u] = s0 + u < ns ? wsh[s] : 0.f;
      const float* src = base + (size_t)s * G * D;
#pragma unroll
      for (int e = 0; e < PER; ++e) xv[u][e] = src[e];
    }
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int e = 0; e < PER; ++e) acc[e] = fmaf(wv[u], xv[u][e], acc[e]);
  }
  const float inv = 1.f / L;
#pragma unroll
  for (int e = 0; e < PER; ++e) out[e] = (bf16)(acc[e] * inv);
  if (lane == 0 && a.lse) a.lse[bh] = (M + __log2f(L)) * kLn2;
}

// Waves per split workgroup: one at d = 64, two at 128 and 256 (each wave
// owning half of the output columns).  At d = 128 with at least 2048
// (b, KV head, chunk) units, one wave per workgroup: enough workgroups to keep the loads in flight, and no score
// recomputation per wave (qwen25-decode 5.56 -> 5.76 TB/s); with fewer
// units the two-wave split keeps more waves per CU (mistral-decode, 1024
// units, is 3 % faster with two).

template <int D, bool CAP>
static hipError_t launch_decode_t(const DecodeArgs& a, hipStream_t stream) {
  constexpr int NW = D == 64 ? 1 : 2;
  const unsigned units = (unsigned)a.B * a.Hkv * a.nsplit;
  bool one = false;
  if constexpr (D == 128 && NW != 1) {
    one = units >= 2048;
    if (one) fa_decode_split_kernel<D, 1, CAP><<<units, 64, 0, stream>>>(a);
  }
  if (!one) fa_decode_split_kernel<D, NW, CAP><<<units, 64 * NW, 0, stream>>>(a);
  stage_mark(stream);
  fa_decode_combine_kernel<D><<<(unsigned)a.B * a.H, 64, 0, stream>>>(a);
  stage_mark(stream);
  return hipGetLastError();
}

hipError_t launch_decode_bf16(const DecodeArgs& a, int d, bool cap, hipStream_t stream) {
  switch (d) {
    case 64: return cap ? launch_decode_t<64, true>(a, stream) : launch_decode_t<64, false>(a, stream);
    case 128: return cap ? launch_decode_t<128, true>(a, stream) : launch_decode_t<128, false>(a, stream);
    case 256: return cap ? launch_decode_t<256, true>(a, stream) : launch_decode_t<256, false>(a, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace fa
