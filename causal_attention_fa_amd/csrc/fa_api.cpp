// C-ABI layer of libfa.so (declared in include/fa.h): argument validation,
// error reporting, window resolution, kernel selection and stream-ordered
// scratch.  Every check runs before any HIP call; no exception crosses the
// interface.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <cmath>
#include <cstdint>
#include <cstdlib>
#include <cstring>
#include <mutex>
#include <string>

#include "fa.h"
#include "internal.h"

namespace {

thread_local std::string g_last_error;

// Stage events armed by fa_set_stage_events (per thread).
constexpr int kMaxStageEvents = 16;
thread_local hipEvent_t g_stage_ev[kMaxStageEvents];
thread_local int g_stage_n = 0;
thread_local int g_stage_next = 0;

void stage_begin(hipStream_t stream) {
  if (g_stage_n <= 0) return;
  hipEventRecord(g_stage_ev[0], stream);
  g_stage_next = 1;
}

int fail(int code, const std::string& msg) {
  g_last_error = msg;
  return code;
}

bool debug_sync() {
  static const bool on = [] {
    const char* e = std::getenv("FA_DEBUG_SYNC");
    return e && e[0] && e[0] != '0';
  }();
  return on;
}

int finish(hipError_t e, hipStream_t stream, const char* what) {
  if (e == hipSuccess && debug_sync()) {
    e = hipStreamSynchronize(stream);
    if (e == hipSuccess) e = hipGetLastError();
  }
  if (e != hipSuccess)
    return fail(FA_ERR_HIP, std::string(what) + ": " + hipGetErrorString(e));
  return FA_OK;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

struct Range {
  const char* name;
  const void* p;
  size_t bytes;
};

// Byte ranges must not overlap (outputs vs everything else).
bool overlap(const Range& a, const Range& b) {
  const uintptr_t a0 = reinterpret_cast<uintptr_t>(a.p), b0 = reinterpret_cast<uintptr_t>(b.p);
  return a0 < b0 + b.bytes && b0 < a0 + a.bytes;
}

// Shared validation of the attention calls.  Returns FA_OK or an error.
int check_attn(const char* fn, int B, int H, int Hkv, int T, int d, float scale, int window,
               int global_every, float softcap, int d_v = -1) {
  if (d_v < 0) d_v = d;
  const std::string f(fn);
  if (B <= 0 || H <= 0 || Hkv <= 0 || T <= 0)
    return fail(FA_ERR_INVALID_ARG, f + ": B, H, Hkv and T must be positive");
  if (H % Hkv != 0) return fail(FA_ERR_INVALID_ARG, f + ": H must be a multiple of Hkv");
  if (d <= 0 || d % 2 != 0) return fail(FA_ERR_INVALID_ARG, f + ": head size d must be even and positive");
  if (d_v <= 0 || d_v % 2 != 0)
    return fail(FA_ERR_INVALID_ARG, f + ": value head size d_v must be even and positive");
  if (d_v == d && d != 64 && d != 128 && d != 256)
    return fail(FA_ERR_UNSUPPORTED, f + ": head size d must be 64, 128 or 256");
  if (d_v != d && !(d == 192 && d_v == 128))
    return fail(FA_ERR_UNSUPPORTED, f + ": (d, d_v) must be equal or (192, 128)");
  if (!(scale > 0.f) || !std::isfinite(scale))
    return fail(FA_ERR_INVALID_ARG, f + ": scale must be positive and finite");
  if (window < 0) return fail(FA_ERR_INVALID_ARG, f + ": window must be >= 0");
  if (global_every < 0) return fail(FA_ERR_INVALID_ARG, f + ": global_every must be >= 0");
  if (!(softcap >= 0.f) || !std::isfinite(softcap))
    return fail(FA_ERR_INVALID_ARG, f + ": softcap must be >= 0 and finite");
  const double elems = (double)B * H * T * d;
  if (elems > 4.0e12) return fail(FA_ERR_INVALID_ARG, f + ": tensor too large");
  // the kernels address one head's [T, d] slice through a buffer resource
  // with a 32-bit byte range
  if ((double)T * std::max(d, d_v) * 2.0 > 2147483647.0)
    return fail(FA_ERR_INVALID_ARG, f + ": one head's [T, d] slice exceeds 2 GiB");
  return FA_OK;
}

int check_ptrs(const char* fn, const Range* rs, int n, int first_out) {
  for (int i = 0; i < n; ++i) {
    if (!rs[i].p) return fail(FA_ERR_INVALID_ARG, std::string(fn) + ": null pointer " + rs[i].name);
    if (!aligned16(rs[i].p))
      return fail(FA_ERR_INVALID_ARG, std::string(fn) + ": " + rs[i].name + " not 16-byte aligned");
  }
  for (int i = first_out; i < n; ++i)
    for (int j = 0; j < n; ++j)
      if (j != i && overlap(rs[i], rs[j]))
        return fail(FA_ERR_INVALID_ARG,
                    std::string(fn) + ": output " + rs[i].name + " overlaps " + rs[j].name);
  return FA_OK;
}

// fa_bwd_noalloc: the backward's [B, H, T] row statistics in a fixed
// device array instead of an allocation.  Each GPU holds its own copy; its
// address on a device comes from hipGetSymbolAddress with that device
// current (the array's name in host code is only a host-side stand-in),
// looked up on the first call that runs on the device and kept.
constexpr size_t kNoAllocRows = size_t(1) << 22;   // B * H * T at most (16 MiB of float)
constexpr int kMaxDevices = 64;

// dQ strategy of the bf16 backward (fa_set_dq_mode): 0 = the measured choice
// (fa::ds_mode_applies), 1 = the dQ pass recomputes S and dP, 2 = dQ from
// stored dS wherever supported.
std::atomic<int> g_dq_mode{0};

// The dS workspace comes from a stream-ordered pool of the library's own per
// device, whose release threshold keeps freed memory for the next call (a
// backward's workspace is GBs: mapping it anew on every call would cost
// more than the pass it serves).  Calls on one device share the pool; the
// stream order keeps their workspaces apart.  A workspace larger than a
// quarter of the device's memory is not taken (the recomputing dQ pass runs
// instead).
std::mutex g_pool_mu;
hipMemPool_t g_pool[kMaxDevices] = {};
size_t g_pool_cap[kMaxDevices] = {};

// the pool of the current device (created on first use) and its cap; null
// when the device has none (then no workspace is taken)
hipMemPool_t ws_pool(size_t* cap) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> lk(g_pool_mu);
  if (!g_pool[dev]) {
    size_t free_b = 0, total_b = 0;
    if (hipMemGetInfo(&free_b, &total_b) != hipSuccess) {
      (void)hipGetLastError();
      return nullptr;
    }
    hipMemPoolProps props{};
    props.allocType = hipMemAllocationTypePinned;
    props.location.type = hipMemLocationTypeDevice;
    props.location.id = dev;
    hipMemPool_t p = nullptr;
    if (hipMemPoolCreate(&p, &props) != hipSuccess) {
      (void)hipGetLastError();
      return nullptr;
    }
    uint64_t keep = UINT64_MAX;
    (void)hipMemPoolSetAttribute(p, hipMemPoolAttrReleaseThreshold, &keep);
    g_pool[dev] = p;
    g_pool_cap[dev] = total_b / 4;
  }
  *cap = g_pool_cap[dev];
  return g_pool[dev];
}
std::mutex g_scratch_mu;
float* g_scratch_dev[kMaxDevices] = {};

}  // namespace

static __device__ __align__(256) float scratch[kNoAllocRows];

namespace {

// scratch's address on the device that runs `stream` (which must be the
// current device) into *out; FA_OK or the error (recorded)
int scratch_on_stream_device(hipStream_t stream, const char* fn, float** out) {
  int cur = -1;
  hipError_t e = hipGetDevice(&cur);
  if (e != hipSuccess) return finish(e, stream, fn);
  int sdev = cur;
  if (stream) {
    e = hipStreamGetDevice(stream, &sdev);
    if (e != hipSuccess) return finish(e, stream, fn);
  }
  if (sdev != cur || cur < 0 || cur >= kMaxDevices)
    return fail(FA_ERR_INVALID_ARG,
                std::string(fn) + ": the stream's device must be the current device (< 64)");
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  if (!g_scratch_dev[cur]) {
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return finish(e, stream, fn);
    if (!ptr) return fail(FA_ERR_HIP, std::string(fn) + ": no device address for the scratch");
    g_scratch_dev[cur] = (float*)ptr;
  }
  *out = g_scratch_dev[cur];
  return FA_OK;
}

int resolve_window(int window, int T) { return window >= T ? 0 : window; }

// Shape of the dS workspace for a resolved window W: ceil(T/32) query tiles
// per head, and the key tiles one query tile can see -- its band:
// keys 32 qt - W + 1 .. 32 qt + 31, i.e. ceil((W - 1) / 32) + 1 tiles under a
// window (each holding a visible pair of the query tile), every earlier tile
// without one (at most ceil(T/32)).
struct DsShape {
  int nqt, nkt;
};
DsShape ds_shape(int T, int W) {
  const int nqt = (T + 31) / 32;
  return {nqt, W > 0 ? std::min(nqt, (W - 1 + 31) / 32 + 1) : nqt};
}

constexpr float kLog2e = 1.4426950408889634f;

int attn_fwd(bool f32, const void* q, const void* k, const void* v, void* o, float* lse, int B,
             int H, int Hkv, int T, int d, float scale, int window, int global_every,
             float softcap, hipStream_t stream, const char* fn = nullptr,
             const float* sinks = nullptr, float* max_logit = nullptr, int d_v = -1,
             const float* rope = nullptr, void* q_rot = nullptr) {
  if (!fn) fn = f32 ? "fa_fwd_f32" : "fa_fwd";
  if (d_v < 0) d_v = d;
  int rc = check_attn(fn, B, H, Hkv, T, d, scale, window, global_every, softcap, d_v);
  if (rc) return rc;
  const size_t es = f32 ? 4 : 2;
  const size_t nq = (size_t)B * H * T * d * es, nk = (size_t)B * Hkv * T * d * es;
  const size_t nv = (size_t)B * Hkv * T * d_v * es, no = (size_t)B * H * T * d_v * es;
  const Range rs[] = {{"q", q, nq}, {"k", k, nk}, {"v", v, nv},
                      {"o", o, no}, {"lse", lse, (size_t)B * H * T * 4}};
  rc = check_ptrs(fn, rs, 5, 3);
  if (rc) return rc;
  if (max_logit) {
    const Range ml{"max_logit", max_logit, (size_t)B * H * 4};
    if (!aligned16(max_logit)) return fail(FA_ERR_INVALID_ARG, std::string(fn) + ": max_logit not 16-byte aligned");
    for (const Range& r : rs)
      if (overlap(ml, r)) return fail(FA_ERR_INVALID_ARG, std::string(fn) + ": max_logit overlaps " + r.name);
  }
  if (q_rot) {
    const Range qr{"q_rot", q_rot, nq};
    if (!aligned16(q_rot)) return fail(FA_ERR_INVALID_ARG, std::string(fn) + ": q_rot not 16-byte aligned");
    for (const Range& r : rs)
      if (overlap(qr, r)) return fail(FA_ERR_INVALID_ARG, std::string(fn) + ": q_rot overlaps " + r.name);
  }
  const int W = resolve_window(window, T);
  hipError_t e;
  if (max_logit) {
    e = fa::launch_fill_f32(max_logit, B * H, -INFINITY, stream);
    if (e != hipSuccess) return finish(e, stream, fn);
  }
  float* rope_cs = nullptr;   // [T, d/2, 2] (cos, sin) for the fused RoPE
  if (rope) {
    e = hipMallocAsync((void**)&rope_cs, (size_t)T * d * sizeof(float), stream);
    if (e != hipSuccess) return finish(e, stream, "fa_fwd_rope table");
    e = fa::launch_rope_table(rope, rope_cs, T, d / 2, stream);
    if (e != hipSuccess) {
      (void)hipFreeAsync(rope_cs, stream);
      return finish(e, stream, fn);
    }
  }
  stage_begin(stream);
  if (f32) {
    fa::F32Args a{};
    a.q = (const float*)q; a.k = (const float*)k; a.v = (const float*)v;
    a.out = (float*)o; a.lse_out = lse;
    a.B = B; a.H = H; a.Hkv = Hkv; a.T = T; a.d = d; a.window = W;
    a.scale = scale; a.softcap = softcap;
    e = fa::launch_fwd_f32(a, stream);
  } else {
    fa::FwdArgs a{};
    a.q = (const fa::bf16*)q; a.k = (const fa::bf16*)k; a.v = (const fa::bf16*)v;
    a.o = (fa::bf16*)o; a.lse = lse;
    a.B = B; a.H = H; a.Hkv = Hkv; a.T = T; a.window = W;
    a.scale_log2e = scale * kLog2e;
    a.two_scale_over_cap_log2e = softcap > 0.f ? 2.f * scale * kLog2e / softcap : 0.f;
    a.cap_log2e = softcap > 0.f ? softcap * kLog2e : 0.f;
    a.sinks = sinks;
    a.max_logit = max_logit;
    a.rope_cs = rope_cs;
    a.q_rot = (fa::bf16*)q_rot;
    e = fa::launch_fwd_bf16(a, d, d_v, stream);
  }
  if (rope_cs) {
    const hipError_t e2 = hipFreeAsync(rope_cs, stream);
    if (e == hipSuccess) e = e2;
  }
  return finish(e, stream, fn);
}

int attn_bwd(bool f32, const void* q, const void* k, const void* v, const void* o,
             const float* lse, const void* dO, void* dq, void* dk, void* dv, int B, int H,
             int Hkv, int T, int d, float scale, int window, int global_every, float softcap,
             hipStream_t stream, const char* fn = nullptr, const float* sinks = nullptr,
             float* dsinks = nullptr, int d_v = -1, const float* rope = nullptr,
             bool static_rows = false) {
  if (!fn) fn = f32 ? "fa_bwd_f32" : "fa_bwd";
  if (d_v < 0) d_v = d;
  int rc = check_attn(fn, B, H, Hkv, T, d, scale, window, global_every, softcap, d_v);
  if (rc) return rc;
  const size_t es = f32 ? 4 : 2;
  const size_t nq = (size_t)B * H * T * d * es, nk = (size_t)B * Hkv * T * d * es;
  const size_t nv = (size_t)B * Hkv * T * d_v * es, no = (size_t)B * H * T * d_v * es;
  const Range rs[] = {{"q", q, nq},   {"k", k, nk},   {"v", v, nv},
                      {"o", o, no},   {"lse", lse, (size_t)B * H * T * 4},
                      {"dO", dO, no}, {"dq", dq, nq}, {"dk", dk, nk},
                      {"dv", dv, nv}};
  rc = check_ptrs(fn, rs, 9, 6);
  if (rc) return rc;
  if ((sinks == nullptr) != (dsinks == nullptr))
    return fail(FA_ERR_INVALID_ARG, std::string(fn) + ": sinks and dsinks must both be given");
  if (dsinks) {
    const Range ds{"dsinks", dsinks, (size_t)H * 4};
    if (!aligned16(dsinks) || !aligned16(sinks))
      return fail(FA_ERR_INVALID_ARG, std::string(fn) + ": sinks/dsinks not 16-byte aligned");
    for (const Range& r : rs)
      if (overlap(ds, r)) return fail(FA_ERR_INVALID_ARG, std::string(fn) + ": dsinks overlaps " + r.name);
    if (overlap(ds, {"sinks", sinks, (size_t)H * 4}))
      return fail(FA_ERR_INVALID_ARG, std::string(fn) + ": dsinks overlaps sinks");
  }
  const int W = resolve_window(window, T);
  // the [B, H, T] row statistics D: the library's fixed array
  // (fa_bwd_noalloc), else stream-ordered scratch
  float* Dst = nullptr;
  hipError_t e = hipSuccess;
  if (static_rows) {
    rc = scratch_on_stream_device(stream, fn, &Dst);
    if (rc) return rc;
  } else {
    e = hipMallocAsync((void**)&Dst, (size_t)B * H * T * sizeof(float), stream);
    if (e != hipSuccess) return finish(e, stream, "fa_bwd scratch");
  }
  auto free_d = [&]() {
    if (!static_rows) (void)hipFreeAsync(Dst, stream);
  };
  if (dsinks) {
    e = fa::launch_fill_f32(dsinks, H, 0.f, stream);
    if (e != hipSuccess) {
      free_d();
      return finish(e, stream, fn);
    }
  }
  float* rope_cs = nullptr;   // [T, d/2, 2] (cos, sin) for the fused RoPE backward
  if (rope) {
    e = hipMallocAsync((void**)&rope_cs, (size_t)T * d * sizeof(float), stream);
    if (e == hipSuccess) e = fa::launch_rope_table(rope, rope_cs, T, d / 2, stream);
    if (e != hipSuccess) {
      if (rope_cs) (void)hipFreeAsync(rope_cs, stream);
      free_d();
      return finish(e, stream, fn);
    }
  }
  // dS workspace: [B, H, ceil(T/32), band] tiles of 2 KB, where band = the
  // key tiles one query tile sees (ceil((W - 1) / 32) + 1 under a window)
  fa::bf16* dsw = nullptr;
  const DsShape dsh = ds_shape(T, W);
  const int nqt = dsh.nqt, nkt = dsh.nkt;
  if (!f32 && !static_rows && !dsinks && fa::ds_mode_applies(g_dq_mode.load(), d, d_v)) {
    const size_t tiles = (size_t)B * H * nqt * nkt;
    size_t cap = 0;
    hipMemPool_t pool = ws_pool(&cap);
    if (pool && tiles < (size_t(1) << 31) && tiles * 2048 <= cap) {
      if (hipMallocFromPoolAsync((void**)&dsw, tiles * 2048, pool, stream) != hipSuccess) {
        (void)hipGetLastError();   // out of memory: the recomputing pass instead
        dsw = nullptr;
      }
    }
  }
  stage_begin(stream);
  if (f32) {
    fa::F32Args a{};
    a.q = (const float*)q; a.k = (const float*)k; a.v = (const float*)v;
    a.o = (const float*)o; a.lse = lse; a.dO = (const float*)dO;
    a.dq = (float*)dq; a.dk = (float*)dk; a.dv = (float*)dv; a.Dst = Dst;
    a.B = B; a.H = H; a.Hkv = Hkv; a.T = T; a.d = d; a.window = W;
    a.scale = scale; a.softcap = softcap;
    e = fa::launch_bwd_f32(a, stream);
  } else {
    fa::BwdArgs a{};
    a.q = (const fa::bf16*)q; a.k = (const fa::bf16*)k; a.v = (const fa::bf16*)v;
    a.o = (const fa::bf16*)o; a.lse = lse; a.dO = (const fa::bf16*)dO;
    a.dq = (fa::bf16*)dq; a.dk = (fa::bf16*)dk; a.dv = (fa::bf16*)dv; a.Dst = Dst;
    a.B = B; a.H = H; a.Hkv = Hkv; a.T = T; a.window = W;
    a.scale = scale;
    a.scale_log2e = scale * kLog2e;
    a.two_scale_over_cap_log2e = softcap > 0.f ? 2.f * scale * kLog2e / softcap : 0.f;
    a.cap_log2e = softcap > 0.f ? softcap * kLog2e : 0.f;
    a.inv_cap = softcap > 0.f ? 1.f / softcap : 0.f;
    a.sinks = sinks;
    a.dsinks = dsinks;
    a.rope_cs = rope_cs;
    a.dsw = dsw;
    a.nqt_ws = nqt;
    a.nkt_ws = nkt;
    e = fa::launch_bwd_bf16(a, d, d_v, stream);
  }
  if (dsw) {
    const hipError_t e3 = hipFreeAsync(dsw, stream);
    if (e == hipSuccess) e = e3;
  }
  hipError_t e2 = static_rows ? hipSuccess : hipFreeAsync(Dst, stream);
  if (e == hipSuccess) e = e2;
  if (rope_cs) {
    e2 = hipFreeAsync(rope_cs, stream);
    if (e == hipSuccess) e = e2;
  }
  return finish(e, stream, fn);
}

// Chunking of the decode: enough (batch, KV head, chunk) units to fill the
// chip several times over, at least 32 tiles of 32 keys per chunk (shorter
// chunks measured slower: 5.25 against 5.74 TB/s on a 4096-key window), at
// most kDecMaxSplits chunks.  max_keys bounds the visible keys of any
// sequence.
void decode_split(int units, int max_keys, int* nsplit, int* chunk) {
  constexpr int kTargetUnits = 4096, kMinChunk = 1024, kTile = 32;
  int ns = (kTargetUnits + units - 1) / units;
  ns = std::min(ns, (max_keys + kMinChunk - 1) / kMinChunk);
  ns = std::max(1, std::min(ns, fa::kDecMaxSplits));
  int c = (max_keys + ns - 1) / ns;
  c = (c + kTile - 1) / kTile * kTile;
  *chunk = c;
  *nsplit = (max_keys + c - 1) / c;
}

int rope(bool f32, bool bwd, const void* x, void* y, const float* inv_freq, int B, int H, int T,
         int d, hipStream_t stream) {
  const char* fn = bwd ? (f32 ? "rope_apply_bwd_f32" : "rope_apply_bwd")
                       : (f32 ? "rope_apply_f32" : "rope_apply");
  const std::string f(fn);
  if (B <= 0 || H <= 0 || T <= 0) return fail(FA_ERR_INVALID_ARG, f + ": B, H and T must be positive");
  if (d <= 0 || d % 2 != 0) return fail(FA_ERR_INVALID_ARG, f + ": d must be even and positive");
  if ((double)B * H * T * d > 4.0e12) return fail(FA_ERR_INVALID_ARG, f + ": tensor too large");
  const size_t n = (size_t)B * H * T * d * (f32 ? 4 : 2);
  if (!x || !y || !inv_freq) return fail(FA_ERR_INVALID_ARG, f + ": null pointer");
  if (!aligned16(x) || !aligned16(y) || !aligned16(inv_freq))
    return fail(FA_ERR_INVALID_ARG, f + ": pointers must be 16-byte aligned");
  if (x != y && overlap({"y", y, n}, {"x", x, n}))
    return fail(FA_ERR_INVALID_ARG, f + ": y partially overlaps x (only y == x is allowed)");
  if (overlap({"inv_freq", inv_freq, (size_t)d / 2 * 4}, {"y", y, n}))
    return fail(FA_ERR_INVALID_ARG, f + ": inv_freq overlaps y");
  fa::RopeArgs a{x, y, inv_freq, B * H, T, d};
  stage_begin(stream);
  const hipError_t e = f32 ? fa::launch_rope_f32(a, bwd, stream) : fa::launch_rope_bf16(a, bwd, stream);
  return finish(e, stream, fn);
}

}  // namespace

namespace fa {
void stage_mark(hipStream_t stream) {
  if (g_stage_next > 0 && g_stage_next < g_stage_n) hipEventRecord(g_stage_ev[g_stage_next++], stream);
}
}  // namespace fa

extern "C" {

int fa_fwd(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H,
           int Hkv, int T, int d, float scale, int window, int global_every, float softcap,
           hipStream_t stream) {
  return attn_fwd(false, q, k, v, o, lse, B, H, Hkv, T, d, scale, window, global_every, softcap,
                  stream);
}

int fa_fwd_f32(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H,
               int Hkv, int T, int d, float scale, int window, int global_every, float softcap,
               hipStream_t stream) {
  return attn_fwd(true, q, k, v, o, lse, B, H, Hkv, T, d, scale, window, global_every, softcap,
                  stream);
}

int fa_bwd(const void* q, const void* k, const void* v, const void* o, const float* lse,
           const void* dO, void* dq, void* dk, void* dv, int B, int H, int Hkv, int T, int d,
           float scale, int window, int global_every, float softcap, hipStream_t stream) {
  return attn_bwd(false, q, k, v, o, lse, dO, dq, dk, dv, B, H, Hkv, T, d, scale, window,
                  global_every, softcap, stream);
}

int fa_bwd_f32(const void* q, const void* k, const void* v, const void* o, const float* lse,
               const void* dO, void* dq, void* dk, void* dv, int B, int H, int Hkv, int T,
               int d, float scale, int window, int global_every, float softcap,
               hipStream_t stream) {
  return attn_bwd(true, q, k, v, o, lse, dO, dq, dk, dv, B, H, Hkv, T, d, scale, window,
                  global_every, softcap, stream);
}

int fa_bwd_noalloc(const void* q, const void* k, const void* v, const void* o, const float* lse,
                   const void* dO, void* dq, void* dk, void* dv, int B, int H, int Hkv, int T,
                   int d, float scale, int window, int global_every, float softcap,
                   hipStream_t stream) {
  const char* fn = "fa_bwd_noalloc";
  const int rc = check_attn(fn, B, H, Hkv, T, d, scale, window, global_every, softcap);
  if (rc) return rc;
  if ((double)B * H * T > (double)kNoAllocRows)
    return fail(FA_ERR_INVALID_ARG, std::string(fn) + ": B*H*T = " +
                                        std::to_string((long long)B * H * T) +
                                        " exceeds its fixed scratch of " +
                                        std::to_string(kNoAllocRows) + " rows");
  return attn_bwd(false, q, k, v, o, lse, dO, dq, dk, dv, B, H, Hkv, T, d, scale, window,
                  global_every, softcap, stream, fn, nullptr, nullptr, -1, nullptr, true);
}

int fa_fwd_sink(const void* q, const void* k, const void* v, void* o, float* lse,
                const float* sinks, float* max_logit, int B, int H, int Hkv, int T, int d,
                float scale, int window, int global_every, float softcap, hipStream_t stream) {
  if (sinks && !aligned16(sinks)) return fail(FA_ERR_INVALID_ARG, "fa_fwd_sink: sinks not 16-byte aligned");
  return attn_fwd(false, q, k, v, o, lse, B, H, Hkv, T, d, scale, window, global_every, softcap,
                  stream, "fa_fwd_sink", sinks, max_logit);
}

int fa_bwd_sink(const void* q, const void* k, const void* v, const void* o, const float* lse,
                const void* dO, const float* sinks, void* dq, void* dk, void* dv, float* dsinks,
                int B, int H, int Hkv, int T, int d, float scale, int window, int global_every,
                float softcap, hipStream_t stream) {
  return attn_bwd(false, q, k, v, o, lse, dO, dq, dk, dv, B, H, Hkv, T, d, scale, window,
                  global_every, softcap, stream, "fa_bwd_sink", sinks, dsinks);
}

int fa_decode(const void* q, const void* k_cache, const void* v_cache, const int* lens, void* o,
              float* lse, const float* sinks, int B, int H, int Hkv, int S, int d, float scale,
              int window, float softcap, hipStream_t stream) {
  const char* fn = "fa_decode";
  int rc = check_attn(fn, B, H, Hkv, S, d, scale, window, 0, softcap);
  if (rc) return rc;
  if (H / Hkv > 32) return fail(FA_ERR_UNSUPPORTED, "fa_decode: at most 32 query heads per KV head");
  const size_t nq = (size_t)B * H * d * 2, nc = (size_t)B * Hkv * S * d * 2;
  const Range rs[] = {{"q", q, nq}, {"k_cache", k_cache, nc}, {"v_cache", v_cache, nc},
                      {"lens", lens, (size_t)B * 4}, {"o", o, nq}};
  rc = check_ptrs(fn, rs, 5, 4);
  if (rc) return rc;
  if (lse) {
    const Range lr{"lse", lse, (size_t)B * H * 4};
    if (!aligned16(lse)) return fail(FA_ERR_INVALID_ARG, "fa_decode: lse not 16-byte aligned");
    for (const Range& r : rs)
      if (overlap(lr, r)) return fail(FA_ERR_INVALID_ARG, std::string("fa_decode: lse overlaps ") + r.name);
  }
  if (sinks && !aligned16(sinks)) return fail(FA_ERR_INVALID_ARG, "fa_decode: sinks not 16-byte aligned");
  const int max_keys = window > 0 ? std::min(window, S) : S;
  int nsplit = 1, chunk = 32;
  decode_split(B * Hkv, max_keys, &nsplit, &chunk);
  if ((double)B * Hkv * nsplit > 2.0e9) return fail(FA_ERR_INVALID_ARG, "fa_decode: too many work units");
  const size_t units = (size_t)B * Hkv * nsplit;
  const size_t part_bytes = units * (H / Hkv) * (size_t)(d + 2) * sizeof(float);
  float* part = nullptr;
  hipError_t e = hipMallocAsync((void**)&part, part_bytes, stream);
  if (e != hipSuccess) return finish(e, stream, "fa_decode scratch");
  fa::DecodeArgs a{};
  a.q = (const fa::bf16*)q; a.kc = (const fa::bf16*)k_cache; a.vc = (const fa::bf16*)v_cache;
  a.lens = lens; a.o = (fa::bf16*)o; a.lse = lse; a.sinks = sinks;
  a.part_o = part;
  a.part_ml = part + units * (H / Hkv) * d;
  a.B = B; a.H = H; a.Hkv = Hkv; a.S = S; a.window = window; a.nsplit = nsplit; a.chunk = chunk;
  a.scale_log2e = scale * kLog2e;
  a.two_scale_over_cap_log2e = softcap > 0.f ? 2.f * scale * kLog2e / softcap : 0.f;
  a.cap_log2e = softcap > 0.f ? softcap * kLog2e : 0.f;
  stage_begin(stream);
  e = fa::launch_decode_bf16(a, d, softcap > 0.f, stream);
  const hipError_t e2 = hipFreeAsync(part, stream);
  if (e == hipSuccess) e = e2;
  return finish(e, stream, fn);
}

const char* fa_bwd_kernels(int d, int d_v) {
  return fa::bwd_kernel_plan(d, d_v, g_dq_mode.load());
}

int fa_bwd_workspace(int B, int H, int T, int d, int d_v, int window, size_t* bytes,
                     int* query_tiles, int* band_tiles) {
  int rc = check_attn("fa_bwd_workspace", B, H, H, T, d, 1.f, window, 0, 0.f, d_v);
  if (rc) return rc;
  if (!bytes || !query_tiles || !band_tiles)
    return fail(FA_ERR_INVALID_ARG, "fa_bwd_workspace: null output pointer");
  const DsShape s = ds_shape(T, resolve_window(window, T));
  *query_tiles = s.nqt;
  *band_tiles = s.nkt;
  *bytes = fa::ds_mode_applies(g_dq_mode.load(), d, d_v) ? (size_t)B * H * s.nqt * s.nkt * 2048 : 0;
  return FA_OK;
}

int fa_set_dq_mode(int mode) {
  if (mode < 0 || mode > 2) return fail(FA_ERR_INVALID_ARG, "fa_set_dq_mode: mode must be 0, 1 or 2");
  return g_dq_mode.exchange(mode);
}

int fa_measure_dq_atomics(int B, int H, int Hkv, int T, int d, int window, float* ms) {
  const char* fn = "fa_measure_dq_atomics";
  int rc = check_attn(fn, B, H, Hkv, T, d, 1.f, window, 0, 0.f);
  if (rc) return rc;
  if (!ms) return fail(FA_ERR_INVALID_ARG, std::string(fn) + ": null pointer ms");
  // the dK/dV pass's key block and query tile for this head size
  const int bkvb = d == 256 ? 64 : 128, bqb = d == 256 ? 32 : 64;
  const int W = resolve_window(window, T);
  const size_t bytes = (size_t)B * H * T * d * sizeof(float);
  float* acc = nullptr;
  hipEvent_t e0 = nullptr, e1 = nullptr;
  hipError_t e = hipMalloc((void**)&acc, bytes);
  if (e == hipSuccess) e = hipMemset(acc, 0, bytes);
  if (e == hipSuccess) e = hipEventCreate(&e0);
  if (e == hipSuccess) e = hipEventCreate(&e1);
  float best = 0.f;
  for (int rep = 0; rep < 3 && e == hipSuccess; ++rep) {   // best of three
    e = hipEventRecord(e0, nullptr);
    if (e == hipSuccess) e = fa::launch_dq_atomic_probe(acc, B, H, Hkv, T, d, W, bkvb, bqb, nullptr);
    if (e == hipSuccess) e = hipEventRecord(e1, nullptr);
    if (e == hipSuccess) e = hipEventSynchronize(e1);
    float t = 0.f;
    if (e == hipSuccess) e = hipEventElapsedTime(&t, e0, e1);
    if (e == hipSuccess && (rep == 0 || t < best)) best = t;
  }
  if (e0) (void)hipEventDestroy(e0);
  if (e1) (void)hipEventDestroy(e1);
  if (acc) (void)hipFree(acc);
  if (e != hipSuccess) return fail(FA_ERR_HIP, std::string(fn) + ": " + hipGetErrorString(e));
  *ms = best;
  return FA_OK;
}

int fa_decode_splits(int B, int Hkv, int S, int window, int* nsplit, int* chunk) {
  if (B <= 0 || Hkv <= 0 || S <= 0 || window < 0 || !nsplit || !chunk)
    return fail(FA_ERR_INVALID_ARG, "fa_decode_splits: invalid arguments");
  decode_split(B * Hkv, window > 0 ? std::min(window, S) : S, nsplit, chunk);
  return FA_OK;
}

int fa_fwd_rope(const void* q, const void* k, const void* v, void* o, float* lse,
                const float* inv_freq, void* q_rot, int B, int H, int Hkv, int T, int d,
                float scale, int window, int global_every, float softcap, hipStream_t stream) {
  if (!inv_freq) return fail(FA_ERR_INVALID_ARG, "fa_fwd_rope: null pointer inv_freq");
  if (!aligned16(inv_freq)) return fail(FA_ERR_INVALID_ARG, "fa_fwd_rope: inv_freq not 16-byte aligned");
  return attn_fwd(false, q, k, v, o, lse, B, H, Hkv, T, d, scale, window, global_every, softcap,
                  stream, "fa_fwd_rope", nullptr, nullptr, -1, inv_freq, q_rot);
}

int fa_bwd_rope(const void* q_rot, const void* k, const void* v, const void* o, const float* lse,
                const void* dO, const float* inv_freq, void* dq, void* dk, void* dv, int B,
                int H, int Hkv, int T, int d, float scale, int window, int global_every,
                float softcap, hipStream_t stream) {
  if (!inv_freq) return fail(FA_ERR_INVALID_ARG, "fa_bwd_rope: null pointer inv_freq");
  if (!aligned16(inv_freq)) return fail(FA_ERR_INVALID_ARG, "fa_bwd_rope: inv_freq not 16-byte aligned");
  return attn_bwd(false, q_rot, k, v, o, lse, dO, dq, dk, dv, B, H, Hkv, T, d, scale, window,
                  global_every, softcap, stream, "fa_bwd_rope", nullptr, nullptr, -1, inv_freq);
}

int fa_fwd_vdim(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H,
                int Hkv, int T, int d, int d_v, float scale, int window, int global_every,
                float softcap, hipStream_t stream) {
  return attn_fwd(false, q, k, v, o, lse, B, H, Hkv, T, d, scale, window, global_every, softcap,
                  stream, "fa_fwd_vdim", nullptr, nullptr, d_v);
}

int fa_bwd_vdim(const void* q, const void* k, const void* v, const void* o, const float* lse,
                const void* dO, void* dq, void* dk, void* dv, int B, int H, int Hkv, int T, int d,
                int d_v, float scale, int window, int global_every, float softcap,
                hipStream_t stream) {
  return attn_bwd(false, q, k, v, o, lse, dO, dq, dk, dv, B, H, Hkv, T, d, scale, window,
                  global_every, softcap, stream, "fa_bwd_vdim", nullptr, nullptr, d_v);
}

int rope_apply(const void* x, void* y, const float* inv_freq, int B, int H, int T, int d,
               hipStream_t stream) {
  return rope(false, false, x, y, inv_freq, B, H, T, d, stream);
}
int rope_apply_bwd(const void* dy, void* dx, const float* inv_freq, int B, int H, int T, int d,
                   hipStream_t stream) {
  return rope(false, true, dy, dx, inv_freq, B, H, T, d, stream);
}
int rope_apply_f32(const void* x, void* y, const float* inv_freq, int B, int H, int T, int d,
                   hipStream_t stream) {
  return rope(true, false, x, y, inv_freq, B, H, T, d, stream);
}
int rope_apply_bwd_f32(const void* dy, void* dx, const float* inv_freq, int B, int H, int T,
                       int d, hipStream_t stream) {
  return rope(true, true, dy, dx, inv_freq, B, H, T, d, stream);
}

int fa_layer_window(int layer, int window, int global_every) {
  if (layer < 0 || window < 0 || global_every < 0)
    return fail(FA_ERR_INVALID_ARG, "fa_layer_window: layer, window and global_every must be >= 0");
  if (global_every > 0 && (layer + 1) % global_every == 0) return 0;
  return window;
}

int fa_rope_inv_freq(float* host_out, int d, double theta) {
  if (!host_out) return fail(FA_ERR_INVALID_ARG, "fa_rope_inv_freq: null pointer");
  if (d <= 0 || d % 2 != 0) return fail(FA_ERR_INVALID_ARG, "fa_rope_inv_freq: d must be even and positive");
  if (!(theta > 0.0) || !std::isfinite(theta))
    return fail(FA_ERR_INVALID_ARG, "fa_rope_inv_freq: theta must be positive and finite");
  for (int i = 0; i < d / 2; ++i) host_out[i] = (float)std::pow(theta, -2.0 * i / d);
  return FA_OK;
}

int fa_rope_inv_freq_llama3(float* host_out, int d, double theta, double factor,
                            double low_freq_factor, double high_freq_factor, double orig_ctx) {
  const int rc = fa_rope_inv_freq(host_out, d, theta);
  if (rc != FA_OK || factor <= 0.0) return rc;
  if (!(high_freq_factor > low_freq_factor) || !(low_freq_factor > 0.0) || !(orig_ctx > 0.0) ||
      !std::isfinite(factor) || !std::isfinite(high_freq_factor) || !std::isfinite(orig_ctx))
    return fail(FA_ERR_INVALID_ARG,
                "fa_rope_inv_freq_llama3: need high_freq_factor > low_freq_factor > 0, orig_ctx > 0");
  const double two_pi = 6.283185307179586;
  const double lo_wave = orig_ctx / low_freq_factor, hi_wave = orig_ctx / high_freq_factor;
  for (int i = 0; i < d / 2; ++i) {
    const double f = std::pow(theta, -2.0 * i / d);
    const double wave = two_pi / f;
    double g;
    if (wave < hi_wave) {
      g = f;
    } else if (wave > lo_wave) {
      g = f / factor;
    } else {
      const double smooth = (orig_ctx / wave - low_freq_factor) / (high_freq_factor - low_freq_factor);
      g = (1.0 - smooth) * f / factor + smooth * f;
    }
    host_out[i] = (float)g;
  }
  return FA_OK;
}

int fa_layer_rope_theta(int layer, double theta, double theta_global, int global_every,
                        double* out) {
  if (!out || layer < 0 || global_every < 0 || !(theta > 0.0))
    return fail(FA_ERR_INVALID_ARG, "fa_layer_rope_theta: bad argument");
  const bool global = global_every > 0 && (layer + 1) % global_every == 0;
  *out = (global && theta_global > 0.0) ? theta_global : theta;
  return FA_OK;
}

int fa_set_stage_events(void* const* events, int count) {
  if (count < 0 || count > kMaxStageEvents || (count > 0 && !events))
    return fail(FA_ERR_INVALID_ARG, "fa_set_stage_events: count must be 0..16 with non-null events");
  for (int i = 0; i < count; ++i) {
    if (!events[i]) return fail(FA_ERR_INVALID_ARG, "fa_set_stage_events: null event");
    g_stage_ev[i] = (hipEvent_t)events[i];
  }
  g_stage_n = count;
  g_stage_next = 0;
  return FA_OK;
}

const char* fa_last_error(void) { return g_last_error.c_str(); }

}  // extern "C"
