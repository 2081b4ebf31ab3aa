// Host/device interface between the C-ABI layer (fa_api.cpp) and the
// kernel launchers.  Not part of the public ABI.
#pragma once

#include <hip/hip_runtime.h>

namespace fa {

typedef __bf16 bf16;

// Forward arguments.  `window` is already resolved (0 = full causal).
// Score constants are folded for the log2-domain softmax:
//   no cap:  s2 = x * scale * log2(e)
//   cap:     s2 = cap * log2(e) * tanh(scale * x / cap), with tanh(y)
//            = 1 - 2 / (exp2(2 y log2(e)) + 1)
struct FwdArgs {
  const bf16* q;
  const bf16* k;
  const bf16* v;
  bf16* o;
  float* lse;
  int B, H, Hkv, T, window;
  float scale_log2e;               // scale * log2(e)
  float two_scale_over_cap_log2e;  // 2 * scale * log2(e) / cap   (cap > 0)
  float cap_log2e;                 // cap * log2(e), 0 when no cap
  const float* sinks;              // [H] sink logits (natural log) or null
  float* max_logit;                // [B, H] largest softmax logit, or null
  const float* rope_cs;            // [T, d/2, 2] (cos, sin) of the RoPE angles: rotate q
                                   // at load (q is un-rotated), or null
  bf16* q_rot;                     // [B, H, T, d] rotated q output, or null
};

// Backward arguments.  Dst holds the per-row D = <dO_i, o_i> scratch
// ([B, H, T] fp32) written by the dq pass and read by the dk/dv pass.
struct BwdArgs {
  const bf16* q;
  const bf16* k;
  const bf16* v;
  const bf16* o;
  const float* lse;
  const bf16* dO;
  bf16* dq;
  bf16* dk;
  bf16* dv;
  float* Dst;
  int B, H, Hkv, T, window;
  float scale;
  float scale_log2e;
  float two_scale_over_cap_log2e;
  float cap_log2e;
  float inv_cap;                   // 1 / cap, 0 when no cap
  const float* sinks;              // [H] sink logits or null
  float* dsinks;                   // [H] gradient of the sinks (accumulated), or null
  const float* rope_cs;            // [T, d/2, 2] RoPE (cos, sin): dq is rotated back
                                   // (gradient w.r.t. the un-rotated q), or null
  // dQ from stored dS: the dK/dV pass writes every visible 32 x 32 tile of
  // bf16 dS to dsw and the dQ pass reads it back (null: the dQ pass
  // recomputes S and dP).  Layout: [B, H, nqt_ws, nkt_ws] tiles of 2 KB;
  // slot j of query tile qt holds key tile qt - nkt_ws + 1 + j.
  bf16* dsw;
  int nqt_ws;                      // query tiles per head, ceil(T / 32)
  int nkt_ws;                      // key tiles a query tile can see
};

// float32 twins (plain pointers, same semantics).
struct F32Args {
  const float* q;
  const float* k;
  const float* v;
  const float* o;
  float* lse_out;      // forward output
  const float* lse;    // backward input
  const float* dO;
  float* out;          // forward o
  float* dq;
  float* dk;
  float* dv;
  float* Dst;
  int B, H, Hkv, T, d, window;
  float scale;
  float softcap;
};

// Decode over a KV cache.  part_o / part_ml: per (batch, KV head, chunk)
// float32 scratch of the split pass -- unnormalised O [G, d] and the
// running (max in log2 units, sum) per query head of the group.
constexpr int kDecMaxSplits = 256;
struct DecodeArgs {
  const bf16* q;      // [B, H, d]
  const bf16* kc;     // [B, Hkv, S, d]
  const bf16* vc;     // [B, Hkv, S, d]
  const int* lens;    // [B] tokens held by each sequence (query at lens-1)
  bf16* o;            // [B, H, d]
  float* lse;         // [B, H] or null
  const float* sinks; // [H] or null
  float* part_o;
  float* part_ml;
  int B, H, Hkv, S, window, nsplit, chunk;
  float scale_log2e;
  float two_scale_over_cap_log2e;
  float cap_log2e;
};

struct RopeArgs {
  const void* x;
  void* y;
  const float* inv_freq;
  int BH, T, d;
};

// Called by the launchers right after each kernel launch; records the
// caller's stage events when fa_set_stage_events() armed them.
void stage_mark(hipStream_t stream);

// Fills n floats with v (initialises accumulated outputs inside a call).
hipError_t launch_fill_f32(float* p, int n, float v, hipStream_t stream);

// d: head size of q and k; d_v: head size of v and o (pairs (x, x) for
// x in {64, 128, 256} and (192, 128)).
hipError_t launch_fwd_bf16(const FwdArgs& a, int d, int d_v, hipStream_t stream);
hipError_t launch_bwd_bf16(const BwdArgs& a, int d, int d_v, hipStream_t stream);
// the software-pipelined dQ pass (fa_bwd_pipe.hip) for d = d_v = 128 or 256,
// launched by launch_bwd_bf16
hipError_t launch_bwd_dq_pipe(const BwdArgs& a, int d, bool cap, hipStream_t stream);
// the d = 128 dK/dV pass (fa_bwd_pipe.hip), launched by launch_bwd_bf16
hipError_t launch_bwd_kv_pipe(const BwdArgs& a, bool cap, hipStream_t stream);
// head sizes whose backward can take dQ from stored dS (fa_bwd_ds.hip)
constexpr bool ds_workspace_sizes(int d, int d_v) { return d == d_v && (d == 128 || d == 256); }
// dQ mode (fa_set_dq_mode): 0 stored dS where it measured faster than the
// recomputing dQ pass (d = 256: gemma-global backward 1.73 against 2.11 ms;
// at d = 128 the dK/dV pass's 2 bytes of stores per visible pair cost about
// what the recomputation saves: mistral 5.19 against 5.01 ms, qwen25 within
// 2 %), 1 recompute everywhere, 2 stored dS wherever supported
constexpr bool ds_mode_applies(int mode, int d, int d_v) {
  return ds_workspace_sizes(d, d_v) && (mode == 2 || (mode == 0 && d == 256));
}
// D prologue and dQ-from-stored-dS pass (fa_bwd_ds.hip), launched by
// launch_bwd_bf16 when a.dsw is set
hipError_t launch_bwd_rowdot(const BwdArgs& a, int d, hipStream_t stream);
hipError_t launch_bwd_dq_ds(const BwdArgs& a, int d, hipStream_t stream);
// kernels launch_bwd_bf16 runs for (d, d_v), in order ("dq,dkdv", or
// "rowdot,dkdv,dq_ds" with a dS workspace); null for unsupported sizes
const char* bwd_kernel_plan(int d, int d_v, int mode);
hipError_t launch_fwd_f32(const F32Args& a, hipStream_t stream);
hipError_t launch_bwd_f32(const F32Args& a, hipStream_t stream);
hipError_t launch_decode_bf16(const DecodeArgs& a, int d, bool cap, hipStream_t stream);
// (cos, sin) of the RoPE angle fl32(t * inv_freq[i]) for t < T, i < half,
// into cs [T, half, 2] -- the same values the RoPE kernels compute.
hipError_t launch_rope_table(const float* inv_freq, float* cs, int T, int half, hipStream_t stream);
hipError_t launch_rope_bf16(const RopeArgs& a, bool bwd, hipStream_t stream);
// the dQ-atomics traffic probe (fa_probe.hip): bkvb keys per workgroup,
// bqb-row query tiles, into acc [B, H, T, d] fp32
hipError_t launch_dq_atomic_probe(float* acc, int B, int H, int Hkv, int T, int d, int W,
                                  int bkvb, int bqb, hipStream_t stream);
hipError_t launch_rope_f32(const RopeArgs& a, bool bwd, hipStream_t stream);

}  // namespace fa
