/*
 * fa.h -- C ABI of the MI355X (gfx950) fused causal flash-attention library
 * (libfa.so).  Plain pointers and sizes only; no C++ or torch types.
 *
 * What the calls compute (sources are web pages, cited by title/section):
 *
 *   For batch b, query head h, key/value head g = h / (H / Hkv):
 *     S[i,j]  = scale * <q[b,h,i,:], k[b,g,j,:]>
 *     S'[i,j] = softcap * tanh(S[i,j] / softcap)   (softcap > 0; else S)
 *               -- Forge ARCHITECTURES.md, implementation plan wave 2,
 *                  item 9: cap*tanh(s/cap) on the pre-softmax scores.
 *     key j is visible to query i iff j <= i and, for 0 < W < T,
 *               j > i - W       -- ARCHITECTURES.md, plan wave 2, item 8:
 *                  the causal mask becomes q-W < k <= q; out-of-window KV
 *                  tiles are skipped by the loop bound, not masked.
 *     lse[i]  = log sum_{j visible} exp(S'[i,j])   (natural log)
 *     o[i]    = sum_{j visible} exp(S'[i,j] - lse[i]) v[b,g,j,:]
 *   fa_bwd returns the gradients of sum(o * dO); the softcap backward uses
 *   the exact derivative 1 - tanh^2 (Forge attention.h commit log, "Wave 2").
 *   GQA (n_kv_heads < n_heads, n_heads % n_kv_heads == 0): Forge README and
 *   forge-studio RESEARCH.md section 2 (config validations).
 *
 * Layouts (all contiguous, row-major, device memory, caller-owned):
 *   q, o, dO, dq : [B, H,   T, d]
 *   k, v, dk, dv : [B, Hkv, T, d]
 *   lse          : [B, H, T] float32
 *   x, y, dy, dx : [B, H, T, d] for rope_* (call once with H query heads for
 *                  Q and once with Hkv heads for K)
 *   inv_freq     : [d/2] float32, device memory (fa_rope_inv_freq fills a
 *                  host array the caller copies over)
 * Element type: bfloat16 for the un-suffixed calls, float32 for the _f32
 * twins (which never round through bf16).  Pointers must be 16-byte aligned.
 * q, k, v, o, lse, dq, dk, dv, dO must not overlap one another; rope's y may
 * equal x (in place), and dx may equal dy.
 *
 * Parameters:
 *   B, H, Hkv, T > 0; H % Hkv == 0; d in {64, 128, 256} for attention,
 *   d even and > 0 for rope (d % 8 == 0 takes the vector path).
 *   scale > 0 (1/sqrt(d) for plain attention; any positive value, e.g. a
 *   query_pre_attn_scalar, is accepted).
 *   window: 0 = full causal; 0 < window < T = sliding window of `window`
 *   keys including the query itself; window >= T = full causal.
 *   global_every >= 0: the model's local:global pattern knob; validated
 *   here, resolved per layer by the caller with fa_layer_window().
 *   softcap: 0 = off, > 0 = cap.
 *
 * Ownership and streams: every call only enqueues work on `stream` (NULL =
 * the default stream) and returns; device faults surface at the caller's
 * next synchronisation.  Calls that need scratch allocate it stream-ordered
 * (hipMallocAsync/hipFreeAsync on `stream`): fa_bwd and its _sink, _vdim
 * and _rope variants (the [B, H, T] float32 row statistics), fa_fwd_rope
 * and fa_bwd_rope (a [T, d/2] float32 (cos, sin) table), fa_decode (the
 * per-chunk partial results).  The bf16 fa_bwd and fa_bwd_rope at
 * d = 128 also take a dS workspace (see fa_bwd_kernels) from a
 * stream-ordered memory pool the library keeps per device: freed at the end
 * of the call, its memory stays in the pool for the next one until the
 * process ends.  fa_bwd_noalloc allocates nothing.  No other state persists
 * between calls.
 *
 * Errors: 0 on success, else a negative FA_ERR_* code; fa_last_error()
 * returns a thread-local message describing the most recent failure.
 * Argument checks run before any HIP call, so an invalid argument never
 * touches the device.  No C++ exception crosses this interface.
 */
#ifndef CAUSAL_FA_H
#define CAUSAL_FA_H

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct ihipStream_t* hipStream_t;

#define FA_OK 0
#define FA_ERR_INVALID_ARG (-1) /* null pointer, non-positive size, H % Hkv,
                                   odd d, window < 0, bad scale/softcap,
                                   global_every < 0 */
#define FA_ERR_UNSUPPORTED (-2) /* attention head size not 64/128/256 */
#define FA_ERR_HIP (-3)         /* HIP runtime or launch error */

/* Forward: o and lse from q, k, v (bf16 tensors, fp32 lse). */
int fa_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
           int B, int H, int Hkv, int T, int d, float scale, int window,
           int global_every, float softcap, hipStream_t stream);

/* Backward: dq, dk, dv from q, k, v, the forward's o and lse, and dO.
 * dk and dv sum over the query heads of each KV group; all three are fully
 * overwritten (no accumulation into the caller's buffers). */
int fa_bwd(const void* q, const void* k, const void* v, const void* o,
           const float* lse, const void* dO, void* dq, void* dk, void* dv,
           int B, int H, int Hkv, int T, int d, float scale, int window,
           int global_every, float softcap, hipStream_t stream);

/* fa_bwd without any allocation, for callers that cannot allocate (code
 * under HIP graph capture, allocation-free serving loops, harnesses that
 * forbid hipMalloc): same parameters and semantics as fa_bwd, and its
 * results bit for bit under dQ mode 1 (fa_set_dq_mode; in the default mode
 * dk and dv are the same bits and dq agrees within the parity bound), with
 * the kernels "dq,dkdv" and the [B, H, T] float32 row statistics in a fixed array
 * in device memory that the library holds for the life of the process on
 * each GPU it runs on (16 MiB).  B * H * T must not exceed 4,194,304
 * (FA_ERR_INVALID_ARG otherwise, before any device work); `stream` must
 * belong to the current device.  The array is fully rewritten by each call
 * before it is read (nothing has to start at zero); calls that overlap on
 * one GPU share it and race -- order them on one stream. */
int fa_bwd_noalloc(const void* q, const void* k, const void* v, const void* o,
                   const float* lse, const void* dO, void* dq, void* dk,
                   void* dv, int B, int H, int Hkv, int T, int d, float scale,
                   int window, int global_every, float softcap,
                   hipStream_t stream);

/* RoPE fused into the attention (bf16 tensors, d = 64, 128, 256).  The
 * query rows are loaded once per workgroup into registers, so their rotation
 * (and the inverse rotation of dq at its store) costs no extra pass over HBM;
 * key tiles are re-read by every query block, so K is rotated beforehand by
 * rope_apply (Forge attention.h commit log, "Wave 1": RoPE reads the host
 * inverse-frequency table; README: interleaved pairs).  Each call builds a
 * [T, d/2] (cos, sin) table of the angles (stream-ordered hipMallocAsync
 * scratch, freed on the stream) with the same arithmetic as rope_apply.
 * fa_fwd_rope: q un-rotated [B,H,T,d]; k already rotated; inv_freq [d/2]
 *   float32 device table; q_rot [B,H,T,d] receives rope_apply(q) bit for bit
 *   (for the backward), or NULL.  o, lse as fa_fwd.
 * fa_bwd_rope: q_rot = rotated q (fa_fwd_rope's q_rot); dq is written as the
 *   gradient with respect to the UN-rotated q (rope_apply_bwd fused, without
 *   the intermediate bf16 rounding); dk and dv as fa_bwd (dk is with respect
 *   to the rotated k: apply rope_apply_bwd to it). */
int fa_fwd_rope(const void* q, const void* k, const void* v, void* o,
                float* lse, const float* inv_freq, void* q_rot, int B, int H,
                int Hkv, int T, int d, float scale, int window,
                int global_every, float softcap, hipStream_t stream);
int fa_bwd_rope(const void* q_rot, const void* k, const void* v,
                const void* o, const float* lse, const void* dO,
                const float* inv_freq, void* dq, void* dk, void* dv, int B,
                int H, int Hkv, int T, int d, float scale, int window,
                int global_every, float softcap, hipStream_t stream);

/* Value head size different from the query/key head size (bf16 tensors):
 * MLA-style heads with the latent decompressed, d = 192 for q and k (128
 * "nope" + 64 rotary dims) and d_v = 128 for v, o, dO, dv, with the caller's
 * scale 1/sqrt(192) (Forge ARCHITECTURES.md family table, DeepSeek-V3 row,
 * and the "Formules clés" note on MLA; plan wave 3 item 13).
 *   q, dq [B,H,T,d]; k, dk [B,Hkv,T,d]; v, dv [B,Hkv,T,d_v];
 *   o, dO [B,H,T,d_v]; lse [B,H,T].
 * Supported (d, d_v): (192, 128), and d == d_v in {64, 128, 256} (then
 * identical to fa_fwd / fa_bwd).  Everything else as fa_fwd / fa_bwd. */
int fa_fwd_vdim(const void* q, const void* k, const void* v, void* o,
                float* lse, int B, int H, int Hkv, int T, int d, int d_v,
                float scale, int window, int global_every, float softcap,
                hipStream_t stream);
int fa_bwd_vdim(const void* q, const void* k, const void* v, const void* o,
                const float* lse, const void* dO, void* dq, void* dk, void* dv,
                int B, int H, int Hkv, int T, int d, int d_v, float scale,
                int window, int global_every, float softcap,
                hipStream_t stream);

/* Attention sinks and the per-head max logit (bf16 tensors).
 * sinks: [H] float32 device array (natural-log logits) or NULL.  A sink is a
 * learned per-head logit in every row's softmax denominator that carries no
 * value (Forge ARCHITECTURES.md family table, GPT-OSS; plan wave 2 item 10:
 * the online softmax starts its (max, sum) from it): lse includes it.
 * max_logit: [B, H] float32 device output or NULL: the largest visible
 * query-key logit (after the cap, if any; = scale*<q,k> without one; the
 * sink is not a query-key logit and is not counted) --
 * the quantity QK-Clip monitors (ARCHITECTURES.md, Kimi K2 MuonClip; plan
 * wave 3 item 12).  fa_fwd_sink with both NULL equals fa_fwd.
 * fa_bwd_sink: sinks and dsinks both NULL (= fa_bwd) or both given; dsinks
 * [H] is overwritten with d sum(o*dO) / d sink summed over the batch
 * (accumulated with float atomics: the last bits may vary run to run). */
int fa_fwd_sink(const void* q, const void* k, const void* v, void* o,
                float* lse, const float* sinks, float* max_logit, int B, int H,
                int Hkv, int T, int d, float scale, int window,
                int global_every, float softcap, hipStream_t stream);
int fa_bwd_sink(const void* q, const void* k, const void* v, const void* o,
                const float* lse, const void* dO, const float* sinks,
                void* dq, void* dk, void* dv, float* dsinks, int B, int H,
                int Hkv, int T, int d, float scale, int window,
                int global_every, float softcap, hipStream_t stream);

/* Single-query decode over a preallocated KV cache (Forge commit "Add HF
 * streaming data pipeline and three research reports", INFERENCE_RESEARCH.md
 * section 2: cache [layer][head][seq][d] preallocated at the maximum length;
 * one query per sequence; split along the cache for long contexts).
 *   q        [B, H, d]        bf16, the new token's query (RoPE applied)
 *   k_cache  [B, Hkv, S, d]   bf16, one layer's cache, S = allocated length
 *   v_cache  [B, Hkv, S, d]   bf16
 *   lens     [B]              int32 device array: tokens held by sequence b,
 *                             the new one included (its query is at position
 *                             lens[b]-1); values are clamped to [0, S]
 *   o        [B, H, d]        bf16 output
 *   lse      [B, H]           float32 output (natural log), or NULL
 *   sinks    [H]              float32 sink logits, or NULL
 * Head h reads KV head h / (H/Hkv) (H/Hkv <= 32); keys j < lens[b] with
 * j > lens[b]-1-window are visible (window 0 = all); softcap as in fa_fwd.
 * Cache rows at or past lens[b] are never read.  lens[b] = 0 gives o = 0
 * and lse = -inf (= the sink with a sink).  The call allocates its float32
 * chunk scratch with hipMallocAsync on `stream` and frees it there.
 * Returns FA_OK, FA_ERR_INVALID_ARG or FA_ERR_UNSUPPORTED (d not 64, 128,
 * 256; more than 32 heads per KV head), FA_ERR_HIP. */
int fa_decode(const void* q, const void* k_cache, const void* v_cache,
              const int* lens, void* o, float* lse, const float* sinks, int B,
              int H, int Hkv, int S, int d, float scale, int window,
              float softcap, hipStream_t stream);

/* The chunking fa_decode uses for these sizes (host only): nsplit chunks of
 * `chunk` keys (a multiple of 32) over the visible range of each sequence. */
int fa_decode_splits(int B, int Hkv, int S, int window, int* nsplit,
                     int* chunk);

/* RoPE on interleaved pairs (x[2i], x[2i+1]) at positions t = 0..T-1 with
 * angle fl32(t * inv_freq[i]) (Forge README: interleaved pairs; Forge
 * attention.h commit log, "Wave 1": kernels read a host-precomputed
 * inverse-frequency table).  rope_apply rotates by +angle, rope_apply_bwd
 * (its transpose) by -angle. */
int rope_apply(const void* x, void* y, const float* inv_freq, int B, int H,
               int T, int d, hipStream_t stream);
int rope_apply_bwd(const void* dy, void* dx, const float* inv_freq, int B,
                   int H, int T, int d, hipStream_t stream);

/* float32 twins: same parameters and semantics, float32 tensors. */
int fa_fwd_f32(const void* q, const void* k, const void* v, void* o,
               float* lse, int B, int H, int Hkv, int T, int d, float scale,
               int window, int global_every, float softcap,
               hipStream_t stream);
int fa_bwd_f32(const void* q, const void* k, const void* v, const void* o,
               const float* lse, const void* dO, void* dq, void* dk,
               void* dv, int B, int H, int Hkv, int T, int d, float scale,
               int window, int global_every, float softcap,
               hipStream_t stream);
int rope_apply_f32(const void* x, void* y, const float* inv_freq, int B,
                   int H, int T, int d, hipStream_t stream);
int rope_apply_bwd_f32(const void* dy, void* dx, const float* inv_freq,
                       int B, int H, int T, int d, hipStream_t stream);

/* Host helpers (no device work). */

/* Effective window of layer `layer` (0-based) of a local:global stack
 * (Forge attention.h commit log, "Wave 2": sliding_window with
 * sliding_global_every; ARCHITECTURES.md family table: Gemma 3 is 5 local
 * to 1 global): returns 0 (global, full causal) when global_every > 0 and
 * (layer + 1) % global_every == 0, else `window`.  Returns FA_ERR_INVALID_ARG
 * for layer < 0, window < 0 or global_every < 0. */
int fa_layer_window(int layer, int window, int global_every);

/* Fills host_out[i] = theta^(-2i/d) for i < d/2 (computed in double,
 * stored as float).  Returns 0, or FA_ERR_INVALID_ARG for a null pointer,
 * odd or non-positive d, or theta <= 0. */
int fa_rope_inv_freq(float* host_out, int d, double theta);

/* Inverse frequencies with the "llama3" context-extension rescaling
 * (Forge ARCHITECTURES.md, "Formules clés"): starting from theta^(-2i/d),
 * a component of wavelength 2*pi/f shorter than orig_ctx/high_freq_factor is
 * kept, one longer than orig_ctx/low_freq_factor is divided by `factor`, and
 * in between s = (orig_ctx/wavelength - low)/(high - low) blends the two:
 * (1-s)*f/factor + s*f.  factor <= 0 means off (plain table; config default
 * rope_scale_factor(0)).  Computed in double, stored as float.  Returns 0 or
 * FA_ERR_INVALID_ARG (bad d/theta, or not high > low > 0, orig_ctx > 0). */
int fa_rope_inv_freq_llama3(float* host_out, int d, double theta, double factor,
                            double low_freq_factor, double high_freq_factor,
                            double orig_ctx);

/* RoPE base of layer `layer`: theta_global for the global layers of a
 * local:global stack (same rule as fa_layer_window) when theta_global > 0,
 * else theta (Forge attention.h commit log, "Wave 2": rope_theta_global).
 * Writes *out; returns 0 or FA_ERR_INVALID_ARG. */
int fa_layer_rope_theta(int layer, double theta, double theta_global,
                        int global_every, double* out);

/* Per-kernel timing for callers that measure (benchmarks, profilers):
 * `events` are `count` (<= 16) hipEvent_t handles created by the caller.
 * While armed (count > 0), every later call on this thread records
 * events[0] on its stream before its first kernel and events[i] right
 * after its i-th kernel launch, for i < count (fa_bwd launches the kernels
 * fa_bwd_kernels names; fa_fwd and rope_* launch 1).  count = 0
 * disarms.  Returns 0, or FA_ERR_INVALID_ARG for count outside 0..16 or a
 * null handle.  Thread-local state; no device work. */
int fa_set_stage_events(void* const* events, int count);

/* The kernels the bf16 fa_bwd (and its _rope and _vdim variants) launches
 * for head sizes (d, d_v), in launch order, comma-separated, under the
 * current dQ mode (fa_set_dq_mode):
 *   "rowdot,dkdv,dq_ds" -- dQ from stored dS: the prologue D = rowsum(dO o)
 *                          alone, the key-parallel dK/dV pass writing every
 *                          visible dS tile (bf16) to a workspace, then the
 *                          query-parallel dQ pass dq = scale dS K reading it
 *                          (d = d_v = 256 in mode 0, 128 and 256 in mode 2;
 *                          taken when the workspace, 2 KB per (query tile,
 *                          key tile) of the band, fits a quarter of the
 *                          device's memory);
 *   "dq,dkdv"           -- the query-parallel dQ pass recomputing S and dP
 *                          (it also writes D), then the dK/dV pass;
 * null for sizes the backward does not support.  fa_bwd_sink and
 * fa_bwd_noalloc always run "dq,dkdv".  Static string owned by the library;
 * host only, no device work.  (Forge attention.h commit log, "Measured
 * findings": register pressure, not bandwidth, dominates the attention
 * backward -- storing dS trades the recomputation's registers and flops
 * for HBM traffic, which pays at d = 256.) */
const char* fa_bwd_kernels(int d, int d_v);

/* The dS workspace the bf16 fa_bwd (and fa_bwd_rope) takes for these sizes
 * under the current dQ mode, for callers that plan device memory: *bytes
 * (0 when the recomputing dQ pass runs), and its shape -- *query_tiles =
 * ceil(T/32) query tiles per (b, h), each with *band_tiles 2 KB slots, one
 * per key tile of 32 that holds a visible key of the query tile (under a
 * window W: ceil((W - 1)/32) + 1, else ceil(T/32); ARCHITECTURES.md,
 * prioritised plan, wave 2, item 8: the mask q - W < k <= q).  The backward
 * takes it from the library's pool when it fits a quarter of the device's
 * memory.  Host only, no device work.  Returns 0, or FA_ERR_INVALID_ARG /
 * FA_ERR_UNSUPPORTED as fa_bwd's size checks (H stands for Hkv). */
int fa_bwd_workspace(int B, int H, int T, int d, int d_v, int window,
                     size_t* bytes, int* query_tiles, int* band_tiles);

/* Process-wide dQ strategy of the bf16 backward, for measurement and tests:
 * 0 (the default) takes dQ from stored dS at d = 256, where it measured
 * faster, 1 always runs the recomputing dQ pass, 2 takes dQ from stored dS
 * at d = 128 and 256.  Both give dq within the parity
 * bound of the oracle; dk and dv are bit for bit the same in both.  Returns
 * the previous mode, or FA_ERR_INVALID_ARG for another value.  Calls
 * already enqueued keep the mode they were enqueued with. */
int fa_set_dq_mode(int mode);

/* Measurement behind the choice of the dQ strategy (host call, synchronous;
 * allocates and frees its own buffer): the time in ms (best of three) of
 * only the global float atomics that accumulating dQ inside the key-parallel
 * dK/dV pass would issue for this shape -- one add per element of each
 * query tile's [rows x d] block per key block that sees it, into a
 * [B, H, T, d] float32 accumulator, in that pass's key blocks and order.  A
 * lower bound on that variant's extra cost, to set beside the time of the
 * separate dQ pass.  Returns 0, FA_ERR_INVALID_ARG/UNSUPPORTED (as fa_fwd's
 * sizes) or FA_ERR_HIP. */
int fa_measure_dq_atomics(int B, int H, int Hkv, int T, int d, int window,
                          float* ms);

/* Thread-local text of the last failure ("" if none yet). */
const char* fa_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* CAUSAL_FA_H */
