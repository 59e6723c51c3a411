/*
 * h2o.h -- C ABI of the chunked H2O (heavy-hitter) sparse attention step on
 * AMD Instinct MI355X (gfx950).
 *
 * Method: "Learning how to Forget: Fine-tuning for Long-Context Sparse
 * Attention" (arXiv 2608.19920), cited below as LHF:
 *   - Fig. 1(a): a row of chunks -- a prefill chunk of length N_C, then
 *     chunks of length S << N_C;
 *   - §1 Introduction ¶1: keys and values live in a fixed-size KV cache whose
 *     slots are evicted once it is full;
 *   - §1 ¶3: grouped query attention (G = Hq / Hkv query heads share a KV
 *     head; query head h reads KV head h / G);
 *   - §1 ¶4, abstract, and the FAQ answer on H2O of the docshare abstract
 *     page: H2O (the heavy-hitter oracle, reference [72]) served by an SDPA
 *     kernel that also returns summed attention weights;
 *   - contributions bullet of §1: the cache buffer follows a linear
 *     recurrence -- each step overwrites some slots of the previous buffer
 *     (the delta of Fig. 1(c)).
 *
 * One step (h2o_chunk_step) on every (batch b, KV head k):
 *   1. attend: query i of the chunk sees every filled cache slot and the
 *      chunk's keys j <= i; z = scale * q.key, softmax, out = P V;
 *      lse = natural-log logsumexp of z over the visible keys;
 *   2. score: every filled slot m gains sum_{g,i} P[g,i,m] (summed over the
 *      chunk's queries and the group's G query heads); chunk key j gets
 *      mu_j = sum_{g, i >= j} P[g,i,j];
 *   3. select: free slots (position < 0) are used first, lowest index first;
 *      the remaining n_e = S - n_free targets are evicted: the n_e filled
 *      slots outside the recent window (position < T - W, T = tokens seen
 *      before the chunk) with the smallest (score, slot index);
 *   4. write: chunk token j goes to the j-th smallest target slot R_j:
 *      K[R_j] = k_j, V[R_j] = v_j, score[R_j] = mu_j, position[R_j] = T + j.
 *   T then advances by S.  The prefill is the same step on an empty cache.
 * The score rule (plain cumulative sum since insertion), the step order, the
 * window test and the tie-break are readings of pages that leave them open.
 *
 * Eviction policy (h2o_config.policy): H2O_POLICY_H2O is the step above.
 * The position policies H2O_POLICY_RECENT and H2O_POLICY_SINK_RECENT (the
 * pages' lr and slr rows among their five KV cache policies, Tables 1 and 6;
 * sinks after the attention-sinks paper in their reference list) skip step
 * 2 and rank the candidates by (position, slot index) instead, so the oldest
 * tokens go; SINK_RECENT never evicts positions below n_sink.  They keep no
 * score: a written slot's score is 0 and the others are left as they are.
 *
 * Conventions for every call:
 *   - Buffer pointers are DEVICE pointers to contiguous, 16-byte aligned
 *     memory owned by the caller; the library never allocates device memory.
 *     A non-NULL buffer pointer that is not 16-byte aligned is refused with
 *     H2O_ERR_ALIGN before anything is enqueued (the kernels move 16-byte
 *     pieces).
 *   - Element type of q/k/v/out/cache is the config's dtype (bf16 or fp32);
 *     scores, lse and masses are fp32; positions and slot ids are int32.
 *   - Layouts: q, out [B, Hq, S, d]; k, v [B, Hkv, S, d]; cache K, V
 *     [B, Hkv, M, d]; scores, positions [B, Hkv, M]; lse [B, Hq, S].
 *   - `stream` is a hipStream_t (NULL = the default stream).  Work is only
 *     enqueued; no call synchronises the device except where stated.
 *   - Arguments are validated on the host before anything is enqueued; on
 *     every error but H2O_ERR_HIP nothing is enqueued and the cache state is
 *     unchanged.  H2O_ERR_HIP means a launch failed part-way through a call:
 *     kernels enqueued before it may have updated the state, so the handle
 *     should be destroyed (a snapshot taken earlier can be adopted again).
 *   - A handle is not thread-safe; calls on one handle must be issued in
 *     order on one stream.
 */
#ifndef H2O_MI355X_H
#define H2O_MI355X_H

#include <stddef.h>
#include <stdint.h>

#if defined(__GNUC__)
#define H2O_API __attribute__((visibility("default")))
#else
#define H2O_API
#endif

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  H2O_OK = 0,
  H2O_ERR_NULL = 1,        /* a required pointer is NULL                        */
  H2O_ERR_CONFIG = 2,      /* config out of range (see h2o_validate_config)      */
  H2O_ERR_SHAPE = 3,       /* chunk length out of range for this call            */
  H2O_ERR_STATE = 4,       /* call not allowed in the current cache state        */
  H2O_ERR_WORKSPACE = 5,   /* workspace smaller than h2o_workspace_bytes()       */
  H2O_ERR_HIP = 6,         /* a HIP call failed; see h2o_last_hip_error()        */
  H2O_ERR_UNSUPPORTED = 7, /* valid request the library does not implement       */
  H2O_ERR_ALIGN = 8,       /* a buffer pointer is not 16-byte aligned            */
  H2O_ERR_TOO_LARGE = 9    /* request exceeds h2o_chunk_backward_static's scratch */
} h2o_status;

typedef enum { H2O_BF16 = 0, H2O_FP32 = 1 } h2o_dtype;
typedef enum { H2O_POLICY_H2O = 0, H2O_POLICY_RECENT = 1, H2O_POLICY_SINK_RECENT = 2 } h2o_policy;

typedef struct {
  int32_t batch;          /* B >= 1                                               */
  int32_t n_q_heads;      /* Hq, a multiple of Hkv                                */
  int32_t n_kv_heads;     /* Hkv >= 1                                             */
  int32_t head_dim;       /* d: 64 or 128                                         */
  int32_t cache_slots;    /* M >= 1 slots per (b, KV head)                        */
  int32_t recent_window;  /* W >= 0; M - W >= max_chunk keeps eviction feasible   */
  int32_t max_chunk;      /* largest S accepted by h2o_chunk_step                 */
  int32_t max_prefill;    /* largest N_C accepted by h2o_prefill (<= M)           */
  int32_t dtype;          /* h2o_dtype                                            */
  float softmax_scale;    /* <= 0 selects 1/sqrt(d)                               */
  int32_t policy;         /* h2o_policy (0 = H2O)                                 */
  int32_t n_sink;         /* SINK_RECENT: positions < n_sink are kept; else 0     */
} h2o_config;

typedef struct h2o_cache h2o_cache;   /* opaque host-side handle */

/* Host only (no HIP call): H2O_OK if the config is usable.  Checks B, Hq, Hkv
 * >= 1, Hq % Hkv == 0, d in {64, 128}, dtype known, 1 <= max_chunk,
 * 1 <= max_prefill <= M, 0 <= W and M - W >= max_chunk (a reading of the pages:
 * with it every eviction finds enough candidates), M, max_chunk and
 * max_prefill <= 16384, (Hq / Hkv) * max(max_chunk, max_prefill) <= 2^20
 * query rows per KV group, every chunk tensor below 2^31 elements, a known
 * policy, n_sink = 0 unless the policy is SINK_RECENT, and for SINK_RECENT
 * 0 <= n_sink and M - W - n_sink >= max_chunk. */
H2O_API h2o_status h2o_validate_config(const h2o_config* cfg);

/* Host only: bytes of device workspace h2o_cache_init needs for `cfg`
 * (0 if the config is invalid).  Holds per-split score partials, an lse
 * buffer for calls that pass lse = NULL, per-head counters and a status
 * word. */
H2O_API size_t h2o_workspace_bytes(const h2o_config* cfg);

/* Creates a handle over caller-owned state buffers.
 * k_cache, v_cache [B,Hkv,M,d] dtype; scores, positions [B,Hkv,M];
 * workspace >= h2o_workspace_bytes(cfg) bytes (kept for the handle's life).
 * adopt = 0: the state is reset on `stream` (positions -1, scores 0; K/V left
 *   as they are) and tokens_seen must be 0.
 * adopt = 1: the buffers already hold a valid state after `tokens_seen`
 *   tokens (resume from a snapshot); nothing but the workspace is touched.
 * In both cases the K/V rows of free slots (position < 0) must hold finite
 *   values (zeros, say): the attention and its backward read them as part of
 *   whole tiles and give them zero weight, which keeps NaN or Inf bit
 *   patterns in unused memory from reaching any output only if the values
 *   themselves are finite.
 * The workspace counters are cleared on `stream` in both cases.
 * The handle belongs to the device current at this call: its compute-unit
 * count sizes the grids of small steps, and every later call on the handle
 * must run with that device current.
 * Errors: H2O_ERR_NULL, H2O_ERR_ALIGN, H2O_ERR_CONFIG, H2O_ERR_WORKSPACE,
 * H2O_ERR_STATE (adopt = 0 with tokens_seen != 0, or tokens_seen < 0),
 * H2O_ERR_HIP (also when the device cannot be queried). */
H2O_API h2o_status h2o_cache_init(const h2o_config* cfg, void* k_cache, void* v_cache,
                          float* scores, int32_t* positions, void* workspace,
                          size_t workspace_bytes, int32_t adopt,
                          int64_t tokens_seen, void* stream, h2o_cache** out);

/* The prefill chunk of length n = N_C (LHF Fig. 1(a)): causal attention over
 * the chunk, then its K/V written to slots 0..n-1 with their masses as scores.
 * q [B,Hq,n,d]; k, v [B,Hkv,n,d]; out [B,Hq,n,d]; lse [B,Hq,n] or NULL.
 * Errors: H2O_ERR_NULL, H2O_ERR_ALIGN; H2O_ERR_SHAPE unless 1 <= n <= max_prefill;
 * H2O_ERR_STATE unless the handle has seen no token yet; H2O_ERR_HIP. */
H2O_API h2o_status h2o_prefill(h2o_cache* c, const void* q, const void* k,
                       const void* v, int32_t n, void* out, float* lse,
                       void* stream);

/* One H2O chunk step of length s (steps 1-4 above).
 * q [B,Hq,s,d]; k_new, v_new [B,Hkv,s,d]; out [B,Hq,s,d]; lse [B,Hq,s] or NULL.
 * Optional outputs (NULL to skip):
 *   slots_out [B,Hkv,s] int32: slot R_j chunk token j was written to;
 *   step_mass [B,Hkv,M+s] fp32: the step's mass per cache slot (0 for slots
 *     that were free) followed by mu_j per chunk key (H2O policy only: a
 *     position policy computes no mass and returns H2O_ERR_UNSUPPORTED);
 *   k_old, v_old [B,Hkv,s,d]: the rows the step overwrote (zeros where a
 *     free slot was filled) -- the buffer delta of LHF Fig. 1(c);
 *   pos_old [B,Hkv,s] int32: the position slot R_j held before the step (-1
 *     where a free slot was filled).  slots_out, k_old/v_old and pos_old
 *     together let h2o_recurrence_backward_step undo the step.
 * Errors: H2O_ERR_NULL (also one of k_old, v_old without the other),
 * H2O_ERR_ALIGN, H2O_ERR_UNSUPPORTED (step_mass with a position policy),
 * H2O_ERR_SHAPE unless 1 <= s <= max_chunk, H2O_ERR_STATE (tokens seen would
 * pass 2^31 - 1), H2O_ERR_HIP.
 * If a state adopted through h2o_cache_init has fewer evictable slots than
 * the step needs, no slot of that (b, head) is written (K/V and positions
 * unchanged; its scores have received the step's mass) and bit 0 of the
 * device status word is set (see h2o_device_status).  The optional outputs
 * of that head are still all written: slots_out and pos_old -1 (a slot
 * outside [0, M), which h2o_recurrence_backward_step skips), k_old/v_old
 * zero, step_mass the masses the step computed. */
H2O_API h2o_status h2o_chunk_step(h2o_cache* c, const void* q, const void* k_new,
                          const void* v_new, int32_t s, void* out, float* lse,
                          int32_t* slots_out, float* step_mass, void* k_old,
                          void* v_old, int32_t* pos_old, void* stream);

/* Enqueues device-to-device copies of the scores [B,Hkv,M] into scores_out
 * and, if positions_out != NULL, of the positions.  Errors: H2O_ERR_NULL,
 * H2O_ERR_ALIGN, H2O_ERR_HIP. */
H2O_API h2o_status h2o_get_scores(const h2o_cache* c, float* scores_out,
                          int32_t* positions_out, void* stream);

/* Frozen-eviction backward of one chunk's attention (the per-cell autograd of
 * LHF Fig. 1(b) for one chunk): gradients of sum(out * d_out) with the
 * visible sets of the forward step (every slot with position >= 0, and chunk
 * keys j <= i) and the scores held constant.  Stateless: uses `cfg` only.
 * Inputs: q [B,Hq,s,d]; the PRE-step cache k_cache, v_cache [B,Hkv,M,d]
 * (free-slot rows finite, as for h2o_cache_init) and positions [B,Hkv,M]; k_new, v_new [B,Hkv,s,d]; the forward's out
 * [B,Hq,s,d] and lse [B,Hq,s]; d_out [B,Hq,s,d].
 * Outputs (every element written): dq [B,Hq,s,d]; dk_cache, dv_cache
 * [B,Hkv,M,d] (zero at free slots); dk_new, dv_new [B,Hkv,s,d]; all bf16.
 * dK/dV of a KV head sum over the G query heads of its group.
 * workspace >= h2o_backward_workspace_bytes(cfg, s) (holds dO . O per row and
 * the fp32 partial dK/dV of the chunk keys; contents need no initialisation).
 * Deterministic (no atomics).  Errors: H2O_ERR_NULL, H2O_ERR_ALIGN, H2O_ERR_CONFIG,
 * H2O_ERR_UNSUPPORTED (fp32 configs), H2O_ERR_SHAPE (s < 1 or s larger than
 * max(max_chunk, max_prefill)), H2O_ERR_WORKSPACE, H2O_ERR_HIP. */
H2O_API h2o_status h2o_chunk_backward(const h2o_config* cfg, const void* q,
                              const void* k_cache, const void* v_cache,
                              const int32_t* positions, const void* k_new,
                              const void* v_new, int32_t s, const void* out,
                              const float* lse, const void* d_out, void* dq,
                              void* dk_cache, void* dv_cache, void* dk_new,
                              void* dv_new, void* workspace,
                              size_t workspace_bytes, void* stream);

/* Host only: workspace bytes h2o_chunk_backward needs for chunk length s
 * (0 if the config is invalid or s < 1). */
H2O_API size_t h2o_backward_workspace_bytes(const h2o_config* cfg, int32_t s);

/* h2o_chunk_backward without a workspace argument, for callers that cannot
 * allocate device memory (code under graph capture, serving loops, harnesses
 * that forbid allocation).  Same arguments (minus workspace), outputs,
 * determinism and errors as h2o_chunk_backward; the kernels are the same.
 * Its scratch is a static device array of 72 MiB that the library holds on
 * every GPU it runs on until the process ends, found once per device with
 * hipGetSymbolAddress on the first call there; the call itself allocates
 * nothing.  Requests whose h2o_backward_workspace_bytes(cfg, s) exceeds
 * 72 MiB are refused with H2O_ERR_TOO_LARGE before anything is enqueued
 * (at d = 128 that allows B * Hkv * ceil(s / 128) * 128 up to 16384 chunk
 * keys, e.g. 8 KV heads of a 2048-token chunk).  Nothing in the scratch
 * needs to start at zero.  Every call on one GPU shares that GPU's scratch:
 * calls that overlap on one GPU (other streams, other threads) race and
 * must be ordered by the caller. */
H2O_API h2o_status h2o_chunk_backward_static(const h2o_config* cfg, const void* q,
                                     const void* k_cache, const void* v_cache,
                                     const int32_t* positions, const void* k_new,
                                     const void* v_new, int32_t s, const void* out,
                                     const float* lse, const void* d_out, void* dq,
                                     void* dk_cache, void* dv_cache, void* dk_new,
                                     void* dv_new, void* stream);

/* One step of the backward walk through the KV buffer over a row of chunks
 * (LHF Fig. 1(b), with the buffer kept as the deltas of Fig. 1(c)): the
 * cache after a step depends on every earlier chunk's keys and values, so a
 * chunk token's key/value gradient collects the gradient of every later step
 * that read the slot the token was written to, up to the step that
 * overwrote it.  Call it for the steps in reverse order (last chunk first,
 * the prefill last).  For step c it
 *   1. undoes the step on the cache: rows slots[b,h,j] of k_cache/v_cache get
 *      k_old/v_old[b,h,j] and their positions pos_old[b,h,j] (the delta that
 *      h2o_chunk_step exported), leaving the cache as step c saw it;
 *   2. routes what later steps owe the step's tokens: for token j written
 *      to slot m = slots[b,h,j], gk[b,h,j] = acc_k[b,h,m], then
 *      acc_k[b,h,m] = 0 (the same for v);
 *   3. runs the frozen-eviction backward of the step on that cache (as
 *      h2o_chunk_backward) in fp32 accumulating form: dq [B,Hq,s,d] (dtype)
 *      is the step's query gradient, the cache gradient is added to every
 *      filled slot (acc_k += dK_c, acc_v += dV_c) and the chunk keys' own
 *      gradient to gk, gv (fp32 [B,Hkv,s,d]), which end as each token's
 *      total key/value gradient.  No gradient is rounded on its way
 *      through the walk.
 * acc_k, acc_v: fp32 [B,Hkv,M,d], zero before the last step's call, carried
 *   between the calls (each slot holds the gradient owed to its occupant).
 * The prefill is undone as a step whose slots are 0..n-1 of every head,
 *   pos_old = -1 and k_old = v_old = zeros.  Scores are neither read nor
 *   changed.  q, k_new, v_new, out, lse, d_out: the step's forward inputs and
 *   outputs and the output gradient, as for h2o_chunk_backward.
 * A slot index outside [0, M) (a step that wrote nothing for that head) is
 *   skipped by the undo and the routing.
 * workspace >= h2o_recurrence_workspace_bytes(cfg, s) (the backward's:
 *   h2o_backward_workspace_bytes).  Deterministic.
 * Errors: H2O_ERR_NULL, H2O_ERR_ALIGN, H2O_ERR_CONFIG, H2O_ERR_UNSUPPORTED
 * (fp32 configs), H2O_ERR_SHAPE (s < 1 or s larger than max(max_chunk,
 * max_prefill)), H2O_ERR_WORKSPACE, H2O_ERR_HIP. */
H2O_API h2o_status h2o_recurrence_backward_step(
    const h2o_config* cfg, void* k_cache, void* v_cache, int32_t* positions,
    const int32_t* slots, const void* k_old, const void* v_old, const int32_t* pos_old,
    const void* q, const void* k_new, const void* v_new, int32_t s, const void* out,
    const float* lse, const void* d_out, float* acc_k, float* acc_v, void* dq, float* gk,
    float* gv, void* workspace, size_t workspace_bytes, void* stream);

/* Host only: workspace bytes h2o_recurrence_backward_step needs for step
 * length s (0 if the config is invalid or s < 1). */
H2O_API size_t h2o_recurrence_workspace_bytes(const h2o_config* cfg, int32_t s);

/* Tokens seen so far (T). */
H2O_API int64_t h2o_tokens_seen(const h2o_cache* c);

/* Synchronises `stream`, returns the device status word in *flags and
 * clears it.  Bit 0: an adopted state had too few evictable slots.  Bit 1:
 * in a step whose selection ran in several workgroups per (b, KV head)
 * (chunks of 257..4096 tokens), the workgroup that rewrites the head's scores
 * and positions waited past its bound (about a second) for the others to
 * finish reading them, and wrote anyway; that step's eviction is then not
 * guaranteed.  Normal steps never set it.  For tests of that bounded wait
 * only, h2o_cache_init reads two environment variables: H2O_SELECT_SPIN_LIMIT
 * (polls before giving up; unset or 0: the default) and H2O_SELECT_SYNC_SKEW
 * (added to the count of reads the wait expects, which makes it wait out its
 * bound). */
H2O_API h2o_status h2o_device_status(h2o_cache* c, void* stream, int32_t* flags);

/* Per-kernel timing with HIP events recorded on the launch stream around
 * the launches of the kernels selected by `kernel_mask` (bit k = kernel id
 * k; -1 = all, 0 = off).  Kernel ids: 0 attention forward, 1 score
 * accumulation, 2 eviction select, 3 state reset, 4 K/V scatter.  Each
 * bracketed launch adds two event records to the stream, so select only
 * the kernels of interest when the step time matters.  h2o_get_timing
 * synchronises on the recorded events and returns the milliseconds and the
 * launch count of kernel_id summed over every bracketed launch since the
 * handle was created (H2O_ERR_SHAPE for an id outside 0..4). */
H2O_API h2o_status h2o_set_timing(h2o_cache* c, int32_t kernel_mask);
H2O_API h2o_status h2o_get_timing(h2o_cache* c, int32_t kernel_id, double* total_ms,
                          int64_t* launches);

H2O_API void h2o_cache_destroy(h2o_cache* c);
H2O_API const char* h2o_status_str(h2o_status s);
H2O_API int32_t h2o_last_hip_error(const h2o_cache* c);   /* last hipError_t, 0 if none */

#ifdef __cplusplus
}
#endif
#endif /* H2O_MI355X_H */
