// Host-side launch interface between the C ABI (api.hip) and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace h2o {

// Shapes of one step.  Cache tensors are [B,Hkv,M,D]; chunk tensors
// [B,H*,S,D]; `n_cache` leading slots are scanned (slots beyond hold nothing).
struct StepShape {
  int B, Hq, Hkv, D, S, M, W;
  int n_cache;
  float scale;      // softmax scale applied to q.k
  int policy = 0;   // 0 H2O (score key), 1 recent, 2 sink_recent (position key)
  int n_sink = 0;   // sink_recent: positions below n_sink are never evicted
  int n_cu = 256;   // compute units of the device (sizes the grids of small steps)
  bool all_filled = false;   // every one of the M slots holds a token (known on the host)
};

struct AttnArgs {
  const void* q;
  const void* k_cache;
  const void* v_cache;
  const int32_t* pos;
  const void* k_new;
  const void* v_new;
  void* out;
  float* lse;
  float* part;      // key-split partial states (workspace; NULL: never split)
};

// rows of key-split partial state the attention may use (bounds its workspace)
constexpr int64_t kSplitRows = 65536;
size_t attn_split_bytes(int B, int Hq, int S, int D);

struct ScoreArgs {
  const void* q;
  const void* k_cache;
  const void* k_new;
  const float* lse;
  float* partial;          // [B*Hkv][R][M + S]: per-split column sums
  int R;                   // row splits
};

struct SelectArgs {
  void* k_cache;
  void* v_cache;
  float* scores;
  int32_t* pos;
  const void* k_new;
  const void* v_new;
  const float* partial;   // [B*Hkv][R][M + S]: per-split masses of cache slots, then chunk keys
  int R;
  int32_t* targets;     // [B*Hkv][S] workspace: target slot of row j (flagged if it was free)
  int32_t* slots_out;   // nullable
  int32_t* pos_old;     // nullable: positions the written slots held before the step
  float* step_mass;     // nullable
  void* k_old;          // nullable
  void* v_old;          // nullable
  int32_t* status;      // device status word
  int32_t T;            // tokens seen before the chunk
  uint32_t* sync;       // [B*Hkv] counters of the parts' reads (workspace, zeroed at init)
  uint32_t sync_target; // running total of those reads once this step's are done
  uint32_t spin_limit;  // bound of part 0's wait (0: the library's default)
};

struct BackwardArgs {
  const void* q;
  const void* k_cache;     // pre-step cache
  const void* v_cache;
  const int32_t* pos;      // pre-step positions
  const void* k_new;
  const void* v_new;
  const void* out;
  const float* lse;
  const void* d_out;
  void* dq;
  void* dk_cache;
  void* dv_cache;
  void* dk_new;
  void* dv_new;
  void* workspace;         // >= backward_workspace_bytes: D_i = dO_i . O_i, partial dK/dV
  // false: dk/dv outputs are bf16 and overwritten.  true: they are fp32 and
  // the step's (scaled) gradients are added to them; free slots add nothing
  bool accumulate = false;
};

// One step of the backward walk through the buffer (recurrence.hip).
struct RecurrenceArgs {
  void* k_cache;          // post-step cache in, pre-step cache out
  void* v_cache;
  int32_t* pos;
  const int32_t* slots;   // [B*Hkv][S] the step's delta
  const void* k_old;
  const void* v_old;
  const int32_t* pos_old;
  float* acc_k;           // [B*Hkv][M][d] carried across the walk
  float* acc_v;
  float* gk;              // [B*Hkv][S][d] total gradients of the step's tokens
  float* gv;
};

enum Dtype { kBF16 = 0, kFP32 = 1 };

hipError_t launch_attn_fwd(const StepShape& sh, const AttnArgs& a, int dtype, hipStream_t st);
// Short-chunk H2O steps (decode.hip): the attention and the column masses in
// one pass over the keys.  decode_fused_halves returns the row splits the
// kernel writes into the masses (1 to 16), or 0 when the step does not take
// it; decode_fused_max_splits bounds them over every S <= s_max.
int decode_fused_halves(const StepShape& sh, int dtype);
int decode_fused_max_splits(int G, int s_max);
hipError_t launch_decode_fused(const StepShape& sh, const AttnArgs& a, float* partial, hipStream_t st);
hipError_t launch_score(const StepShape& sh, const ScoreArgs& a, int dtype, hipStream_t st);
hipError_t launch_select(const StepShape& sh, const SelectArgs& a, int dtype, hipStream_t st);
bool select_copies_rows(const StepShape& sh);   // the select kernel also writes the K/V rows
int select_parts(const StepShape& sh);          // select workgroups per (b, KV head)
hipError_t launch_scatter(const StepShape& sh, const SelectArgs& a, int dtype, hipStream_t st);
hipError_t launch_backward(const StepShape& sh, const BackwardArgs& a, hipStream_t st);
size_t backward_workspace_bytes(int B, int Hq, int Hkv, int S, int D);
// undo the step on the cache and move each written slot's accumulator into
// its token's gradient (before the step's backward adds into both)
hipError_t launch_undo_gather(const StepShape& sh, const RecurrenceArgs& a, int dtype, hipStream_t st);
hipError_t launch_reset(float* scores, int32_t* pos, int64_t n_slots, int32_t* counters,
                        int64_t n_counters, hipStream_t st);

// Row splits the score kernel uses for a step of this shape (host heuristic).
int score_row_splits(const StepShape& sh, int dtype);
// Upper bound of score_row_splits over every S <= s_max (workspace sizing).
int score_row_splits_max();

}  // namespace h2o
