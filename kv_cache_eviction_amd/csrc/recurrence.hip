// Backward walk over a row of chunks through the KV buffer
// (h2o_recurrence_backward_step).
//
// "Learning how to Forget: Fine-tuning for Long-Context Sparse Attention"
// (arXiv 2608.19920) trains through the lattice of chunks of its Fig. 1(b):
// the cache after a chunk depends on the keys and values of every earlier
// chunk, so the gradient of a chunk token's key (value) collects, besides its
// own step's term, the gradient of every later step that read the slot the
// token was written to, up to the step that overwrote the slot.  Fig. 1(c)
// keeps the buffer as deltas (the rows each step overwrote); the walk below
// replays them backward.
//
// Per step c, walking c = last .. 0:
//   undo:  cache row slots[j] <- (k_old[j], v_old[j]), its position <-
//          pos_old[j]: the cache as step c saw it;
//   the frozen-eviction backward of step c on that cache (attn_bwd.hip);
//   route: gk[j] = dk_new[j] + acc_k[slots[j]]   (total gradient of token j)
//          acc_k[slots[j]] = 0, then acc_k[m] += dk_cache[m] for every slot m,
//          so acc_k[m] is again the gradient owed to slot m's occupant (the
//          occupant before step c, for the slots step c wrote);
//   the same for v.  acc_k, acc_v are fp32 [B,Hkv,M,d] carried by the caller.
#include "h2o_device.h"
#include "h2o_launch.h"

namespace h2o {
namespace {

constexpr int kRecThreads = 256;

// Workgroup = (head, a group of rows); thread = one 16-byte chunk of a row.
// A slot outside [0, M) (a step that wrote nothing for the head) is skipped.
__global__ __launch_bounds__(kRecThreads) void undo_step_kernel(
    char* __restrict__ kc, char* __restrict__ vc, int32_t* __restrict__ pos,
    const int32_t* __restrict__ slots, const char* __restrict__ k_old,
    const char* __restrict__ v_old, const int32_t* __restrict__ pos_old, int S, int M,
    int row_bytes, int rows_per_wg, int parts) {
  const int cpr = row_bytes >> 4;
  const int bh = static_cast<int>(blockIdx.x) / parts, part = static_cast<int>(blockIdx.x) % parts;
  const int rr = static_cast<int>(threadIdx.x) / cpr, ch = static_cast<int>(threadIdx.x) % cpr;
  const int j = part * rows_per_wg + rr;
  if (rr >= rows_per_wg || j >= S) return;
  const size_t r = static_cast<size_t>(bh) * S + j;
  const int slot = slots[r];
  if (slot < 0 || slot >= M) return;
  const size_t dst = (static_cast<size_t>(bh) * M + slot) * row_bytes + 16 * ch;
  const size_t src = r * row_bytes + 16 * ch;
  store_u32x4(kc + dst, load_u32x4(k_old + src));
  store_u32x4(vc + dst, load_u32x4(v_old + src));
  if (ch == 0) pos[static_cast<size_t>(bh) * M + slot] = pos_old[r];
}

// gk[j] = dk_new[j] + acc_k[slot_j]; acc_k[slot_j] = 0 (and v).  One thread
// per 4 elements of a chunk row.
__global__ __launch_bounds__(kRecThreads) void route_gather_kernel(
    const int32_t* __restrict__ slots, const bf16_t* __restrict__ dk_new,
    const bf16_t* __restrict__ dv_new, float* __restrict__ acc_k, float* __restrict__ acc_v,
    float* __restrict__ gk, float* __restrict__ gv, int S, int M, int D, int64_t n) {
  const int64_t idx = static_cast<int64_t>(blockIdx.x) * kRecThreads + threadIdx.x;
  if (idx >= n) return;
  const int c4 = D >> 2;
  const int64_t r = idx / c4;                      // bh * S + j
  const int e = 4 * static_cast<int>(idx - r * c4);
  const int bh = static_cast<int>(r / S);
  const int slot = slots[r];
  f32x4 gkv = __builtin_convertvector(*reinterpret_cast<const bf16x4*>(dk_new + r * D + e), f32x4);
  f32x4 gvv = __builtin_convertvector(*reinterpret_cast<const bf16x4*>(dv_new + r * D + e), f32x4);
  if (slot >= 0 && slot < M) {
    const size_t a = (static_cast<size_t>(bh) * M + slot) * D + e;
    gkv += *reinterpret_cast<const f32x4*>(acc_k + a);
    gvv += *reinterpret_cast<const f32x4*>(acc_v + a);
    *reinterpret_cast<f32x4*>(acc_k + a) = f32x4{0.f, 0.f, 0.f, 0.f};
    *reinterpret_cast<f32x4*>(acc_v + a) = f32x4{0.f, 0.f, 0.f, 0.f};
  }
  *reinterpret_cast<f32x4*>(gk + r * D + e) = gkv;
  *reinterpret_cast<f32x4*>(gv + r * D + e) = gvv;
}

// acc_k[m] += dk_cache[m] for every slot (and v).  One thread per 4 elements.
__global__ __launch_bounds__(kRecThreads) void route_accum_kernel(
    const bf16_t* __restrict__ dk_cache, const bf16_t* __restrict__ dv_cache,
    float* __restrict__ acc_k, float* __restrict__ acc_v, int64_t n4) {
  const int64_t idx = static_cast<int64_t>(blockIdx.x) * kRecThreads + threadIdx.x;
  if (idx >= n4) return;
  const int64_t e = 4 * idx;
  *reinterpret_cast<f32x4*>(acc_k + e) +=
      __builtin_convertvector(*reinterpret_cast<const bf16x4*>(dk_cache + e), f32x4);
  *reinterpret_cast<f32x4*>(acc_v + e) +=
      __builtin_convertvector(*reinterpret_cast<const bf16x4*>(dv_cache + e), f32x4);
}

}  // namespace

hipError_t launch_undo_step(const StepShape& sh, const RecurrenceArgs& a, int dtype, hipStream_t st) {
  const int n_heads = sh.B * sh.Hkv;
  const int row_bytes = sh.D * (dtype == kBF16 ? 2 : 4);
  const int rows_per_wg = kRecThreads / (row_bytes / 16);
  const int parts = (sh.S + rows_per_wg - 1) / rows_per_wg;
  hipLaunchKernelGGL(undo_step_kernel, dim3(n_heads * parts), dim3(kRecThreads), 0, st,
                     static_cast<char*>(a.k_cache), static_cast<char*>(a.v_cache), a.pos, a.slots,
                     static_cast<const char*>(a.k_old), static_cast<const char*>(a.v_old), a.pos_old,
                     sh.S, sh.M, row_bytes, rows_per_wg, parts);
  return hipGetLastError();
}

hipError_t launch_route(const StepShape& sh, const RecurrenceArgs& a, hipStream_t st) {
  const int n_heads = sh.B * sh.Hkv;
  const int64_t n_g = static_cast<int64_t>(n_heads) * sh.S * (sh.D / 4);
  hipLaunchKernelGGL(route_gather_kernel, dim3(static_cast<unsigned>((n_g + kRecThreads - 1) / kRecThreads)),
                     dim3(kRecThreads), 0, st, a.slots, static_cast<const bf16_t*>(a.dk_new),
                     static_cast<const bf16_t*>(a.dv_new), a.acc_k, a.acc_v, a.gk, a.gv, sh.S, sh.M, sh.D,
                     n_g);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int64_t n_a = static_cast<int64_t>(n_heads) * sh.M * (sh.D / 4);
  hipLaunchKernelGGL(route_accum_kernel, dim3(static_cast<unsigned>((n_a + kRecThreads - 1) / kRecThreads)),
                     dim3(kRecThreads), 0, st, static_cast<const bf16_t*>(a.dk_cache),
                     static_cast<const bf16_t*>(a.dv_cache), a.acc_k, a.acc_v, n_a);
  return hipGetLastError();
}

}  // namespace h2o
