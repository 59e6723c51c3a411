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
//   undo + gather (this file): cache row slots[j] <- (k_old[j], v_old[j]),
//          its position <- pos_old[j] (the cache as step c saw it), and
//          gk[j] = acc_k[slots[j]], acc_k[slots[j]] = 0: what later steps
//          owe token j leaves the slot before the slot's earlier occupant
//          collects step c's gradient;
//   the frozen-eviction backward of step c on that cache (attn_bwd.hip) in
//          its accumulating form: acc_k[m] += dK_c[m] for every filled slot
//          m, and gk[j] += dk_new[j];
//   the same for v.  acc_k, acc_v, gk, gv are fp32 throughout: no gradient
//   is rounded on its way through the walk.
#include "h2o_device.h"
#include "h2o_launch.h"

namespace h2o {
namespace {

constexpr int kRecThreads = 256;

// One thread per 4 floats of a chunk row (bh * S + j): the token's
// accumulator row is gathered and cleared, and the threads of the row's
// first row_bytes / 16 chunks also put the old K/V row back.  A slot outside
// [0, M) (a step that wrote nothing for the head) undoes nothing and
// gathers zeros.
__global__ __launch_bounds__(kRecThreads) void undo_gather_kernel(
    char* __restrict__ kc, char* __restrict__ vc, int32_t* __restrict__ pos,
    const int32_t* __restrict__ slots, const char* __restrict__ k_old,
    const char* __restrict__ v_old, const int32_t* __restrict__ pos_old, float* __restrict__ acc_k,
    float* __restrict__ acc_v, float* __restrict__ gk, float* __restrict__ gv, int S, int M, int D,
    int row_bytes, int64_t n) {
  const int64_t idx = static_cast<int64_t>(blockIdx.x) * kRecThreads + threadIdx.x;
  if (idx >= n) return;
  const int c4n = D >> 2;
  const int64_t r = idx / c4n;                     // bh * S + j
  const int c4 = static_cast<int>(idx - r * c4n);
  const int bh = static_cast<int>(r / S);
  const int slot = slots[r];
  f32x4 a = {0.f, 0.f, 0.f, 0.f}, b = {0.f, 0.f, 0.f, 0.f};
  if (slot >= 0 && slot < M) {
    const size_t srow = static_cast<size_t>(bh) * M + slot;
    f32x4* ak = reinterpret_cast<f32x4*>(acc_k + srow * D + 4 * c4);
    f32x4* av = reinterpret_cast<f32x4*>(acc_v + srow * D + 4 * c4);
    a = *ak;
    b = *av;
    *ak = f32x4{0.f, 0.f, 0.f, 0.f};
    *av = f32x4{0.f, 0.f, 0.f, 0.f};
    if (16 * c4 < row_bytes) {
      const size_t dst = srow * row_bytes + 16 * c4;
      const size_t src = static_cast<size_t>(r) * row_bytes + 16 * c4;
      store_u32x4(kc + dst, load_u32x4(k_old + src));
      store_u32x4(vc + dst, load_u32x4(v_old + src));
    }
    if (c4 == 0) pos[srow] = pos_old[r];
  }
  *reinterpret_cast<f32x4*>(gk + r * D + 4 * c4) = a;
  *reinterpret_cast<f32x4*>(gv + r * D + 4 * c4) = b;
}

}  // namespace

hipError_t launch_undo_gather(const StepShape& sh, const RecurrenceArgs& a, int dtype, hipStream_t st) {
  const int n_heads = sh.B * sh.Hkv;
  const int row_bytes = sh.D * (dtype == kBF16 ? 2 : 4);
  const int64_t n = static_cast<int64_t>(n_heads) * sh.S * (sh.D / 4);
  hipLaunchKernelGGL(undo_gather_kernel, dim3(static_cast<unsigned>((n + kRecThreads - 1) / kRecThreads)),
                     dim3(kRecThreads), 0, st, static_cast<char*>(a.k_cache), static_cast<char*>(a.v_cache),
                     a.pos, a.slots, static_cast<const char*>(a.k_old), static_cast<const char*>(a.v_old),
                     a.pos_old, a.acc_k, a.acc_v, a.gk, a.gv, sh.S, sh.M, sh.D, row_bytes, n);
  return hipGetLastError();
}

}  // namespace h2o
