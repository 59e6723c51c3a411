// Eviction select + scatter (steps 3 and 4 of h2o_chunk_step).
//
// "Learning how to Forget: Fine-tuning for Long-Context Sparse Attention"
// (arXiv 2608.19920): the KV cache has a fixed number of slots, evicted once
// it is full (§1 Introduction ¶1); the H2O policy (§1 ¶4, reference [72])
// evicts the slots with the lowest accumulated score; the new cache is the
// old one with some slots overwritten (the linear buffer recurrence of the
// §1 contributions bullet, whose delta Fig. 1(c) encodes).  Readings where
// the pages are silent: free slots are filled first in ascending order; a
// filled slot is evictable when its position is below T - W; victims are the
// smallest (score, slot index); chunk token j goes to the j-th smallest
// target slot.
//
// One workgroup handles a share of the chunk's rows for one (b, KV head).
// Every workgroup of a head recomputes the same selection from the same
// inputs (deterministic), copies its share of K/V rows, then counts itself
// done on a per-head counter; the last one to finish writes the new scores
// and positions (no workgroup still reads them at that point) and clears the
// counter for the next launch.  Scores are mapped to order-preserving 32-bit
// keys; the n_e-th smallest candidate is found by a 4-pass, 8-bit LDS radix
// select; equal scores resolve to the lowest slot by an exclusive scan over
// slot order.
#include "h2o_device.h"
#include "h2o_launch.h"

namespace h2o {
namespace {

constexpr int kThreads = 512;
constexpr int kWavesSel = kThreads / 64;
constexpr int kRowsPerPart = 64;
constexpr int kMaxParts = 64;

enum : uint8_t { kFree = 0, kCand = 1, kKeep = 2, kTarget = 4 };

// Order-preserving key of a float: unsigned comparison of keys matches the
// numeric order (scores are non-negative by construction; adopted states may
// carry any finite value).
__device__ __forceinline__ uint32_t order_key(float f) {
  const uint32_t u = __float_as_uint(f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ int wave_incl_scan(int v, int lane) {
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int t = __shfl_up(v, o);
    if (lane >= o) v += t;
  }
  return v;
}

// Exclusive prefix of v over the threads of the block (thread order); also
// returns the block total.  `tmp` holds kWavesSel ints of LDS.
__device__ int block_excl_scan(int v, int* tmp, int& total) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int incl = wave_incl_scan(v, lane);
  __syncthreads();
  if (lane == 63) tmp[wave] = incl;
  __syncthreads();
  int before = 0, tot = 0;
#pragma unroll
  for (int w = 0; w < kWavesSel; ++w) {
    const int x = tmp[w];
    before += (w < wave) ? x : 0;
    tot += x;
  }
  total = tot;
  return before + incl - v;
}

__global__ __launch_bounds__(kThreads) void select_scatter_kernel(
    char* __restrict__ kc, char* __restrict__ vc, float* __restrict__ scores,
    int32_t* __restrict__ pos, const char* __restrict__ kn, const char* __restrict__ vn,
    const float* __restrict__ partial, int R, int32_t* __restrict__ slots_out,
    float* __restrict__ step_mass, char* __restrict__ k_old, char* __restrict__ v_old,
    int32_t* __restrict__ counters, int32_t* __restrict__ status, int T, int W, int S, int M,
    int n_cache, int row_bytes, int n_heads, int n_parts) {
  extern __shared__ __attribute__((aligned(16))) char smem[];
  float* s_sig = reinterpret_cast<float*>(smem);                 // [M]
  int* s_R = reinterpret_cast<int*>(smem + 4 * static_cast<size_t>(M));   // [S]
  uint8_t* s_fl = reinterpret_cast<uint8_t*>(smem + 4 * static_cast<size_t>(M) + 4 * static_cast<size_t>(S));
  __shared__ uint32_t hist[256];
  __shared__ int s_tmp[kWavesSel];
  __shared__ int s_sel[2];
  __shared__ int s_last;

  const int tid = threadIdx.x, lane = tid & 63;
  const int bh = blockIdx.x % n_heads;
  const int part = static_cast<int>(blockIdx.x) / n_heads;
  const size_t PS = static_cast<size_t>(M) + S;        // partial row length
  const float* ph = partial + static_cast<size_t>(bh) * R * PS;
  float* sc_h = scores + static_cast<size_t>(bh) * M;
  int32_t* pos_h = pos + static_cast<size_t>(bh) * M;

  // 1. scores after this step's mass; slot classes
  int my_free = 0, my_cand = 0;
  for (int m = tid; m < M; m += kThreads) {
    const int p = pos_h[m];
    float s = sc_h[m];
    uint8_t fl;
    if (p < 0) {
      fl = kFree;
    } else {
      fl = (p < T - W) ? kCand : kKeep;
      if (m < n_cache) {
        float ds = 0.f;
        for (int r = 0; r < R; ++r) ds += ph[static_cast<size_t>(r) * PS + m];
        s += ds;
      }
    }
    s_sig[m] = s;
    s_fl[m] = fl;
    my_free += fl == kFree;
    my_cand += fl == kCand;
  }
  int n_free, n_cand;
  block_excl_scan(my_free, s_tmp, n_free);
  block_excl_scan(my_cand, s_tmp, n_cand);
  const int n_f = min(S, n_free);
  const int n_e = S - n_f;
  if (n_cand < n_e) {                      // infeasible adopted state: leave it untouched
    if (part == 0 && tid == 0) atomicOr(status, 1);
    return;
  }

  // 2. radix select of the n_e-th smallest candidate score (bit pattern)
  uint32_t thr = 0;
  int k_eq = 0;
  if (n_e > 0) {
    uint32_t prefix = 0, pmask = 0;
    int kk = n_e;
    for (int pass = 0; pass < 4; ++pass) {
      const int shift = 24 - 8 * pass;
      __syncthreads();
      if (tid < 256) hist[tid] = 0;
      __syncthreads();
      for (int m = tid; m < M; m += kThreads) {
        if (s_fl[m] != kCand) continue;
        const uint32_t u = order_key(s_sig[m]);
        if ((u & pmask) == prefix) atomicAdd(&hist[(u >> shift) & 255u], 1u);
      }
      __syncthreads();
      if (tid < 64) {
        int c[4], tot = 0;
#pragma unroll
        for (int q = 0; q < 4; ++q) { c[q] = static_cast<int>(hist[4 * tid + q]); tot += c[q]; }
        int cb = wave_incl_scan(tot, lane) - tot;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          if (cb < kk && kk <= cb + c[q]) { s_sel[0] = 4 * tid + q; s_sel[1] = cb; }
          cb += c[q];
        }
      }
      __syncthreads();
      prefix |= static_cast<uint32_t>(s_sel[0]) << shift;
      pmask |= 0xffu << shift;
      kk -= s_sel[1];
    }
    thr = prefix;
    k_eq = kk;      // how many candidates scoring exactly thr are taken (lowest slots)
  }

  // 3. targets in ascending slot order: each thread owns a contiguous slot range
  const int per = (M + kThreads - 1) / kThreads;
  const int lo = min(M, tid * per), hi = min(M, lo + per);
  int c_free = 0, c_eq = 0;
  for (int m = lo; m < hi; ++m) {
    const uint8_t fl = s_fl[m];
    c_free += fl == kFree;
    c_eq += (n_e > 0 && fl == kCand && order_key(s_sig[m]) == thr);
  }
  int dummy;
  int fr = block_excl_scan(c_free, s_tmp, dummy);
  int eq = block_excl_scan(c_eq, s_tmp, dummy);
  int c_t = 0;
  for (int m = lo; m < hi; ++m) {
    const uint8_t fl = s_fl[m];
    bool t = false;
    if (fl == kFree) {
      t = fr < n_f;
      ++fr;
    } else if (fl == kCand && n_e > 0) {
      const uint32_t u = order_key(s_sig[m]);
      t = (u < thr) || (u == thr && eq < k_eq);
      eq += u == thr;
    }
    if (t) s_fl[m] = fl | kTarget;
    c_t += t;
  }
  int j = block_excl_scan(c_t, s_tmp, dummy);
  for (int m = lo; m < hi; ++m)
    if ((s_fl[m] & kTarget) && j < S) s_R[j++] = m;
  __syncthreads();

  // 4. scatter this workgroup's share of the chunk's rows
  const int rows_per = (S + n_parts - 1) / n_parts;
  const int j0 = min(S, part * rows_per), j1 = min(S, j0 + rows_per);
  const int cpr = row_bytes / 16;
  for (int idx = tid; idx < (j1 - j0) * cpr; idx += kThreads) {
    const int jj = j0 + idx / cpr, c = idx % cpr;
    const int slot = s_R[jj];
    const size_t src = (static_cast<size_t>(bh) * S + jj) * row_bytes + 16 * c;
    const size_t dst = (static_cast<size_t>(bh) * M + slot) * row_bytes + 16 * c;
    const bool was_free = (s_fl[slot] & 3) == kFree;
    if (k_old) {
      const u32x4 z = {0, 0, 0, 0};
      store_u32x4(k_old + src, was_free ? z : load_u32x4(kc + dst));
      store_u32x4(v_old + src, was_free ? z : load_u32x4(vc + dst));
    }
    store_u32x4(kc + dst, load_u32x4(kn + src));
    store_u32x4(vc + dst, load_u32x4(vn + src));
  }

  // 5. the last workgroup of this head writes scores, positions and outputs
  __syncthreads();
  if (tid == 0) {
    __threadfence();
    const int prev = atomicAdd(&counters[bh], 1);
    s_last = prev == n_parts - 1;
  }
  __syncthreads();
  if (!s_last) return;
  if (tid == 0) counters[bh] = 0;
  for (int m = tid; m < M; m += kThreads) {
    const uint8_t fl = s_fl[m];
    if (!(fl & kTarget) && (fl & 3) != kFree) sc_h[m] = s_sig[m];
    if (step_mass) {
      float ds = 0.f;
      if ((fl & 3) != kFree && m < n_cache)
        for (int r = 0; r < R; ++r) ds += ph[static_cast<size_t>(r) * PS + m];
      step_mass[static_cast<size_t>(bh) * PS + m] = ds;
    }
  }
  for (int jj = tid; jj < S; jj += kThreads) {
    const int slot = s_R[jj];
    float mu = 0.f;
    for (int r = 0; r < R; ++r) mu += ph[static_cast<size_t>(r) * PS + M + jj];
    sc_h[slot] = mu;
    pos_h[slot] = T + jj;
    if (slots_out) slots_out[static_cast<size_t>(bh) * S + jj] = slot;
    if (step_mass) step_mass[static_cast<size_t>(bh) * PS + M + jj] = mu;
  }
}

__global__ void reset_kernel(float* scores, int32_t* pos, int64_t n, int32_t* counters, int64_t nc) {
  const int64_t stride = static_cast<int64_t>(gridDim.x) * blockDim.x;
  for (int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; i < n; i += stride) {
    if (scores) scores[i] = 0.f;
    if (pos) pos[i] = -1;
  }
  for (int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; i < nc; i += stride)
    counters[i] = 0;
}

}  // namespace

hipError_t launch_select_scatter(const StepShape& sh, const SelectArgs& a, int dtype, hipStream_t st) {
  const int n_heads = sh.B * sh.Hkv;
  int n_parts = (sh.S + kRowsPerPart - 1) / kRowsPerPart;
  n_parts = n_parts < 1 ? 1 : (n_parts > kMaxParts ? kMaxParts : n_parts);
  const int row_bytes = sh.D * (dtype == kBF16 ? 2 : 4);
  const size_t lds = 4 * static_cast<size_t>(sh.M) + 4 * static_cast<size_t>(sh.S) +
                     static_cast<size_t>(sh.M) + 16;
  if (lds > 64 * 1024) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&select_scatter_kernel),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(lds));
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL(select_scatter_kernel, dim3(n_heads * n_parts), dim3(kThreads), lds, st,
                     static_cast<char*>(a.k_cache), static_cast<char*>(a.v_cache), a.scores, a.pos,
                     static_cast<const char*>(a.k_new), static_cast<const char*>(a.v_new), a.partial,
                     a.R, a.slots_out, a.step_mass, static_cast<char*>(a.k_old),
                     static_cast<char*>(a.v_old), a.counters, a.status, a.T, sh.W, sh.S, sh.M,
                     sh.n_cache, row_bytes, n_heads, n_parts);
  return hipGetLastError();
}

hipError_t launch_reset(float* scores, int32_t* pos, int64_t n_slots, int32_t* counters,
                        int64_t n_counters, hipStream_t st) {
  const int64_t big = n_slots > n_counters ? n_slots : n_counters;
  int64_t blocks = (big + 255) / 256;
  blocks = blocks < 1 ? 1 : (blocks > 4096 ? 4096 : blocks);
  hipLaunchKernelGGL(reset_kernel, dim3(static_cast<unsigned>(blocks)), dim3(256), 0, st, scores, pos,
                     n_slots, counters, n_counters);
  return hipGetLastError();
}

}  // namespace h2o
