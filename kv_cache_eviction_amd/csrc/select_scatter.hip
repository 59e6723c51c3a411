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
// Position policies (recent, sink_recent: the pages' lr and slr rows among
// their five KV cache policies, Tables 1 and 6; sinks after the attention-
// sinks paper in their reference list): the same select with the position as
// the key, so the oldest candidates go; positions below n_sink are never
// candidates; no score is read, and a written slot gets score 0.
//
// Two kernels.  The select kernel runs one 512-thread workgroup per
// (b, KV head): no other workgroup reads or writes that head's scores,
// positions or slots, so it needs no inter-workgroup synchronisation.  It
//   1. adds the score kernel's R per-split masses to the filled slots'
//      scores (fixed split order: deterministic);
//   2. selects the targets: scores map to order-preserving 32-bit keys, the
//      bits every candidate shares are found with an AND/OR reduction and
//      skipped, and 8-bit LDS radix passes over the remaining bits (one
//      barrier each) find the n_e-th smallest key; equal keys resolve to the
//      lowest slot through one exclusive scan in slot order;
//   3. writes scores, positions and the target list R (with a flag for
//      targets that were free).
// The scatter kernel then copies the chunk's K/V rows into their slots with
// many workgroups per head (a pure bandwidth copy, 16-byte accesses); chunks
// of at most kSelectCopyRows tokens are copied by the select kernel itself.
#include <type_traits>

#include "h2o_device.h"
#include "h2o_launch.h"

namespace h2o {
namespace {

constexpr int kThreads = 512;
constexpr int kWavesSel = kThreads / 64;
constexpr int kMaxSplits = 8;  // upper bound of the score kernel's row splits
constexpr int kMuRegs = 2;     // chunk keys per thread whose masses are prefetched
// chunks up to this length copy their K/V rows inside the select kernel (one
// workgroup per head keeps up with that little data, and a launch is saved);
// longer chunks use the many-workgroup scatter kernel
constexpr int kSelectCopyRows = 256;

enum : uint8_t { kFree = 0, kCand = 1, kKeep = 2, kTarget = 4 };
constexpr int32_t kWasFree = 0x40000000;   // flag bit of a target-list entry

// Order-preserving key of a float: unsigned comparison of keys matches the
// numeric order (scores are non-negative by construction; adopted states may
// carry any finite value).
__device__ __forceinline__ uint32_t order_key(float f) {
  const uint32_t u = __float_as_uint(f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ float key_value(uint32_t k) {
  return __uint_as_float((k & 0x80000000u) ? (k & 0x7fffffffu) : ~k);
}

// wave64 inclusive prefix on DPP: shifts within 16-lane rows (lanes without
// a source add the identity), then row broadcasts across rows
__device__ __forceinline__ int wave_incl_scan(int x) {
  x += __builtin_amdgcn_update_dpp(0, x, 0x111, 0xf, 0xf, false);   // row_shr:1
  x += __builtin_amdgcn_update_dpp(0, x, 0x112, 0xf, 0xf, false);   // row_shr:2
  x += __builtin_amdgcn_update_dpp(0, x, 0x114, 0xf, 0xf, false);   // row_shr:4
  x += __builtin_amdgcn_update_dpp(0, x, 0x118, 0xf, 0xf, false);   // row_shr:8
  x += __builtin_amdgcn_update_dpp(0, x, 0x142, 0xa, 0xf, false);   // row_bcast:15 -> rows 1, 3
  x += __builtin_amdgcn_update_dpp(0, x, 0x143, 0xc, 0xf, false);   // row_bcast:31 -> rows 2, 3
  return x;
}
__device__ __forceinline__ uint32_t wave_and(uint32_t v) {
  int x = static_cast<int>(v);
  x &= __builtin_amdgcn_update_dpp(-1, x, 0x111, 0xf, 0xf, false);
  x &= __builtin_amdgcn_update_dpp(-1, x, 0x112, 0xf, 0xf, false);
  x &= __builtin_amdgcn_update_dpp(-1, x, 0x114, 0xf, 0xf, false);
  x &= __builtin_amdgcn_update_dpp(-1, x, 0x118, 0xf, 0xf, false);
  x &= __builtin_amdgcn_update_dpp(-1, x, 0x142, 0xa, 0xf, false);
  x &= __builtin_amdgcn_update_dpp(-1, x, 0x143, 0xc, 0xf, false);
  return static_cast<uint32_t>(__builtin_amdgcn_readlane(x, 63));
}
__device__ __forceinline__ uint32_t wave_or(uint32_t v) {
  int x = static_cast<int>(v);
  x |= __builtin_amdgcn_update_dpp(0, x, 0x111, 0xf, 0xf, false);
  x |= __builtin_amdgcn_update_dpp(0, x, 0x112, 0xf, 0xf, false);
  x |= __builtin_amdgcn_update_dpp(0, x, 0x114, 0xf, 0xf, false);
  x |= __builtin_amdgcn_update_dpp(0, x, 0x118, 0xf, 0xf, false);
  x |= __builtin_amdgcn_update_dpp(0, x, 0x142, 0xa, 0xf, false);
  x |= __builtin_amdgcn_update_dpp(0, x, 0x143, 0xc, 0xf, false);
  return static_cast<uint32_t>(__builtin_amdgcn_readlane(x, 63));
}

// Exclusive prefix over the threads of the block (thread order) of two ints
// at once, one barrier; `tmp` (2 * kWavesSel ints) must not be in use by
// another call until the next barrier.
__device__ void block_excl_scan2(int a, int b, int* tmp, int& pa, int& pb) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int ia = wave_incl_scan(a), ib = wave_incl_scan(b);
  if (lane == 63) {
    tmp[wave] = ia;
    tmp[kWavesSel + wave] = ib;
  }
  __syncthreads();
  int ba = 0, bb = 0;
#pragma unroll
  for (int w = 0; w < kWavesSel; ++w) {
    ba += (w < wave) ? tmp[w] : 0;
    bb += (w < wave) ? tmp[kWavesSel + w] : 0;
  }
  pa = ba + ia - a;
  pb = bb + ib - b;
}

// Thread t owns the SPT consecutive slots t*SPT .. t*SPT+SPT-1 (SPT*512 >= M)
// and keeps their keys and classes in registers through every phase.
template <int SPT, bool POS>
__global__ __launch_bounds__(kThreads) void select_kernel(
    float* __restrict__ scores, int32_t* __restrict__ pos, const float* __restrict__ partial,
    int R, int32_t* __restrict__ targets, int32_t* __restrict__ slots_out,
    int32_t* __restrict__ pos_old, float* __restrict__ step_mass, int32_t* __restrict__ status, int T, int W, int S, int M,
    int n_cache, int vec, int n_floor, char* __restrict__ kc, char* __restrict__ vc,
    const char* __restrict__ kn, const char* __restrict__ vn, char* __restrict__ k_old,
    char* __restrict__ v_old, int row_bytes) {
  extern __shared__ __attribute__((aligned(16))) char smem[];
  int* s_R = reinterpret_cast<int*>(smem);                 // [S]: target of chunk row j (flagged)
  __shared__ __attribute__((aligned(16))) uint32_t hist[3][kWavesSel / 2][256];   // per wave pair, 3 rotating
  __shared__ int s_red[3][kWavesSel];
  __shared__ int s_scan[2 * kWavesSel];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int bh = blockIdx.x;
  const size_t PS = static_cast<size_t>(M) + S;
  const float* ph = partial + static_cast<size_t>(bh) * R * PS;
  float* sc_h = scores + static_cast<size_t>(bh) * M;
  int32_t* pos_h = pos + static_cast<size_t>(bh) * M;
  const int m0 = tid * SPT;

  // 0. every load up front: the chunk keys' masses (first kMuRegs keys per
  // thread, summed at the end), then the thread's slots (position, score
  // and the R per-split masses; splits past R re-read split R-1)
  float mup[kMuRegs][kMaxSplits];
#pragma unroll
  for (int k = 0; k < kMuRegs; ++k) {
    const int jj = min(tid + k * kThreads, S - 1);
#pragma unroll
    for (int r = 0; r < kMaxSplits; ++r)
      mup[k][r] = POS ? 0.f : ph[static_cast<size_t>(min(r, R - 1)) * PS + M + jj];
  }
  int pv[SPT];
  float sv[SPT], dv[SPT];
  if constexpr (POS) {
    // positions only: no score is read or kept
#pragma unroll
    for (int i = 0; i < SPT; ++i) {
      pv[i] = pos_h[min(m0 + i, M - 1)];
      sv[i] = 0.f;
      dv[i] = 0.f;
    }
  } else if (SPT % 4 == 0 && vec && m0 + SPT <= M) {
    // 16-byte loads of the thread's slots (rows aligned: M, S multiples of 4)
#pragma unroll
    for (int i = 0; i < SPT; i += 4) {
      const int4 p4 = *reinterpret_cast<const int4*>(pos_h + m0 + i);
      const float4 s4 = *reinterpret_cast<const float4*>(sc_h + m0 + i);
      pv[i] = p4.x; pv[i + 1] = p4.y; pv[i + 2] = p4.z; pv[i + 3] = p4.w;
      sv[i] = s4.x; sv[i + 1] = s4.y; sv[i + 2] = s4.z; sv[i + 3] = s4.w;
      float4 part[kMaxSplits];
#pragma unroll
      for (int r = 0; r < kMaxSplits; ++r)
        part[r] = *reinterpret_cast<const float4*>(ph + static_cast<size_t>(min(r, R - 1)) * PS + m0 + i);
      float4 ds = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int r = 0; r < kMaxSplits; ++r) {
        if (r < R) {
          ds.x += part[r].x;
          ds.y += part[r].y;
          ds.z += part[r].z;
          ds.w += part[r].w;
        }
      }
      dv[i] = ds.x; dv[i + 1] = ds.y; dv[i + 2] = ds.z; dv[i + 3] = ds.w;
    }
  } else {
#pragma unroll
    for (int i = 0; i < SPT; ++i) {
      const int m = min(m0 + i, M - 1);
      pv[i] = pos_h[m];
      sv[i] = sc_h[m];
      float part[kMaxSplits];
#pragma unroll
      for (int r = 0; r < kMaxSplits; ++r) part[r] = ph[static_cast<size_t>(min(r, R - 1)) * PS + m];
      float ds = 0.f;
#pragma unroll
      for (int r = 0; r < kMaxSplits; ++r) ds += (r < R) ? part[r] : 0.f;
      dv[i] = ds;
    }
  }

  // 1. scores after this step's mass, slot classes (bit masks), candidate
  // AND/OR, counts
  uint32_t key[SPT];
  uint32_t fmask = 0, cmask = 0;
  uint32_t k_and = 0xffffffffu, k_or = 0u;
#pragma unroll
  for (int i = 0; i < SPT; ++i) {
    const int m = m0 + i;
    const bool exists = m < M;
    float ds = m < n_cache ? dv[i] : 0.f;
    float sc = sv[i];
    if (pv[i] >= 0) {
      sc += ds;
      if (pv[i] >= n_floor && pv[i] < T - W) cmask |= 1u << i;
    } else {
      ds = 0.f;
      if (exists) fmask |= 1u << i;
    }
    if (!exists) cmask &= ~(1u << i);
    if (step_mass && exists) step_mass[static_cast<size_t>(bh) * PS + m] = ds;
    key[i] = POS ? static_cast<uint32_t>(pv[i]) : order_key(sc);
    if ((cmask >> i) & 1u) {
      k_and &= key[i];
      k_or |= key[i];
    }
  }
  for (int i = tid; i < 2 * (kWavesSel / 2) * 256; i += kThreads) (&hist[0][0][0])[i] = 0;
  // 2. counts (free | candidates << 16: each at most M <= 16384) and the
  // candidates' common bits, one barrier
  {
    const int cnt = __builtin_popcount(fmask) | (__builtin_popcount(cmask) << 16);
    const int wsum = __builtin_amdgcn_readlane(wave_incl_scan(cnt), 63);
    const uint32_t wa = wave_and(k_and), wo = wave_or(k_or);
    if (lane == 0) {
      s_red[0][wave] = wsum;
      s_red[1][wave] = static_cast<int>(wa);
      s_red[2][wave] = static_cast<int>(wo);
    }
  }
  __syncthreads();
  int tot = 0;
  uint32_t all_and = 0xffffffffu, all_or = 0u;
#pragma unroll
  for (int w = 0; w < kWavesSel; ++w) {
    tot += s_red[0][w];
    all_and &= static_cast<uint32_t>(s_red[1][w]);
    all_or |= static_cast<uint32_t>(s_red[2][w]);
  }
  const int n_free = tot & 0xffff, n_cand = tot >> 16;
  const int n_f = min(S, n_free);
  const int n_e = S - n_f;
  if (n_cand < n_e) {                      // infeasible adopted state: no slot is written
    if constexpr (!POS) {
#pragma unroll
      for (int i = 0; i < SPT; ++i)
        if (m0 + i < M && !((fmask >> i) & 1u)) sc_h[m0 + i] = key_value(key[i]);
    }
    for (int jj = tid; jj < S; jj += kThreads) targets[static_cast<size_t>(bh) * S + jj] = -1;
    if (tid == 0) atomicOr(status, 1);
    return;
  }

  // 3. radix select of the n_e-th smallest candidate key over the bits the
  // candidates do not all share, 8 bits per pass, one barrier per pass:
  // histograms rotate through three buffers (a buffer is cleared two passes
  // before its use, after every wave has read it) and every wave finds the
  // digit itself
  uint32_t thr = 0;
  int k_eq = 0;
  if (n_e > 0) {
    const uint32_t differ = all_and ^ all_or;
    uint32_t prefix = all_and & ~differ, pmask = ~differ;
    int kk = n_e;
    int top = differ ? 31 - __builtin_clz(differ) : -1;  // highest differing bit
    int pass = 0;
    while (top >= 0) {
      const int shift = top >= 7 ? top - 7 : 0;
      const uint32_t dmask = (top >= 7 ? 0xffu : ((1u << (top + 1)) - 1u)) << shift;
      uint32_t (*h)[256] = hist[pass % 3];
      uint32_t* hw = h[wave >> 1];
#pragma unroll
      for (int i = 0; i < SPT; ++i)
        if (((cmask >> i) & 1u) && (key[i] & pmask) == prefix) atomicAdd(&hw[(key[i] & dmask) >> shift], 1u);
      __syncthreads();
#pragma unroll
      for (int i = 0; i < (kWavesSel / 2) * 256 / kThreads; ++i) (&hist[(pass + 2) % 3][0][0])[tid + i * kThreads] = 0;
      int c[4] = {0, 0, 0, 0}, sum = 0;
#pragma unroll
      for (int wp = 0; wp < kWavesSel / 2; ++wp) {
        const uint4 v = *reinterpret_cast<const uint4*>(&h[wp][4 * lane]);
        c[0] += static_cast<int>(v.x);
        c[1] += static_cast<int>(v.y);
        c[2] += static_cast<int>(v.z);
        c[3] += static_cast<int>(v.w);
      }
#pragma unroll
      for (int q = 0; q < 4; ++q) sum += c[q];
      // the cumulative counts are monotone, so exactly one (lane, q) has
      // kk in (cb, cb + c[q]]: no ordering between the q tests is needed
      int cb = wave_incl_scan(sum) - sum;
      int digit = 0, before = 0;
      bool found = false;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const bool hit = cb < kk && kk <= cb + c[q];
        digit = hit ? 4 * lane + q : digit;
        before = hit ? cb : before;
        found = found || hit;
        cb += c[q];
      }
      const uint64_t bal = __ballot(found);
      const int src = bal ? static_cast<int>(__builtin_ctzll(bal)) : 0;   // exactly one lane finds it
      digit = __builtin_amdgcn_readlane(digit, src);
      before = __builtin_amdgcn_readlane(before, src);
      prefix |= static_cast<uint32_t>(digit) << shift;
      pmask |= dmask;
      kk -= before;
      top = shift - 1;
      ++pass;
    }
    thr = prefix;
    k_eq = kk;      // how many candidates with key == thr are taken (lowest slots)
  }

  // 4. targets in ascending slot order.  One scan of (free | equal << 16,
  // below) gives each thread's first target index: the free targets are the
  // first n_f free slots and the equal ones the first k_eq candidates with
  // key == thr.
  int c_eq = 0, c_lt = 0;
  if (n_e > 0) {
#pragma unroll
    for (int i = 0; i < SPT; ++i) {
      const bool cand = (cmask >> i) & 1u;
      c_lt += cand && key[i] < thr;
      c_eq += cand && key[i] == thr;
    }
  }
  int p_fe, p_lt;
  block_excl_scan2(__builtin_popcount(fmask) | (c_eq << 16), c_lt, s_scan, p_fe, p_lt);
  int fr = p_fe & 0xffff, eq = p_fe >> 16;
  int j = min(fr, n_f) + p_lt + min(eq, k_eq);
  float nsc[SPT];                      // new scores of kept slots (targets: rewritten below)
#pragma unroll
  for (int i = 0; i < SPT; ++i) {
    const int m = m0 + i;
    const bool fre = (fmask >> i) & 1u;
    bool t = false;
    if (fre) {
      t = fr < n_f;
      ++fr;
    } else if (((cmask >> i) & 1u) && n_e > 0) {
      t = (key[i] < thr) || (key[i] == thr && eq < k_eq);
      eq += key[i] == thr;
    }
    if (t) s_R[j++] = fre ? (m | kWasFree) : m;
    nsc[i] = fre ? sv[i] : key_value(key[i]);
  }
  if constexpr (POS) {
    // scores are not kept
  } else if (SPT % 4 == 0 && vec && m0 + SPT <= M) {
#pragma unroll
    for (int i = 0; i < SPT; i += 4)
      *reinterpret_cast<float4*>(sc_h + m0 + i) = float4{nsc[i], nsc[i + 1], nsc[i + 2], nsc[i + 3]};
  } else {
#pragma unroll
    for (int i = 0; i < SPT; ++i)
      if (m0 + i < M && !((fmask >> i) & 1u)) sc_h[m0 + i] = nsc[i];
  }
  __syncthreads();                     // orders these stores before the target stores below

  // 5. targets: score = mass from the chunk's own queries, position T + j
  auto write_target = [&](int jj, float mu) __attribute__((always_inline)) {
    const int v = s_R[jj];
    const int slot = v & ~kWasFree;
    sc_h[slot] = mu;
    if (pos_old) pos_old[static_cast<size_t>(bh) * S + jj] = pos_h[slot];
    pos_h[slot] = T + jj;
    targets[static_cast<size_t>(bh) * S + jj] = v;
    if (slots_out) slots_out[static_cast<size_t>(bh) * S + jj] = slot;
    if (step_mass) step_mass[static_cast<size_t>(bh) * PS + M + jj] = mu;
  };
#pragma unroll
  for (int k = 0; k < kMuRegs; ++k) {
    const int jj = tid + k * kThreads;
    float mu = 0.f;
#pragma unroll
    for (int r = 0; r < kMaxSplits; ++r) mu += (r < R) ? mup[k][r] : 0.f;
    if (jj < S) write_target(jj, mu);
  }
  for (int jj = tid + kMuRegs * kThreads; jj < S; jj += kThreads) {
    float part[kMaxSplits];
#pragma unroll
    for (int r = 0; r < kMaxSplits; ++r) part[r] = POS ? 0.f : ph[static_cast<size_t>(min(r, R - 1)) * PS + M + jj];
    float mu = 0.f;
#pragma unroll
    for (int r = 0; r < kMaxSplits; ++r) mu += (r < R) ? part[r] : 0.f;
    write_target(jj, mu);
  }

  // short chunks (row_bytes > 0): the chunk's K/V rows go to their targets
  // here, as scatter_kernel would copy them (the target list is complete in
  // LDS since the barrier after step 4; each slot has one writer)
  if (row_bytes > 0) {
    const int cpr = row_bytes >> 4;
    for (int idx = tid; idx < S * cpr; idx += kThreads) {
      const int jj = idx / cpr, c = idx - jj * cpr;
      const int t = s_R[jj];
      const int slot = t & ~kWasFree;
      const size_t src = (static_cast<size_t>(bh) * S + jj) * row_bytes + 16 * c;
      const size_t dst = (static_cast<size_t>(bh) * M + slot) * row_bytes + 16 * c;
      const u32x4 kv = load_u32x4(kn + src);
      const u32x4 vv = load_u32x4(vn + src);
      if (k_old) {
        const u32x4 z = {0, 0, 0, 0};
        const bool was_free = (t & kWasFree) != 0;
        store_u32x4(k_old + src, was_free ? z : load_u32x4(kc + dst));
        store_u32x4(v_old + src, was_free ? z : load_u32x4(vc + dst));
      }
      store_u32x4(kc + dst, kv);
      store_u32x4(vc + dst, vv);
    }
  }
}

// Copies chunk row j of every (b, KV head) into its target slot; the rows of
// a head are spread over `parts` workgroups.  With k_old/v_old, the row a
// target held before is saved first (zeros for a slot that was free).
__global__ __launch_bounds__(256) void scatter_kernel(
    char* __restrict__ kc, char* __restrict__ vc, const char* __restrict__ kn,
    const char* __restrict__ vn, const int32_t* __restrict__ targets, char* __restrict__ k_old,
    char* __restrict__ v_old, int S, int M, int row_bytes, int n_heads, int rows_per) {
  const int bh = blockIdx.x % n_heads;
  const int part = static_cast<int>(blockIdx.x) / n_heads;
  const int cpr = row_bytes / 16;
  const int j0 = part * rows_per, j1 = min(S, j0 + rows_per);
  const int n = (j1 - j0) * cpr;
  for (int idx = threadIdx.x; idx < n; idx += blockDim.x) {
    const int jj = j0 + idx / cpr, c = idx % cpr;
    const int t = targets[static_cast<size_t>(bh) * S + jj];
    if (t < 0) continue;                          // infeasible head: nothing is written
    const int slot = t & ~kWasFree;
    const size_t src = (static_cast<size_t>(bh) * S + jj) * row_bytes + 16 * c;
    const size_t dst = (static_cast<size_t>(bh) * M + slot) * row_bytes + 16 * c;
    const u32x4 kv = load_u32x4(kn + src);
    const u32x4 vv = load_u32x4(vn + src);
    if (k_old) {
      const u32x4 z = {0, 0, 0, 0};
      const bool was_free = (t & kWasFree) != 0;
      store_u32x4(k_old + src, was_free ? z : load_u32x4(kc + dst));
      store_u32x4(v_old + src, was_free ? z : load_u32x4(vc + dst));
    }
    store_u32x4(kc + dst, kv);
    store_u32x4(vc + dst, vv);
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

size_t select_lds_bytes(int M, int S) {
  (void)M;
  return 4 * static_cast<size_t>(S) + 16;
}

bool select_copies_rows(const StepShape& sh) { return sh.S <= kSelectCopyRows; }

hipError_t launch_select(const StepShape& sh, const SelectArgs& a, int dtype, hipStream_t st) {
  const int row_bytes = select_copies_rows(sh) ? sh.D * (dtype == kBF16 ? 2 : 4) : 0;
  const int n_heads = sh.B * sh.Hkv;
  const size_t lds = select_lds_bytes(sh.M, sh.S);
  auto al16 = [](const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; };
  const bool vec = sh.M % 4 == 0 && sh.S % 4 == 0 && al16(a.scores) && al16(a.pos) && al16(a.partial);
  auto go = [&](auto kern) -> hipError_t {
    if (lds > 48 * 1024) {
      hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                         hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(lds));
      if (e != hipSuccess) return e;
    }
    hipLaunchKernelGGL(kern, dim3(n_heads), dim3(kThreads), lds, st, a.scores, a.pos, a.partial, a.R,
                       a.targets, a.slots_out, a.pos_old, a.step_mass, a.status, a.T, sh.W, sh.S, sh.M, sh.n_cache,
                       vec ? 1 : 0, sh.policy == 2 ? sh.n_sink : 0, static_cast<char*>(a.k_cache),
                       static_cast<char*>(a.v_cache), static_cast<const char*>(a.k_new),
                       static_cast<const char*>(a.v_new), static_cast<char*>(a.k_old),
                       static_cast<char*>(a.v_old), row_bytes);
    return hipGetLastError();
  };
  // slots per thread: the smallest power of two with 512 * SPT >= M (M <= 16384)
  auto pick = [&](auto pos_key) -> hipError_t {
    constexpr bool P = decltype(pos_key)::value;
    if (sh.M <= kThreads) return go(select_kernel<1, P>);
    if (sh.M <= 2 * kThreads) return go(select_kernel<2, P>);
    if (sh.M <= 4 * kThreads) return go(select_kernel<4, P>);
    if (sh.M <= 8 * kThreads) return go(select_kernel<8, P>);
    if (sh.M <= 16 * kThreads) return go(select_kernel<16, P>);
    return go(select_kernel<32, P>);
  };
  return sh.policy == 0 ? pick(std::false_type{}) : pick(std::true_type{});
}

hipError_t launch_scatter(const StepShape& sh, const SelectArgs& a, int dtype, hipStream_t st) {
  const int n_heads = sh.B * sh.Hkv;
  const int row_bytes = sh.D * (dtype == kBF16 ? 2 : 4);
  // about 512 workgroups of 32 rows or more
  int rows_per = (sh.S * n_heads + 511) / 512;
  rows_per = rows_per < 16 ? 16 : rows_per;
  const int parts = (sh.S + rows_per - 1) / rows_per;
  hipLaunchKernelGGL(scatter_kernel, dim3(n_heads * parts), dim3(256), 0, st,
                     static_cast<char*>(a.k_cache), static_cast<char*>(a.v_cache),
                     static_cast<const char*>(a.k_new), static_cast<const char*>(a.v_new), a.targets,
                     static_cast<char*>(a.k_old), static_cast<char*>(a.v_old), sh.S, sh.M, row_bytes,
                     n_heads, rows_per);
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
