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
// Two kernels.  The select kernel runs P 512-thread workgroups ("parts")
// per (b, KV head), each of which
//   1. adds the score kernel's R per-split masses to the filled slots'
//      scores (fixed split order: deterministic);
//   2. selects the targets: scores map to order-preserving 32-bit keys, the
//      bits every candidate shares are found with an AND/OR reduction and
//      skipped, and 11-bit LDS radix passes over the remaining bits (one
//      barrier each, stopping as soon as the bin holding the cut is taken
//      whole) find the n_e-th smallest key; equal keys resolve to the lowest
//      slot through one exclusive scan in slot order;
//   3. writes scores, positions and the target list R (with a flag for
//      targets that were free) -- part 0 only;
//   4. copies its share of the chunk's K/V rows (tokens part * S / P ..)
//      into their target slots.
// Every part computes the whole selection from the same inputs, so they
// agree bit for bit; the only exchange between them is a per-head counter:
// part p > 0 adds one to it once its reads of the old scores and positions
// are done, and part 0 rewrites those arrays only after the counter has
// reached the running total of reads the host expects.  That wait is
// bounded: past kSelectSpin polls part 0 sets bit 1 of the status word and
// writes anyway.  Chunks of at most kSelectCopyRows tokens take one part
// per head.  Chunks longer than kSelectPartRows tokens (whose target lists
// would not fit LDS), or whose slot count or length is not a multiple of 4,
// or whose heads are so many that one part per head already fills half the
// CUs, keep one part that copies no rows, and the scatter kernel copies them
// with many workgroups per head.
#include <algorithm>
#include <type_traits>

#include "h2o_device.h"
#include "h2o_launch.h"

namespace h2o {
namespace {

constexpr int kThreads = 512;
constexpr int kWavesSel = kThreads / 64;
constexpr int kMaxSplits = 16; // upper bound of the row splits of the masses
constexpr int kDigitBits = 11; // radix digit: 2048-bin histograms
constexpr int kBins = 1 << kDigitBits;
// chunks up to this length copy their K/V rows inside the select kernel (one
// workgroup per head keeps up with that little data, and a launch is saved);
// longer chunks take several parts or the many-workgroup scatter kernel
constexpr int kSelectCopyRows = 256;
// longer chunks, up to this length, are selected by several parts per head
// that each copy a share of the rows; beyond it the scatter kernel copies
constexpr int kSelectPartRows = 4096;
// bound of part 0's wait for the other parts' reads: polls of a device-scope
// load and a short sleep, about 1 us each, so about a second in all (in a
// normal step the other parts have read long before part 0 asks; they only
// need a CU slot, and none of them waits on anything)
constexpr uint32_t kSelectSpin = 1u << 20;
// 16-byte pieces of chunk rows per thread loaded at the start of the select
constexpr int kRowPre = 4;

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
  barrier_lds();
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
// RMAX bounds the row splits R of the masses (1, 2, 4, 8 or 16; R <= RMAX, splits
// past R re-read split R-1 and are not added); RMAX = 0 selects a position
// policy (no masses).  VEC: M and S are multiples of 4 and the buffers are
// 16-byte aligned, so slot rows and chunk masses move in 16-byte pieces.
// MP: several parts per head (the template keeps the single-part kernel free
// of the parts' registers and handshake).
template <int SPT, int RMAX, bool VEC, bool MP>
__global__ __launch_bounds__(kThreads) void select_kernel(
    float* __restrict__ scores, int32_t* __restrict__ pos, const float* __restrict__ partial,
    int R, int32_t* __restrict__ targets, int32_t* __restrict__ slots_out,
    int32_t* __restrict__ pos_old, float* __restrict__ step_mass, int32_t* __restrict__ status, int T, int W,
    int S, int M, int n_cache, int n_floor, char* __restrict__ kc, char* __restrict__ vc,
    const char* __restrict__ kn, const char* __restrict__ vn, char* __restrict__ k_old,
    char* __restrict__ v_old, int row_bytes, int parts, uint32_t* __restrict__ sync, uint32_t sync_target,
    uint32_t spin_limit) {
  constexpr bool POS = RMAX == 0;
  constexpr int NR = POS ? 1 : RMAX;
  constexpr bool VSLOT = VEC && SPT % 4 == 0;
  extern __shared__ __attribute__((aligned(16))) char smem[];
  float* s_mu = reinterpret_cast<float*>(smem);                      // [S] chunk keys' masses (H2O)
  int* s_R = reinterpret_cast<int*>(smem + (POS ? 0 : 4 * static_cast<size_t>(S)));   // [S] row copy
  __shared__ __attribute__((aligned(16))) uint32_t hist[3][kBins];   // 3 rotating histograms
  __shared__ int s_red[3][kWavesSel];
  __shared__ int s_scan[2 * kWavesSel];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  // workgroup -> (head, part): the parts of a head share its XCD when the
  // head count is a multiple of 8 (round-robin dispatch), so their reads of
  // the same scores and masses hit one L2
  const int n_parts = MP ? parts : 1;
  const int n_heads = static_cast<int>(gridDim.x) / n_parts;
  const int bh = MP ? static_cast<int>(blockIdx.x) % n_heads : static_cast<int>(blockIdx.x);
  const int pid = MP ? static_cast<int>(blockIdx.x) / n_heads : 0;
  const size_t PS = static_cast<size_t>(M) + S;
  const float* ph = partial + static_cast<size_t>(bh) * R * PS;
  float* sc_h = scores + static_cast<size_t>(bh) * M;
  int32_t* pos_h = pos + static_cast<size_t>(bh) * M;
  const int m0 = tid * SPT;
  auto split_of = [&](int r) __attribute__((always_inline)) { return static_cast<size_t>(min(r, R - 1)) * PS; };

  // this part's tokens and their K/V rows' 16-byte pieces; with several
  // parts the first kRowPre * kThreads pieces are loaded now (the sources do
  // not depend on the selection), so that only their stores are left at the
  // end (a single part per head, i.e. a chunk of at most 256 tokens, loads
  // them at the end)
  const int cpr = row_bytes >> 4;
  const int j_lo = static_cast<int>(static_cast<int64_t>(pid) * S / n_parts);
  const int j_hi = static_cast<int>(static_cast<int64_t>(pid + 1) * S / n_parts);
  const int n_items = row_bytes > 0 ? (j_hi - j_lo) * cpr : 0;
  auto item_src = [&](int idx) __attribute__((always_inline)) {
    const int jj = j_lo + idx / cpr, c = idx - (idx / cpr) * cpr;
    return (static_cast<size_t>(bh) * S + jj) * row_bytes + 16 * c;
  };
  constexpr int NPRE = MP ? kRowPre : 1;
  const int n_pre = MP ? min(n_items, kRowPre * kThreads) : 0;
  u32x4 rk[NPRE], rv[NPRE];
#pragma unroll
  for (int u = 0; u < NPRE; ++u) {
    const int idx = tid + u * kThreads;
    if (idx < n_pre) {
      rk[u] = load_u32x4(kn + item_src(idx));
      rv[u] = load_u32x4(vn + item_src(idx));
    }
  }

  // 0. loads.  The thread's slots first (position, score, the per-split
  // masses), then the chunk keys' masses, summed in split order into s_mu;
  // every load is unconditional (out-of-range threads re-read a valid row
  // that they do not use), so the two sets are in flight together and the
  // wait for the second covers the first.
  int pv[SPT];
  float sv[SPT], dv[SPT];
  if constexpr (VSLOT) {
#pragma unroll
    for (int i = 0; i < SPT; i += 4) {
      const int g = min(m0 + i, M - 4);
      const int4 p4 = *reinterpret_cast<const int4*>(pos_h + g);
      pv[i] = p4.x; pv[i + 1] = p4.y; pv[i + 2] = p4.z; pv[i + 3] = p4.w;
      if constexpr (POS) {
        sv[i] = sv[i + 1] = sv[i + 2] = sv[i + 3] = 0.f;
        dv[i] = dv[i + 1] = dv[i + 2] = dv[i + 3] = 0.f;
      } else {
        const float4 s4 = *reinterpret_cast<const float4*>(sc_h + g);
        sv[i] = s4.x; sv[i + 1] = s4.y; sv[i + 2] = s4.z; sv[i + 3] = s4.w;
        float4 part[NR];
#pragma unroll
        for (int r = 0; r < NR; ++r) part[r] = *reinterpret_cast<const float4*>(ph + split_of(r) + g);
        float4 ds = part[0];
#pragma unroll
        for (int r = 1; r < NR; ++r) {
          if (r < R) {
            ds.x += part[r].x;
            ds.y += part[r].y;
            ds.z += part[r].z;
            ds.w += part[r].w;
          }
        }
        dv[i] = ds.x; dv[i + 1] = ds.y; dv[i + 2] = ds.z; dv[i + 3] = ds.w;
      }
    }
  } else {
#pragma unroll
    for (int i = 0; i < SPT; ++i) {
      const int m = min(m0 + i, M - 1);
      pv[i] = pos_h[m];
      if constexpr (POS) {
        sv[i] = 0.f;
        dv[i] = 0.f;
      } else {
        sv[i] = sc_h[m];
        float part[NR];
#pragma unroll
        for (int r = 0; r < NR; ++r) part[r] = ph[split_of(r) + m];
        float ds = part[0];
#pragma unroll
        for (int r = 1; r < NR; ++r) ds += (r < R) ? part[r] : 0.f;
        dv[i] = ds;
      }
    }
  }
  if constexpr (!POS) {
    if constexpr (VEC) {
      for (int j0 = 4 * tid; j0 < S; j0 += 4 * kThreads) {
        float4 part[NR];
#pragma unroll
        for (int r = 0; r < NR; ++r) part[r] = *reinterpret_cast<const float4*>(ph + split_of(r) + M + j0);
        float4 mu = part[0];
#pragma unroll
        for (int r = 1; r < NR; ++r) {
          if (r < R) {
            mu.x += part[r].x;
            mu.y += part[r].y;
            mu.z += part[r].z;
            mu.w += part[r].w;
          }
        }
        *reinterpret_cast<float4*>(s_mu + j0) = mu;
      }
    } else {
      for (int jj = tid; jj < S; jj += kThreads) {
        float part[NR];
#pragma unroll
        for (int r = 0; r < NR; ++r) part[r] = ph[split_of(r) + M + jj];
        float mu = part[0];
#pragma unroll
        for (int r = 1; r < NR; ++r) mu += (r < R) ? part[r] : 0.f;
        s_mu[jj] = mu;
      }
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
    if (step_mass && exists && pid == 0) step_mass[static_cast<size_t>(bh) * PS + m] = ds;
    key[i] = POS ? static_cast<uint32_t>(pv[i]) : order_key(sc);
    if ((cmask >> i) & 1u) {
      k_and &= key[i];
      k_or |= key[i];
    }
  }
  // the first two passes' histograms start at zero (each pass clears the
  // one two passes ahead)
  for (int i = tid; i < 2 * kBins / 4; i += kThreads) reinterpret_cast<uint4*>(&hist[0][0])[i] = uint4{0, 0, 0, 0};
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
  if constexpr (MP) wait_vmem_all();
  barrier_lds();
  // every thread's reads of the old scores, positions and masses are done:
  // a part other than 0 says so
  if constexpr (MP) {
    if (pid > 0 && tid == 0) __hip_atomic_fetch_add(sync + bh, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  // part 0, before it rewrites scores or positions: wait until every other
  // part has read them (the host's running total of such reads), bounded
  auto wait_readers = [&]() __attribute__((always_inline)) {
    if constexpr (MP) {
      if (tid == 0) {
        uint32_t it = 0;
        while (static_cast<int32_t>(__hip_atomic_load(sync + bh, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) -
                                    sync_target) < 0) {
          if (++it > spin_limit) {
            atomicOr(status, 2);
            break;
          }
          __builtin_amdgcn_s_sleep(2);
        }
      }
      barrier_lds();
    }
  };
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
  if (n_cand < n_e) {
    // infeasible adopted state: no slot is written.  Every optional output
    // is still defined: slot and old position -1 (outside [0, M), so the
    // backward walk skips the token), the chunk keys' masses as computed,
    // zero old rows (the scatter kernel zeroes them for longer chunks).
    // Part 0 writes all of it.
    if (pid != 0) return;
    wait_readers();
    if constexpr (!POS) {
#pragma unroll
      for (int i = 0; i < SPT; ++i)
        if (m0 + i < M && !((fmask >> i) & 1u)) sc_h[m0 + i] = key_value(key[i]);
    }
    for (int jj = tid; jj < S; jj += kThreads) {
      const size_t r = static_cast<size_t>(bh) * S + jj;
      targets[r] = -1;
      if (slots_out) slots_out[r] = -1;
      if (pos_old) pos_old[r] = -1;
      if (step_mass) step_mass[static_cast<size_t>(bh) * PS + M + jj] = POS ? 0.f : s_mu[jj];
    }
    if (row_bytes > 0 && k_old) {
      const int cpr = row_bytes >> 4;
      const u32x4 z = {0, 0, 0, 0};
      for (int idx = tid; idx < S * cpr; idx += kThreads) {
        const size_t off = static_cast<size_t>(bh) * S * row_bytes + static_cast<size_t>(idx) * 16;
        store_u32x4(k_old + off, z);
        store_u32x4(v_old + off, z);
      }
    }
    if (tid == 0) atomicOr(status, 1);
    return;
  }

  // 3. radix select of the n_e-th smallest candidate key over the bits the
  // candidates do not all share, kDigitBits bits per pass, one barrier per
  // pass: histograms rotate through three buffers (a buffer is cleared two
  // passes before its use, after every wave has read it) and every wave
  // finds the digit itself.  The walk stops early once the bin holding the
  // cut is taken whole: the bits seen so far then decide every candidate
  // (cmp_mask below), and the order inside the bin no longer matters.
  uint32_t thr = 0, cmp_mask = 0xffffffffu;
  int k_eq = 0;
  if (n_e > 0) {
    const uint32_t differ = all_and ^ all_or;
    uint32_t prefix = all_and & ~differ, pmask = ~differ;
    int kk = n_e;
    int top = differ ? 31 - __builtin_clz(differ) : -1;  // highest differing bit
    int pass = 0;
    while (top >= 0) {
      const int nb = top + 1 < kDigitBits ? top + 1 : kDigitBits;
      const int shift = top + 1 - nb;
      const uint32_t dmask = ((1u << nb) - 1u) << shift;
      uint32_t* h = hist[pass % 3];
      // histogram: the lanes of a wave whose digit equals the first active
      // lane's add together in one atomic (scores cluster, so many lanes of
      // a wave often share a bin), the others one by one
#pragma unroll
      for (int i = 0; i < SPT; ++i) {
        const bool c = ((cmask >> i) & 1u) && (key[i] & pmask) == prefix;
        const uint32_t d = (key[i] & dmask) >> shift;
        const uint64_t act = __ballot(c);
        if (act) {
          const int lead = static_cast<int>(__builtin_ctzll(act));
          const uint32_t d0 = static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(d), lead));
          const uint64_t same = __ballot(c && d == d0);
          if (lane == lead) atomicAdd(&h[d0], static_cast<uint32_t>(__builtin_popcountll(same)));
          else if (c && d != d0) atomicAdd(&h[d], 1u);
        }
      }
      barrier_lds();
      {
        uint4* hc = reinterpret_cast<uint4*>(hist[(pass + 2) % 3]);
#pragma unroll
        for (int i = 0; i < kBins / 4 / kThreads; ++i) hc[tid + i * kThreads] = uint4{0, 0, 0, 0};
      }
      // two levels: lane l sums bins kPer l .. kPer l + kPer - 1 and the
      // lane holding the cut is found; then its bins, one per lane, give the
      // digit (the cumulative counts are monotone: exactly one bin holds it)
      // (each lane walks its 16-byte pieces starting at piece lane % 8: with
      // the natural order the 64 lanes' reads, 128 bytes apart, fall in two
      // LDS banks and serialise 32-way)
      constexpr int kPer = kBins / 64;
      int sum = 0;
#pragma unroll
      for (int v = 0; v < kPer / 4; ++v) {
        const int pc = (v + lane) & (kPer / 4 - 1);
        const uint4 x = *reinterpret_cast<const uint4*>(&h[kPer * lane + 4 * pc]);
        sum += static_cast<int>(x.x + x.y + x.z + x.w);
      }
      const int run = wave_incl_scan(sum) - sum;
      const uint64_t bal = __ballot(run < kk && kk <= run + sum);
      const int src = bal ? static_cast<int>(__builtin_ctzll(bal)) : 0;   // exactly one lane holds it
      const int base = __builtin_amdgcn_readlane(run, src);
      const int cq = lane < kPer ? static_cast<int>(h[kPer * src + lane]) : 0;
      const int r2 = base + wave_incl_scan(cq) - cq;
      const uint64_t bal2 = __ballot(lane < kPer && r2 < kk && kk <= r2 + cq);
      const int q = bal2 ? static_cast<int>(__builtin_ctzll(bal2)) : 0;
      const int digit = kPer * src + q;
      const int before = __builtin_amdgcn_readlane(r2, q);
      const int cnt = __builtin_amdgcn_readlane(cq, q);
      prefix |= static_cast<uint32_t>(digit) << shift;
      pmask |= dmask;
      kk -= before;
      top = shift - 1;
      ++pass;
      if (kk == cnt) break;   // the whole bin is taken
    }
    thr = prefix;
    cmp_mask = pmask;
    k_eq = kk;      // how many candidates whose masked key equals thr are taken (lowest slots)
  }

  // 4. targets in ascending slot order.  One scan of (free | equal << 16,
  // below) gives each thread its first target index: the free targets are
  // the first n_f free slots and the equal ones the first k_eq candidates
  // whose masked key equals thr.  The owner of a target slot then writes
  // everything about it -- the slot's new score (the chunk key's mass) and
  // position, and the token's slot, old position, mass and list entry -- so
  // every address has one writer and no ordering between threads is needed.
  int c_eq = 0, c_lt = 0;
  if (n_e > 0) {
#pragma unroll
    for (int i = 0; i < SPT; ++i) {
      const bool cand = (cmask >> i) & 1u;
      c_lt += cand && (key[i] & cmp_mask) < thr;
      c_eq += cand && (key[i] & cmp_mask) == thr;
    }
  }
  int p_fe, p_lt;
  block_excl_scan2(__builtin_popcount(fmask) | (c_eq << 16), c_lt, s_scan, p_fe, p_lt);
  int fr = p_fe & 0xffff, eq = p_fe >> 16;
  int j = min(fr, n_f) + p_lt + min(eq, k_eq);
  float nsc[SPT];
  int npos[SPT];
  uint32_t tmask = 0;
#pragma unroll
  for (int i = 0; i < SPT; ++i) {
    const int m = m0 + i;
    const bool fre = (fmask >> i) & 1u;
    bool t = false;
    if (fre) {
      t = fr < n_f;
      ++fr;
    } else if (((cmask >> i) & 1u) && n_e > 0) {
      const uint32_t km = key[i] & cmp_mask;
      t = (km < thr) || (km == thr && eq < k_eq);
      eq += km == thr;
    }
    nsc[i] = fre ? sv[i] : key_value(key[i]);
    npos[i] = pv[i];
    if (t) {
      const int jj = j++;
      const float mu = POS ? 0.f : s_mu[jj];
      const size_t r = static_cast<size_t>(bh) * S + jj;
      const int v = fre ? (m | kWasFree) : m;
      nsc[i] = mu;
      npos[i] = T + jj;
      tmask |= 1u << i;
      if (pid == 0) {
        targets[r] = v;
        if (slots_out) slots_out[r] = m;
        if (pos_old) pos_old[r] = pv[i];
        if (step_mass) step_mass[static_cast<size_t>(bh) * PS + M + jj] = mu;
      }
      if (row_bytes > 0) s_R[jj] = v;
    }
  }
  if (pid == 0) wait_readers();
  if (pid != 0) {
    // only part 0 rewrites the head's scores and positions
  } else if constexpr (POS) {
    // scores are not kept: a written slot's score is 0, the rest untouched
#pragma unroll
    for (int i = 0; i < SPT; ++i)
      if ((tmask >> i) & 1u) {
        sc_h[m0 + i] = 0.f;
        pos_h[m0 + i] = npos[i];
      }
  } else if constexpr (VSLOT) {
#pragma unroll
    for (int i = 0; i < SPT; i += 4) {
      if (m0 + i < M) {
        *reinterpret_cast<float4*>(sc_h + m0 + i) = float4{nsc[i], nsc[i + 1], nsc[i + 2], nsc[i + 3]};
        *reinterpret_cast<int4*>(pos_h + m0 + i) = int4{npos[i], npos[i + 1], npos[i + 2], npos[i + 3]};
      }
    }
  } else {
#pragma unroll
    for (int i = 0; i < SPT; ++i) {
      if (m0 + i < M && !((fmask >> i) & 1u && !((tmask >> i) & 1u))) sc_h[m0 + i] = nsc[i];
      if ((tmask >> i) & 1u) pos_h[m0 + i] = npos[i];
    }
  }

  // chunks up to kSelectPartRows (row_bytes > 0): this part's share of the
  // chunk's K/V rows goes to their targets here, as scatter_kernel would copy
  // them (each slot has one writer; the target list is complete in LDS after
  // the barrier)
  if (row_bytes > 0) {
    barrier_lds();
    auto put = [&](int idx, const u32x4& kv, const u32x4& vv) __attribute__((always_inline)) {
      const int jj = j_lo + idx / cpr, c = idx - (idx / cpr) * cpr;
      const int t = s_R[jj];
      const int slot = t & ~kWasFree;
      const size_t src = item_src(idx);
      const size_t dst = (static_cast<size_t>(bh) * M + slot) * row_bytes + 16 * c;
      if (k_old) {
        const u32x4 z = {0, 0, 0, 0};
        const bool was_free = (t & kWasFree) != 0;
        store_u32x4(k_old + src, was_free ? z : load_u32x4(kc + dst));
        store_u32x4(v_old + src, was_free ? z : load_u32x4(vc + dst));
      }
      store_u32x4(kc + dst, kv);
      store_u32x4(vc + dst, vv);
    };
#pragma unroll
    for (int u = 0; u < NPRE; ++u) {
      const int idx = tid + u * kThreads;
      if (idx < n_pre) put(idx, rk[u], rv[u]);
    }
    for (int idx = n_pre + tid; idx < n_items; idx += kThreads)
      put(idx, load_u32x4(kn + item_src(idx)), load_u32x4(vn + item_src(idx)));
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
    const size_t src = (static_cast<size_t>(bh) * S + jj) * row_bytes + 16 * c;
    // the row's loads go out with the target's (they do not depend on it)
    const u32x4 kv = load_u32x4(kn + src);
    const u32x4 vv = load_u32x4(vn + src);
    const int t = targets[static_cast<size_t>(bh) * S + jj];
    if (t < 0) {                                  // infeasible head: nothing is overwritten
      if (k_old) {
        const u32x4 z = {0, 0, 0, 0};
        store_u32x4(k_old + src, z);
        store_u32x4(v_old + src, z);
      }
      continue;
    }
    const int slot = t & ~kWasFree;
    const size_t dst = (static_cast<size_t>(bh) * M + slot) * row_bytes + 16 * c;
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

// Several parts need the 16-byte slot and mass loads (M and S multiples of
// 4; the buffers are 16-byte aligned by validation); other shapes keep one
// part and the scatter kernel above kSelectCopyRows.
static bool parts_shape(const StepShape& sh) { return sh.M % 4 == 0 && sh.S % 4 == 0 && sh.S <= kSelectPartRows; }

// Parts per head: one up to kSelectCopyRows tokens (one workgroup keeps up
// with that little data); for longer chunks, enough for about half a
// workgroup per CU over all heads, at least 32 rows each.  A long chunk left
// with one part (many heads) is copied by the scatter kernel instead: one
// workgroup per head would be bound by its own copy bandwidth.
int select_parts(const StepShape& sh) {
  if (sh.S <= kSelectCopyRows || !parts_shape(sh)) return 1;
  const int n_heads = sh.B * sh.Hkv;
  int p = (sh.n_cu + 2 * n_heads - 1) / (2 * n_heads);
  p = std::min(p, (sh.S + 31) / 32);
  return std::max(p, 1);
}

bool select_copies_rows(const StepShape& sh) { return sh.S <= kSelectCopyRows || select_parts(sh) > 1; }

// dynamic LDS of the select kernel: the chunk keys' masses (H2O), then the
// target list of a chunk whose rows it copies
size_t select_lds_bytes(const StepShape& sh) {
  const size_t S = static_cast<size_t>(sh.S);
  return (sh.policy == 0 ? 4 * S : 0) + (select_copies_rows(sh) ? 4 * S : 0) + 16;
}

hipError_t launch_select(const StepShape& sh, const SelectArgs& a, int dtype, hipStream_t st) {
  const int row_bytes = select_copies_rows(sh) ? sh.D * (dtype == kBF16 ? 2 : 4) : 0;
  const int n_heads = sh.B * sh.Hkv;
  const int parts = select_parts(sh);
  const size_t lds = select_lds_bytes(sh);
  auto al16 = [](const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; };
  const bool vec = sh.M % 4 == 0 && sh.S % 4 == 0 && al16(a.scores) && al16(a.pos) && al16(a.partial);
  auto go = [&](auto kern) -> hipError_t {
    if (lds > 48 * 1024) {
      hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                         hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(lds));
      if (e != hipSuccess) return e;
    }
    hipLaunchKernelGGL(kern, dim3(n_heads * parts), dim3(kThreads), lds, st, a.scores, a.pos, a.partial, a.R,
                       a.targets, a.slots_out, a.pos_old, a.step_mass, a.status, a.T, sh.W, sh.S, sh.M, sh.n_cache,
                       sh.policy == 2 ? sh.n_sink : 0, static_cast<char*>(a.k_cache),
                       static_cast<char*>(a.v_cache), static_cast<const char*>(a.k_new),
                       static_cast<const char*>(a.v_new), static_cast<char*>(a.k_old),
                       static_cast<char*>(a.v_old), row_bytes, parts, a.sync, a.sync_target,
                       a.spin_limit ? a.spin_limit : kSelectSpin);
    return hipGetLastError();
  };
  // slots per thread: the smallest power of two with 512 * SPT >= M (M <= 16384);
  // split bound: the smallest power of two >= R (0: position policy)
  auto by_spt = [&](auto rmax, auto vv, auto mp) -> hipError_t {
    constexpr int RM = decltype(rmax)::value;
    constexpr bool V = decltype(vv)::value;
    constexpr bool MPv = decltype(mp)::value;
    if (sh.M <= kThreads) return go(select_kernel<1, RM, V, MPv>);
    if (sh.M <= 2 * kThreads) return go(select_kernel<2, RM, V, MPv>);
    if (sh.M <= 4 * kThreads) return go(select_kernel<4, RM, V, MPv>);
    if (sh.M <= 8 * kThreads) return go(select_kernel<8, RM, V, MPv>);
    if (sh.M <= 16 * kThreads) return go(select_kernel<16, RM, V, MPv>);
    return go(select_kernel<32, RM, V, MPv>);
  };
  auto by_r = [&](auto vv, auto mp) -> hipError_t {
    if (sh.policy != 0) return by_spt(std::integral_constant<int, 0>{}, vv, mp);
    if (a.R <= 1) return by_spt(std::integral_constant<int, 1>{}, vv, mp);
    if (a.R <= 2) return by_spt(std::integral_constant<int, 2>{}, vv, mp);
    if (a.R <= 4) return by_spt(std::integral_constant<int, 4>{}, vv, mp);
    if (a.R <= 8) return by_spt(std::integral_constant<int, 8>{}, vv, mp);
    return by_spt(std::integral_constant<int, kMaxSplits>{}, vv, mp);
  };
  // several parts only with the 16-byte loads (parts_shape)
  if (parts > 1) {
    if (!vec) return hipErrorInvalidValue;
    return by_r(std::true_type{}, std::true_type{});
  }
  return vec ? by_r(std::true_type{}, std::false_type{}) : by_r(std::false_type{}, std::false_type{});
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
