// H2O score accumulation (step 2 of h2o_chunk_step): the attention mass
// every key received in this step, summed over the chunk's queries and the
// G query heads of its KV group -- the "summed attention weights" served
// alongside the SDPA kernel ("Learning how to Forget: Fine-tuning for
// Long-Context Sparse Attention", arXiv 2608.19920, §1 ¶4 and the docshare
// FAQ answer on H2O; the score itself is the heavy-hitter oracle of its
// reference [72]).
//
// P = exp(z - lse) is recomputed from Q, K and the forward's lse (the
// forward's online softmax cannot normalise a column before every row is
// done), and reduced over rows without atomics: each workgroup owns a tile
// of 256 key columns and one contiguous range of query rows (a "row split")
// and writes one partial sum per column.  The select kernel adds the R
// partials of a column in split order, so the result is deterministic.
//
// bf16 path: S = Q K^T on v_mfma_f32_32x32x16_bf16 with the wave's 64 keys
// as the B operand held in registers for the whole kernel; 64-row query
// blocks are the A operand, each 16-byte fragment read from LDS feeding two
// MFMAs (the wave's two 32-key halves).  Each accumulator column belongs to
// one key, so the column sum is one fp32 add per element inside the lane
// plus one exchange with lane l^32 at the end.
//   * Rows: a cache-key tile takes every (query head, query) row of the KV
//     group; a chunk-key tile only the rows whose query index reaches its
//     first key, so no staged block is wasted.  Rows are numbered g * L + i
//     over the needed queries and split into contiguous ranges: R for a
//     cache tile, and for a chunk tile the share of R its rows call for
//     (chunk_tile_splits), so that every workgroup holds about the same
//     number of blocks.  The last split of a chunk tile writes zeros into
//     the partial rows it does not use, so the select still adds R partials
//     per column.
//   * Query blocks reach LDS through direct copies (buffer_load ... lds)
//     into a 3-stage ring, the row swizzle applied on the source side; the
//     rows' lse values are staged one block ahead through registers.
//   * Each 64-row block is computed in two 32-row halves, software
//     pipelined: the MFMAs of the next half are issued beside the exp and
//     column adds of the current one, with one barrier per block.
//   * Blocks where some query of the block precedes some key of the wave
//     take a masked variant; all others no per-element test.
#include <cstdint>
#include <type_traits>

#include "h2o_device.h"
#include "h2o_launch.h"

namespace h2o {
namespace {

constexpr int kCT = 256;        // key columns per workgroup (4 waves x 64)
constexpr int kRB = 64;         // query rows per staged block (2 MFMA row blocks)
constexpr int kStages = 3;
constexpr int kRowSplitsMax = 8;     // the select kernel sums up to this many splits

// Row splits of chunk tile tp (keys 256 tp ..) when a cache tile takes R:
// R scaled by the tile's share of the 64-row blocks of a cache tile (whose
// G * S rows are the most any tile has), rounded up, at least 1.
__host__ __device__ inline int chunk_tile_splits(int R, int G, int S, int tp) {
  const int n_c = (G * S + kRB - 1) / kRB;
  const int n_t = (G * (S - kCT * tp) + kRB - 1) / kRB;
  const int r = (R * n_t + n_c - 1) / n_c;
  return r < 1 ? 1 : (r > R ? R : r);
}

template <int CPR>
__device__ __forceinline__ int q_chunk(int row, int c) { return c ^ (row & (CPR - 1)); }

template <int D>
__global__ __launch_bounds__(256, 2) void score_bf16_kernel(
    const bf16_t* __restrict__ Q, const bf16_t* __restrict__ Kc,
    const bf16_t* __restrict__ Kn, const float* __restrict__ lse,
    float* __restrict__ partial, int Hq, int Hkv, int S, int M, int n_cache, float c2,
    int n_heads, int n_ct, int n_jt, int R) {
  constexpr int DS = D / 16;
  constexpr int CPR = D / 8;
  constexpr int RBY = 2 * D;                  // bytes per query row
  constexpr int BLK = kRB * RBY;              // bytes per staged block
  constexpr int NDMA = BLK / 1024 / 4;        // 1 KB copies per wave per block
  // one array per stage: the compiler can then tell that a copy in flight
  // into one stage does not alias the reads of another (and inserts no wait)
  __shared__ __attribute__((aligned(1024))) char qs0[BLK];
  __shared__ __attribute__((aligned(1024))) char qs1[BLK];
  __shared__ __attribute__((aligned(1024))) char qs2[BLK];
  __shared__ __attribute__((aligned(16))) float s_l2[kStages][kRB];
  __shared__ __attribute__((aligned(16))) int s_qi[kStages][kRB];

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63, hf = lane >> 5, col = lane & 31;
  const int bh = blockIdx.x % n_heads;
  const int b = bh / Hkv, kvh = bh - b * Hkv;
  const int G = Hq / Hkv;
  // workgroup -> (tile, split): the n_ct cache tiles' R splits each, then
  // the chunk tiles' chunk_tile_splits each (the host sized the grid so)
  int tile, split, n_split;
  {
    int u = static_cast<int>(blockIdx.x) / n_heads;
    if (u < n_ct * R) {
      tile = u / R;
      split = u - tile * R;
      n_split = R;
    } else {
      u -= n_ct * R;
      int tp = 0;
      n_split = chunk_tile_splits(R, G, S, 0);
      while (u >= n_split && tp + 1 < n_jt) {
        u -= n_split;
        ++tp;
        n_split = chunk_tile_splits(R, G, S, tp);
      }
      tile = n_ct + tp;
      split = u;
    }
  }
  if (split >= n_split) return;
  const bool is_cache = tile < n_ct;
  const int base = (is_cache ? tile : tile - n_ct) * kCT;
  const int lim = is_cache ? n_cache : S;
  const bf16_t* khead = is_cache ? Kc + static_cast<size_t>(bh) * M * D
                                 : Kn + static_cast<size_t>(bh) * S * D;
  const int key0 = base + wave * 64;          // first key of this wave

  // The wave's 64 keys: B operand (lane: key column, d 8hf..+8).
  bf16x8 kf[2][DS];
#pragma unroll
  for (int kb = 0; kb < 2; ++kb) {
    const int key = key0 + kb * 32 + col;
    const bool ok = key < lim;
    const bf16_t* krow = khead + static_cast<size_t>(ok ? key : 0) * D;
#pragma unroll
    for (int st = 0; st < DS; ++st) {
      const bf16x8 v = load_bf16x8(krow + 16 * st + 8 * hf);
      kf[kb][st] = ok ? v : bf16x8{};
    }
  }

  // needed rows: u = g * L + (i - i_off), i_off = 0 (cache tile) or base
  const int i_off = is_cache ? 0 : base;
  const int L = S - i_off;
  const int n_need = G * L;
  const int n_blk = (n_need + kRB - 1) / kRB;
  const int blk_lo = static_cast<int>(static_cast<int64_t>(split) * n_blk / n_split);
  const int blk_hi = static_cast<int>(static_cast<int64_t>(split + 1) * n_blk / n_split);
  const float invL = 1.f / static_cast<float>(L);
  // row u (< n_need) -> row g * S + i of the group's Q / lse
  // (u < G L <= 2^20 and every product stays below 2^24: 24-bit multiplies)
  auto row_of = [&](int u, int& i) __attribute__((always_inline)) {
    int g = static_cast<int>(static_cast<float>(u) * invL);
    int rel = u - __mul24(g, L);
    g = rel < 0 ? g - 1 : g;
    rel = rel < 0 ? rel + L : rel;
    g = rel >= L ? g + 1 : g;
    rel = rel >= L ? rel - L : rel;
    i = i_off + rel;
    return __mul24(g, S) + i;
  };
  const bf16_t* qhead = Q + static_cast<size_t>(b * Hq + kvh * G) * S * D;
  const float* lhead = lse + static_cast<size_t>(b * Hq + kvh * G) * S;
  const __amdgpu_buffer_rsrc_t rq = make_rsrc(qhead, static_cast<uint32_t>(G) * S * RBY);

  // copies of block bk into stage stg: LDS byte 1024 j' + 16 i (j' = wave NDMA
  // + j) is row r, physical chunk c' of the block; the lane fetches that row's
  // logical chunk c' ^ (r mod CPR)
  // Per lane: its rows r0 + RK j, j < NDMA, of every block; the swizzled
  // chunk of row r0 + RK j is c ^ (r mod CPR) = (its value for j = 0) with
  // two bits flipped by j (CPR = 16) or unchanged (CPR = 8).
  constexpr int RK = 1024 / RBY;              // rows per 1 KB copy
  const int r0 = wave * NDMA * RK + lane / CPR;
  const uint32_t chunk0 = 16 * q_chunk<CPR>(r0, lane % CPR);
  const int row_last = (n_need - 1) / L * S + i_off + (n_need - 1) % L;
  auto stage_buf = [&](auto stg) __attribute__((always_inline)) {
    constexpr int SG = decltype(stg)::value;
    return SG == 0 ? qs0 : SG == 1 ? qs1 : qs2;
  };
  auto issue_blk = [&](int bk, auto stg) __attribute__((always_inline)) {
    const char* dst = stage_buf(stg) + wave * NDMA * 1024;
    const int u0 = bk * kRB + r0;
    if (is_cache) {                 // every query row of the group: row u is row u
#pragma unroll
      for (int j = 0; j < NDMA; ++j) {
        const uint32_t chunk = CPR == 16 ? (chunk0 ^ (64u * j)) : chunk0;
        dma16(rq, dst + j * 1024, static_cast<uint32_t>(min(u0 + j * RK, n_need - 1)) * RBY + chunk, 0);
      }
      return;
    }
    int i0;
    const int row0 = row_of(min(u0, n_need - 1), i0);
    int rows[NDMA];
    if (L >= kRB) {                 // a block's rows cross at most one head boundary
#pragma unroll
      for (int j = 0; j < NDMA; ++j) rows[j] = row0 + j * RK + (i0 + j * RK >= S ? S - L : 0);
    } else {
#pragma unroll
      for (int j = 0; j < NDMA; ++j) {
        int i;
        rows[j] = row_of(min(u0 + j * RK, n_need - 1), i);
      }
    }
#pragma unroll
    for (int j = 0; j < NDMA; ++j) {
      const int row = u0 + j * RK < n_need ? rows[j] : row_last;
      const uint32_t chunk = CPR == 16 ? (chunk0 ^ (64u * j)) : chunk0;
      dma16(rq, dst + j * 1024, static_cast<uint32_t>(row) * RBY + chunk, 0);
    }
  };
  // lse (log2 domain) and query index of row tid of block bk; rows past the
  // end get +inf (P = 0)
  // (the loaded lse is first used at the next barrier, so the load does not
  // hold up the copies issued just before it)
  struct RowInfo {
    float lv;
    int qi;     // query index, or 1 << 30 for rows past the end
  };
  auto load_rows = [&](int bk) __attribute__((always_inline)) {
    RowInfo ri{0.f, 1 << 30};
    if (tid < kRB) {
      const int u = bk * kRB + tid;
      if (is_cache) {               // row u is row u; its query index is never tested
        ri.lv = lhead[min(u, n_need - 1)];
        ri.qi = u < n_need ? 0 : (1 << 30);
      } else {
        int i;
        const int row = row_of(min(u, n_need - 1), i);
        ri.lv = lhead[row];
        ri.qi = u < n_need ? i : (1 << 30);
      }
    }
    return ri;
  };
  auto store_rows = [&](const RowInfo& ri, int stg) __attribute__((always_inline)) {
    if (tid < kRB) {
      s_l2[stg][tid] = ri.qi < (1 << 30) ? ri.lv * kLog2e : __builtin_huge_valf();
      s_qi[stg][tid] = ri.qi;
    }
  };

  // per-lane LDS offsets of the A-operand fragments (row 32h + col, logical chunk 2st + hf)
  uint32_t q_rd[DS];
#pragma unroll
  for (int st = 0; st < DS; ++st) q_rd[st] = col * RBY + 16 * q_chunk<CPR>(col, 2 * st + hf);

  auto mfma_half = [&](auto stg, int h, f32x16& a0, f32x16& a1) __attribute__((always_inline)) {
    const char* qb = stage_buf(stg) + h * 32 * RBY;
    a0 = zero16();
    a1 = zero16();
#pragma unroll
    for (int st = 0; st < DS; ++st) {
      const bf16x8 qa = *reinterpret_cast<const bf16x8*>(qb + q_rd[st]);
      a0 = mfma32x32x16(qa, kf[0][st], a0);
      a1 = mfma32x32x16(qa, kf[1][st], a1);
    }
  };
  // column sums of this lane's two key columns, four partial sums each
  // (short dependency chains)
  float cs0[4] = {0.f, 0.f, 0.f, 0.f}, cs1[4] = {0.f, 0.f, 0.f, 0.f};
  // accumulator register r of lane l: row 32h + 8(r/4) + 4hf + r%4 of the
  // block; the 4 rows of each group of 4 registers are consecutive
  auto valu_half = [&](const f32x16& a0, const f32x16& a1, int stg, int h, auto masked) __attribute__((always_inline)) {
    constexpr bool MASKED = decltype(masked)::value;
#pragma unroll
    for (int a4 = 0; a4 < 4; ++a4) {
      const int row0 = h * 32 + 8 * a4 + 4 * hf;
      const f32x4 l2v = *reinterpret_cast<const f32x4*>(&s_l2[stg][row0]);
      int4 qiv = {0, 0, 0, 0};
      if (MASKED) qiv = *reinterpret_cast<const int4*>(&s_qi[stg][row0]);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int r = 4 * a4 + e;
        float p0 = fast_exp2(fmaf(a0[r], c2, -l2v[e]));
        float p1 = fast_exp2(fmaf(a1[r], c2, -l2v[e]));
        if (MASKED) {
          const int qi = e == 0 ? qiv.x : e == 1 ? qiv.y : e == 2 ? qiv.z : qiv.w;
          p0 = (key0 + col <= qi) ? p0 : 0.f;
          p1 = (key0 + 32 + col <= qi) ? p1 : 0.f;
        }
        cs0[e] += p0;
        cs1[e] += p1;
      }
    }
  };
  // smallest query index among block bk's rows (scalar): the first row's
  // index, or i_off when the block reaches the start of another head
  auto block_masked = [&](int bk) __attribute__((always_inline)) {
    const int u0 = bk * kRB;
    const int r = u0 % L;
    const int min_qi = (r + kRB - 1 >= L && u0 + L - r < n_need) ? i_off : i_off + r;
    return !is_cache && min_qi < key0 + 63;
  };

  if (blk_lo < blk_hi) {
    using S0 = std::integral_constant<int, 0>;
    using S1 = std::integral_constant<int, 1>;
    using S2 = std::integral_constant<int, 2>;
    // prologue: blocks lo (stage 0) and lo + 1 (stage 1) in flight, rows of
    // lo staged, MFMAs of lo's first half
    issue_blk(blk_lo, S0{});
    if (blk_lo + 1 < blk_hi) issue_blk(blk_lo + 1, S1{});
    const RowInfo r0 = load_rows(blk_lo);
    RowInfo rn = load_rows(blk_lo + 1);
    wait_vmem_all();
    store_rows(r0, 0);
    barrier_lds();
    f32x16 A0, A1, B0, B1;
    mfma_half(S0{}, 0, A0, A1);
    bool masked = block_masked(blk_lo);
    // block bk in stage STG (= (bk - lo) mod 3, compile-time after unrolling)
    auto block = [&](int bk, auto stg) __attribute__((always_inline)) {
      constexpr int STG = decltype(stg)::value;
      using N1 = std::integral_constant<int, (STG + 1) % kStages>;
      using N2 = std::integral_constant<int, (STG + 2) % kStages>;
      // second half's MFMAs beside the first half's exp and column sums
      if (masked) {
        mfma_half(stg, 1, B0, B1);
        valu_half(A0, A1, STG, 0, std::true_type{});
      } else {
        mfma_half(stg, 1, B0, B1);
        valu_half(A0, A1, STG, 0, std::false_type{});
      }
      // block bk+1 landed (copies and rows issued one block ago); then
      // fetch block bk+2 into the stage block bk-1 used
      wait_vmem_all();
      if (bk + 1 < blk_hi) store_rows(rn, N1::value);
      barrier_lds();
      if (bk + 2 < blk_hi) {
        issue_blk(bk + 2, N2{});
        rn = load_rows(bk + 2);
      }
      const bool masked_next = bk + 1 < blk_hi && block_masked(bk + 1);
      // next block's first-half MFMAs beside this block's second half
      if (bk + 1 < blk_hi) {
        if (masked) {
          mfma_half(N1{}, 0, A0, A1);
          valu_half(B0, B1, STG, 1, std::true_type{});
        } else {
          mfma_half(N1{}, 0, A0, A1);
          valu_half(B0, B1, STG, 1, std::false_type{});
        }
      } else {
        if (masked) valu_half(B0, B1, STG, 1, std::true_type{});
        else valu_half(B0, B1, STG, 1, std::false_type{});
      }
      masked = masked_next;
    };
    // whole triples without conditions between the blocks (so the wait
    // analysis sees every copy into a stage waited before that stage is
    // read), then the remaining one or two blocks
    int bk = blk_lo;
    for (; bk + kStages <= blk_hi; bk += kStages) {
      block(bk, S0{});
      block(bk + 1, S1{});
      block(bk + 2, S2{});
    }
    if (bk < blk_hi) block(bk, S0{});
    if (bk + 1 < blk_hi) block(bk + 1, S1{});
  }
  float t0 = (cs0[0] + cs0[1]) + (cs0[2] + cs0[3]);
  float t1 = (cs1[0] + cs1[1]) + (cs1[2] + cs1[3]);
  t0 += xor32(t0);
  t1 += xor32(t1);
  const size_t PS = static_cast<size_t>(M) + S;
  if (hf == 0) {
    float* out = partial + (static_cast<size_t>(bh) * R + split) * PS + (is_cache ? 0 : M);
    const int k0 = key0 + col, k1 = key0 + 32 + col;
    if (k0 < lim) out[k0] = t0;
    if (k1 < lim) out[k1] = t1;
    // a chunk tile with fewer splits than R: its unused partial rows are zero
    if (split == n_split - 1) {
      for (int s2 = n_split; s2 < R; ++s2) {
        float* z = out + static_cast<size_t>(s2 - split) * PS;
        if (k0 < lim) z[k0] = 0.f;
        if (k1 < lim) z[k1] = 0.f;
      }
    }
  }
}

// Short chunks (G*S <= 64 rows per KV group): one 64-row block holds every
// query row, so it is staged once and each wave walks its keys in 64-key
// groups, loading the next group's K fragments while it computes the
// current one.  A workgroup takes kDecKeys consecutive keys of the head's
// key sequence (the n_cache cache slots, then the S chunk keys), so the
// cache streams once per step (one row split).  The groups are walked last
// first: the attention kernel has just read every head's keys in ascending
// order, so the highest keys are the most recently fetched and the likeliest
// to still sit in the memory-side cache (6 % less score time per decode step
// than ascending order).
constexpr int kDecKeys = 2304;        // keys per workgroup: 4 waves x 9 groups x 64

template <int D>
__global__ __launch_bounds__(256, 1) void score_dec_kernel(
    const bf16_t* __restrict__ Q, const bf16_t* __restrict__ Kc, const bf16_t* __restrict__ Kn,
    const float* __restrict__ lse, float* __restrict__ partial, int Hq, int Hkv, int S, int M,
    int n_cache, float c2, int n_heads) {
  constexpr int DS = D / 16, CPR = D / 8, RBY = 2 * D;
  constexpr int NG = kDecKeys / 256;          // key groups per wave
  constexpr int NQ = kRB * CPR / 256;         // 16-byte query chunks per thread
  __shared__ __attribute__((aligned(16))) char qs[kRB * RBY];
  __shared__ __attribute__((aligned(16))) float s_l2[kRB];
  __shared__ __attribute__((aligned(16))) int s_qi[kRB];

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63, hf = lane >> 5, col = lane & 31;
  const int bh = blockIdx.x % n_heads;
  const int wgi = static_cast<int>(blockIdx.x) / n_heads;
  const int b = bh / Hkv, kvh = bh - b * Hkv;
  const int G = Hq / Hkv;
  const int n_rows = G * S;                   // <= kRB; row u is query row u of the group
  const int n_keys = n_cache + S;             // key v: cache slot v, or chunk key v - n_cache
  const int base = wgi * kDecKeys;
  const bf16_t* kc_head = Kc + static_cast<size_t>(bh) * M * D;
  const bf16_t* kn_head = Kn + static_cast<size_t>(bh) * S * D;
  const bf16_t* qhead = Q + static_cast<size_t>(b * Hq + kvh * G) * S * D;
  const float* lhead = lse + static_cast<size_t>(b * Hq + kvh * G) * S;

  // the wave's key groups: keys base + 256 k + 64 wave + (0..63), k < NG;
  // a key past the end reads the head's first chunk row (its column is
  // never stored)
  auto load_keys = [&](int k, bf16x8 (&kf)[2][DS]) __attribute__((always_inline)) {
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      const int v = base + 256 * (NG - 1 - k) + 64 * wave + 32 * kb + col;
      const bf16_t* krow = v < n_cache ? kc_head + static_cast<size_t>(v) * D
                                       : kn_head + static_cast<size_t>(v < n_keys ? v - n_cache : 0) * D;
#pragma unroll
      for (int st = 0; st < DS; ++st) kf[kb][st] = load_bf16x8(krow + 16 * st + 8 * hf);
    }
  };
  // kSets register sets in rotation: kSets - 1 groups are in flight while
  // one is computed (a group's compute is shorter than a load's latency).
  // Every wave walks all NG groups (a key past the end is computed and not
  // stored), so the loads are unconditional and the waits exact.
  constexpr int kSets = 3;
  static_assert(NG % kSets == 0, "whole passes over the register sets");
  bf16x8 kset[kSets][2][DS];

  // the rows (zero past the end, lse +inf so that P = 0 there); loaded
  // before the first key groups so that staging them waits for these only
  u32x4 qx[NQ];
#pragma unroll
  for (int c = 0; c < NQ; ++c) {
    const int idx = c * 256 + tid, row = idx / CPR, ch = idx % CPR;
    qx[c] = load_u32x4(qhead + static_cast<size_t>(min(row, n_rows - 1)) * D + ch * 8);
  }
  const float l_in = tid < kRB ? lhead[min(tid, n_rows - 1)] : 0.f;
#pragma unroll
  for (int p0 = 0; p0 < kSets - 1; ++p0) load_keys(p0, kset[p0]);
#pragma unroll
  for (int c = 0; c < NQ; ++c) {
    const int idx = c * 256 + tid, row = idx / CPR, ch = idx % CPR;
    const u32x4 z = {0, 0, 0, 0};
    store_u32x4(qs + row * RBY + 16 * q_chunk<CPR>(row, ch), row < n_rows ? qx[c] : z);
  }
  if (tid < kRB) {
    const bool ok = tid < n_rows;
    s_l2[tid] = ok ? l_in * kLog2e : __builtin_huge_valf();
    s_qi[tid] = ok ? tid % S : -1;
  }
  barrier_lds();

  uint32_t q_rd[DS];
#pragma unroll
  for (int st = 0; st < DS; ++st) q_rd[st] = col * RBY + 16 * q_chunk<CPR>(col, 2 * st + hf);
  float* out = partial + static_cast<size_t>(bh) * (static_cast<size_t>(M) + S);

  // one 64-key group: S = Q K^T over both 32-row halves, P, column sums
  auto group = [&](int k, const bf16x8 (&kf)[2][DS]) __attribute__((always_inline)) {
    const int v0 = base + 256 * (NG - 1 - k) + 64 * wave + col, v1 = v0 + 32;   // this lane's two keys
    const int j0 = v0 - n_cache, j1 = v1 - n_cache;                   // chunk index (< 0: cache)
    float cs0[4] = {0.f, 0.f, 0.f, 0.f}, cs1[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      f32x16 a0 = zero16(), a1 = zero16();
#pragma unroll
      for (int st = 0; st < DS; ++st) {
        const bf16x8 qa = *reinterpret_cast<const bf16x8*>(qs + h * 32 * RBY + q_rd[st]);
        a0 = mfma32x32x16(qa, kf[0][st], a0);
        a1 = mfma32x32x16(qa, kf[1][st], a1);
      }
      // accumulator register r of lane l: row 32h + 8(r/4) + 4hf + r%4;
      // a chunk key j is seen by rows whose query index reaches j
#pragma unroll
      for (int a4 = 0; a4 < 4; ++a4) {
        const int row0 = h * 32 + 8 * a4 + 4 * hf;
        const f32x4 l2v = *reinterpret_cast<const f32x4*>(&s_l2[row0]);
        const int4 qiv = *reinterpret_cast<const int4*>(&s_qi[row0]);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int r = 4 * a4 + e;
          const int qi = e == 0 ? qiv.x : e == 1 ? qiv.y : e == 2 ? qiv.z : qiv.w;
          const float p0 = fast_exp2(fmaf(a0[r], c2, -l2v[e]));
          const float p1 = fast_exp2(fmaf(a1[r], c2, -l2v[e]));
          cs0[e] += j0 <= qi ? p0 : 0.f;
          cs1[e] += j1 <= qi ? p1 : 0.f;
        }
      }
    }
    float t0 = (cs0[0] + cs0[1]) + (cs0[2] + cs0[3]);
    float t1 = (cs1[0] + cs1[1]) + (cs1[2] + cs1[3]);
    t0 += xor32(t0);
    t1 += xor32(t1);
    if (hf == 0) {
      if (v0 < n_keys) out[v0 < n_cache ? v0 : M + j0] = t0;
      if (v1 < n_keys) out[v1 < n_cache ? v1 : M + j1] = t1;
    }
  };
  // the last pass reloads the last group into the sets it frees (unused)
#pragma unroll 1
  for (int k = 0; k < NG; k += kSets) {
#pragma unroll
    for (int u = 0; u < kSets; ++u) {
      load_keys(min(k + u + kSets - 1, NG - 1), kset[(u + kSets - 1) % kSets]);
      group(k + u, kset[u]);
    }
  }
}

// fp32: one thread per key column, query rows streamed through LDS; one row
// split, so each workgroup finalizes its own columns.
template <int D>
__global__ __launch_bounds__(64) void score_f32_kernel(
    const float* __restrict__ Q, const float* __restrict__ Kc, const float* __restrict__ Kn,
    const float* __restrict__ lse, float* __restrict__ partial, int Hq, int Hkv, int S, int M,
    int n_cache, float c2, int n_heads, int n_ct, int n_tiles) {
  constexpr int RT = 16;
  __shared__ float Qs[RT][D];
  __shared__ float ls[RT];
  __shared__ int is[RT];
  const int lane = threadIdx.x;
  const int bh = blockIdx.x % n_heads;
  const int tile = static_cast<int>(blockIdx.x) / n_heads;
  const int b = bh / Hkv, kvh = bh - b * Hkv;
  const int G = Hq / Hkv;
  const bool is_cache = tile < n_ct;
  const int key = (is_cache ? tile : tile - n_ct) * 64 + lane;
  const int lim = is_cache ? n_cache : S;
  const bool ok = key < lim;
  const float* krow = (is_cache ? Kc + static_cast<size_t>(bh) * M * D : Kn + static_cast<size_t>(bh) * S * D) +
                      static_cast<size_t>(ok ? key : 0) * D;
  float k[D];
#pragma unroll
  for (int e = 0; e < D; ++e) k[e] = krow[e];
  const int n_rows = G * S;
  const float* qhead = Q + static_cast<size_t>(b * Hq + kvh * G) * S * D;
  const float* lhead = lse + static_cast<size_t>(b * Hq + kvh * G) * S;
  float cs = 0.f;
  for (int r0 = 0; r0 < n_rows; r0 += RT) {
    __syncthreads();
    for (int idx = lane; idx < RT * D; idx += 64) {
      const int rr = idx / D, e = idx % D;
      Qs[rr][e] = (r0 + rr < n_rows) ? qhead[static_cast<size_t>(r0 + rr) * D + e] : 0.f;
    }
    if (lane < RT) {
      const int r = r0 + lane;
      ls[lane] = (r < n_rows) ? lhead[r] * kLog2e : __builtin_huge_valf();
      is[lane] = (r < n_rows) ? r % S : -1;
    }
    __syncthreads();
    for (int rr = 0; rr < RT; ++rr) {
      if (!is_cache && key > is[rr]) continue;
      float z = 0.f;
#pragma unroll
      for (int e = 0; e < D; ++e) z = fmaf(Qs[rr][e], k[e], z);
      cs += fast_exp2(fmaf(z, c2, -ls[rr]));
    }
  }
  if (ok) partial[static_cast<size_t>(bh) * (M + S) + (is_cache ? 0 : M) + key] = cs;
}

}  // namespace

int score_row_splits_max() { return kRowSplitsMax; }

// Workgroups of one (b, KV head) of the bf16 score kernel for row splits R:
// R per cache tile, chunk_tile_splits per chunk tile.
static int64_t score_head_workgroups(const StepShape& sh, int R) {
  const int G = sh.Hq / sh.Hkv;
  const int n_ct = (sh.n_cache + kCT - 1) / kCT, n_jt = (sh.S + kCT - 1) / kCT;
  int64_t n = static_cast<int64_t>(n_ct) * R;
  for (int tp = 0; tp < n_jt; ++tp) n += chunk_tile_splits(R, G, sh.S, tp);
  return n;
}

// Row splits R: a workgroup costs a start-up of about kStartBlocks block
// times (K fragments, first copies) plus one block time per 64-row block
// when it has its CU to itself, two per block beside a second resident
// workgroup.  R minimises the start-ups of the rounds of two workgroups per
// CU plus the blocks queued on the busiest CU, the largest workgroup (a cache
// tile's, or a chunk tile's when there is no cache yet) times the
// workgroups per CU.
int score_row_splits(const StepShape& sh, int dtype) {
  if (dtype != kBF16) return 1;
  constexpr int kStartBlocks = 4;
  const int64_t n_cu = sh.n_cu;
  const int64_t heads = static_cast<int64_t>(sh.B) * sh.Hkv;
  const int n_blk = (sh.Hq / sh.Hkv * sh.S + kRB - 1) / kRB;
  int best = 1;
  int64_t best_cost = INT64_MAX;
  for (int R = 1; R <= kRowSplitsMax && R <= n_blk; ++R) {
    const int64_t n_wg = heads * score_head_workgroups(sh, R);
    const int64_t cost = kStartBlocks * ((n_wg + 2 * n_cu - 1) / (2 * n_cu)) +
                         static_cast<int64_t>((n_blk + R - 1) / R) * ((n_wg + n_cu - 1) / n_cu);
    if (cost < best_cost) {
      best_cost = cost;
      best = R;
    }
  }
  return best;
}

hipError_t launch_score(const StepShape& sh, const ScoreArgs& a, int dtype, hipStream_t st) {
  const int n_heads = sh.B * sh.Hkv;
  const float c2 = sh.scale * kLog2e;
  if (dtype == kBF16 && sh.Hq / sh.Hkv * sh.S <= kRB) {
    // short chunks: every query row in one block, keys streamed per wave
    const int n_wg = (sh.n_cache + sh.S + kDecKeys - 1) / kDecKeys;
#define H2O_LAUNCH_SCORE_DEC(DD)                                                                   \
  hipLaunchKernelGGL(score_dec_kernel<DD>, dim3(n_heads * n_wg), dim3(256), 0, st,                 \
                     static_cast<const bf16_t*>(a.q), static_cast<const bf16_t*>(a.k_cache),      \
                     static_cast<const bf16_t*>(a.k_new), a.lse, a.partial, sh.Hq, sh.Hkv, sh.S,   \
                     sh.M, sh.n_cache, c2, n_heads)
    if (sh.D == 128) H2O_LAUNCH_SCORE_DEC(128);
    else H2O_LAUNCH_SCORE_DEC(64);
#undef H2O_LAUNCH_SCORE_DEC
  } else if (dtype == kBF16) {
    const int n_ct = (sh.n_cache + kCT - 1) / kCT;
    const int n_jt = (sh.S + kCT - 1) / kCT;
    const dim3 grid(static_cast<unsigned>(n_heads * score_head_workgroups(sh, a.R))), block(256);
#define H2O_LAUNCH_SCORE(DD)                                                                      \
  hipLaunchKernelGGL(score_bf16_kernel<DD>, grid, block, 0, st, static_cast<const bf16_t*>(a.q), \
                     static_cast<const bf16_t*>(a.k_cache), static_cast<const bf16_t*>(a.k_new), \
                     a.lse, a.partial, sh.Hq, sh.Hkv, sh.S, sh.M, sh.n_cache, c2, n_heads, n_ct, \
                     n_jt, a.R)
    if (sh.D == 128) H2O_LAUNCH_SCORE(128);
    else H2O_LAUNCH_SCORE(64);
#undef H2O_LAUNCH_SCORE
  } else {
    const int n_ct = (sh.n_cache + 63) / 64;
    const int n_tiles = n_ct + (sh.S + 63) / 64;
    const dim3 grid(n_heads * n_tiles), block(64);
#define H2O_LAUNCH_SCORE32(DD)                                                                  \
  hipLaunchKernelGGL(score_f32_kernel<DD>, grid, block, 0, st, static_cast<const float*>(a.q), \
                     static_cast<const float*>(a.k_cache), static_cast<const float*>(a.k_new), \
                     a.lse, a.partial, sh.Hq, sh.Hkv, sh.S, sh.M, sh.n_cache, c2, n_heads, n_ct, \
                     n_tiles)
    if (sh.D == 128) H2O_LAUNCH_SCORE32(128);
    else H2O_LAUNCH_SCORE32(64);
#undef H2O_LAUNCH_SCORE32
  }
  return hipGetLastError();
}

}  // namespace h2o
