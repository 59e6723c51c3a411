// Chunk attention forward of the H2O step (step 1 of h2o_chunk_step):
// every query of the chunk attends to the filled cache slots and to the
// chunk's keys j <= i; writes the output and the natural-log logsumexp that
// the score kernel reuses.
//
// Method: "Learning how to Forget: Fine-tuning for Long-Context Sparse
// Attention" (arXiv 2608.19920) -- §1 Introduction ¶1 (fixed-size KV cache),
// §1 ¶3 (grouped query attention), §1 ¶4 and the docshare FAQ answer on H2O
// (SDPA kernel that also serves the summed attention weights).  The pages
// describe no kernel; the design below is this library's own, for CDNA4.
//
// bf16 path (v_mfma_f32_32x32x16_bf16, fp32 accumulation):
//   * A workgroup is 8 waves in two groups of 4.  Wave w of a group owns one
//     row block = 32 consecutive queries of one query head; row blocks are
//     numbered (query block, head in group), so the 4 row blocks of a
//     workgroup share their query range, causal extent and K/V tiles.  The
//     two groups split the 64-key tiles between them (even / odd tiles) and
//     merge their softmax states through LDS at the end; with two waves per
//     SIMD, one wave's softmax arithmetic overlaps the other's MFMAs.
//   * The kernel computes S^T = K Q^T: K is the A operand read from LDS, the
//     wave's 32 queries are the B operand held in registers for the whole
//     kernel.  Each lane then owns one query column, so the row softmax
//     needs no cross-lane work except one exchange with lane l^32.
//   * K rows are stored in LDS in MFMA-row order, chosen so that accumulator
//     register r of lane l holds key 16(l/32) + r.  The probabilities then
//     feed O^T = V^T P^T as the B operand straight from registers.  V stays
//     row-major in LDS and the A operand V^T is read with the gfx950 LDS
//     transpose load (ds_read_b64_tr_b16): in each 16-lane group, lane i
//     receives element i%4 of the 8-byte pieces addressed by lanes
//     4r + i/4, r = 0..3 -- four consecutive keys of one d column.
//   * 16-byte chunks of every LDS row are XOR-swizzled (per row) so that the
//     K reads (16 rows, one chunk) and the transpose reads (4 rows, 2-4
//     chunks) hit distinct banks.
//   * Online softmax in the log2 domain (exp2 on v_exp_f32); the O rescale
//     is skipped when no lane's running maximum moved.
//   * Tiles pass through registers into a double-buffered LDS ring: the
//     loads of the next pair of tiles are issued before the current pair is
//     computed, and one barrier per pair separates the stages.  Loads are
//     unconditional: rows past the end of a tile read its last row (masked).
//   * blockIdx -> (head, row group) keeps every workgroup of one (b, KV head)
//     on one XCD when B*Hkv is a multiple of 8 (dispatch is round-robin over
//     the 8 XCDs), so that head's K/V stays in that XCD's L2; the row groups
//     with the longest causal extent are dispatched first.
// fp32 path: one thread per query row, scalar online softmax over K/V rows
// broadcast from LDS (used for fp32 workloads, which are tiny).
#include <algorithm>
#include <type_traits>

#include "h2o_device.h"
#include "h2o_launch.h"

namespace h2o {
namespace {

// buffer_load_dword ... lds: lane i copies the 4 bytes at voff + soff of the
// resource to LDS address lds_base + 4 i; untracked by the compiler like
// dma16 (h2o_device.h), so only the kernel's own vmcnt waits order it.
__device__ __forceinline__ void dma4_lds(__amdgpu_buffer_rsrc_t r, const void* lds_base, uint32_t voff,
                                         uint32_t soff) {
  const uint32_t m0 = static_cast<uint32_t>(reinterpret_cast<uintptr_t>(
      (__attribute__((address_space(3))) const void*)(lds_base)));
  asm volatile("buffer_load_dword %0, %1, %2 offen lds" ::"v"(voff), "s"(r), "s"(soff), "{m0}"(m0) : "memory");
}

constexpr int kKT = 64;        // keys per tile
constexpr int kRowBlocks = 4;  // row blocks (32 queries of one head) per workgroup
constexpr int kMaxKeySplits = 4;
constexpr int kFwdThreads = 512;
constexpr float kRescaleSlack = 8.f;   // log2 headroom before the running maximum must move
constexpr float kNoMax = -1e30f;       // running maximum of a query that has seen no key yet

// K rows of a 32-key block sit in LDS in MFMA A-operand row order: row
// 8q + 4h + r holds key 16h + 4q + r, so that accumulator register r' of
// lane l corresponds to key 16(l/32) + r'.  The tile copies below apply this
// permutation on the source side (their per-lane and scalar offsets).

// Swizzled 16-byte chunk of a K row / V row (CPR chunks per row); both maps
// are involutions in the chunk index.
template <int CPR>
__device__ __forceinline__ int k_chunk(int row, int c) { return c ^ (row & (CPR - 1)); }
template <int CPR>
__device__ __forceinline__ int v_chunk(int row, int c) {
  return c ^ ((row & 3) << (CPR == 16 ? 2 : 1));
}

// ALLF: every cache slot holds a token (known on the host once the cache has
// filled), so no tile needs its keys' positions: no position copies, and
// only keys past the last slot are masked.
template <int D, bool DEC, bool SKIP, bool ALLF>
__global__ __launch_bounds__(kFwdThreads, 1) void attn_fwd_bf16_kernel(
    const bf16_t* __restrict__ Q, const bf16_t* __restrict__ Kc,
    const bf16_t* __restrict__ Vc, const int32_t* __restrict__ pos,
    const bf16_t* __restrict__ Kn, const bf16_t* __restrict__ Vn,
    bf16_t* __restrict__ O, float* __restrict__ lse, int Hq, int Hkv, int S,
    int M, int n_cache, float c2, int n_heads, int wg_per_head, int n_split, float* __restrict__ part) {
  constexpr int DS = D / 16;              // MFMA k-steps over d
  constexpr int DB = D / 32;              // 32-row blocks of O^T
  constexpr int CPR = D / 8;              // 16-byte chunks per row
  constexpr int RB = 2 * D;               // bytes per K or V row
  constexpr int TB = kKT * RB;            // bytes per K or V tile
  constexpr int NDMA = TB / 4096;         // 1 KB copies per wave per tile (4 waves per group)
  // K and V slots, one array per (group, slot): the compiler can then tell
  // that a copy in flight into one slot does not alias reads of another, and
  // inserts no wait for it
  __shared__ __attribute__((aligned(1024))) char k00[TB];
  __shared__ __attribute__((aligned(1024))) char k01[TB];
  __shared__ __attribute__((aligned(1024))) char k10[TB];
  __shared__ __attribute__((aligned(1024))) char k11[TB];
  __shared__ __attribute__((aligned(1024))) char v00[TB];
  __shared__ __attribute__((aligned(1024))) char v01[TB];
  __shared__ __attribute__((aligned(1024))) char v10[TB];
  __shared__ __attribute__((aligned(1024))) char v11[TB];
  // compile-time (group, slot) -> buffer
  auto kbuf = [&](auto g, auto sl) __attribute__((always_inline)) {
    constexpr int GG = decltype(g)::value, SL = decltype(sl)::value;
    return GG == 0 ? (SL == 0 ? k00 : k01) : (SL == 0 ? k10 : k11);
  };
  auto vbuf = [&](auto g, auto sl) __attribute__((always_inline)) {
    constexpr int GG = decltype(g)::value, SL = decltype(sl)::value;
    return GG == 0 ? (SL == 0 ? v00 : v01) : (SL == 0 ? v10 : v11);
  };
  // positions of the cache tiles, per wave: a ring of 4 tiles of its group
  // (slot (local tile / 2) & 3), copied with the tile's K
  __shared__ int s_pos[2][kRowBlocks][4][kKT];
  using I0 = std::integral_constant<int, 0>;
  using I1 = std::integral_constant<int, 1>;

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63, hf = lane >> 5, col = lane & 31;
  const int grp = wave >> 2, rbw = wave & 3;
  const int bh = blockIdx.x % n_heads;
  const int wsp = static_cast<int>(blockIdx.x) / n_heads;     // (row group, key split)
  const int wgi = wg_per_head - 1 - wsp / n_split;
  const int split = wsp - (wsp / n_split) * n_split;
  const int b = bh / Hkv, kvh = bh - b * Hkv;
  const int G = Hq / Hkv;
  const int n_rb = DEC ? (G * S + 31) >> 5 : G * ((S + 31) >> 5);
  // Row blocks.  Chunk layout: row block = 32 consecutive queries of one
  // head, numbered (query block, head); the workgroup's 4 waves of a group
  // own 4 row blocks.  Short-chunk layout (DEC, S < 32): the G*S rows
  // (head, query) of the KV group are packed 32 to a row block, and the
  // group's waves are 2 row blocks x 2 key halves: wave kh takes keys
  // 32 kh..32 kh+31 of every tile, so no MFMA works on padding rows.
  constexpr int RBW = DEC ? 2 : kRowBlocks;     // row blocks per workgroup
  const int rbp = DEC ? (rbw >> 1) : rbw;
  const int kh = DEC ? (rbw & 1) : 0;
  const int rb = wgi * RBW + rbp;
  const bool active = rb < n_rb;
  int g, qb, qi;
  bool row_ok;                                  // this lane's row exists
  if constexpr (DEC) {
    const int R = rb * 32 + col;
    row_ok = active && R < G * S;
    g = row_ok ? R / S : 0;
    qi = row_ok ? R - g * S : 0;
    qb = 0;
  } else {
    g = active ? rb % G : 0;
    qb = active ? rb / G : 0;
    qi = qb * 32 + col;
    row_ok = active && qi < S;
  }
  const int hq = kvh * G + g;
  const int rb_last = min(wgi * RBW + RBW - 1, n_rb - 1);
  const int n_chunk_keys = DEC ? S : min(S, (rb_last / G + 1) * 32);
  const int n_ct = (n_cache + kKT - 1) / kKT;
  const int n_tiles_all = n_ct + (n_chunk_keys + kKT - 1) / kKT;
  // Key split (small grids): this workgroup takes global tiles
  // [T0, T0 + n_tiles) of the row group's cache-then-chunk tile list and
  // leaves its partial softmax state for the merge kernel.  Below, tile
  // indices are local to that range.
  const int T0 = split * n_tiles_all / n_split;
  const int n_tiles = (split + 1) * n_tiles_all / n_split - T0;
  // group g takes tiles 2t + g, t < n_iter (even: the loop body is unrolled
  // by two so that LDS slot parities are compile-time); tiles past the end
  // are fully masked
  const int n_iter = ((n_tiles + 3) >> 2) << 1;
  // SKIP (key-split launches, whose workgroups walk only a few tiles): local
  // tile Tl needs no work from this wave when it is past the range (fully
  // masked) or a chunk tile after the wave's last query (wave-uniform).
  // The long-walk variant does not test: the branches cost its main loop more
  // than the padding tiles they would save.
  auto skip_tile = [&](int Tl) __attribute__((always_inline)) {
    if constexpr (!SKIP) return false;
    if (Tl >= n_tiles) return true;
    if constexpr (DEC) {
      return false;
    } else {
      const int Tg = T0 + Tl;
      return Tg >= n_ct && (Tg - n_ct) * kKT > qb * 32 + 31;
    }
  };

  const bf16_t* kc_head = Kc + static_cast<size_t>(bh) * M * D;
  const bf16_t* vc_head = Vc + static_cast<size_t>(bh) * M * D;
  const bf16_t* kn_head = Kn + static_cast<size_t>(bh) * S * D;
  const bf16_t* vn_head = Vn + static_cast<size_t>(bh) * S * D;
  const __amdgpu_buffer_rsrc_t r_pos = make_rsrc(pos + static_cast<size_t>(bh) * M, static_cast<uint32_t>(M) * 4);
  const __amdgpu_buffer_rsrc_t rk_c = make_rsrc(kc_head, static_cast<uint32_t>(M) * RB);
  const __amdgpu_buffer_rsrc_t rv_c = make_rsrc(vc_head, static_cast<uint32_t>(M) * RB);
  const __amdgpu_buffer_rsrc_t rk_n = make_rsrc(kn_head, static_cast<uint32_t>(S) * RB);
  const __amdgpu_buffer_rsrc_t rv_n = make_rsrc(vn_head, static_cast<uint32_t>(S) * RB);

  // The wave's queries: B operand of S^T = K Q^T (lane: query col, d 8hf..+8).
  bf16x8 qf[DS];
  {
    const bool qok = row_ok;
    const bf16_t* qrow = Q + (static_cast<size_t>(b * Hq + hq) * S + (qok ? qi : 0)) * D;
#pragma unroll
    for (int st = 0; st < DS; ++st) {
      bf16x8 v = load_bf16x8(qrow + 16 * st + 8 * hf);
      qf[st] = qok ? v : bf16x8{};
    }
  }
  f32x16 o[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) o[db] = zero16();
  float m_run = kNoMax, l_run = 0.f;

  // ---- tile copies (global -> LDS, no registers).  LDS byte 1024 j' + 16 i
  // of a tile (j' = rbw NDMA + j, lane i) is row r, physical chunk c'; the
  // lane fetches the source row and logical chunk that belong there.  Worked
  // out for the two row sizes, the source offset splits into a per-lane part
  // (one register; for K rows of 256 bytes the copy index flips two bits of
  // it) and a wave-uniform part passed as the scalar offset.
  // lane_src(l, &k, &v): per-lane parts for lane l
  auto lane_src = [](int l, uint32_t& k, uint32_t& v) __attribute__((always_inline)) {
    if constexpr (D == 128) {
      const int q = l >> 4;
      k = 256 * q + 16 * ((l & 15) ^ q);
      v = 256 * q + 16 * ((l & 15) ^ (4 * q));
    } else {
      const int q8 = l >> 3, c = l & 7;
      k = 128 * (16 * ((q8 >> 2) & 1) + (q8 & 3)) + 16 * (c ^ q8);
      v = 128 * q8 + 16 * (c ^ ((q8 & 3) << 1));
    }
  };
  uint32_t dk_lane, dv_lane;
  lane_src(lane, dk_lane, dv_lane);
  auto dk_voff = [&](int j) __attribute__((always_inline)) {
    return D == 128 ? (dk_lane ^ (64u * j)) : dk_lane;
  };
  auto dk_soff = [&](int j) __attribute__((always_inline)) {
    return static_cast<uint32_t>(D == 128 ? 256 * (32 * (rbw >> 1) + 8 * (rbw & 1) + 16 * (j & 1) + 4 * (j >> 1))
                                          : 128 * (32 * (rbw >> 1) + 4 * (2 * (rbw & 1) + j)));
  };
  auto dv_soff = [&](int j) __attribute__((always_inline)) {
    return static_cast<uint32_t>(D == 128 ? 256 * (16 * rbw + 4 * j) : 128 * 8 * (2 * rbw + j));
  };
  // rows past the end of a partial tile re-read its last row (masked later)
  auto clamp_row = [](uint32_t off, int n) __attribute__((always_inline)) {
    const int key = static_cast<int>(off / RB);
    return key < n ? off : off - static_cast<uint32_t>(key - n + 1) * RB;
  };
  auto issue_k = [&](int T, auto g, auto slot) __attribute__((always_inline)) {
    T = T0 + min(T, n_tiles - 1);     // past the end: reload the last tile (masked)
    const bool is_cache = T < n_ct;
    const int base = is_cache ? T * kKT : (T - n_ct) * kKT;
    const int n = (is_cache ? n_cache : S) - base;
    const __amdgpu_buffer_rsrc_t r = is_cache ? rk_c : rk_n;
    const char* dst = kbuf(g, slot) + rbw * NDMA * 1024;
    const uint32_t soff = static_cast<uint32_t>(base) * RB;
    if (n >= kKT) {
#pragma unroll
      for (int j = 0; j < NDMA; ++j) dma16(r, dst + j * 1024, dk_voff(j), soff + dk_soff(j));
    } else {      // rare: recomputed here so that the clamped offsets hold no registers
      int l = lane;
      asm volatile("" : "+v"(l));
      uint32_t kl, vl;
      lane_src(l, kl, vl);
#pragma unroll
      for (int j = 0; j < NDMA; ++j) {
        const uint32_t ko = D == 128 ? (kl ^ (64u * j)) : kl;
        dma16(r, dst + j * 1024, clamp_row(ko + dk_soff(j), n), soff);
      }
    }
  };
  auto issue_v = [&](int T, auto g, auto slot) __attribute__((always_inline)) {
    T = T0 + min(T, n_tiles - 1);     // past the end: reload the last tile (masked)
    const bool is_cache = T < n_ct;
    const int base = is_cache ? T * kKT : (T - n_ct) * kKT;
    const int n = (is_cache ? n_cache : S) - base;
    const __amdgpu_buffer_rsrc_t r = is_cache ? rv_c : rv_n;
    const char* dst = vbuf(g, slot) + rbw * NDMA * 1024;
    const uint32_t soff = static_cast<uint32_t>(base) * RB;
    if (n >= kKT) {
#pragma unroll
      for (int j = 0; j < NDMA; ++j) dma16(r, dst + j * 1024, dv_lane, soff + dv_soff(j));
    } else {      // rare: as for K
      int l = lane;
      asm volatile("" : "+v"(l));
      uint32_t kl, vl;
      lane_src(l, kl, vl);
#pragma unroll
      for (int j = 0; j < NDMA; ++j) dma16(r, dst + j * 1024, clamp_row(vl + dv_soff(j), n), soff);
    }
  };
  // Positions of local tile T's keys into this wave's ring slot, issued just
  // before the tile's K copies (so they complete no later than K, which the
  // tile's QK^T already waits for; the mask reads them after that).  A
  // position read through an ordinary load would be tracked by the
  // compiler, whose wait for it would also wait for the untracked tile
  // copies issued after it (vmcnt retires in order).
  auto issue_pos = [&](int T) __attribute__((always_inline)) {
    if constexpr (!ALLF) {
      const int Tc = T0 + min(T, n_tiles - 1);
      dma4_lds(r_pos, s_pos[grp][rbw][(T >> 1) & 3], 4u * static_cast<uint32_t>(min(Tc * kKT + lane, M - 1)), 0u);
    }
  };
  // position of this lane's key in local tile T (cache tiles; -1 = free or past the end)
  auto pos_of = [&](int T) __attribute__((always_inline)) {
    const int key = (T0 + T) * kKT + lane;
    if constexpr (ALLF) return key < n_cache ? 0 : -1;
    const int p = s_pos[grp][rbw][(T >> 1) & 3][lane];
    return key < n_cache ? p : -1;
  };

  // ---- LDS fragment addresses (bytes from the group's slot 0)
  uint32_t k_rd[DS], v_rd[DB];
  {
#pragma unroll
    for (int st = 0; st < DS; ++st) k_rd[st] = (32 * kh + col) * RB + 16 * k_chunk<CPR>(col, 2 * st + hf);
    const int tr_j = lane & 15, tr_r = tr_j >> 2, tr_q = tr_j & 3, tr_dg = (lane >> 4) & 1;
#pragma unroll
    for (int db = 0; db < DB; ++db) {
      const int d = db * 32 + tr_dg * 16 + 4 * tr_q;
      v_rd[db] = (32 * kh + 16 * hf + tr_r) * RB + 16 * v_chunk<CPR>(tr_r, d >> 3) + 2 * (d & 7);
    }
  }

  // S^T of one tile: register r of a0 (a1) <-> key 16(l/32) + r (+32); in
  // the short-chunk layout only a0, for the wave's key half
  auto qk = [&](auto g, auto slot, f32x16& a0, f32x16& a1) __attribute__((always_inline)) {
    const char* kt = kbuf(g, slot);
    a0 = zero16();
    if constexpr (!DEC) a1 = zero16();
#pragma unroll
    for (int st = 0; st < DS; ++st) {
      const bf16x8 ka = *reinterpret_cast<const bf16x8*>(kt + k_rd[st]);
      a0 = mfma32x32x16(ka, qf[st], a0);
      if constexpr (!DEC) {
        const bf16x8 kb = *reinterpret_cast<const bf16x8*>(kt + 32 * RB + k_rd[st]);
        a1 = mfma32x32x16(kb, qf[st], a1);
      }
    }
  };
  // O^T += V^T P^T; MFMA (kb,u) covers keys 32kb + 16(l/32) + 8u + e.  The A
  // operand V^T comes from two transpose reads: lane j = 4r + q of a 16-lane
  // group addresses V[key0 + r][d0 + 4q .. +4).
  auto pv = [&](auto g, auto slot, const bf16x8 (&pb)[4]) __attribute__((always_inline)) {
    // one base address per 32-row block of O^T; the key offsets of the
    // reads go in their offset fields (the V slots lie above 64 KB of LDS)
    const uint32_t vt = lds_addr(vbuf(g, slot));
    uint32_t vb[DB];
#pragma unroll
    for (int db = 0; db < DB; ++db) vb[db] = vt + v_rd[db];
#pragma unroll
    for (int kb = 0; kb < (DEC ? 1 : 2); ++kb)
#pragma unroll
      for (int u = 0; u < 2; ++u)
#pragma unroll
        for (int db = 0; db < DB; ++db) {
          const uint32_t p = vb[db] + (32 * kb + 8 * u) * RB;
          const bf16x4 h0 = lds_read_tr16_at(p);
          const bf16x4 h1 = lds_read_tr16_at(p + 4 * RB);
          const bf16x8 a = __builtin_shufflevector(h0, h1, 0, 1, 2, 3, 4, 5, 6, 7);
          o[db] = mfma32x32x16(a, pb[2 * kb + u], o[db]);
        }
  };
  // probabilities of the current tile against the running maximum
  auto softmax = [&](const f32x16& a0, const f32x16& a1, bf16x8 (&pb)[4]) __attribute__((always_inline)) {
    f32x8 t[4];
    float rs0 = 0.f, rs1 = 0.f;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const float p0 = fast_exp2(fmaf(a0[r], c2, -m_run));
      t[r >> 3][r & 7] = p0;
      rs0 += p0;
      if constexpr (!DEC) {
        const float p1 = fast_exp2(fmaf(a1[r], c2, -m_run));
        t[2 + (r >> 3)][r & 7] = p1;
        rs1 += p1;
      }
    }
    l_run += rs0 + rs1;
#pragma unroll
    for (int i = 0; i < (DEC ? 2 : 4); ++i) pb[i] = to_bf16x8(t[i]);
  };
  // largest raw score of the lane's 32 entries (v_maximum3_f32; NaN-propagating)
  auto tile_max = [&](const f32x16& a0, const f32x16& a1) __attribute__((always_inline)) {
    if constexpr (DEC) {
      float mx = __builtin_elementwise_maximum(a0[0], a0[1]);
#pragma unroll
      for (int r = 2; r < 16; r += 2) mx = __builtin_elementwise_maximum(mx, __builtin_elementwise_maximum(a0[r], a0[r + 1]));
      return mx;
    } else {
      float mx = __builtin_elementwise_maximum(a0[0], a1[0]);
#pragma unroll
      for (int r = 1; r < 16; ++r) mx = __builtin_elementwise_maximum(mx, __builtin_elementwise_maximum(a0[r], a1[r]));
      return mx;
    }
  };
  // masks global tile T's scores (then the maximum mx of the raw scores is
  // recomputed over the visible ones), and moves the running maximum (with
  // O and l rescaled) only if some score exceeds it by the slack
  auto mask_and_check = [&](f32x16& a0, f32x16& a1, float mx, int Tl, int posv) __attribute__((always_inline)) {
    const bool exists = Tl < n_tiles;
    const int T = T0 + Tl;
    const bool is_cache = T < n_ct;
    const int base = is_cache ? T * kKT : (T - n_ct) * kKT;
    uint64_t vm;
    if (!exists) {
      vm = 0;
    } else if (is_cache) {
      vm = __ballot(posv >= 0);
    } else {
      const int n = S - base;
      vm = n >= 64 ? ~0ull : ((1ull << n) - 1);
    }
    const bool causal = exists && !is_cache && (DEC || base + kKT - 1 > qb * 32);
    if constexpr (DEC) vm = (vm >> (32 * kh)) & 0xffffffffull;   // the wave's key half
    if (vm != (DEC ? 0xffffffffull : ~0ull) || causal) {
      const uint32_t bits0 = static_cast<uint32_t>(vm >> (16 * hf)) & 0xffffu;
      const uint32_t bits1 = static_cast<uint32_t>(vm >> (32 + 16 * hf)) & 0xffffu;
      const int lim_i = causal ? qi - base - 16 * hf - 32 * kh : (1 << 30);   // key offset bound
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const bool ok0 = ((bits0 >> r) & 1u) && (r <= lim_i);
        a0[r] = ok0 ? a0[r] : kNegInf;
        if constexpr (!DEC) {
          const bool ok1 = ((bits1 >> r) & 1u) && (32 + r <= lim_i);
          a1[r] = ok1 ? a1[r] : kNegInf;
        }
      }
      mx = tile_max(a0, a1);
    }
    if (__ballot(mx * c2 > m_run + kRescaleSlack)) {
      const float m_new = fmaxf(m_run, fmaxf(mx, xor32(mx)) * c2);
      const float alpha = fast_exp2(m_run - m_new);
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) o[db][r] *= alpha;
      l_run *= alpha;
      m_run = m_new;
    }
  };

  // ---- prologue: K and V of the group's tiles 0 and 1, scores of tile 0.
  // Every slot receives a real tile before its first use (tile indices past
  // the end reload the last tile, masked), so masked P = 0 always meets
  // finite V.
  f32x16 sc0, sc1;
  bf16x8 pb[4];

  // Ping-pong: iteration t has an MFMA phase M(t) = {S^T of tile t+1 from K
  // slot (t+1)&1, O += PV of tile t from V slot t&1} and a VALU phase
  // V(t') = {mask, check and softmax of tile t'} producing P(t').  Group 0
  // runs M(t) then V(t+1); group 1 runs V(t) then M(t), one phase behind, so
  // that of the two waves sharing a SIMD one issues MFMAs while the other
  // does the softmax.  A barrier separates the phases.  Each wave issues the
  // same number of loads per iteration (position + K and V tile copies), so
  // a fixed vmcnt waits for exactly the previous iteration's copies: after
  // its MFMA phase a group fetches K of tile t+3 and V of tile t+2 into the
  // slots it just read, three phases before their use.  Each group runs its
  // own loop (same barrier count), so that each carries only its own state
  // across iterations (group 0 P, group 1 S) and its buffers are fixed.
  constexpr int kLoadsPerIter = (ALLF ? 0 : 1) + 2 * NDMA;
  constexpr int kWaitPrev = 0x0f70 | (kLoadsPerIter & 15) | ((kLoadsPerIter >> 4) << 14);
  auto run_group = [&](auto g) __attribute__((always_inline)) {
    constexpr int GG = decltype(g)::value;
    issue_pos(GG);
    issue_k(GG, g, I0{});
    issue_pos(2 + GG);
    issue_k(2 + GG, g, I1{});
    issue_v(GG, g, I0{});
    issue_v(2 + GG, g, I1{});
    wait_vmem_all();
    barrier_lds();
    if (!skip_tile(GG)) qk(g, I0{}, sc0, sc1);
    barrier_lds();
    issue_pos(4 + GG);
    issue_k(4 + GG, g, I0{});
    // S^T of tile tq (K slot PN) and O += P V of tile tp (V slot par)
    auto m_phase = [&](auto par, int tq, int tp) __attribute__((always_inline)) {
      using PN = std::integral_constant<int, decltype(par)::value ^ 1>;
      if (!skip_tile(tq)) {
        f32x16 sn0, sn1;
        qk(g, PN{}, sn0, sn1);
        if (!skip_tile(tp)) pv(g, par, pb);
        sc0 = sn0;
        sc1 = sn1;
        if constexpr (D == 128 && !DEC && !SKIP) {
          // Issue order of the phase's 32 MFMAs and 48 LDS reads: 4 reads
          // first, then 3 reads behind every MFMA pair, so that each K
          // fragment and V^T half is requested about two MFMA pairs before
          // its use (left to itself the compiler reads one fragment ahead
          // and every MFMA waits for LDS).  Measured at 64k context (G = 4,
          // 1024-token chunks, 2048 slots): 60.7 -> 58.1 us per launch.
          __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);     // LDS reads
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);   // MFMAs
            __builtin_amdgcn_sched_group_barrier(0x100, 3, 0);
          }
        }
      } else if (!skip_tile(tp)) {
        pv(g, par, pb);
      }
    };
    auto v_phase = [&](int T) __attribute__((always_inline)) {
      if (skip_tile(T)) return;
      mask_and_check(sc0, sc1, tile_max(sc0, sc1), T, pos_of(T));
      softmax(sc0, sc1, pb);
    };
    if constexpr (GG == 0) {
      v_phase(0);                       // P(0)
      auto iteration = [&](int t, auto par) __attribute__((always_inline)) {
        using PN = std::integral_constant<int, decltype(par)::value ^ 1>;
        m_phase(par, 2 * (t + 1), 2 * t);
        barrier_lds();
        issue_pos(2 * (t + 3));
        issue_k(2 * (t + 3), g, PN{});
        issue_v(2 * (t + 2), g, par);
        v_phase(2 * (t + 1));
        __builtin_amdgcn_s_waitcnt(kWaitPrev);
        barrier_lds();
      };
      for (int t = 0; t < n_iter; t += 2) {
        iteration(t, I0{});
        iteration(t + 1, I1{});
      }
    } else {
      auto iteration = [&](int t, auto par) __attribute__((always_inline)) {
        using PN = std::integral_constant<int, decltype(par)::value ^ 1>;
        v_phase(2 * t + 1);
        __builtin_amdgcn_s_waitcnt(kWaitPrev);
        barrier_lds();
        m_phase(par, 2 * (t + 1) + 1, 2 * t + 1);
        barrier_lds();
        issue_pos(2 * (t + 3) + 1);
        issue_k(2 * (t + 3) + 1, g, PN{});
        issue_v(2 * (t + 2) + 1, g, par);
      };
      for (int t = 0; t < n_iter; t += 2) {
        iteration(t, I0{});
        iteration(t + 1, I1{});
      }
    }
  };
  if (n_tiles > 0) {                  // workgroup-uniform
    if (grp == 0) run_group(I0{});
    else run_group(I1{});
  }

  // ---- merge the partial softmax states of a row block: writer waves pass
  // (m, l, O^T) through LDS (one 32-row block of O^T per round, through a K
  // slot) to the reader wave that holds the same rows.  Chunk layout: group
  // 1 -> group 0.  Short-chunk layout: key half 1 -> key half 0 in each
  // group, then group 1 -> group 0.
  wait_vmem_all();
  barrier_lds();
  constexpr int NX = kRowBlocks * 64;                     // exchange slots
  constexpr int XR = TB / (NX * 4) < 16 ? TB / (NX * 4) : 16;   // O registers per round
  static_assert(XR >= 1 && 16 % XR == 0 && 2 * NX * 4 <= TB, "exchange fits a K slot");
  float* xo = reinterpret_cast<float*>(k00);              // XR x NX floats (one K slot)
  float* xm = reinterpret_cast<float*>(k01);              // m, l
  auto fold = [&](bool writer, bool reader, int slot) __attribute__((always_inline)) {
    if (writer) {
      xm[slot] = m_run;
      xm[NX + slot] = l_run;
    }
    barrier_lds();
    float a0 = 1.f, a1 = 0.f;
    if (reader) {
      const float m1 = xm[slot];
      const float l1 = xm[NX + slot];
      const float m = fmaxf(m_run, m1);
      a0 = fast_exp2(m_run - m);
      a1 = fast_exp2(m1 - m);
      l_run = l_run * a0 + l1 * a1;
      m_run = m;
    }
#pragma unroll
    for (int db = 0; db < DB; ++db) {
#pragma unroll
      for (int r0 = 0; r0 < 16; r0 += XR) {
        if (writer) {
#pragma unroll
          for (int r = 0; r < XR; ++r) xo[r * NX + slot] = o[db][r0 + r];
        }
        barrier_lds();
        if (reader) {
#pragma unroll
          for (int r = 0; r < XR; ++r) o[db][r0 + r] = o[db][r0 + r] * a0 + xo[r * NX + slot] * a1;
        }
        barrier_lds();
      }
    }
  };
  if constexpr (DEC) {
    fold(kh == 1, kh == 0, (grp * 2 + rbp) * 64 + lane);
    fold(grp == 1 && kh == 0, grp == 0 && kh == 0, rbp * 64 + lane);
  } else {
    fold(grp == 1, grp == 0, rbw * 64 + lane);
  }
  if (grp == 1 || kh == 1 || !active) return;
  const float l_tot = l_run + xor32(l_run);
  if (!row_ok) return;
  if (n_split > 1) {
    // partial state of this row and split: O unnormalised against m_run
    // (log2 units), then m_run and the row sum; record = D + 4 floats
    float* rec = part + ((static_cast<size_t>(b * Hq + hq) * S + qi) * n_split + split) * (D + 4);
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int a = 0; a < 4; ++a)
        *reinterpret_cast<f32x4*>(rec + db * 32 + 8 * a + 4 * hf) =
            f32x4{o[db][4 * a], o[db][4 * a + 1], o[db][4 * a + 2], o[db][4 * a + 3]};
    if (hf == 0) *reinterpret_cast<f32x4*>(rec + D) = f32x4{m_run, l_tot, 0.f, 0.f};
    return;
  }
  const float inv = 1.f / l_tot;
  bf16_t* orow = O + (static_cast<size_t>(b * Hq + hq) * S + qi) * D;
#pragma unroll
  for (int db = 0; db < DB; ++db) {
#pragma unroll
    for (int a = 0; a < 4; ++a) {
      f32x4 v = {o[db][4 * a] * inv, o[db][4 * a + 1] * inv, o[db][4 * a + 2] * inv,
                 o[db][4 * a + 3] * inv};
      *reinterpret_cast<bf16x4*>(orow + db * 32 + 8 * a + 4 * hf) = to_bf16x4(v);
    }
  }
  if (hf == 0) lse[static_cast<size_t>(b * Hq + hq) * S + qi] = (m_run + log2f(l_tot)) * kLn2;
}

// Key-split merge: row r's splits combine as m = max_s m_s, weights
// w_s = 2^(m_s - m), O = sum_s w_s O_s / sum_s w_s l_s (splits in order, so
// the result is deterministic), lse = (m + log2 l) ln 2.  One thread per 4
// elements of a row.
template <int D>
__global__ __launch_bounds__(256) void attn_merge_kernel(const float* __restrict__ part,
                                                         bf16_t* __restrict__ O, float* __restrict__ lse,
                                                         int n_split, int64_t n_rows) {
  constexpr int C4 = D / 4, REC = D + 4;
  const int64_t idx = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  if (idx >= n_rows * C4) return;
  const int64_t row = idx / C4;
  const int c4 = static_cast<int>(idx - row * C4);
  const float* rec = part + row * n_split * REC;
  float m = kNoMax;
  for (int sp = 0; sp < n_split; ++sp) m = fmaxf(m, rec[sp * REC + D]);
  float l = 0.f;
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  for (int sp = 0; sp < n_split; ++sp) {
    const float* r = rec + sp * REC;
    const float w = fast_exp2(r[D] - m);
    l = fmaf(w, r[D + 1], l);
    acc += w * *reinterpret_cast<const f32x4*>(r + 4 * c4);
  }
  const float inv = 1.f / l;
  *reinterpret_cast<bf16x4*>(O + row * D + 4 * c4) = to_bf16x4(acc * inv);
  if (c4 == 0) lse[row] = (m + log2f(l)) * kLn2;
}

// fp32: one thread per (query head in group, query) row; 64 rows per wave.
template <int D>
__global__ __launch_bounds__(64) void attn_fwd_f32_kernel(
    const float* __restrict__ Q, const float* __restrict__ Kc, const float* __restrict__ Vc,
    const int32_t* __restrict__ pos, const float* __restrict__ Kn, const float* __restrict__ Vn,
    float* __restrict__ O, float* __restrict__ lse, int Hq, int Hkv, int S, int M, int n_cache,
    float c2, int n_heads, int wg_per_head) {
  constexpr int KT = 32;
  __shared__ float Ks[KT][D];
  __shared__ float Vs[KT][D];
  __shared__ int okey[KT];
  const int lane = threadIdx.x;
  const int bh = blockIdx.x % n_heads;
  const int wgi = static_cast<int>(blockIdx.x) / n_heads;
  const int b = bh / Hkv, kvh = bh - b * Hkv;
  const int G = Hq / Hkv;
  const int row = wgi * 64 + lane;
  const bool active = row < G * S;
  const int g = active ? row / S : 0, qi = active ? row % S : 0;
  const int hq = kvh * G + g;
  const int last_row = min(wgi * 64 + 63, G * S - 1);
  // largest query index among this wave's rows
  const int max_i = (last_row / S > (wgi * 64) / S) ? S - 1 : last_row % S;
  float q[D], o[D];
  const float* qrow = Q + (static_cast<size_t>(b * Hq + hq) * S + qi) * D;
#pragma unroll
  for (int e = 0; e < D; ++e) { q[e] = active ? qrow[e] : 0.f; o[e] = 0.f; }
  float m = kNegInf, l = 0.f;
  const int n_ct = (n_cache + KT - 1) / KT;
  const int n_tiles = n_ct + (max_i + 1 + KT - 1) / KT;
  for (int t = 0; t < n_tiles; ++t) {
    const bool is_cache = t < n_ct;
    const int base = is_cache ? t * KT : (t - n_ct) * KT;
    const int lim = is_cache ? n_cache : S;
    const float* ks = is_cache ? Kc + static_cast<size_t>(bh) * M * D : Kn + static_cast<size_t>(bh) * S * D;
    const float* vs = is_cache ? Vc + static_cast<size_t>(bh) * M * D : Vn + static_cast<size_t>(bh) * S * D;
    __syncthreads();
    for (int idx = lane; idx < KT * D; idx += 64) {
      const int k = idx / D, e = idx % D;
      const bool ok = base + k < lim;
      Ks[k][e] = ok ? ks[static_cast<size_t>(base + k) * D + e] : 0.f;
      Vs[k][e] = ok ? vs[static_cast<size_t>(base + k) * D + e] : 0.f;
    }
    if (lane < KT) {
      const int key = base + lane;
      okey[lane] = (key < lim) && (!is_cache || pos[static_cast<size_t>(bh) * M + key] >= 0);
    }
    __syncthreads();
    for (int k = 0; k < KT; ++k) {
      if (!okey[k]) continue;
      if (!is_cache && base + k > qi) continue;
      float z = 0.f;
#pragma unroll
      for (int e = 0; e < D; ++e) z = fmaf(q[e], Ks[k][e], z);
      z *= c2;
      if (z > m) {
        const float a = fast_exp2(m - z);
        l *= a;
#pragma unroll
        for (int e = 0; e < D; ++e) o[e] *= a;
        m = z;
      }
      const float p = fast_exp2(z - m);
      l += p;
#pragma unroll
      for (int e = 0; e < D; ++e) o[e] = fmaf(p, Vs[k][e], o[e]);
    }
  }
  if (!active) return;
  float* orow = O + (static_cast<size_t>(b * Hq + hq) * S + qi) * D;
  const float inv = 1.f / l;
#pragma unroll
  for (int e = 0; e < D; ++e) orow[e] = o[e] * inv;
  lse[static_cast<size_t>(b * Hq + hq) * S + qi] = (m + log2f(l)) * kLn2;
}

}  // namespace

size_t attn_split_bytes(int B, int Hq, int S, int D) {
  const int64_t rows = std::min<int64_t>(kSplitRows, static_cast<int64_t>(B) * Hq * S * kMaxKeySplits);
  return static_cast<size_t>(rows) * (D + 4) * sizeof(float);
}

hipError_t launch_attn_fwd(const StepShape& sh, const AttnArgs& a, int dtype, hipStream_t st) {
  const int n_heads = sh.B * sh.Hkv;
  const int G = sh.Hq / sh.Hkv;
  const float c2 = sh.scale * kLog2e;
  if (dtype == kBF16) {
    // short chunks pack the G*S rows of a KV group densely (see the kernel)
    const bool dec = sh.S < 32;
    const int n_rb = dec ? (G * sh.S + 31) / 32 : G * ((sh.S + 31) / 32);
    const int rbw = dec ? 2 : kRowBlocks;
    const int wgp = (n_rb + rbw - 1) / rbw;
    // small grids (under half the CUs) split the keys of each row group over
    // several workgroups (about one round of the CUs, at least 4 tiles each)
    // and merge after
    int n_split = 1;
    if (!dec && a.part != nullptr && 2 * n_heads * wgp < sh.n_cu) {
      const int n_tiles_min = (sh.n_cache + 63) / 64 + 1;
      n_split = std::min(kMaxKeySplits, std::min(sh.n_cu / (n_heads * wgp), std::max(1, n_tiles_min / 4)));
      while (n_split > 1 && static_cast<int64_t>(sh.B) * sh.Hq * sh.S * n_split > kSplitRows) --n_split;
    }
    const dim3 grid(n_heads * wgp * n_split), block(kFwdThreads);
#define H2O_LAUNCH_FWD1(DD, DEC, SK, AF)                                                            \
  hipLaunchKernelGGL(HIP_KERNEL_NAME(attn_fwd_bf16_kernel<DD, DEC, SK, AF>), grid, block, 0, st,    \
                     static_cast<const bf16_t*>(a.q), static_cast<const bf16_t*>(a.k_cache),        \
                     static_cast<const bf16_t*>(a.v_cache), a.pos,                                  \
                     static_cast<const bf16_t*>(a.k_new), static_cast<const bf16_t*>(a.v_new),      \
                     static_cast<bf16_t*>(a.out), a.lse, sh.Hq, sh.Hkv, sh.S, sh.M, sh.n_cache, c2, \
                     n_heads, wgp, n_split, a.part)
#define H2O_LAUNCH_FWD(DD)                                    \
  if (dec) H2O_LAUNCH_FWD1(DD, true, false, false);           \
  else if (n_split > 1) H2O_LAUNCH_FWD1(DD, false, true, false); \
  else if (sh.all_filled) H2O_LAUNCH_FWD1(DD, false, false, true); \
  else H2O_LAUNCH_FWD1(DD, false, false, false)
    if (sh.D == 128) {
      H2O_LAUNCH_FWD(128);
    } else {
      H2O_LAUNCH_FWD(64);
    }
#undef H2O_LAUNCH_FWD
#undef H2O_LAUNCH_FWD1
    if (n_split > 1) {
      const hipError_t e = hipGetLastError();
      if (e != hipSuccess) return e;
      const int64_t n_rows = static_cast<int64_t>(sh.B) * sh.Hq * sh.S;
      const unsigned blocks = static_cast<unsigned>((n_rows * (sh.D / 4) + 255) / 256);
      if (sh.D == 128)
        hipLaunchKernelGGL(attn_merge_kernel<128>, dim3(blocks), dim3(256), 0, st, a.part,
                           static_cast<bf16_t*>(a.out), a.lse, n_split, n_rows);
      else
        hipLaunchKernelGGL(attn_merge_kernel<64>, dim3(blocks), dim3(256), 0, st, a.part,
                           static_cast<bf16_t*>(a.out), a.lse, n_split, n_rows);
    }
  } else {
    const int wgp = (G * sh.S + 63) / 64;
    const dim3 grid(n_heads * wgp), block(64);
#define H2O_LAUNCH_FWD32(DD)                                                                     \
  hipLaunchKernelGGL(attn_fwd_f32_kernel<DD>, grid, block, 0, st,                                \
                     static_cast<const float*>(a.q), static_cast<const float*>(a.k_cache),       \
                     static_cast<const float*>(a.v_cache), a.pos,                                \
                     static_cast<const float*>(a.k_new), static_cast<const float*>(a.v_new),     \
                     static_cast<float*>(a.out), a.lse, sh.Hq, sh.Hkv, sh.S, sh.M, sh.n_cache, c2, \
                     n_heads, wgp)
    if (sh.D == 128) H2O_LAUNCH_FWD32(128);
    else H2O_LAUNCH_FWD32(64);
#undef H2O_LAUNCH_FWD32
  }
  return hipGetLastError();
}

}  // namespace h2o
