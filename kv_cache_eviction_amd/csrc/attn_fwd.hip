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
//   * A workgroup is 4 waves, one per SIMD.  Wave w owns one row block = 32
//     consecutive queries of one query head; row blocks are numbered
//     (query block, head in group), so the 4 row blocks of a workgroup share
//     their query range, causal extent and K/V tiles.
//   * Every wave runs two independent online-softmax chains, one over the
//     even and one over the odd 64-key tiles, merged at the end.  Both chains
//     sit in one instruction stream, so the MFMAs of one chain overlap the
//     softmax arithmetic of the other without the waves of a SIMD having to
//     fall out of step.
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
//   * Tile pairs go from global memory straight into a double-buffered LDS
//     ring with the gfx950 direct-to-LDS load (global_load_lds_dwordx4: lane
//     i of a wave writes bytes 16i..16i+15 of a 1 KB block); each lane picks
//     the source chunk that belongs at its LDS position, so the swizzled
//     layout costs nothing.  The next pair is requested before the current
//     pair is computed, and one wait + barrier per pair separates stages.
//     Rows past the end of a tile are clamped to a valid row and masked.
//   * Which cache slots hold a token (position >= 0) is read once per
//     workgroup into a bit mask in LDS.
//   * blockIdx -> (head, row group) keeps every workgroup of one (b, KV head)
//     on one XCD when B*Hkv is a multiple of 8 (dispatch is round-robin over
//     the 8 XCDs), so that head's K/V stays in that XCD's L2; the row groups
//     with the longest causal extent are dispatched first.
// fp32 path: one thread per query row, scalar online softmax over K/V rows
// broadcast from LDS (used for fp32 workloads, which are tiny).
#include "h2o_device.h"
#include "h2o_launch.h"

namespace h2o {
namespace {

constexpr int kKT = 64;        // keys per LDS tile
constexpr int kRowBlocks = 4;  // row blocks (32 queries of one head) per workgroup
constexpr int kFwdThreads = 256;

// Key k (0..31) of a 32-key block -> LDS row = MFMA A-operand row that reads
// it.  Row 8q + 4h + r holds key 16h + 4q + r, so that accumulator register
// r' of lane l corresponds to key 16(l/32) + r'.
__device__ __forceinline__ int krow_of_key(int k) {
  return ((k & 15) >> 2) * 8 + (k >> 4) * 4 + (k & 3);
}

// Swizzled 16-byte chunk of a K row / V row (CPR chunks per row).
template <int CPR>
__device__ __forceinline__ int k_chunk(int row, int c) { return c ^ (row & (CPR - 1)); }
template <int CPR>
__device__ __forceinline__ int v_chunk(int row, int c) {
  return c ^ ((row & 3) << (CPR == 16 ? 2 : 1));
}

// One online-softmax chain of a wave: running max (log2 domain), the lane's
// partial row sum and the O^T accumulators.
template <int DB>
struct Chain {
  f32x16 o[DB];
  float m, l;
};

// Scores S^T (64 keys x 32 queries) of one tile: accumulator register r of
// lane l holds key kb*32 + 16(l/32) + r against query l%32.
template <int D>
__device__ __forceinline__ void tile_scores(const bf16_t* Kt, const bf16x8 (&qf)[D / 16], int col,
                                            int hf, f32x16& s0, f32x16& s1) {
  constexpr int CPR = D / 8;
  s0 = zero16();
  s1 = zero16();
#pragma unroll
  for (int st = 0; st < D / 16; ++st) {
    const bf16x8 a0 = *reinterpret_cast<const bf16x8*>(Kt + col * D + 8 * k_chunk<CPR>(col, 2 * st + hf));
    const bf16x8 a1 =
        *reinterpret_cast<const bf16x8*>(Kt + (32 + col) * D + 8 * k_chunk<CPR>(32 + col, 2 * st + hf));
    s0 = mfma32x32x16(a0, qf[st], s0);
    s1 = mfma32x32x16(a1, qf[st], s1);
  }
}

// Masks (validity bits of the tile, causal bound), online-softmax update of
// the chain and conversion of the probabilities to the PV B operands.
template <int DB>
__device__ __forceinline__ void tile_softmax(f32x16& s0, f32x16& s1, Chain<DB>& ch, uint64_t vm,
                                             bool causal, int lim_i, int hf, float c2,
                                             bf16x8 (&pb)[4]) {
  if (vm != ~0ull || causal) {
    const uint32_t bits0 = static_cast<uint32_t>(vm >> (16 * hf)) & 0xffffu;
    const uint32_t bits1 = static_cast<uint32_t>(vm >> (32 + 16 * hf)) & 0xffffu;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const bool ok0 = ((bits0 >> r) & 1u) && (r <= lim_i);
      const bool ok1 = ((bits1 >> r) & 1u) && (32 + r <= lim_i);
      s0[r] = ok0 ? s0[r] : kNegInf;
      s1[r] = ok1 ? s1[r] : kNegInf;
    }
  }
  float mx = kNegInf;
#pragma unroll
  for (int r = 0; r < 16; ++r) mx = fmaxf(mx, fmaxf(s0[r], s1[r]));
  mx = fmaxf(mx, xor32(mx));
  const float m_new = fmaxf(ch.m, mx * c2);
  const float m_use = (m_new == kNegInf) ? 0.f : m_new;
  const float alpha = fast_exp2(ch.m - m_use);
  float rs = 0.f;
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    s0[r] = fast_exp2(fmaf(s0[r], c2, -m_use));
    s1[r] = fast_exp2(fmaf(s1[r], c2, -m_use));
    rs += s0[r] + s1[r];
  }
  ch.l = fmaf(ch.l, alpha, rs);
  ch.m = m_new;
  if (__ballot(alpha != 1.f)) {
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int r = 0; r < 16; ++r) ch.o[db][r] *= alpha;
  }
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    f32x8 v0, v1;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      v0[e] = s0[8 * u + e];
      v1[e] = s1[8 * u + e];
    }
    pb[u] = to_bf16x8(v0);
    pb[2 + u] = to_bf16x8(v1);
  }
}

// O^T += V^T P^T for one tile.  MFMA (kb,u) covers keys 32kb + 16(l/32) +
// 8u + e; its A operand comes from two transpose reads in which lane
// j = 4r + q of a 16-lane group addresses V[key0 + r][d0 + 4q .. +4).
template <int D>
__device__ __forceinline__ void tile_pv(const bf16_t* Vt, const bf16x8 (&pb)[4], f32x16 (&o)[D / 32],
                                        int hf, int tr_r, int tr_q, int tr_dg) {
  constexpr int CPR = D / 8;
#pragma unroll
  for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
    for (int u = 0; u < 2; ++u) {
#pragma unroll
      for (int db = 0; db < D / 32; ++db) {
        const int d = db * 32 + tr_dg * 16 + 4 * tr_q;
        const int key0 = kb * 32 + 16 * hf + 8 * u + tr_r;
        const bf16x4 h0 = lds_read_tr16(Vt + key0 * D + 8 * v_chunk<CPR>(key0, d >> 3) + (d & 7));
        const bf16x4 h1 = lds_read_tr16(Vt + (key0 + 4) * D + 8 * v_chunk<CPR>(key0 + 4, d >> 3) + (d & 7));
        const bf16x8 a = __builtin_shufflevector(h0, h1, 0, 1, 2, 3, 4, 5, 6, 7);
        o[db] = mfma32x32x16(a, pb[2 * kb + u], o[db]);
      }
    }
  }
}

template <int D>
__global__ __launch_bounds__(kFwdThreads, 1) void attn_fwd_bf16_kernel(
    const bf16_t* __restrict__ Q, const bf16_t* __restrict__ Kc,
    const bf16_t* __restrict__ Vc, const int32_t* __restrict__ pos,
    const bf16_t* __restrict__ Kn, const bf16_t* __restrict__ Vn,
    bf16_t* __restrict__ O, float* __restrict__ lse, int Hq, int Hkv, int S,
    int M, int n_cache, float c2, int n_heads, int wg_per_head) {
  constexpr int DS = D / 16;              // MFMA k-steps over d
  constexpr int DB = D / 32;              // 32-row blocks of O^T
  constexpr int CPR = D / 8;              // 16-byte chunks per row
  constexpr int TILE = kKT * D;           // elements per K or V tile
  // [stage][tile of the pair][K,V][TILE]
  __shared__ __attribute__((aligned(16))) bf16_t lds[2 * 2 * 2 * TILE];
  __shared__ uint64_t s_vbits[16384 / kKT];

  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63, hf = lane >> 5, col = lane & 31;
  const int bh = blockIdx.x % n_heads;
  const int wgi = wg_per_head - 1 - static_cast<int>(blockIdx.x) / n_heads;
  const int b = bh / Hkv, kvh = bh - b * Hkv;
  const int G = Hq / Hkv;
  const int n_rb = G * ((S + 31) >> 5);
  const int rb = wgi * kRowBlocks + wave;
  const bool active = rb < n_rb;
  const int g = active ? rb % G : 0;
  const int qb = active ? rb / G : 0;
  const int qi = qb * 32 + col;
  const int hq = kvh * G + g;
  const int rb_last = min(wgi * kRowBlocks + kRowBlocks - 1, n_rb - 1);
  const int n_chunk_keys = min(S, (rb_last / G + 1) * 32);
  const int n_ct = (n_cache + kKT - 1) / kKT;
  const int n_tiles = n_ct + (n_chunk_keys + kKT - 1) / kKT;
  const int n_pairs = (n_tiles + 1) >> 1;

  const bf16_t* kc_head = Kc + static_cast<size_t>(bh) * M * D;
  const bf16_t* vc_head = Vc + static_cast<size_t>(bh) * M * D;
  const bf16_t* kn_head = Kn + static_cast<size_t>(bh) * S * D;
  const bf16_t* vn_head = Vn + static_cast<size_t>(bh) * S * D;
  const int32_t* pos_head = pos + static_cast<size_t>(bh) * M;

  // The wave's queries: B operand of S^T = K Q^T (lane: query col, d 8hf..+8).
  bf16x8 qf[DS];
  {
    const bool qok = active && qi < S;
    const bf16_t* qrow = Q + (static_cast<size_t>(b * Hq + hq) * S + (qok ? qi : 0)) * D;
#pragma unroll
    for (int st = 0; st < DS; ++st) {
      bf16x8 v = load_bf16x8(qrow + 16 * st + 8 * hf);
      qf[st] = qok ? v : bf16x8{};
    }
  }
  Chain<DB> ch0, ch1;
#pragma unroll
  for (int db = 0; db < DB; ++db) {
    ch0.o[db] = zero16();
    ch1.o[db] = zero16();
  }
  ch0.m = ch1.m = kNegInf;
  ch0.l = ch1.l = 0.f;

  // ---- validity of the cache slots: one 64-bit mask per cache tile
  for (int t = wave; t < n_ct; t += kRowBlocks) {
    const int key = t * kKT + lane;
    const int pv = pos_head[min(key, M - 1)];
    const uint64_t m = __ballot(key < n_cache && pv >= 0);
    if (lane == 0) s_vbits[t] = m;
  }

  // ---- staging: tile pair p = tiles (2p, 2p+1).  Wave w fills matrix
  // (w & 1 ? V : K) of tile 2p + (w >> 1): its instruction j writes LDS rows
  // RPI*j .. RPI*j + RPI-1 of that matrix (1 KB), lane i landing on row
  // RPI*j + i/CPR, physical chunk i%CPR.  The lane loads the logical chunk and
  // key that belong there.  Rows past the tile's end read its last row; a
  // tile past the last one reads chunk row 0 (never used).
  constexpr int RPI = 64 / CPR;                       // rows per 1 KB instruction
  const int dma_mat = wave & 1, dma_tt = wave >> 1;
  const int dma_row_in = lane / CPR, dma_pc = lane % CPR;
  const bf16_t* dma_cache = dma_mat ? vc_head : kc_head;
  const bf16_t* dma_new = dma_mat ? vn_head : kn_head;
  auto load_pair = [&](int p) __attribute__((always_inline)) {
    const int t = 2 * p + dma_tt;
    const bool is_cache = t < n_ct;
    const bool exists = t < n_tiles;
    const int base = is_cache ? t * kKT : (t - n_ct) * kKT;
    const int n = exists ? (is_cache ? n_cache : S) - base : 1;
    const bf16_t* src = ((exists && is_cache) ? dma_cache : dma_new) + (exists ? static_cast<size_t>(base) * D : 0);
    bf16_t* dst = lds + (((p & 1) * 2 + dma_tt) * 2 + dma_mat) * TILE;
#pragma unroll
    for (int j = 0; j < CPR; ++j) {
      const int row = RPI * j + dma_row_in;
      int key, c;
      if (dma_mat == 0) {
        key = (row & ~31) | (16 * ((row >> 2) & 1) + 4 * ((row & 31) >> 3) + (row & 3));
        c = k_chunk<CPR>(row, dma_pc);
      } else {
        key = row;
        c = v_chunk<CPR>(row, dma_pc);
      }
      key = min(key, n - 1);
      __builtin_amdgcn_global_load_lds(src + key * D + c * 8, dst + j * (RPI * D), 16, 0, 0);
    }
  };
  auto wait_pair = [&]() __attribute__((always_inline)) {
    __builtin_amdgcn_s_waitcnt(0x0f70);               // vmcnt(0): this wave's copies landed
    __syncthreads();                                  // ... and every other wave's
  };

  const int tr_j = lane & 15, tr_r = tr_j >> 2, tr_q = tr_j & 3, tr_dg = (lane >> 4) & 1;

  struct TileInfo {
    int base;
    bool work, causal;
    uint64_t vmask;
  };
  auto tile_info = [&](int t) __attribute__((always_inline)) {
    TileInfo i;
    const bool is_cache = t < n_ct;
    i.base = is_cache ? t * kKT : (t - n_ct) * kKT;
    i.work = active && t < n_tiles && (is_cache || i.base <= qb * 32 + 31);
    i.causal = !is_cache && (i.base + kKT - 1 > qb * 32);
    const int nk = S - i.base;
    i.vmask = is_cache ? s_vbits[min(t, n_ct - 1)]
                       : (nk >= 64 ? ~0ull : ((1ull << (nk > 0 ? nk : 0)) - 1ull));
    return i;
  };

  if (n_pairs > 0) load_pair(0);
  wait_pair();
  for (int p = 0; p < n_pairs; ++p) {
    const int stage = p & 1;
    if (p + 1 < n_pairs) load_pair(p + 1);          // into the stage computed last iteration
    // tiles 2p (chain 0) and 2p+1 (chain 1); skip tiles past the end or past
    // this wave's causal extent
    const TileInfo i0 = tile_info(2 * p), i1 = tile_info(2 * p + 1);
    const bf16_t* K0 = lds + ((stage * 2 + 0) * 2 + 0) * TILE;
    const bf16_t* V0 = lds + ((stage * 2 + 0) * 2 + 1) * TILE;
    const bf16_t* K1 = lds + ((stage * 2 + 1) * 2 + 0) * TILE;
    const bf16_t* V1 = lds + ((stage * 2 + 1) * 2 + 1) * TILE;
    if (i0.work && i1.work) {
      // both chains: interleavable MFMA / VALU streams
      f32x16 a0, a1, b0, b1;
      bf16x8 pa[4], pbb[4];
      tile_scores<D>(K0, qf, col, hf, a0, a1);
      tile_scores<D>(K1, qf, col, hf, b0, b1);
      tile_softmax<DB>(a0, a1, ch0, i0.vmask, i0.causal, qi - i0.base - 16 * hf, hf, c2, pa);
      tile_softmax<DB>(b0, b1, ch1, i1.vmask, i1.causal, qi - i1.base - 16 * hf, hf, c2, pbb);
      tile_pv<D>(V0, pa, ch0.o, hf, tr_r, tr_q, tr_dg);
      tile_pv<D>(V1, pbb, ch1.o, hf, tr_r, tr_q, tr_dg);
    } else if (i0.work) {
      f32x16 a0, a1;
      bf16x8 pa[4];
      tile_scores<D>(K0, qf, col, hf, a0, a1);
      tile_softmax<DB>(a0, a1, ch0, i0.vmask, i0.causal, qi - i0.base - 16 * hf, hf, c2, pa);
      tile_pv<D>(V0, pa, ch0.o, hf, tr_r, tr_q, tr_dg);
    } else if (i1.work) {
      f32x16 b0, b1;
      bf16x8 pbb[4];
      tile_scores<D>(K1, qf, col, hf, b0, b1);
      tile_softmax<DB>(b0, b1, ch1, i1.vmask, i1.causal, qi - i1.base - 16 * hf, hf, c2, pbb);
      tile_pv<D>(V1, pbb, ch1.o, hf, tr_r, tr_q, tr_dg);
    }
    wait_pair();
  }
  if (!active) return;

  // ---- merge the two chains
  const float m = fmaxf(ch0.m, ch1.m);
  const float mu = (m == kNegInf) ? 0.f : m;
  const float w0 = fast_exp2(ch0.m - mu), w1 = fast_exp2(ch1.m - mu);
  const float l_lane = ch0.l * w0 + ch1.l * w1;
  const float l_tot = l_lane + xor32(l_lane);
  if (qi >= S) return;
  const float inv = 1.f / l_tot;
  bf16_t* orow = O + (static_cast<size_t>(b * Hq + hq) * S + qi) * D;
#pragma unroll
  for (int db = 0; db < DB; ++db) {
#pragma unroll
    for (int a = 0; a < 4; ++a) {
      f32x4 v;
#pragma unroll
      for (int e = 0; e < 4; ++e) v[e] = (ch0.o[db][4 * a + e] * w0 + ch1.o[db][4 * a + e] * w1) * inv;
      *reinterpret_cast<bf16x4*>(orow + db * 32 + 8 * a + 4 * hf) = to_bf16x4(v);
    }
  }
  if (hf == 0) lse[static_cast<size_t>(b * Hq + hq) * S + qi] = (m + log2f(l_tot)) * kLn2;
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

hipError_t launch_attn_fwd(const StepShape& sh, const AttnArgs& a, int dtype, hipStream_t st) {
  const int n_heads = sh.B * sh.Hkv;
  const int G = sh.Hq / sh.Hkv;
  const float c2 = sh.scale * kLog2e;
  if (dtype == kBF16) {
    const int n_rb = G * ((sh.S + 31) / 32);
    const int wgp = (n_rb + kRowBlocks - 1) / kRowBlocks;
    const dim3 grid(n_heads * wgp), block(kFwdThreads);
#define H2O_LAUNCH_FWD(DD)                                                                          \
  hipLaunchKernelGGL(attn_fwd_bf16_kernel<DD>, grid, block, 0, st,                                  \
                     static_cast<const bf16_t*>(a.q), static_cast<const bf16_t*>(a.k_cache),        \
                     static_cast<const bf16_t*>(a.v_cache), a.pos,                                  \
                     static_cast<const bf16_t*>(a.k_new), static_cast<const bf16_t*>(a.v_new),      \
                     static_cast<bf16_t*>(a.out), a.lse, sh.Hq, sh.Hkv, sh.S, sh.M, sh.n_cache, c2, \
                     n_heads, wgp)
    if (sh.D == 128) H2O_LAUNCH_FWD(128);
    else H2O_LAUNCH_FWD(64);
#undef H2O_LAUNCH_FWD
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
