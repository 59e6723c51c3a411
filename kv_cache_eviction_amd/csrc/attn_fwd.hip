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
#include "h2o_device.h"
#include "h2o_launch.h"

namespace h2o {
namespace {

constexpr int kKT = 64;        // keys per LDS tile
constexpr int kRowBlocks = 4;  // row blocks (32 queries of one head) per workgroup
constexpr int kFwdThreads = 512;

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
  constexpr int NCH = 2 * 2 * kKT * CPR / kFwdThreads;   // chunks per thread per tile pair
  // [stage][group][K,V][TILE]
  __shared__ __attribute__((aligned(16))) bf16_t lds[2 * 2 * 2 * TILE];
  __shared__ uint64_t s_valid[2][2];

  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63, hf = lane >> 5, col = lane & 31;
  const int grp = wave >> 2, rbw = wave & 3;
  const int bh = blockIdx.x % n_heads;
  const int wgi = wg_per_head - 1 - static_cast<int>(blockIdx.x) / n_heads;
  const int b = bh / Hkv, kvh = bh - b * Hkv;
  const int G = Hq / Hkv;
  const int n_rb = G * ((S + 31) >> 5);
  const int rb = wgi * kRowBlocks + rbw;
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
  f32x16 o[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) o[db] = zero16();
  float m_run = kNegInf, l_run = 0.f;

  // ---- staging: tile pair p = tiles (2p, 2p+1).  Chunk r of a thread is
  // c = tid + 512 r; its tile (tt), matrix (K or V) and row follow from r at
  // compile time, so every source pointer is a uniform per-tile value.
  struct TileSrc {
    const bf16_t* k;
    const bf16_t* v;
    int n;            // rows of the tile that exist (keys < lim)
  };
  auto tile_src = [&](int t) __attribute__((always_inline)) {
    TileSrc r;
    const bool is_cache = t < n_ct;
    const bool exists = t < n_tiles;
    const int base = is_cache ? t * kKT : (t - n_ct) * kKT;
    const size_t off = exists ? static_cast<size_t>(base) * D : 0;
    r.k = ((exists && is_cache) ? kc_head : kn_head) + off;
    r.v = ((exists && is_cache) ? vc_head : vn_head) + off;
    r.n = exists ? (is_cache ? n_cache : S) - base : 1;   // a tile past the end reads chunk row 0
    return r;
  };
  constexpr int RPT = NCH / 2;                  // chunks per thread per tile
  constexpr int RPM = RPT / 2;                  // chunks per thread per matrix of a tile
  const int ch = tid % CPR;                     // 16-byte chunk within the row
  const int row0 = tid / CPR;                   // first row; chunk r adds (r % RPM) * (512 / CPR)
  u32x4 reg[NCH];
  int preg = -1;
  auto load_pair = [&](int p) __attribute__((always_inline)) {
#pragma unroll
    for (int tt = 0; tt < 2; ++tt) {
      const TileSrc ts = tile_src(2 * p + tt);
#pragma unroll
      for (int mat = 0; mat < 2; ++mat) {
#pragma unroll
        for (int i = 0; i < RPM; ++i) {
          const int row = row0 + i * (kFwdThreads / CPR);
          // rows past the end of a tile read its last row (masked later): no branches
          const bf16_t* src = (mat ? ts.v : ts.k) + min(row, ts.n - 1) * D + ch * 8;
          reg[(tt * 2 + mat) * RPM + i] = load_u32x4(src);
        }
      }
    }
    if (wave < 2) {                       // wave tt fetches the positions of tile 2p+tt
      const int t = 2 * p + wave;
      const bool is_cache = t < n_ct;
      const int base = is_cache ? t * kKT : (t - n_ct) * kKT;
      const int lim = t < n_tiles ? (is_cache ? n_cache : S) : base;
      const int key = base + lane;
      const int pv = pos_head[is_cache ? min(key, M - 1) : 0];
      preg = key < lim ? (is_cache ? pv : 0) : -1;
    }
  };
  auto store_pair = [&](int stage) __attribute__((always_inline)) {
#pragma unroll
    for (int tt = 0; tt < 2; ++tt) {
#pragma unroll
      for (int mat = 0; mat < 2; ++mat) {
        bf16_t* dst = lds + ((stage * 2 + tt) * 2 + mat) * TILE;
#pragma unroll
        for (int i = 0; i < RPM; ++i) {
          const int row = row0 + i * (kFwdThreads / CPR);
          const u32x4 v = reg[(tt * 2 + mat) * RPM + i];
          if (mat == 0) {
            const int krow = (row & ~31) | krow_of_key(row & 31);
            store_u32x4(dst + krow * D + 8 * k_chunk<CPR>(krow, ch), v);
          } else {
            store_u32x4(dst + row * D + 8 * v_chunk<CPR>(row, ch), v);
          }
        }
      }
    }
    if (wave < 2) {
      const uint64_t m = __ballot(preg >= 0);
      if (lane == 0) s_valid[stage][wave] = m;
    }
  };

  // per-lane parts of the transpose-read addresses (see the V^T operand below)
  const int tr_j = lane & 15, tr_r = tr_j >> 2, tr_q = tr_j & 3, tr_dg = (lane >> 4) & 1;

  if (n_pairs > 0) {
    load_pair(0);
    store_pair(0);
    if (n_pairs > 1) load_pair(1);
  }
  __syncthreads();
  for (int p = 0; p < n_pairs; ++p) {
    const int stage = p & 1;
    const int t = 2 * p + grp;
    const bool is_cache = t < n_ct;
    const int base = is_cache ? t * kKT : (t - n_ct) * kKT;
    const bool work = active && t < n_tiles && (is_cache || base <= qb * 32 + 31);
    if (work) {
      const bf16_t* Kt = lds + ((stage * 2 + grp) * 2 + 0) * TILE;
      const bf16_t* Vt = lds + ((stage * 2 + grp) * 2 + 1) * TILE;
      f32x16 s0 = zero16(), s1 = zero16();
#pragma unroll
      for (int st = 0; st < DS; ++st) {
        const bf16x8 a0 = *reinterpret_cast<const bf16x8*>(Kt + col * D + 8 * k_chunk<CPR>(col, 2 * st + hf));
        const bf16x8 a1 =
            *reinterpret_cast<const bf16x8*>(Kt + (32 + col) * D + 8 * k_chunk<CPR>(32 + col, 2 * st + hf));
        s0 = mfma32x32x16(a0, qf[st], s0);
        s1 = mfma32x32x16(a1, qf[st], s1);
      }
      const uint64_t vm = s_valid[stage][grp];
      const bool causal = !is_cache && (base + kKT - 1 > qb * 32);
      if (vm != ~0ull || causal) {
        const uint32_t bits0 = static_cast<uint32_t>(vm >> (16 * hf)) & 0xffffu;
        const uint32_t bits1 = static_cast<uint32_t>(vm >> (32 + 16 * hf)) & 0xffffu;
        const int lim_i = causal ? qi - base - 16 * hf : 1 << 30;   // key offset bound
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
      const float m_new = fmaxf(m_run, mx * c2);
      const float m_use = (m_new == kNegInf) ? 0.f : m_new;
      const float alpha = fast_exp2(m_run - m_use);
      float rs = 0.f;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        s0[r] = fast_exp2(fmaf(s0[r], c2, -m_use));
        s1[r] = fast_exp2(fmaf(s1[r], c2, -m_use));
        rs += s0[r] + s1[r];
      }
      l_run = fmaf(l_run, alpha, rs);
      m_run = m_new;
      if (__ballot(alpha != 1.f)) {
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
          for (int r = 0; r < 16; ++r) o[db][r] *= alpha;
      }
      // O^T += V^T P^T; MFMA (kb,u) covers keys 32kb + 16(l/32) + 8u + e.  The
      // A operand V^T comes from two transpose reads: lane j = 4r + q of a
      // 16-lane group addresses V[key0 + r][d0 + 4q .. +4).
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
        for (int u = 0; u < 2; ++u) {
          const f32x16& sv = kb ? s1 : s0;
          f32x8 pv;
#pragma unroll
          for (int e = 0; e < 8; ++e) pv[e] = sv[8 * u + e];
          const bf16x8 pb = to_bf16x8(pv);
#pragma unroll
          for (int db = 0; db < DB; ++db) {
            const int d = db * 32 + tr_dg * 16 + 4 * tr_q;
            bf16x4 h0, h1;
#pragma unroll
            for (int t2 = 0; t2 < 2; ++t2) {
              const int key = kb * 32 + 16 * hf + 8 * u + 4 * t2 + tr_r;
              const bf16x4 v = lds_read_tr16(Vt + key * D + 8 * v_chunk<CPR>(key, d >> 3) + (d & 7));
              if (t2 == 0) h0 = v; else h1 = v;
            }
            const bf16x8 a = __builtin_shufflevector(h0, h1, 0, 1, 2, 3, 4, 5, 6, 7);
            o[db] = mfma32x32x16(a, pb, o[db]);
          }
        }
      }
    }
    // stage the next pair into the other buffer, prefetch the one after
    if (p + 1 < n_pairs) store_pair(stage ^ 1);
    if (p + 2 < n_pairs) load_pair(p + 2);
    __syncthreads();
  }

  // ---- merge the two groups' softmax states (group 1 -> LDS -> group 0)
  float* xch = reinterpret_cast<float*>(lds);            // [DB*16 + 2][kRowBlocks*64]
  const int slot = rbw * 64 + lane;
  constexpr int NX = kRowBlocks * 64;
  if (grp == 1) {
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int r = 0; r < 16; ++r) xch[(db * 16 + r) * NX + slot] = o[db][r];
    xch[(DB * 16) * NX + slot] = m_run;
    xch[(DB * 16 + 1) * NX + slot] = l_run;
  }
  __syncthreads();
  if (grp == 1 || !active) return;
  {
    const float m1 = xch[(DB * 16) * NX + slot];
    const float l1 = xch[(DB * 16 + 1) * NX + slot];
    const float m = fmaxf(m_run, m1);
    const float mu = (m == kNegInf) ? 0.f : m;
    const float a0 = fast_exp2(m_run - mu), a1 = fast_exp2(m1 - mu);
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int r = 0; r < 16; ++r) o[db][r] = o[db][r] * a0 + xch[(db * 16 + r) * NX + slot] * a1;
    l_run = l_run * a0 + l1 * a1;
    m_run = m;
  }
  const float l_tot = l_run + xor32(l_run);
  if (qi >= S) return;
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
