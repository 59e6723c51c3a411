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
//   * A workgroup is 4 waves; wave w owns one row block = 32 consecutive
//     queries of one query head.  Row blocks are numbered (query block, head
//     in group), so the waves of a workgroup share their query range and
//     therefore their causal extent and every K/V tile.
//   * The kernel computes S^T = K Q^T: K (64-key tiles) is the A operand read
//     from LDS, the wave's 32 queries are the B operand held in registers for
//     the whole kernel.  Each lane then owns one query column, so the row
//     softmax needs no cross-lane work except one exchange with lane l^32.
//   * K rows are stored in LDS in MFMA-row order, chosen so that accumulator
//     register r of lane l holds key 16(l/32) + r.  The probabilities then
//     feed O^T = V^T P^T as the B operand straight from registers, and V^T
//     (transposed into LDS when the tile is staged) is the A operand.
//   * Online softmax in the log2 domain (exp2 on v_exp_f32); the O rescale
//     is skipped when no lane's running maximum moved.
//   * Tiles are staged through registers: the next tile's global loads are
//     issued before the current tile's MFMAs.
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

constexpr int kKT = 64;     // keys per LDS tile
constexpr int kWaves = 4;   // row blocks (waves) per workgroup

// Key k (0..31) of a 32-key block -> LDS row = MFMA A-operand row that reads
// it.  Row 8q + 4h + r holds key 16h + 4q + r, so that accumulator register
// r' of lane l corresponds to key 16(l/32) + r'.
__device__ __forceinline__ int krow_of_key(int k) {
  return ((k & 15) >> 2) * 8 + (k >> 4) * 4 + (k & 3);
}

// Column of element (d, key) in the transposed V tile: 8-key groups are
// XOR-swizzled by (d/8) % 8 to spread the transposing stores over banks;
// every aligned 8-key group stays contiguous (one 16-byte read).
__device__ __forceinline__ int vt_col(int d, int k) {
  return ((((k >> 3) ^ (d >> 3)) & 7) << 3) | (k & 7);
}

template <int D>
__global__ __launch_bounds__(256, 1) void attn_fwd_bf16_kernel(
    const bf16_t* __restrict__ Q, const bf16_t* __restrict__ Kc,
    const bf16_t* __restrict__ Vc, const int32_t* __restrict__ pos,
    const bf16_t* __restrict__ Kn, const bf16_t* __restrict__ Vn,
    bf16_t* __restrict__ O, float* __restrict__ lse, int Hq, int Hkv, int S,
    int M, int n_cache, float c2, int n_heads, int wg_per_head) {
  constexpr int DS = D / 16;          // MFMA k-steps over d
  constexpr int DB = D / 32;          // 32-row blocks of O^T
  constexpr int KLD = D + 8;          // K tile row stride (elements)
  constexpr int VLD = kKT + 8;        // V^T tile row stride (elements)
  constexpr int CPR = D / 8;          // 16-byte chunks per key row
  constexpr int NCH = kKT * CPR / 256;
  __shared__ __attribute__((aligned(16))) bf16_t Ks[kKT * KLD];
  __shared__ __attribute__((aligned(16))) bf16_t Vt[D * VLD];
  __shared__ uint64_t s_valid;

  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63, hf = lane >> 5, col = lane & 31;
  const int bh = blockIdx.x % n_heads;
  const int wgi = wg_per_head - 1 - static_cast<int>(blockIdx.x) / n_heads;
  const int b = bh / Hkv, kvh = bh - b * Hkv;
  const int G = Hq / Hkv;
  const int n_rb = G * ((S + 31) >> 5);
  const int rb = wgi * kWaves + wave;
  const bool active = rb < n_rb;
  const int g = active ? rb % G : 0;
  const int qb = active ? rb / G : 0;
  const int qi = qb * 32 + col;
  const int hq = kvh * G + g;
  const int rb_last = min(wgi * kWaves + kWaves - 1, n_rb - 1);
  const int n_chunk_keys = min(S, (rb_last / G + 1) * 32);
  const int n_ct = (n_cache + kKT - 1) / kKT;
  const int n_tiles = n_ct + (n_chunk_keys + kKT - 1) / kKT;

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

  u32x4 kreg[NCH], vreg[NCH];
  int preg = 0;
  auto load_tile = [&](int t) {
    const bool is_cache = t < n_ct;
    const int base = is_cache ? t * kKT : (t - n_ct) * kKT;
    const int lim = is_cache ? n_cache : S;
    const bf16_t* ks = is_cache ? kc_head : kn_head;
    const bf16_t* vs = is_cache ? vc_head : vn_head;
#pragma unroll
    for (int r = 0; r < NCH; ++r) {
      const int c = r * 256 + tid, key = c / CPR, dc = c % CPR;
      if (base + key < lim) {
        kreg[r] = load_u32x4(ks + static_cast<size_t>(base + key) * D + dc * 8);
        vreg[r] = load_u32x4(vs + static_cast<size_t>(base + key) * D + dc * 8);
      } else {
        kreg[r] = u32x4{0, 0, 0, 0};
        vreg[r] = u32x4{0, 0, 0, 0};
      }
    }
    if (wave == 0) {
      const int key = base + lane;
      preg = (key < lim) ? (is_cache ? pos_head[key] : 0) : -1;
    }
  };
  auto store_tile = [&]() {
#pragma unroll
    for (int r = 0; r < NCH; ++r) {
      const int c = r * 256 + tid, key = c / CPR, dc = c % CPR;
      const int krow = (key & ~31) | krow_of_key(key & 31);
      store_u32x4(&Ks[krow * KLD + dc * 8], kreg[r]);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int d = dc * 8 + e;
        const uint32_t w = vreg[r][e >> 1];
        Vt[d * VLD + vt_col(d, key)] = static_cast<bf16_t>((e & 1) ? (w >> 16) : (w & 0xffffu));
      }
    }
    if (wave == 0) {
      const uint64_t m = __ballot(preg >= 0);
      if (lane == 0) s_valid = m;
    }
  };

  if (n_tiles > 0) load_tile(0);
  for (int t = 0; t < n_tiles; ++t) {
    __syncthreads();
    store_tile();
    __syncthreads();
    if (t + 1 < n_tiles) load_tile(t + 1);
    if (!active) continue;
    const bool is_cache = t < n_ct;
    const int base = is_cache ? t * kKT : (t - n_ct) * kKT;
    if (!is_cache && base > qb * 32 + 31) continue;   // beyond this wave's causal extent

    f32x16 s0 = zero16(), s1 = zero16();
#pragma unroll
    for (int st = 0; st < DS; ++st) {
      const bf16x8 a0 = *reinterpret_cast<const bf16x8*>(&Ks[col * KLD + 16 * st + 8 * hf]);
      const bf16x8 a1 = *reinterpret_cast<const bf16x8*>(&Ks[(32 + col) * KLD + 16 * st + 8 * hf]);
      s0 = mfma32x32x16(a0, qf[st], s0);
      s1 = mfma32x32x16(a1, qf[st], s1);
    }
    const uint64_t vm = s_valid;
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
    // O^T += V^T P^T; MFMA (kb,u) covers keys 32kb + 16(l/32) + 8u + e.
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const f32x16& s = kb ? s1 : s0;
        f32x8 pv;
#pragma unroll
        for (int e = 0; e < 8; ++e) pv[e] = s[8 * u + e];
        const bf16x8 pb = to_bf16x8(pv);
        const int key = kb * 32 + 16 * hf + 8 * u;
#pragma unroll
        for (int db = 0; db < DB; ++db) {
          const int d = db * 32 + col;
          const bf16x8 a = *reinterpret_cast<const bf16x8*>(&Vt[d * VLD + vt_col(d, key)]);
          o[db] = mfma32x32x16(a, pb, o[db]);
        }
      }
    }
  }
  if (!active) return;
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
    const int wgp = (n_rb + kWaves - 1) / kWaves;
    const dim3 grid(n_heads * wgp), block(256);
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
