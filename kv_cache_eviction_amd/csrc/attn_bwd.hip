// Frozen-eviction backward of one chunk's attention (h2o_chunk_backward).
//
// "Learning how to Forget: Fine-tuning for Long-Context Sparse Attention"
// (arXiv 2608.19920) trains through the chunk lattice of its Fig. 1 by
// running autograd per cell (Fig. 1(b)); the gradient of one chunk step's
// attention with the eviction decisions held fixed is the building block.
// The visible sets are those of the forward step: every filled slot of the
// pre-step cache and the chunk's keys j <= i; the scores are not
// differentiated.  With P = softmax(scale * q.key) over the visible keys:
//   dP = dO V^T,  D_i = sum_j P_ij dP_ij (= dO_i . O_i),  dS = P * (dP - D),
//   dq = scale * dS K,  dK = scale * dS^T Q,  dV = P^T dO,
// where dK and dV of a KV head sum over the G query heads of its group.
//
// Three kernels, all deterministic (no atomics):
//   * bwd_dq_kernel: one wave per 32-query row block, 8 per workgroup (the forward's layout:
//     S^T = K Q^T, lane = query), loops over the key tiles.  Its dS uses
//     D_i = dO_i . O_i from the stored output; it accumulates the exact
//     sum_j P_ij dP_ij on the way and writes that D for the dK/dV kernel.
//     K rows sit in LDS in MFMA-row order, which keeps every aligned group of
//     4 keys in 4 consecutive rows, so the same tile serves the K rows of S^T
//     (16-byte reads) and K^T of dQ^T = K^T dS^T (transpose reads).
//   * bwd_dkdv_kernel: 128 keys per workgroup (K and V rows in LDS), one wave
//     per 32 keys and row set; the two row sets split the query rows of the
//     KV group (S = Q K^T, lane = key), accumulating dV^T += dO^T P and
//     dK^T += Q^T dS with dO^T and Q^T from transpose reads of the staged
//     row block, and fold their sums at the end.  Chunk-key tiles split
//     their query rows into pieces that write fp32 partials;
//   * bwd_chunk_reduce_kernel sums those partials in piece order.
#include <type_traits>

#include "h2o_device.h"
#include "h2o_launch.h"

namespace h2o {
namespace {

constexpr int kBKT = 64;     // keys per LDS tile (dq kernel)
constexpr int kBWaves = 8;     // row blocks (waves) per dQ workgroup

// LDS row r of a 32-key block holds key key_of_bkrow(r) (MFMA A-operand row
// order: row 8q + 4h + r' holds key 16h + 4q + r').
__device__ __forceinline__ int key_of_bkrow(int r) {
  return ((r >> 2) & 1) * 16 + (r >> 3) * 4 + (r & 3);
}
// Swizzled 16-byte chunk of a tile row (CPR chunks per row).  A tile here is
// read two ways: by rows (16 lanes, 16 consecutive rows, one chunk each) and
// by transpose reads (32 lanes, 4 consecutive rows x 4 consecutive chunks).
// The XOR mask is a bijection over each 16 rows and gives the 4 rows of an
// aligned group distinct high chunk bits, so both patterns hit all 64 banks
// once.  Rows of D = 64 are 128 bytes: even and odd rows use opposite bank
// halves and the mask runs over row / 2.
template <int CPR>
__device__ __forceinline__ int bchunk(int row, int c) {
  static_assert(CPR == 8 || CPR == 16, "head dims 64 and 128");
  if constexpr (CPR == 16) return c ^ (((row & 3) << 2) | ((row >> 2) & 3));
  return c ^ ((((row >> 1) & 1) << 2) | ((row >> 2) & 3));
}

// ---------------------------------------------------------------- dQ and D
template <int D>
__global__ __launch_bounds__(512, 1) void bwd_dq_kernel(
    const bf16_t* __restrict__ Q, const bf16_t* __restrict__ Kc, const bf16_t* __restrict__ Vc,
    const int32_t* __restrict__ pos, const bf16_t* __restrict__ Kn, const bf16_t* __restrict__ Vn,
    const bf16_t* __restrict__ Oo, const bf16_t* __restrict__ dO, const float* __restrict__ lse,
    float* __restrict__ Dws, bf16_t* __restrict__ dQ, int Hq, int Hkv, int S, int M, float c2,
    float scale, int n_heads, int wg_per_head) {
  constexpr int DS = D / 16, DB = D / 32, CPR = D / 8;
  constexpr int RB = 2 * D;                        // bytes per row
  constexpr int NCH = kBKT * CPR / 512;            // 16-byte copies per thread per tile and tensor
  // two buffers: the next key tile is copied into one while the current one
  // is computed from the other; one array per buffer, so reads of one never
  // wait for copies into the other
  __shared__ __attribute__((aligned(16))) char k_b0[kBKT * RB], k_b1[kBKT * RB];
  __shared__ __attribute__((aligned(16))) char v_b0[kBKT * RB], v_b1[kBKT * RB];
  __shared__ uint64_t s_valid2[2];

  const int tid = threadIdx.x, lane = tid & 63, hf = lane >> 5, col = lane & 31;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int bh = blockIdx.x % n_heads;
  const int wgi = wg_per_head - 1 - static_cast<int>(blockIdx.x) / n_heads;
  const int b = bh / Hkv, kvh = bh - b * Hkv;
  const int G = Hq / Hkv;
  const int n_rb = G * ((S + 31) >> 5);
  const int rb = wgi * kBWaves + wave;
  const bool active = rb < n_rb;
  const int g = active ? rb % G : 0;
  const int qb = active ? rb / G : 0;
  const int qi = qb * 32 + col;
  const int hq = kvh * G + g;
  const bool qok = active && qi < S;
  const int rb_last = min(wgi * kBWaves + kBWaves - 1, n_rb - 1);
  const int n_chunk_keys = min(S, (rb_last / G + 1) * 32);
  const int n_ct = (M + kBKT - 1) / kBKT;
  const int n_tiles = n_ct + (n_chunk_keys + kBKT - 1) / kBKT;

  // the wave's queries and output gradients (B operands, lane = query)
  const size_t row_off = (static_cast<size_t>(b * Hq + hq) * S + (qok ? qi : 0)) * D;
  bf16x8 qf[DS], dof[DS];
  float dsum = 0.f;
#pragma unroll
  for (int st = 0; st < DS; ++st) {
    const bf16x8 q = load_bf16x8(Q + row_off + 16 * st + 8 * hf);
    const bf16x8 go = load_bf16x8(dO + row_off + 16 * st + 8 * hf);
    const bf16x8 o = load_bf16x8(Oo + row_off + 16 * st + 8 * hf);
    qf[st] = qok ? q : bf16x8{};
    dof[st] = qok ? go : bf16x8{};
#pragma unroll
    for (int e = 0; e < 8; ++e) dsum = fmaf(static_cast<float>(go[e]), static_cast<float>(o[e]), dsum);
  }
  dsum += xor32(dsum);
  // D_i for dS here is dO_i . O_i with the stored (bf16) output, as it must be
  // known before the keys are walked; the exact D_i = sum_j P_ij dP_ij is
  // accumulated along the walk and written for the dK/dV kernel, where the
  // output's rounding would otherwise be amplified wherever dP - D cancels
  const float Di = qok ? dsum : 0.f;
  float dex[4] = {0.f, 0.f, 0.f, 0.f};
  const float lse2 = qok ? lse[static_cast<size_t>(b * Hq + hq) * S + qi] * kLog2e : __builtin_huge_valf();

  f32x16 acc[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) acc[db] = zero16();

  const bf16_t* kc_head = Kc + static_cast<size_t>(bh) * M * D;
  const bf16_t* vc_head = Vc + static_cast<size_t>(bh) * M * D;
  const bf16_t* kn_head = Kn + static_cast<size_t>(bh) * S * D;
  const bf16_t* vn_head = Vn + static_cast<size_t>(bh) * S * D;
  const int32_t* pos_head = pos + static_cast<size_t>(bh) * M;
  const int tr_j = lane & 15, tr_r = tr_j >> 2, tr_q = tr_j & 3, tr_dg = (lane >> 4) & 1;

  const __amdgpu_buffer_rsrc_t rkc = make_rsrc(kc_head, static_cast<uint32_t>(M) * RB);
  const __amdgpu_buffer_rsrc_t rvc = make_rsrc(vc_head, static_cast<uint32_t>(M) * RB);
  const __amdgpu_buffer_rsrc_t rkn = make_rsrc(kn_head, static_cast<uint32_t>(S) * RB);
  const __amdgpu_buffer_rsrc_t rvn = make_rsrc(vn_head, static_cast<uint32_t>(S) * RB);
  // Tile rows sit in MFMA-row order (LDS row R holds key (R & ~31) | key_of_bkrow(R & 31)),
  // chunks swizzled.  Copy lanes: slot s = R*CPR + physical chunk receives the
  // logical chunk the swizzle puts there; keys past the end read as zeros.
  uint32_t cp_off[NCH];
#pragma unroll
  for (int c = 0; c < NCH; ++c) {
    const int sl = c * 512 + wave * 64 + lane, R = sl / CPR;
    const int key = (R & ~31) | key_of_bkrow(R & 31);
    cp_off[c] = key * RB + 16 * bchunk<CPR>(R, sl % CPR);
  }
  // Lane byte offsets (a constant change of the chunk is an XOR of the offset):
  //   a_row: row col, chunk hf (chunk 2st+hf: ^ 32st; rows +32kb: + 32kb*RB)
  //   a_tr : transpose read of rows 4hf+tr_r, element 16 tr_dg + 4 tr_q
  //          (+32 db: ^ 64db; rows +16u+32kb: + that*RB; rows +8: ^ 32, + 8*RB)
  const uint32_t a_row = col * RB + 16 * bchunk<CPR>(col, hf);
  const int trow = 4 * hf + tr_r;
  const uint32_t a_tr = trow * RB + 16 * bchunk<CPR>(trow, 2 * tr_dg + (tr_q >> 1)) + 8 * (tr_q & 1);

  int f_pos = 0;
  auto fetch = [&](int t, auto bfc) __attribute__((always_inline)) {
    constexpr int bf = decltype(bfc)::value;
    const bool is_cache = t < n_ct;
    const int base = is_cache ? t * kBKT : (t - n_ct) * kBKT;
    const uint32_t soff = static_cast<uint32_t>(base) * RB;
    char* kd = (bf ? k_b1 : k_b0) + wave * 1024;
    char* vd = (bf ? v_b1 : v_b0) + wave * 1024;
#pragma unroll
    for (int c = 0; c < NCH; ++c) {
      dma16(is_cache ? rkc : rkn, kd + c * 8192, cp_off[c], soff);
      dma16(is_cache ? rvc : rvn, vd + c * 8192, cp_off[c], soff);
    }
    if (wave == 0) f_pos = pos_head[is_cache ? min(base + lane, M - 1) : 0];
  };
  auto commit = [&](int t, auto bfc) __attribute__((always_inline)) {
    constexpr int bf = decltype(bfc)::value;
    const bool is_cache = t < n_ct;
    const int base = is_cache ? t * kBKT : (t - n_ct) * kBKT;
    const int lim = is_cache ? M : S;
    if (wave == 0) {
      const uint64_t m = __ballot(base + lane < lim && (!is_cache || f_pos >= 0));
      if (lane == 0) s_valid2[bf] = m;
    }
  };
  auto compute = [&](int t, auto bfc) __attribute__((always_inline)) {
    constexpr int bf = decltype(bfc)::value;
    const bool is_cache = t < n_ct;
    const int base = is_cache ? t * kBKT : (t - n_ct) * kBKT;
    if (!active || (!is_cache && base > qb * 32 + 31)) return;
    const char* ks = bf ? k_b1 : k_b0;
    const char* vs = bf ? v_b1 : v_b0;
    uint32_t ar = a_row, at = a_tr;
    asm volatile("" : "+v"(ar), "+v"(at));       // per-step offsets stay in the loop
    const uint64_t vm = s_valid2[bf];
    const bool causal = !is_cache && (base + kBKT - 1 > qb * 32);
    const int lim_i = causal ? qi - base - 16 * hf : 1 << 30;
    // one 32-key half at a time (keeps two accumulators live, not four)
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      // S^T and dP^T of keys 32kb..: register r of lane l <-> key 32kb + 16(l/32) + r
      f32x16 sh = zero16(), ph = zero16();
#pragma unroll
      for (int st = 0; st < DS; ++st) {
        const uint32_t o = (ar ^ (32 * st)) + 32 * kb * RB;
        const bf16x8 ka = *reinterpret_cast<const bf16x8*>(ks + o);
        const bf16x8 va = *reinterpret_cast<const bf16x8*>(vs + o);
        sh = mfma32x32x16(ka, qf[st], sh);
        ph = mfma32x32x16(va, dof[st], ph);
      }
      const uint32_t bits = static_cast<uint32_t>(vm >> (32 * kb + 16 * hf)) & 0xffffu;
      f32x8 d8[2];
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const bool ok = ((bits >> r) & 1u) && (32 * kb + r <= lim_i);
        // masked keys: pa = 0 against a finite dP (free-slot rows are finite,
        // rows past the end read as zeros), so both products are exactly 0
        const float pa = ok ? fast_exp2(fmaf(sh[r], c2, -lse2)) : 0.f;
        d8[r >> 3][r & 7] = pa * (ph[r] - Di);
        dex[r & 3] = fmaf(pa, ph[r], dex[r & 3]);
      }
      // dQ^T += K^T dS^T: MFMA u covers keys 32kb + 16(l/32) + 8u + e, which
      // sit in tile rows 32kb + 16u + 4(l/32) + {0..3} and those + 8
      const uint32_t at1 = at ^ 32;
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const bf16x8 ds = to_bf16x8(d8[u]);
#pragma unroll
        for (int db = 0; db < DB; ++db) {
          const uint32_t o0 = (at ^ (64 * db)) + (32 * kb + 16 * u) * RB;
          const uint32_t o1 = (at1 ^ (64 * db)) + (32 * kb + 16 * u + 8) * RB;
          const bf16x4 h0 = lds_read_tr16(reinterpret_cast<const bf16_t*>(ks + o0));
          const bf16x4 h1 = lds_read_tr16(reinterpret_cast<const bf16_t*>(ks + o1));
          const bf16x8 a = __builtin_shufflevector(h0, h1, 0, 1, 2, 3, 4, 5, 6, 7);
          acc[db] = mfma32x32x16(a, ds, acc[db]);
        }
      }
    }
    if constexpr (D == 128) {
      // Issue order of a tile's LDS reads against its MFMAs: 4 reads first,
      // then 2 behind every S^T/dP^T MFMA pair and 2 behind every dQ MFMA,
      // so that fragments are requested ahead of use (the compiler's own
      // order waits for each one).  Measured at 128k context (G = 8,
      // 2048-token chunks, 8192 slots): the backward of a row of chunks
      // 128.9 -> 127.6 ms.
      __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);       // LDS reads
#pragma unroll
      for (int h = 0; h < 2; ++h) {
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);     // MFMAs
          __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
        }
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
          __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
        }
      }
    }
  };

  using I0 = std::integral_constant<int, 0>;
  using I1 = std::integral_constant<int, 1>;
  // a buffer is refilled one tile after it was read, behind that tile's barrier
  if (n_tiles > 0) fetch(0, I0{});
  int t = 0;
  auto step = [&](auto bfc) __attribute__((always_inline)) {
    using BN = std::integral_constant<int, decltype(bfc)::value ^ 1>;
    if (t >= n_tiles) return false;
    commit(t, bfc);
    wait_vmem_all();                   // this wave's copies of tile t have landed
    barrier_lds();                     // ... and every wave's
    if (t + 1 < n_tiles) fetch(t + 1, BN{});
    compute(t, bfc);
    ++t;
    return true;
  };
  while (step(I0{}) && step(I1{})) {
  }
  float dx = (dex[0] + dex[1]) + (dex[2] + dex[3]);
  dx += xor32(dx);
  if (qok && hf == 0) Dws[static_cast<size_t>(b * Hq + hq) * S + qi] = dx;
  if (!qok) return;
  bf16_t* out = dQ + row_off;
#pragma unroll
  for (int db = 0; db < DB; ++db) {
#pragma unroll
    for (int a = 0; a < 4; ++a) {
      f32x4 v = {acc[db][4 * a] * scale, acc[db][4 * a + 1] * scale, acc[db][4 * a + 2] * scale,
                 acc[db][4 * a + 3] * scale};
      *reinterpret_cast<bf16x4*>(out + db * 32 + 8 * a + 4 * hf) = to_bf16x4(v);
    }
  }
}

// ---------------------------------------------------------------- dK and dV
constexpr int kKeysPerWG = 128;     // 4 key groups x 32 keys
// A chunk-key tile only sees the queries at or after its first key, so its
// work shrinks along the chunk; each chunk tile's query rows are split into
// kPieces equal pieces, taken by separate workgroups that write fp32 partial
// dK/dV for a reduction kernel.  With the cache tiles whole, the workgroups
// then fill the CUs evenly instead of leaving a last, half-empty round.
constexpr int kPieces = 4;

// 8 waves: key group kg = wave % 4 owns 32 keys (lane = key column), row set
// rs = wave / 4 takes every other needed query row block; the two row sets
// fold their dK/dV at the end.  The workgroup's K and V rows sit in LDS and
// are read as the B operands of every block, so a wave holds only its dK/dV
// accumulators and the block in flight: two waves fit on each SIMD.
// ACC: the cache tiles add their (scaled) dK/dV into fp32 accumulators
// [B*Hkv][M][d] instead of writing bf16 rows; a free slot adds nothing.
template <int D, bool ACC>
__global__ __launch_bounds__(512, 1) void bwd_dkdv_kernel(
    const bf16_t* __restrict__ Q, const bf16_t* __restrict__ Kc, const bf16_t* __restrict__ Vc,
    const int32_t* __restrict__ pos, const bf16_t* __restrict__ Kn, const bf16_t* __restrict__ Vn,
    const bf16_t* __restrict__ dO, const float* __restrict__ lse, const float* __restrict__ Dws,
    void* __restrict__ dKc, void* __restrict__ dVc, float* __restrict__ part, int Hq,
    int Hkv, int S, int M, float c2, float scale, int n_heads, int n_ct, int n_cht) {
  constexpr int DS = D / 16, DB = D / 32, CPR = D / 8;
  constexpr int RB = 2 * D;                        // bytes per row
  constexpr int TB = 32 * RB;                      // bytes per 32-row block
  constexpr int NCH = 32 * CPR / 256;              // 16-byte copies per thread of a row set per block
  constexpr int NKV = kKeysPerWG * CPR / 512;      // chunks per thread of the key rows
  // LDS: Q and dO blocks of the two row sets in two buffers -- the next block
  // is copied in while the current one is computed; one array per buffer, so
  // the compiler sees that reads of one do not wait for copies into the
  // other --, the workgroup's K and V rows, and the per-row scalars
  // [buffer][row set][32]
  __shared__ __attribute__((aligned(16))) char q_b0[2 * TB], q_b1[2 * TB], g_b0[2 * TB], g_b1[2 * TB];
  __shared__ __attribute__((aligned(16))) char kv_rows[2 * kKeysPerWG * RB];
  __shared__ __attribute__((aligned(16))) float s_lse2[2][64], s_D[2][64];
  __shared__ __attribute__((aligned(16))) int s_irow[2][64];
  constexpr int kV = kKeysPerWG * RB;              // V rows after the K rows

  const int tid = threadIdx.x, lane = tid & 63, hf = lane >> 5, col = lane & 31;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int kg = wave & 3, rs = wave >> 2;
  const int ltid = tid & 255;                      // thread index within the row set
  const int bh = blockIdx.x % n_heads;
  const int tix = static_cast<int>(blockIdx.x) / n_heads;     // cache tiles, then (chunk tile, piece)
  const int b = bh / Hkv, kvh = bh - b * Hkv;
  const int G = Hq / Hkv;
  const bool is_cache = tix < n_ct;
  const int cti = is_cache ? 0 : (tix - n_ct) / kPieces;
  const int piece = is_cache ? 0 : tix - n_ct - cti * kPieces;
  const int base = (is_cache ? tix : cti) * kKeysPerWG;
  const int lim = is_cache ? M : S;
  const int key = base + kg * 32 + col;            // this lane's key column
  const bf16_t* kh = is_cache ? Kc + static_cast<size_t>(bh) * M * D : Kn + static_cast<size_t>(bh) * S * D;
  const bf16_t* vh = is_cache ? Vc + static_cast<size_t>(bh) * M * D : Vn + static_cast<size_t>(bh) * S * D;
  const int pv = pos[static_cast<size_t>(bh) * M + (is_cache ? min(key, M - 1) : 0)];
  const bool key_ok = key < lim && (!is_cache || pv >= 0);
  const bool has_keys = base + kg * 32 < lim;      // some key of this wave exists

  // the workgroup's K and V rows (row r = key base + r; rows past the end
  // repeat the last row and get zero weight)
#pragma unroll
  for (int c = 0; c < NKV; ++c) {
    const int idx = c * 512 + tid, row = idx / CPR, ch = idx % CPR;
    const size_t src = static_cast<size_t>(min(base + row, lim - 1)) * D + ch * 8;
    const int o = row * RB + 16 * bchunk<CPR>(row, ch);
    store_u32x4(kv_rows + o, load_u32x4(kh + src));
    store_u32x4(kv_rows + kV + o, load_u32x4(vh + src));
  }
  f32x16 dk[DB], dv[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) {
    dk[db] = zero16();
    dv[db] = zero16();
  }

  const int n_rows = G * S;
  // rows [r_lo, r_hi) of the group are this workgroup's: all of them for a
  // cache tile; for a chunk tile, piece p of the needed rows (g, i >= base)
  // numbered o = g*(S - base) + i - base, o in [p*N/P, (p+1)*N/P)
  int r_lo = 0, r_hi = n_rows;
  if (!is_cache) {
    const int L = S - base, N = G * L;
    const int o_lo = piece * N / kPieces, o_hi = (piece + 1) * N / kPieces;
    r_lo = o_lo < N ? (o_lo / L) * S + base + o_lo % L : n_rows;
    r_hi = o_hi < N ? (o_hi / L) * S + base + o_hi % L : n_rows;
  }
  const bf16_t* qhead = Q + static_cast<size_t>(b * Hq + kvh * G) * S * D;   // rows g*S + i
  const bf16_t* ghead = dO + static_cast<size_t>(b * Hq + kvh * G) * S * D;
  const float* lhead = lse + static_cast<size_t>(b * Hq + kvh * G) * S;
  const float* dhead = Dws + static_cast<size_t>(b * Hq + kvh * G) * S;
  // rows past the group's end read as zeros (and get lse = +inf below)
  const __amdgpu_buffer_rsrc_t rq = make_rsrc(qhead, static_cast<uint32_t>(n_rows) * RB);
  const __amdgpu_buffer_rsrc_t rg = make_rsrc(ghead, static_cast<uint32_t>(n_rows) * RB);
  const int tr_j = lane & 15, tr_r = tr_j >> 2, tr_q = tr_j & 3, tr_dg = (lane >> 4) & 1;
  const int krow = kg * 32 + col;                  // LDS row of this lane's key

  // Lane byte offsets into a block or the key rows.  Swizzled chunk c of row
  // r sits at r*RB + 16*(c ^ mask(r)); a constant change of c is then an XOR
  // of the offset, so each read below costs one v_xor from these bases.
  //   a_row: row col, chunk hf (chunk 2st+hf = a_row ^ 32st)
  //   a_key: K row krow, chunk hf
  //   a_tr : transpose read of rows 4hf+tr_r, element 16 tr_dg + 4 tr_q
  //          (+32 db: ^ 64db; rows +16u: + 16u*RB; rows +8: ^ 32, + 8*RB)
  const uint32_t a_row = col * RB + 16 * bchunk<CPR>(col, hf);
  const uint32_t a_key = krow * RB + 16 * bchunk<CPR>(krow, hf);
  const int trow = 4 * hf + tr_r;
  const uint32_t a_tr = trow * RB + 16 * bchunk<CPR>(trow, 2 * tr_dg + (tr_q >> 1)) + 8 * (tr_q & 1);
  // copy lanes: slot s = row*CPR + physical chunk of a block receives the
  // logical chunk that the swizzle puts there
  const int wl = wave & 3;                         // wave within the row set
  uint32_t cp_off[NCH];
#pragma unroll
  for (int c = 0; c < NCH; ++c) {
    const int sl = c * 256 + wl * 64 + lane, row = sl / CPR;
    cp_off[c] = row * RB + 16 * bchunk<CPR>(row, sl % CPR);
  }

  // chunk keys only see queries i >= key: blocks whose queries all precede
  // the tile are skipped; next_block(r0) is the first block after r0 to do
  auto skipped = [&](int r0) __attribute__((always_inline)) {
    const int r1 = min(r0 + 31, n_rows - 1);
    return !is_cache && r0 / S == r1 / S && (r1 % S) < base;
  };
  auto next_block = [&](int r0) __attribute__((always_inline)) {
    r0 += 32;
    while (r0 < r_hi && skipped(r0)) r0 += 32;
    return r0;
  };
  float f_l = 0.f, f_d = 0.f;
  // block r0 of this row set -> buffer bf (copies land in LDS asynchronously)
  auto fetch = [&](int r0, auto bfc) __attribute__((always_inline)) {
    constexpr int bf = decltype(bfc)::value;
    const uint32_t soff = static_cast<uint32_t>(r0) * RB;
    char* qd = (bf ? q_b1 : q_b0) + rs * TB + wl * 1024;
    char* gd = (bf ? g_b1 : g_b0) + rs * TB + wl * 1024;
#pragma unroll
    for (int c = 0; c < NCH; ++c) {
      dma16(rq, qd + c * 4096, cp_off[c], soff);
      dma16(rg, gd + c * 4096, cp_off[c], soff);
    }
    if (ltid < 32) {
      const int rc = min(r0 + ltid, n_rows - 1);
      f_l = lhead[rc];
      f_d = dhead[rc];
    }
  };
  auto commit = [&](int r0, auto bfc) __attribute__((always_inline)) {
    constexpr int bf = decltype(bfc)::value;
    if (ltid < 32) {
      const int r = r0 + ltid, o = rs * 32 + ltid;
      const bool mine = r >= r_lo && r < r_hi;
      s_lse2[bf][o] = mine ? f_l * kLog2e : __builtin_huge_valf();
      s_D[bf][o] = mine ? f_d : 0.f;
      s_irow[bf][o] = mine ? r % S : -1;
    }
  };
  // chunk tiles: key k sees query i only if k <= i (rows past the group's end
  // carry i = -1 and lse = +inf).  Cache tiles need no mask per element: a
  // key's dK/dV columns depend on no other key, so a lane whose slot is empty
  // just stores zeros at the end (its K/V rows are finite).
  const int key_thr = key_ok ? key : 0x7fffffff;
  auto compute = [&](auto bfc, auto causal_c) __attribute__((always_inline)) {
    constexpr int bf = decltype(bfc)::value;
    constexpr bool causal = decltype(causal_c)::value;
    const char* qs = bf ? q_b1 : q_b0;
    const char* gs = bf ? g_b1 : g_b0;
    const uint32_t blk = rs * TB;
    uint32_t ak = a_key;
    asm volatile("" : "+v"(ak));                   // per-step offsets stay in the loop
    const uint32_t aq = a_row + blk;
    // S and dP (queries x keys): register r of lane l <-> row 8(r/4) + 4(l/32) + r%4
    f32x16 s = zero16(), p = zero16();
#pragma unroll
    for (int st = 0; st < DS; ++st) {
      const uint32_t oq = aq ^ (32 * st), ok = ak ^ (32 * st);
      const bf16x8 qa = *reinterpret_cast<const bf16x8*>(qs + oq);
      const bf16x8 ga = *reinterpret_cast<const bf16x8*>(gs + oq);
      const bf16x8 kb = *reinterpret_cast<const bf16x8*>(kv_rows + ok);
      const bf16x8 vb = *reinterpret_cast<const bf16x8*>(kv_rows + kV + ok);
      s = mfma32x32x16(qa, kb, s);
      p = mfma32x32x16(ga, vb, p);
    }
    f32x8 pp[2], dd[2];
#pragma unroll
    for (int a4 = 0; a4 < 4; ++a4) {
      const int row0 = rs * 32 + 8 * a4 + 4 * hf;
      const f32x4 l2 = *reinterpret_cast<const f32x4*>(&s_lse2[bf][row0]);
      const f32x4 dv4 = *reinterpret_cast<const f32x4*>(&s_D[bf][row0]);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int r = 4 * a4 + e;
        const float pe = fast_exp2(fmaf(s[r], c2, -l2[e]));
        if constexpr (causal) {
          const int4 iv = *reinterpret_cast<const int4*>(&s_irow[bf][row0]);
          const int qi = e == 0 ? iv.x : e == 1 ? iv.y : e == 2 ? iv.z : iv.w;
          const bool ok = key_thr <= qi;
          const float pr = ok ? pe : 0.f;
          pp[r >> 3][r & 7] = pr;
          dd[r >> 3][r & 7] = ok ? pr * (p[r] - dv4[e]) : 0.f;
        } else {
          pp[r >> 3][r & 7] = pe;
          dd[r >> 3][r & 7] = pe * (p[r] - dv4[e]);
        }
      }
    }
    // dV^T += dO^T P and dK^T += Q^T dS: MFMA u contracts over the rows held
    // in registers 8u..8u+7, i.e. rows 16u + 4(l/32) + {0..3, 8..11}
    const uint32_t at0 = a_tr + blk, at1 = at0 ^ 32;
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const bf16x8 pb = to_bf16x8(pp[u]);
      const bf16x8 db8 = to_bf16x8(dd[u]);
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        const uint32_t o0 = (at0 ^ (64 * db)) + 16 * u * RB;
        const uint32_t o1 = (at1 ^ (64 * db)) + (16 * u + 8) * RB;
        const bf16x4 g0 = lds_read_tr16(reinterpret_cast<const bf16_t*>(gs + o0));
        const bf16x4 g1 = lds_read_tr16(reinterpret_cast<const bf16_t*>(gs + o1));
        const bf16x4 q0 = lds_read_tr16(reinterpret_cast<const bf16_t*>(qs + o0));
        const bf16x4 q1 = lds_read_tr16(reinterpret_cast<const bf16_t*>(qs + o1));
        dv[db] = mfma32x32x16(__builtin_shufflevector(g0, g1, 0, 1, 2, 3, 4, 5, 6, 7), pb, dv[db]);
        dk[db] = mfma32x32x16(__builtin_shufflevector(q0, q1, 0, 1, 2, 3, 4, 5, 6, 7), db8, dk[db]);
      }
    }
  };

  // The needed blocks in order are split alternately: row set 0 takes the
  // 1st, 3rd, ..., row set 1 the 2nd, 4th, ... (ra, rb: the two sets'
  // current blocks, tracked by every wave).  A buffer is refilled one
  // iteration after it was read, behind that iteration's barrier.
  using I0 = std::integral_constant<int, 0>;
  using I1 = std::integral_constant<int, 1>;
  const int r_first = r_lo & ~31;
  int ra = r_lo >= r_hi ? r_hi : skipped(r_first) ? next_block(r_first) : r_first;
  int rb = ra < r_hi ? next_block(ra) : r_hi;
  int r0 = rs ? rb : ra;
  if (r0 < r_hi) fetch(r0, I0{});
  // one iteration on buffer bf; false once every block is done
  auto step = [&](auto bfc, auto causal_c) __attribute__((always_inline)) {
    using BN = std::integral_constant<int, decltype(bfc)::value ^ 1>;
    if (ra >= r_hi) return false;
    if (r0 < r_hi) commit(r0, bfc);
    wait_vmem_all();                   // this wave's copies of the block have landed
    barrier_lds();                     // ... and every wave's; also orders the key rows' stores
    const int na = rb < r_hi ? next_block(rb) : r_hi;
    const int nb = na < r_hi ? next_block(na) : r_hi;
    const int rn = rs ? nb : na;
    if (rn < r_hi) fetch(rn, BN{});
    if (r0 < r_hi && has_keys) compute(bfc, causal_c);
    ra = na;
    rb = nb;
    r0 = rn;
    return true;
  };
  if (is_cache) {
    while (step(I0{}, std::false_type{}) && step(I1{}, std::false_type{})) {
    }
  } else {
    while (step(I0{}, std::true_type{}) && step(I1{}, std::true_type{})) {
    }
  }

  // fold row set 1's dK, dV into row set 0's, one 32-row block of the
  // accumulators per round through the query buffers
  __syncthreads();
  float* xo = reinterpret_cast<float*>(kv_rows);     // 16 x 256 floats per round
  const int xs = kg * 64 + lane;
#pragma unroll
  for (int h = 0; h < 2; ++h) {
#pragma unroll
    for (int db = 0; db < DB; ++db) {
      f32x16& acc = h ? dv[db] : dk[db];
      if (rs == 1) {
#pragma unroll
        for (int r = 0; r < 16; ++r) xo[r * 256 + xs] = acc[r];
      }
      __syncthreads();
      if (rs == 0) {
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[r] += xo[r * 256 + xs];
      }
      __syncthreads();
    }
  }
  if (rs == 1 || key >= lim) return;
  if (ACC && is_cache && !key_ok) return;          // a free slot's accumulator is left as it is
  if (!key_ok) {
#pragma unroll
    for (int db = 0; db < DB; ++db) {
      dk[db] = zero16();
      dv[db] = zero16();
    }
  }
  // accumulator register r of lane l: d = 32 db + 8(r/4) + 4(l/32) + r%4, key column l%32
  if (ACC && is_cache) {
    // each slot belongs to one workgroup: a plain read-modify-write
    float* ko = static_cast<float*>(dKc) + (static_cast<size_t>(bh) * M + key) * D;
    float* vo = static_cast<float*>(dVc) + (static_cast<size_t>(bh) * M + key) * D;
#pragma unroll
    for (int db = 0; db < DB; ++db) {
#pragma unroll
      for (int a = 0; a < 4; ++a) {
        f32x4* kp = reinterpret_cast<f32x4*>(ko + db * 32 + 8 * a + 4 * hf);
        f32x4* vp = reinterpret_cast<f32x4*>(vo + db * 32 + 8 * a + 4 * hf);
        const f32x4 kold = *kp, vold = *vp;
        *kp = kold + f32x4{dk[db][4 * a] * scale, dk[db][4 * a + 1] * scale, dk[db][4 * a + 2] * scale,
                           dk[db][4 * a + 3] * scale};
        *vp = vold + f32x4{dv[db][4 * a], dv[db][4 * a + 1], dv[db][4 * a + 2], dv[db][4 * a + 3]};
      }
    }
  } else if (is_cache) {
    bf16_t* ko = static_cast<bf16_t*>(dKc) + (static_cast<size_t>(bh) * M + key) * D;
    bf16_t* vo = static_cast<bf16_t*>(dVc) + (static_cast<size_t>(bh) * M + key) * D;
#pragma unroll
    for (int db = 0; db < DB; ++db) {
#pragma unroll
      for (int a = 0; a < 4; ++a) {
        f32x4 kv = {dk[db][4 * a] * scale, dk[db][4 * a + 1] * scale, dk[db][4 * a + 2] * scale,
                    dk[db][4 * a + 3] * scale};
        f32x4 vv = {dv[db][4 * a], dv[db][4 * a + 1], dv[db][4 * a + 2], dv[db][4 * a + 3]};
        *reinterpret_cast<bf16x4*>(ko + db * 32 + 8 * a + 4 * hf) = to_bf16x4(kv);
        *reinterpret_cast<bf16x4*>(vo + db * 32 + 8 * a + 4 * hf) = to_bf16x4(vv);
      }
    }
  } else {
    // partials [dK | dV][piece][head][key < n_cht * 128][d], unscaled
    const size_t s_pad = static_cast<size_t>(n_cht) * kKeysPerWG;
    float* ko = part + ((static_cast<size_t>(piece) * n_heads + bh) * s_pad + key) * D;
    float* vo = ko + static_cast<size_t>(kPieces) * n_heads * s_pad * D;
#pragma unroll
    for (int db = 0; db < DB; ++db) {
#pragma unroll
      for (int a = 0; a < 4; ++a) {
        f32x4 kv = {dk[db][4 * a], dk[db][4 * a + 1], dk[db][4 * a + 2], dk[db][4 * a + 3]};
        f32x4 vv = {dv[db][4 * a], dv[db][4 * a + 1], dv[db][4 * a + 2], dv[db][4 * a + 3]};
        *reinterpret_cast<f32x4*>(ko + db * 32 + 8 * a + 4 * hf) = kv;
        *reinterpret_cast<f32x4*>(vo + db * 32 + 8 * a + 4 * hf) = vv;
      }
    }
  }
}

// dK/dV of the chunk keys: sum of the kPieces partials in piece order
// (deterministic), dK scaled, written in bf16 -- or, with ACC, added to the
// fp32 rows already in dKn/dVn.  One thread per 4 elements.
template <int D, bool ACC>
__global__ __launch_bounds__(256) void bwd_chunk_reduce_kernel(const float* __restrict__ part,
                                                               void* __restrict__ dKn,
                                                               void* __restrict__ dVn, int S,
                                                               int n_heads, int n_cht, float scale) {
  constexpr int C4 = D / 4;
  const int64_t idx = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  if (idx >= static_cast<int64_t>(n_heads) * S * C4) return;
  const int c4 = static_cast<int>(idx % C4);
  const int64_t kr = idx / C4;                     // bh * S + key
  const int key = static_cast<int>(kr % S), bh = static_cast<int>(kr / S);
  const size_t s_pad = static_cast<size_t>(n_cht) * kKeysPerWG;
  const size_t ps = static_cast<size_t>(n_heads) * s_pad * D;      // one piece
  const float* src = part + (static_cast<size_t>(bh) * s_pad + key) * D + 4 * c4;
  f32x4 sk = *reinterpret_cast<const f32x4*>(src);
  f32x4 sv = *reinterpret_cast<const f32x4*>(src + kPieces * ps);
#pragma unroll
  for (int p = 1; p < kPieces; ++p) {
    sk += *reinterpret_cast<const f32x4*>(src + p * ps);
    sv += *reinterpret_cast<const f32x4*>(src + kPieces * ps + p * ps);
  }
  if constexpr (ACC) {
    f32x4* kp = reinterpret_cast<f32x4*>(static_cast<float*>(dKn) + kr * D + 4 * c4);
    f32x4* vp = reinterpret_cast<f32x4*>(static_cast<float*>(dVn) + kr * D + 4 * c4);
    *kp = *kp + sk * scale;
    *vp = *vp + sv;
  } else {
    *reinterpret_cast<bf16x4*>(static_cast<bf16_t*>(dKn) + kr * D + 4 * c4) = to_bf16x4(sk * scale);
    *reinterpret_cast<bf16x4*>(static_cast<bf16_t*>(dVn) + kr * D + 4 * c4) = to_bf16x4(sv);
  }
}

}  // namespace

// D_i per query row, then the chunk tiles' partial dK/dV
static size_t backward_d_bytes(int B, int Hq, int S) {
  return (static_cast<size_t>(B) * Hq * S * sizeof(float) + 255) & ~static_cast<size_t>(255);
}
size_t backward_workspace_bytes(int B, int Hq, int Hkv, int S, int D) {
  const size_t n_cht = (static_cast<size_t>(S) + kKeysPerWG - 1) / kKeysPerWG;
  return backward_d_bytes(B, Hq, S) +
         2 * static_cast<size_t>(kPieces) * B * Hkv * n_cht * kKeysPerWG * D * sizeof(float);
}

hipError_t launch_backward(const StepShape& sh, const BackwardArgs& a, hipStream_t st) {
  const int n_heads = sh.B * sh.Hkv;
  const int G = sh.Hq / sh.Hkv;
  const float c2 = sh.scale * kLog2e;
  const int n_rb = G * ((sh.S + 31) / 32);
  const int wgp = (n_rb + kBWaves - 1) / kBWaves;
  float* Dws = static_cast<float*>(a.workspace);
  float* part = reinterpret_cast<float*>(static_cast<char*>(a.workspace) + backward_d_bytes(sh.B, sh.Hq, sh.S));
#define H2O_LAUNCH_DQ(DD)                                                                              \
  hipLaunchKernelGGL(bwd_dq_kernel<DD>, dim3(n_heads * wgp), dim3(512), 0, st,                         \
                     static_cast<const bf16_t*>(a.q), static_cast<const bf16_t*>(a.k_cache),          \
                     static_cast<const bf16_t*>(a.v_cache), a.pos, static_cast<const bf16_t*>(a.k_new), \
                     static_cast<const bf16_t*>(a.v_new), static_cast<const bf16_t*>(a.out),          \
                     static_cast<const bf16_t*>(a.d_out), a.lse, Dws, static_cast<bf16_t*>(a.dq),     \
                     sh.Hq, sh.Hkv, sh.S, sh.M, c2, sh.scale, n_heads, wgp)
  if (sh.D == 128) H2O_LAUNCH_DQ(128);
  else H2O_LAUNCH_DQ(64);
#undef H2O_LAUNCH_DQ
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int n_ct = (sh.M + kKeysPerWG - 1) / kKeysPerWG;
  const int n_cht = (sh.S + kKeysPerWG - 1) / kKeysPerWG;
#define H2O_LAUNCH_DKDV(DD, AC)                                                                        \
  hipLaunchKernelGGL(HIP_KERNEL_NAME(bwd_dkdv_kernel<DD, AC>), dim3(n_heads * (n_ct + n_cht * kPieces)),  \
                     dim3(512), 0, st, static_cast<const bf16_t*>(a.q),                                \
                     static_cast<const bf16_t*>(a.k_cache), static_cast<const bf16_t*>(a.v_cache), a.pos, \
                     static_cast<const bf16_t*>(a.k_new), static_cast<const bf16_t*>(a.v_new),         \
                     static_cast<const bf16_t*>(a.d_out), a.lse, Dws, a.dk_cache, a.dv_cache, part,    \
                     sh.Hq, sh.Hkv, sh.S, sh.M, c2, sh.scale, n_heads, n_ct, n_cht)
  if (sh.D == 128) {
    if (a.accumulate) H2O_LAUNCH_DKDV(128, true);
    else H2O_LAUNCH_DKDV(128, false);
  } else {
    if (a.accumulate) H2O_LAUNCH_DKDV(64, true);
    else H2O_LAUNCH_DKDV(64, false);
  }
#undef H2O_LAUNCH_DKDV
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int64_t n_red = static_cast<int64_t>(n_heads) * sh.S * (sh.D / 4);
  const unsigned red_blocks = static_cast<unsigned>((n_red + 255) / 256);
#define H2O_LAUNCH_RED(DD, AC)                                                                           \
  hipLaunchKernelGGL(HIP_KERNEL_NAME(bwd_chunk_reduce_kernel<DD, AC>), dim3(red_blocks), dim3(256), 0, st, \
                     part, a.dk_new, a.dv_new, sh.S, n_heads, n_cht, sh.scale)
  if (sh.D == 128) {
    if (a.accumulate) H2O_LAUNCH_RED(128, true);
    else H2O_LAUNCH_RED(128, false);
  } else {
    if (a.accumulate) H2O_LAUNCH_RED(64, true);
    else H2O_LAUNCH_RED(64, false);
  }
#undef H2O_LAUNCH_RED
  return hipGetLastError();
}

}  // namespace h2o
