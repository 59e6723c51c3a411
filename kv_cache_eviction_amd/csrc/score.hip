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
// as the B operand held in registers for the whole kernel and 64-row query
// blocks as the A operand, staged in a double-buffered LDS ring shared by
// the 4 waves and prefetched two blocks ahead through registers.  Each
// accumulator column belongs to one key, so the column sum is one fp32 add
// per element inside the lane plus one exchange with lane l^32 at the end.
#include "h2o_device.h"
#include "h2o_launch.h"

namespace h2o {
namespace {

constexpr int kCT = 256;        // key columns per workgroup (4 waves x 64)
constexpr int kRB = 64;         // query rows per staged block (2 MFMA row blocks)
constexpr int kRowSplitsMax = 16;

template <int D>
__global__ __launch_bounds__(256, 2) void score_bf16_kernel(
    const bf16_t* __restrict__ Q, const bf16_t* __restrict__ Kc,
    const bf16_t* __restrict__ Kn, const float* __restrict__ lse,
    float* __restrict__ partial, int Hq, int Hkv, int S, int M, int n_cache, float c2,
    int n_heads, int n_ct, int n_tiles, int R) {
  constexpr int DS = D / 16;
  constexpr int QLD = D + 8;
  constexpr int CPR = D / 8;
  constexpr int NCH = kRB * CPR / 256;  // 16-byte chunks per thread per row block
  __shared__ __attribute__((aligned(16))) bf16_t Qs[2][kRB * QLD];
  __shared__ __attribute__((aligned(16))) float s_lse2[2][kRB];
  __shared__ __attribute__((aligned(16))) int s_irow[2][kRB];

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int hf = lane >> 5, col = lane & 31;
  const int bh = blockIdx.x % n_heads;
  const int rest = static_cast<int>(blockIdx.x) / n_heads;
  const int tile = rest % n_tiles, split = rest / n_tiles;
  const int b = bh / Hkv, kvh = bh - b * Hkv;
  const int G = Hq / Hkv;
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

  const int n_rows = G * S;
  const int n_blk = (n_rows + kRB - 1) / kRB;
  const int blk_lo = static_cast<int>(static_cast<int64_t>(split) * n_blk / R);
  const int blk_hi = static_cast<int>(static_cast<int64_t>(split + 1) * n_blk / R);
  const bf16_t* qhead = Q + static_cast<size_t>(b * Hq + kvh * G) * S * D;  // rows g*S + i
  const float* lhead = lse + static_cast<size_t>(b * Hq + kvh * G) * S;

  // A row block contributes to chunk keys only if one of its queries i >= base.
  auto block_needed = [&](int blk) __attribute__((always_inline)) {
    if (is_cache) return true;
    const int r0 = blk * kRB, r1 = min(r0 + kRB - 1, n_rows - 1);
    if (r0 / S != r1 / S) return true;
    return (r1 % S) >= base;
  };
  auto next_needed = [&](int blk) __attribute__((always_inline)) {
    ++blk;
    while (blk < blk_hi && !block_needed(blk)) ++blk;
    return blk;
  };

  struct Stage {
    u32x4 q[NCH];
    float l;
    int i;
  };
  auto load_blk = [&](int blk, Stage& s) __attribute__((always_inline)) {
    const int r0 = blk * kRB;
#pragma unroll
    for (int c = 0; c < NCH; ++c) {
      const int idx = c * 256 + tid, row = idx / CPR, dc = idx % CPR;
      // rows past the end read the last row; their lse of +inf zeroes them
      const int r = min(r0 + row, n_rows - 1);
      s.q[c] = load_u32x4(qhead + static_cast<size_t>(r) * D + dc * 8);
    }
    if (tid < kRB) {
      const int r = r0 + tid;
      const float lv = lhead[min(r, n_rows - 1)];
      s.l = (r < n_rows) ? lv * kLog2e : __builtin_huge_valf();
      s.i = (r < n_rows) ? r % S : -1;
    }
  };
  auto store_blk = [&](const Stage& s, int buf) __attribute__((always_inline)) {
#pragma unroll
    for (int c = 0; c < NCH; ++c) {
      const int idx = c * 256 + tid, row = idx / CPR, dc = idx % CPR;
      store_u32x4(&Qs[buf][row * QLD + dc * 8], s.q[c]);
    }
    if (tid < kRB) {
      s_lse2[buf][tid] = s.l;
      s_irow[buf][tid] = s.i;
    }
  };

  float cs0 = 0.f, cs1 = 0.f;     // column sums of this lane's two key columns
  // Ping-pong register stages: while block `cur` is computed from LDS buffer
  // `buf`, one stage holds block n1 (stored to the other buffer after the
  // MFMAs) and the other block n2; each stage's loads get two blocks of
  // compute to land.
  Stage st0, st1;
  int cur = next_needed(blk_lo - 1);
  int n1 = cur < blk_hi ? next_needed(cur) : blk_hi;
  int n2 = n1 < blk_hi ? next_needed(n1) : blk_hi;
  if (cur < blk_hi) {
    load_blk(cur, st0);
    store_blk(st0, 0);
  }
  if (n1 < blk_hi) load_blk(n1, st0);
  if (n2 < blk_hi) load_blk(n2, st1);
  __syncthreads();
  int buf = 0;
  auto iter = [&](Stage& st) __attribute__((always_inline)) {
    if (key0 < lim) {
#pragma unroll
      for (int half = 0; half < 2; ++half) {
        f32x16 a0 = zero16(), a1 = zero16();
#pragma unroll
        for (int q = 0; q < DS; ++q) {
          const bf16x8 qa = *reinterpret_cast<const bf16x8*>(
              &Qs[buf][(half * 32 + col) * QLD + 16 * q + 8 * hf]);
          a0 = mfma32x32x16(qa, kf[0][q], a0);
          a1 = mfma32x32x16(qa, kf[1][q], a1);
        }
        // accumulator register r of lane l: query row 8(r/4) + 4hf + r%4 of this half block;
        // the 4 rows of each group of 4 registers are consecutive (one 16-byte LDS read)
#pragma unroll
        for (int a4 = 0; a4 < 4; ++a4) {
          const int row0 = half * 32 + 8 * a4 + 4 * hf;
          const f32x4 l2v = *reinterpret_cast<const f32x4*>(&s_lse2[buf][row0]);
          int4 qiv = {0, 0, 0, 0};
          if (!is_cache) qiv = *reinterpret_cast<const int4*>(&s_irow[buf][row0]);
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int r = 4 * a4 + e;
            float p0 = fast_exp2(fmaf(a0[r], c2, -l2v[e]));
            float p1 = fast_exp2(fmaf(a1[r], c2, -l2v[e]));
            if (!is_cache) {
              const int qi = e == 0 ? qiv.x : e == 1 ? qiv.y : e == 2 ? qiv.z : qiv.w;
              p0 = (key0 + col <= qi) ? p0 : 0.f;
              p1 = (key0 + 32 + col <= qi) ? p1 : 0.f;
            }
            cs0 += p0;
            cs1 += p1;
          }
        }
      }
    }
    if (n1 < blk_hi) store_blk(st, buf ^ 1);      // st holds block n1
    const int n3 = n2 < blk_hi ? next_needed(n2) : blk_hi;
    if (n3 < blk_hi) load_blk(n3, st);             // st now carries block n3
    __syncthreads();
    cur = n1;
    n1 = n2;
    n2 = n3;
    buf ^= 1;
  };
  while (cur < blk_hi) {
    iter(st0);
    if (cur >= blk_hi) break;
    iter(st1);
  }
  cs0 += xor32(cs0);
  cs1 += xor32(cs1);
  const size_t PS = static_cast<size_t>(M) + S;
  if (hf == 0) {
    float* out = partial + (static_cast<size_t>(bh) * R + split) * PS + (is_cache ? 0 : M);
    const int k0 = key0 + col, k1 = key0 + 32 + col;
    if (k0 < lim) out[k0] = cs0;
    if (k1 < lim) out[k1] = cs1;
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

int score_tiles(const StepShape& sh, int dtype) {
  const int ct = dtype == kBF16 ? kCT : 64;
  return (sh.n_cache + ct - 1) / ct + (sh.S + ct - 1) / ct;
}

int score_row_splits(const StepShape& sh, int dtype) {
  if (dtype != kBF16) return 1;
  const int n_heads = sh.B * sh.Hkv;
  const int n_tiles = score_tiles(sh, dtype);
  const int n_blk = (sh.Hq / sh.Hkv * sh.S + kRB - 1) / kRB;
  const int target = 512;   // two resident workgroups per CU
  int R = target / (n_heads * n_tiles);
  R = R < 1 ? 1 : R;
  R = R > kRowSplitsMax ? kRowSplitsMax : R;
  R = R > n_blk ? n_blk : R;
  return R;
}

hipError_t launch_score(const StepShape& sh, const ScoreArgs& a, int dtype, hipStream_t st) {
  const int n_heads = sh.B * sh.Hkv;
  const float c2 = sh.scale * kLog2e;
  if (dtype == kBF16) {
    const int n_ct = (sh.n_cache + kCT - 1) / kCT;
    const int n_tiles = n_ct + (sh.S + kCT - 1) / kCT;
    const dim3 grid(n_heads * n_tiles * a.R), block(256);
#define H2O_LAUNCH_SCORE(DD)                                                                      \
  hipLaunchKernelGGL(score_bf16_kernel<DD>, grid, block, 0, st, static_cast<const bf16_t*>(a.q), \
                     static_cast<const bf16_t*>(a.k_cache), static_cast<const bf16_t*>(a.k_new), \
                     a.lse, a.partial, sh.Hq, sh.Hkv, sh.S, sh.M, sh.n_cache, c2, n_heads, n_ct, \
                     n_tiles, a.R)
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
