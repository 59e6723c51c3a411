// Attention and H2O column masses of a short-chunk step in one pass over the
// keys (steps 1 and 2 of h2o_chunk_step when the G*S query rows of a KV
// group fit 16 parts of 32 rows and the head's keys fit the register stash).
//
// Method: "Learning how to Forget: Fine-tuning for Long-Context Sparse
// Attention" (arXiv 2608.19920) -- §1 ¶1 (fixed-size KV cache), §1 ¶3
// (grouped query attention), §1 ¶4 and the docshare FAQ answer on H2O (the
// summed attention weights served with the attention output).  The kernel
// design is this library's own, for CDNA4.
//
// A column mass sum_i P[i, j] needs every row's final logsumexp before any
// probability of the column is normalised.  The two-kernel path gets it by
// recomputing Q K^T after the attention, which reads the K cache a second
// time; in the decode regime, where the step streams the whole cache, that
// second read is a third of the step's traffic.  Here a workgroup owns one
// 32-row half of a KV group's rows and every key of the head, and keeps the
// half's scaled logits for all its keys in registers:
//   1. K pass: each wave walks its own 32-key blocks (every 8th block of the
//      head's cache-then-chunk block list) through a private two-slot LDS
//      ring, computes S^T = K Q^T on v_mfma_f32_32x32x16_bf16 (K rows in
//      MFMA A-operand row order, so accumulator register r of lane l holds
//      key 16(l/32) + r of the block and column l%32 is the lane's query
//      row), masks, and stashes the 16 logits of each block.
//      The exps are taken in this pass against the lane's running row
//      maximum (online-softmax style), so they overlap the block copies.
//   2. The rows' maximum and sum over all keys: with lane l^32, then across
//      the 8 waves through LDS; P = e 2^(m_block - m) / l exactly, in fp32.
//   3. Column masses of the half's rows: a reduce-scatter over each 16-lane
//      row (DPP pairings) and one exchange between the two rows of a lane
//      half leave key 16(l/32) + l%16's sum in lane l; written as row split
//      `half` of the masses.
//   4. V pass: O^T += V^T P^T from the same ring (V rows read with the
//      gfx950 transpose load), P as the B operand straight from registers.
//   5. The 8 waves' O^T partials are summed through LDS in wave order and
//      the rows written; lse as the natural log.
// All halves of a head are dispatched to one XCD (round-robin dispatch,
// ids 8 apart), so that their identical K/V streams share that XCD's L2
// fills.  Every block's copy goes through
// buffer_load ... lds with the row order and XOR swizzle applied on the
// source side; rows past the end of a block re-read its last valid row
// (masked), so masked probabilities always meet finite V.
#include <algorithm>
#include <type_traits>

#include "h2o_device.h"
#include "h2o_launch.h"

namespace h2o {
namespace {

constexpr int kDW = 8;          // waves per workgroup
constexpr int kDMaxHalves = 16; // 32-row parts of a KV group's rows (G*S <= 512)
constexpr int kDNB = 9;         // 32-key blocks per wave at most (2304 keys per head)
constexpr float kDNoMax = -1e30f;

// buffer_load_dword ... lds: lane i copies the 4 bytes at voff + soff of the
// resource to LDS address lds_base + 4 i (issued like dma16: untracked by the
// compiler, ordered by the kernel's own vmcnt waits and barriers).
__device__ __forceinline__ void dma4(__amdgpu_buffer_rsrc_t r, const void* lds_base, uint32_t voff, uint32_t soff) {
  const uint32_t m0 = static_cast<uint32_t>(reinterpret_cast<uintptr_t>(
      (__attribute__((address_space(3))) const void*)(lds_base)));
  asm volatile("buffer_load_dword %0, %1, %2 offen lds" ::"v"(voff), "s"(r), "s"(soff), "{m0}"(m0) : "memory");
}

// ALLF: every cache slot holds a token (known on the host once the cache has
// filled): no position copies, and only keys past the last slot are masked.
template <int D, bool ALLF>
__global__ __launch_bounds__(kDW * 64, 1) void decode_fused_kernel(
    const bf16_t* __restrict__ Q, const bf16_t* __restrict__ Kc, const bf16_t* __restrict__ Vc,
    const int32_t* __restrict__ pos, const bf16_t* __restrict__ Kn, const bf16_t* __restrict__ Vn,
    bf16_t* __restrict__ O, float* __restrict__ lse, float* __restrict__ partial, int Hq, int Hkv, int S,
    int M, int n_cache, float c2, int n_heads, int halves) {
  constexpr int DS = D / 16;            // MFMA k-steps over d
  constexpr int DB = D / 32;            // 32-row blocks of O^T
  constexpr int CPR = D / 8;            // 16-byte chunks per row
  constexpr int RB = 2 * D;             // bytes per K or V row
  constexpr int BB = 32 * RB;           // bytes per 32-key block
  constexpr int NC = BB / 1024;         // 1 KB copies per block
  constexpr int RPC = 1024 / RB;        // rows per copy
  __shared__ __attribute__((aligned(1024))) char ring[kDW][2][BB];
  __shared__ __attribute__((aligned(1024))) char qs[32 * RB];     // the half's query rows
  __shared__ int s_pos[kDW][2][64];                                 // positions of a cache block
  __shared__ float s_m[kDW][32];
  __shared__ float s_l[kDW][32];

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63, hf = lane >> 5, col = lane & 31;
  // workgroup -> (head, half).  With 8 | n_heads, head h's halves all run on
  // XCD h % 8 (dispatch is round-robin over the 8 XCDs), so that their
  // identical K/V streams share that XCD's L2 fills.
  int bh, half;
  if ((n_heads & 7) == 0) {
    const int w = blockIdx.x, x = w & 7, k = w >> 3;
    const int lh = k / halves;
    half = k - lh * halves;
    bh = 8 * lh + x;
  } else {
    bh = static_cast<int>(blockIdx.x) / halves;
    half = static_cast<int>(blockIdx.x) - bh * halves;
  }
  const int b = bh / Hkv, kvh = bh - b * Hkv;
  const int G = Hq / Hkv;
  const int n_rows = G * S;
  const int row = 32 * half + col;                 // this lane's query row (g * S + qi)
  const bool row_ok = row < n_rows;
  const int g = row_ok ? row / S : 0;
  const int qi = row_ok ? row - g * S : 0;
  const int hq = kvh * G + g;

  const int ncb = (n_cache + 31) >> 5;             // cache blocks, then chunk blocks
  const int nblk = ncb + ((S + 31) >> 5);
  const int nbw = nblk > wave ? (nblk - wave + kDW - 1) / kDW : 0;   // this wave's blocks (<= kDNB)

  const bf16_t* kc_head = Kc + static_cast<size_t>(bh) * M * D;
  const bf16_t* vc_head = Vc + static_cast<size_t>(bh) * M * D;
  const bf16_t* kn_head = Kn + static_cast<size_t>(bh) * S * D;
  const bf16_t* vn_head = Vn + static_cast<size_t>(bh) * S * D;
  const __amdgpu_buffer_rsrc_t rk_c = make_rsrc(kc_head, static_cast<uint32_t>(M) * RB);
  const __amdgpu_buffer_rsrc_t rv_c = make_rsrc(vc_head, static_cast<uint32_t>(M) * RB);
  const __amdgpu_buffer_rsrc_t rk_n = make_rsrc(kn_head, static_cast<uint32_t>(S) * RB);
  const __amdgpu_buffer_rsrc_t rv_n = make_rsrc(vn_head, static_cast<uint32_t>(S) * RB);
  const __amdgpu_buffer_rsrc_t r_pos = make_rsrc(pos + static_cast<size_t>(bh) * M, static_cast<uint32_t>(M) * 4);
  const __amdgpu_buffer_rsrc_t r_q = make_rsrc(Q + static_cast<size_t>(b * Hq + kvh * G) * S * D,
                                               static_cast<uint32_t>(n_rows) * RB);

  // ---- block copies (global -> LDS, no registers).  LDS byte 1024 j + 16 l
  // of a block holds row rho = RPC j + l / CPR, physical chunk l % CPR: for
  // K the key in MFMA A-operand row order (row 8q + 4h + r holds key
  // 16h + 4q + r) with chunk c ^ (rho % CPR), for V key rho with chunk
  // c ^ ((rho % 4) << (CPR == 16 ? 2 : 1)).  The source offset splits into a
  // per-lane part and a copy-uniform part (scalar offset); a block with fewer
  // than 32 valid rows recomputes the clamped per-lane offsets.
  uint32_t k_lane, v_lane;
  if constexpr (D == 128) {
    const int t = lane >> 4, pc = lane & 15;
    k_lane = 256 * t + 16 * (pc ^ t);
    v_lane = 256 * t + 16 * (pc ^ (4 * t));
  } else {
    const int t = lane >> 3, pc = lane & 7;
    k_lane = 128 * (16 * (t >> 2) + (t & 3)) + 16 * (pc ^ t);
    v_lane = 128 * t + 16 * (pc ^ ((t & 3) << 1));
  }
  auto k_key = [](int rho) { return 16 * ((rho >> 2) & 1) + 4 * (rho >> 3) + (rho & 3); };
  auto issue_k = [&](int i, int slot) __attribute__((always_inline)) {
    const int bi = wave + kDW * i;
    const bool is_cache = bi < ncb;
    const int base = is_cache ? 32 * bi : 32 * (bi - ncb);
    const int n_valid = (is_cache ? n_cache : S) - base;
    const __amdgpu_buffer_rsrc_t r = is_cache ? rk_c : rk_n;
    const char* dst = ring[wave][slot];
    const uint32_t soff = static_cast<uint32_t>(base) * RB;
    // the block's positions (lane k < 32: slot base + k; chunk blocks copy
    // positions they never read)
    if constexpr (!ALLF)
      dma4(r_pos, s_pos[wave][slot], 4u * static_cast<uint32_t>(min(base + (lane & 31), M - 1)), 0u);
    if (n_valid >= 32) {
#pragma unroll
      for (int j = 0; j < NC; ++j) {
        if constexpr (D == 128)
          dma16(r, dst + 1024 * j, k_lane ^ (64u * (j & 3)), soff + RB * (16 * (j & 1) + 4 * (j >> 1)));
        else
          dma16(r, dst + 1024 * j, k_lane, soff + RB * 4 * j);
      }
    } else {
#pragma unroll
      for (int j = 0; j < NC; ++j) {
        const int rho = RPC * j + lane / CPR, pc = lane % CPR;
        const uint32_t voff = static_cast<uint32_t>(min(k_key(rho), n_valid - 1)) * RB + 16 * (pc ^ (rho & (CPR - 1)));
        dma16(r, dst + 1024 * j, voff, soff);
      }
    }
  };
  auto issue_v = [&](int i, int slot) __attribute__((always_inline)) {
    const int bi = wave + kDW * i;
    const bool is_cache = bi < ncb;
    const int base = is_cache ? 32 * bi : 32 * (bi - ncb);
    const int n_valid = (is_cache ? n_cache : S) - base;
    const __amdgpu_buffer_rsrc_t r = is_cache ? rv_c : rv_n;
    const char* dst = ring[wave][slot];
    const uint32_t soff = static_cast<uint32_t>(base) * RB;
    if (n_valid >= 32) {
#pragma unroll
      for (int j = 0; j < NC; ++j) dma16(r, dst + 1024 * j, v_lane, soff + RB * RPC * j);
    } else {
#pragma unroll
      for (int j = 0; j < NC; ++j) {
        const int rho = RPC * j + lane / CPR, pc = lane % CPR;
        const uint32_t voff = static_cast<uint32_t>(min(rho, n_valid - 1)) * RB +
                              16 * (pc ^ ((rho & 3) << (CPR == 16 ? 2 : 1)));
        dma16(r, dst + 1024 * j, voff, soff);
      }
    }
  };

  // LDS fragment addresses within a slot (K rows and the query rows share
  // the layout)
  uint32_t k_rd[DS], v_rd[DB];
#pragma unroll
  for (int st = 0; st < DS; ++st) k_rd[st] = col * RB + 16 * ((2 * st + hf) ^ (col & (CPR - 1)));
  {
    const int tr_j = lane & 15, tr_r = tr_j >> 2, tr_q = tr_j & 3, tr_dg = (lane >> 4) & 1;
#pragma unroll
    for (int db = 0; db < DB; ++db) {
      const int d = db * 32 + tr_dg * 16 + 4 * tr_q;
      v_rd[db] = (16 * hf + tr_r) * RB + 16 * ((d >> 3) ^ ((tr_r & 3) << (CPR == 16 ? 2 : 1))) + 2 * (d & 7);
    }
  }

  // Stream of this wave: item s < nbw is K block s (with its positions),
  // item nbw + i is V block i; item s sits in ring slot s & 1.  Items s and
  // s + 1 are in flight while the wave waits for s; once s is consumed (and
  // its LDS reads are done), s + 2 goes into its slot.  Every global read
  // is a copy into LDS, so the compiler inserts no waits of its own and each
  // wait below is exact: the copies of the items issued after s.
  constexpr int KOPS = NC + (ALLF ? 0 : 1);              // copies of a K item (rows, positions)
  auto ops = [&](int s) { return s < nbw ? KOPS : NC; };
  auto issue = [&](int s) __attribute__((always_inline)) {
    if (s < nbw) issue_k(s, s & 1);
    else if (s < 2 * nbw) issue_v(s - nbw, s & 1);
  };
  auto wait_for = [&](int s) __attribute__((always_inline)) {
    if (s + 1 < 2 * nbw) {
      if (ops(s + 1) == KOPS) __builtin_amdgcn_s_waitcnt(0x0f70 | (KOPS & 15) | ((KOPS >> 4) << 14));
      else __builtin_amdgcn_s_waitcnt(0x0f70 | (NC & 15) | ((NC >> 4) << 14));
    } else {
      wait_vmem_all();
    }
  };
  auto refill = [&](int s) __attribute__((always_inline)) {
    __builtin_amdgcn_s_waitcnt(0xc07f);                   // lgkmcnt(0): the slot's reads are done
    if (s + 2 < 2 * nbw) issue(s + 2);
  };

  // prologue: the query rows (one 1 KB copy per wave: row block 32 half,
  // rows past the group clamped, in the K row layout), then items 0 and 1
  {
    const int jq = wave % (32 * RB / 1024);
    const int rho = RPC * jq + lane / CPR, pc = lane % CPR;
    const int qrow = min(32 * half + rho, n_rows - 1);
    dma16(r_q, qs + 1024 * jq, static_cast<uint32_t>(qrow) * RB + 16 * (pc ^ (rho & (CPR - 1))), 0u);
  }
  issue(0);
  issue(1);
  if (nbw >= 2) {                                            // items 0 and 1 (both K)
    constexpr int N2 = 2 * KOPS;
    __builtin_amdgcn_s_waitcnt(0x0f70 | (N2 & 15) | ((N2 >> 4) << 14));
  } else if (nbw == 1) {                                     // items 0 (K) and 1 (V)
    constexpr int N2 = KOPS + NC;
    __builtin_amdgcn_s_waitcnt(0x0f70 | (N2 & 15) | ((N2 >> 4) << 14));
  } else {
    wait_vmem_all();
  }
  barrier_lds();
  bf16x8 qf[DS];
#pragma unroll
  for (int st = 0; st < DS; ++st) {
    const bf16x8 v = *reinterpret_cast<const bf16x8*>(qs + k_rd[st]);
    qf[st] = row_ok ? v : bf16x8{};
  }

  // ---- 1. K pass: per block, the logits z (log2 domain, masked), the
  // lane's running row maximum m_run, and the stash e = 2^(z - m_run) with
  // m_run as it stands after the block (kept per block in mb); l_run sums e
  // against the current maximum (online-softmax rescale).  The exps thus run
  // while the next blocks are in flight.
  f32x16 z[kDNB];
  float mb[kDNB];
  float m_run = kDNoMax, l_run = 0.f;
#pragma unroll
  for (int i = 0; i < kDNB; ++i) {
    if (i < nbw) {
      wait_for(i);
      const char* kt = ring[wave][i & 1];
      f32x16 acc = zero16();
#pragma unroll
      for (int st = 0; st < DS; ++st) {
        const bf16x8 ka = *reinterpret_cast<const bf16x8*>(kt + k_rd[st]);
        acc = mfma32x32x16(ka, qf[st], acc);
      }
      const int bi = wave + kDW * i;
      uint32_t vis;                                       // bit k: key k of the block is visible to this row
      if (bi < ncb) {
        const int n_valid = n_cache - 32 * bi;
        uint32_t filled = 0xffffffffu;
        if constexpr (!ALLF) {
          const int pk = s_pos[wave][i & 1][lane];
          filled = static_cast<uint32_t>(__ballot(lane < 32 && pk >= 0));
        }
        vis = filled & (n_valid >= 32 ? 0xffffffffu : ((1u << n_valid) - 1u));
      } else {
        const int j0 = 32 * (bi - ncb);
        const int lim = min(S - 1, qi) - j0;              // last visible key offset
        vis = lim < 0 ? 0u : (lim >= 31 ? 0xffffffffu : ((2u << lim) - 1u));
      }
      if (!row_ok) vis = 0u;
      vis >>= 16 * hf;
      float bmx = kNegInf;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float v = ((vis >> r) & 1u) ? acc[r] * c2 : kNegInf;
        acc[r] = v;
        bmx = fmaxf(bmx, v);
      }
      const float m_new = fmaxf(m_run, bmx);
      float bs = 0.f;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float e = fast_exp2(acc[r] - m_new);
        z[i][r] = e;
        bs += e;
      }
      l_run = l_run * fast_exp2(m_run - m_new) + bs;
      m_run = m_new;
      mb[i] = m_new;
      refill(i);
    }
  }

  // ---- 2. the rows' maximum and sum over all keys: the two lane halves
  // (other keys of the same row), then the 8 waves through LDS
  {
    const float m2 = xor32(m_run), l2 = xor32(l_run);
    const float mm = fmaxf(m_run, m2);
    l_run = l_run * fast_exp2(m_run - mm) + l2 * fast_exp2(m2 - mm);
    m_run = mm;
  }
  if (hf == 0) {
    s_m[wave][col] = m_run;
    s_l[wave][col] = l_run;
  }
  barrier_lds();
  float m = s_m[0][col];
#pragma unroll
  for (int w = 1; w < kDW; ++w) m = fmaxf(m, s_m[w][col]);
  float l = 0.f;
#pragma unroll
  for (int w = 0; w < kDW; ++w) l += s_l[w][col] * fast_exp2(s_m[w][col] - m);
  const float inv_l = row_ok ? 1.f / l : 0.f;
  if (row_ok && wave == 0 && hf == 0)
    lse[static_cast<size_t>(b * Hq + hq) * S + qi] = (m + log2f(l)) * kLn2;

  // ---- 3. exact probabilities p = e 2^(mb - m) / l, column masses over the
  // half's rows, bf16 P.  The column sum is a reduce-scatter within each
  // 16-lane row with DPP pairings (lane i with 15 - i, then with 7 - i in
  // its 8-lane half, then i ^ 2, i ^ 1): at each step the lane whose index
  // bit (3, 2, 1, 0) is set keeps the upper half of its values and adds the
  // partner's copy of them, so that lane i ends with register i % 16 summed
  // over its row; one exchange with lane i ^ 16 adds the other row of the
  // 32-lane half.
  const int R = halves;
  float* out = partial + (static_cast<size_t>(bh) * R + half) * (static_cast<size_t>(M) + S);
  auto dpp_f = [](float v, auto ctrl) __attribute__((always_inline)) {
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v),
                                                                 decltype(ctrl)::value, 0xf, 0xf, false));
  };
  using kMirror = std::integral_constant<int, 0x140>;      // row_mirror: lane 15 - i of the row
  using kHalfMirror = std::integral_constant<int, 0x141>;  // row_half_mirror: lane 7 - i of the 8-lane half
  using kXor2 = std::integral_constant<int, 0x4e>;         // quad_perm [2, 3, 0, 1]
  using kXor1 = std::integral_constant<int, 0xb1>;         // quad_perm [1, 0, 3, 2]
  const bool b3 = (lane & 8) != 0, b2 = (lane & 4) != 0, b1 = (lane & 2) != 0, b0 = (lane & 1) != 0;
  bf16x8 pb[kDNB][2];
  // block i: p, its masses (written) and the bf16 B operand of PV
  auto masses = [&](int i) __attribute__((always_inline)) {
    const float f = fast_exp2(mb[i] - m) * inv_l;
    float p[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) p[r] = z[i][r] * f;
    f32x8 t0, t1;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      t0[e] = p[e];
      t1[e] = p[8 + e];
    }
    pb[i][0] = to_bf16x8(t0);
    pb[i][1] = to_bf16x8(t1);
    float v8[8], v4[4], v2[2], v1;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float keep = b3 ? p[8 + e] : p[e], send = b3 ? p[e] : p[8 + e];
      v8[e] = keep + dpp_f(send, kMirror{});
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float keep = b2 ? v8[4 + e] : v8[e], send = b2 ? v8[e] : v8[4 + e];
      v4[e] = keep + dpp_f(send, kHalfMirror{});
    }
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      const float keep = b1 ? v4[2 + e] : v4[e], send = b1 ? v4[e] : v4[2 + e];
      v2[e] = keep + dpp_f(send, kXor2{});
    }
    {
      const float keep = b0 ? v2[1] : v2[0], send = b0 ? v2[0] : v2[1];
      v1 = keep + dpp_f(send, kXor1{});
    }
    v1 += __shfl_xor(v1, 16);
    const int bi = wave + kDW * i;
    const int k = 16 * hf + (lane & 15);                // key of the block this lane holds
    if ((lane & 16) == 0) {
      if (bi < ncb) {
        const int slot = 32 * bi + k;
        if (slot < n_cache) out[slot] = v1;
      } else {
        const int j = 32 * (bi - ncb) + k;
        if (j < S) out[M + j] = v1;
      }
    }
  };
  // the first kEarly blocks here; the rest inside the V pass, each before
  // its block's wait, so that their VALU work runs while V blocks are in
  // flight (the stash of the later blocks and O^T then share the registers)
  constexpr int kEarly = 3;
#pragma unroll
  for (int i = 0; i < kEarly; ++i)
    if (i < nbw) masses(i);

  // ---- 4. V pass: O^T += V^T P^T over the wave's blocks
  f32x16 o[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) o[db] = zero16();
#pragma unroll
  for (int i = 0; i < kDNB; ++i) {
    if (i < nbw) {
      if (i >= kEarly) masses(i);
      wait_for(nbw + i);
      const char* vt = ring[wave][(nbw + i) & 1];
#pragma unroll
      for (int u = 0; u < 2; ++u)
#pragma unroll
        for (int db = 0; db < DB; ++db) {
          const char* p = vt + v_rd[db] + 8 * u * RB;
          const bf16x4 h0 = lds_read_tr16(reinterpret_cast<const bf16_t*>(p));
          const bf16x4 h1 = lds_read_tr16(reinterpret_cast<const bf16_t*>(p + 4 * RB));
          const bf16x8 a = __builtin_shufflevector(h0, h1, 0, 1, 2, 3, 4, 5, 6, 7);
          o[db] = mfma32x32x16(a, pb[i][u], o[db]);
        }
      refill(nbw + i);
    }
  }

  // ---- 5. sum the waves' O^T partials (wave order) and write the rows.
  // Wave w's partial goes to its own ring slots as [d][row] floats.
  wait_vmem_all();
  float* xo = reinterpret_cast<float*>(ring[wave][0]);
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) xo[(db * 32 + 8 * (r >> 2) + 4 * hf + (r & 3)) * 32 + col] = o[db][r];
  barrier_lds();
  // thread: row tid % 32, EPT consecutive d from EPT * (tid / 32)
  constexpr int EPT = 32 * D / (kDW * 64);              // 8 (D = 128) or 4 (D = 64)
  const int orow = tid & 31, od = EPT * (tid >> 5);
  float acc[EPT];
#pragma unroll
  for (int e = 0; e < EPT; ++e) acc[e] = 0.f;
#pragma unroll
  for (int w = 0; w < kDW; ++w) {
    const float* src = reinterpret_cast<const float*>(ring[w][0]);
#pragma unroll
    for (int e = 0; e < EPT; ++e) acc[e] += src[(od + e) * 32 + orow];
  }
  const int R_ = 32 * half + orow;
  if (R_ < n_rows) {
    const int og = R_ / S, oqi = R_ - og * S;
    bf16_t* dst = O + (static_cast<size_t>(b * Hq + kvh * G + og) * S + oqi) * D + od;
    if constexpr (EPT == 8) {
      f32x8 t;
#pragma unroll
      for (int e = 0; e < 8; ++e) t[e] = acc[e];
      *reinterpret_cast<bf16x8*>(dst) = to_bf16x8(t);
    } else {
      f32x4 t = {acc[0], acc[1], acc[2], acc[3]};
      *reinterpret_cast<bf16x4*>(dst) = to_bf16x4(t);
    }
  }
}

}  // namespace

int decode_fused_halves(const StepShape& sh, int dtype) {
  if (dtype != kBF16 || sh.policy != 0) return 0;
  if (sh.D != 64 && sh.D != 128) return 0;
  const int rows = sh.Hq / sh.Hkv * sh.S;
  if (rows > 32 * kDMaxHalves) return 0;
  const int nblk = (sh.n_cache + 31) / 32 + (sh.S + 31) / 32;
  if (nblk > kDW * kDNB) return 0;
  return (rows + 31) / 32;
}

int decode_fused_max_splits(int G, int s_max) {
  const int rows = std::min(G * s_max, 32 * kDMaxHalves);
  return (rows + 31) / 32;
}

hipError_t launch_decode_fused(const StepShape& sh, const AttnArgs& a, float* partial, hipStream_t st) {
  const int halves = decode_fused_halves(sh, kBF16);
  if (halves == 0) return hipErrorInvalidValue;
  const int n_heads = sh.B * sh.Hkv;
  const float c2 = sh.scale * kLog2e;
  const dim3 grid(n_heads * halves), block(kDW * 64);
#define H2O_LAUNCH_DEC1(DD, AF)                                                                          \
  hipLaunchKernelGGL(HIP_KERNEL_NAME(decode_fused_kernel<DD, AF>), grid, block, 0, st, static_cast<const bf16_t*>(a.q), \
                     static_cast<const bf16_t*>(a.k_cache), static_cast<const bf16_t*>(a.v_cache), a.pos, \
                     static_cast<const bf16_t*>(a.k_new), static_cast<const bf16_t*>(a.v_new),          \
                     static_cast<bf16_t*>(a.out), a.lse, partial, sh.Hq, sh.Hkv, sh.S, sh.M, sh.n_cache, c2, \
                     n_heads, halves)
#define H2O_LAUNCH_DEC(DD)                  \
  if (sh.all_filled) H2O_LAUNCH_DEC1(DD, true); \
  else H2O_LAUNCH_DEC1(DD, false)
  if (sh.D == 128) {
    H2O_LAUNCH_DEC(128);
  } else {
    H2O_LAUNCH_DEC(64);
  }
#undef H2O_LAUNCH_DEC
#undef H2O_LAUNCH_DEC1
  return hipGetLastError();
}

}  // namespace h2o
