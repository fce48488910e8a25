// Backward pass of the tiled online-softmax attention for CDNA4 (gfx950).
//
// Given Q, K, V, the forward outputs O and L and the gradient dO of a loss
// with respect to O, computes dQ, dK and dV of O = softmax(scale Q K^T) V
// (keys after the query excluded when causal) without storing the N x N
// probability matrix:
//
//  * The probabilities are recomputed tile by tile from the stored logsumexp,
//    P = exp(S - L) ("FlashAttention-2 from PyTorch to Triton", section "What
//    We Are Building": exp(S - m) / l = exp(S - m - log l) = exp(S - L)), in
//    base 2 with log2 e folded into the scale as in the forward kernels.
//  * The work is split into a dQ kernel and a dK/dV kernel, each owning its
//    outputs outright, so no atomics are needed (the split the "Case Study:
//    metal-flash-attention" page describes for that project's backward pass).
//  * dS = P o (dP - D) with dP = dO V^T and D_i = sum_c dO[i][c] O[i][c]: the
//    Jacobian of a row softmax applied to dP, using sum_j P[i][j] dP[i][j] =
//    dO_i . sum_j P[i][j] V_j = dO_i . O_i. D and the base-2 logsumexp
//    L * log2 e are formed once per row: by the bf16 dQ kernel, which holds the
//    row's dO already (it also stores them for the dK/dV kernel that runs
//    after it), and by a preprocessing kernel for fp32.
//
// gfx950 mapping (bf16; v_mfma_f32_32x32x16_bf16, fp32 accumulation; P and dS
// rounded to bf16 only as MFMA operands):
//  * dQ kernel: a workgroup of four waves owns 128 query rows (32 per wave)
//    and streams 64-key tiles of K and V through LDS (double-buffered, LDS
//    DMA). Q and dO stay in VGPRs as B operands of S^T = K Q^T and
//    dP^T = V dO^T, so in the result a lane holds 16 keys of one query and L,
//    D are per-lane scalars; dQ^T += K^T dS^T reads K transposed
//    (ds_read_b64_tr_b16) from the same tile.
//  * dK/dV kernel: a workgroup of eight waves owns 128 keys and streams
//    64-row tiles of Q and dO (with their L and D) through LDS; wave w takes
//    keys 32 (w % 4) .. and query block w / 4 of each tile. K and V of the 128
//    keys stay in LDS as B operands of S = Q K^T and dP = dO V^T, so a lane
//    holds 16 queries of one key; dV^T += dO^T P and dK^T += Q^T dS read dO and
//    Q transposed. The two query-block halves are summed at the end.
//  * Causal: the dQ kernel stops at the diagonal key tile, the dK/dV kernel
//    starts at the diagonal query tile; only tiles that straddle the diagonal
//    or the ragged end are masked.

#include <hip/hip_runtime.h>

#include <math.h>
#include <stddef.h>
#include <stdint.h>

#include <mutex>
#include <type_traits>

#include "fa.h"
#include "fa_device.h"

namespace {

constexpr float kLog2e = 1.44269504088896340736f;
constexpr int kBwdRows = 128;  // query rows (dQ kernel) or keys (dK/dV kernel) per workgroup
constexpr int kBwdTile = 64;   // streamed rows per LDS tile

// One dword per lane from rsrc + voffset into LDS at `lds` (via M0) + 4 * lane
// (buffer_load_dword ... lds); same M0 wait state as load_lds_share.
__device__ __forceinline__ void load_lds_4(__amdgpu_buffer_rsrc_t rsrc, uint32_t lds, int voffset) {
#if defined(__HIP_DEVICE_COMPILE__)
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dword %1, %2, 0 offen lds"
               :
               : "s"(lds), "v"(voffset), "s"(rsrc)
               : "memory", "m0");
#else
  (void)rsrc, (void)lds, (void)voffset;
#endif
}

// Per-lane addressing of a bf16 tile laid out with swz_b (BfLayout): every tile
// of the backward is read as rows, and the streamed K, Q and dO tiles also
// transposed.
//  * row reads: lane (l32, hh) reads chunk 2cc + hh of row 32 blk + l32 at
//    tile + 32 blk ROW + (row_base ^ 32 cc);
//  * transposing reads (ds_read_b64_tr_b16): the 16-lane group g reads rows
//    16 mm + 8 hi + 4 hh + (lane % 16) / 4 (+ 32 blk) at column bytes
//    64 db + 32 (g % 2) + 8 (lane % 4), i.e. tile + (32 blk + 16 mm) ROW +
//    (tr_base[hi] ^ 64 db). Each lane then holds 4 consecutive rows of column
//    32 db + l32: rows 16 mm + 4 hh + 0..3 (hi = 0) and + 8 (hi = 1), the
//    order in which the MFMA result layout lists a lane's 16 rows.
template <class LY>
struct TileAddr {
  static_assert(LY::CPR == 8 || LY::CPR == 16, "swz_b is defined for d = 64 and 128");
  int row_base;
  int tr_base[2];
  __device__ TileAddr(int lane) {
    const int l32 = lane % 32, hh = lane / 32;
    row_base = l32 * LY::ROW + 16 * (hh ^ LY::swz_b(l32));
    const int trow = 4 * hh + (lane % 16) / 4;
    const int tcol = 32 * ((lane / 16) % 2) + 8 * (lane % 4);
#pragma unroll
    for (int hi = 0; hi < 2; ++hi) {
      const int r = 8 * hi + trow;
      tr_base[hi] = r * LY::ROW + 16 * ((tcol >> 4) ^ LY::swz_b(r)) + (tcol & 15);
    }
  }
  __device__ bf16x8 row(const char *tile, int blk, int cc) const {
    return *(const bf16x8 *)(tile + 32 * blk * LY::ROW + (row_base ^ (32 * cc)));
  }
  __device__ bf16x8 tr(const char *tile, int blk, int mm, int db) const {
    const char *p = tile + (32 * blk + 16 * mm) * LY::ROW;
    const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4 *)(p + (tr_base[0] ^ (64 * db))));
    const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4 *)(p + (tr_base[1] ^ (64 * db))));
    return __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
  }
};

// Per-lane global byte offsets of this wave's share of a 64-row tile load (LDS
// slot p = 1024 gi + 16 lane holds chunk slot ^ swz_b(row) of row p / ROW);
// load i adds 1024 i through its instruction offset, so it is taken out here.
template <class LY>
__device__ __forceinline__ void tile_load_offsets(int wave, int lane, int (&vo)[LY::LPW]) {
#pragma unroll
  for (int i = 0; i < LY::LPW; ++i) {
    const int p = 64 * (wave * LY::LPW + i) + lane;
    const int r = p / LY::CPR, j = p % LY::CPR;
    vo[i] = r * LY::ROW + 16 * (j ^ LY::swz_b(r)) - 1024 * i;
  }
}

// D[r] = sum_c dO[r][c] O[r][c] and L2[r] = L[r] log2 e for every row r of all
// heads; work = [D (rows floats) | L2 (rows floats)]. Consecutive lanes read 16
// bytes each of one row (whole rows per wave instruction), and their partial
// sums are combined by a fixed butterfly of lane exchanges.
template <class T, int D>
__global__ __launch_bounds__(256) void fa_bwd_prep_kernel(const T *__restrict__ O,
                                                          const T *__restrict__ dO,
                                                          const float *__restrict__ L,
                                                          float *__restrict__ work, int64_t rows) {
  constexpr int EPL = 16 / sizeof(T);  // elements per lane
  constexpr int LPR = D / EPL;         // lanes per row
  constexpr int RPB = 256 / LPR;       // rows per workgroup
  typedef T vec __attribute__((ext_vector_type(EPL)));
  const int64_t r = (int64_t)blockIdx.x * RPB + threadIdx.x / LPR;
  const int part = threadIdx.x % LPR;
  float acc = 0.f;
  if (r < rows) {
    const vec a = *(const vec *)(O + r * D + EPL * part);
    const vec b = *(const vec *)(dO + r * D + EPL * part);
#pragma unroll
    for (int e = 0; e < EPL; ++e) acc = fmaf((float)a[e], (float)b[e], acc);
  }
#pragma unroll
  for (int off = LPR / 2; off > 0; off /= 2) acc += __shfl_xor(acc, off);
  if (r < rows && part == 0) {
    work[r] = acc;
    work[rows + r] = L[r] * kLog2e;
  }
}

// dQ = scale * dS K for 128 query rows of one head.
template <int D, bool CAUSAL>
__global__ __launch_bounds__(256, 2) void fa_bwd_dq_bf16_kernel(
    const bf16 *__restrict__ Q, const bf16 *__restrict__ K, const bf16 *__restrict__ V,
    const bf16 *__restrict__ dO, const bf16 *__restrict__ O, const float *__restrict__ L,
    float *__restrict__ work, bf16 *__restrict__ dQ, int N, int n_qtiles, int64_t rows, float c,
    float scale, int group) {
  using LY = BfLayout<D, kBwdTile, 4>;
  constexpr int BN = kBwdTile;
  constexpr int NKB = BN / 32;
  constexpr int NDB = D / 32;
  constexpr int NCC = D / 16;
  __shared__ __attribute__((aligned(1024))) char smem[2 * LY::STAGE];

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid / 64);
  const int lane = tid % 64;
  const int l32 = lane % 32, hh = lane / 32;

  int bh, qt;
  map_block(blockIdx.x, gridDim.x, n_qtiles, CAUSAL, group, bh, qt);
  const size_t head = (size_t)bh * (size_t)N * D;
  const bf16 *Kh = K + head;
  const bf16 *Vh = V + head;
  const int q0 = qt * kBwdRows;
  const int qw = q0 + kRowsPerWave * wave;
  const int qrow = qw + l32;
  const bool row_ok = qrow < N;

  // Q and dO rows as the B operands of S^T = K Q^T and dP^T = V dO^T.
  bf16x8 qf[NCC], gf[NCC];
#pragma unroll
  for (int cc = 0; cc < NCC; ++cc) {
    const size_t off = head + (size_t)qrow * D + 16 * cc + 8 * hh;
    qf[cc] = row_ok ? *(const bf16x8 *)(Q + off) : bf16x8{};
    gf[cc] = row_ok ? *(const bf16x8 *)(dO + off) : bf16x8{};
  }
  // D = sum_c dO[c] O[c] of this row (the two half-waves hold its two column halves) and
  // L2 = L log2 e, also stored in `work` for the dK/dV kernel that runs next.
  float dpart = 0.f;
#pragma unroll
  for (int cc = 0; cc < NCC; ++cc) {
    const bf16x8 of = row_ok ? *(const bf16x8 *)(O + head + (size_t)qrow * D + 16 * cc + 8 * hh) : bf16x8{};
#pragma unroll
    for (int e = 0; e < 8; ++e) dpart = fmaf((float)gf[cc][e], (float)of[e], dpart);
  }
  const float dd = halves_sum(dpart);
  const float l2 = row_ok ? L[(size_t)bh * N + qrow] * kLog2e : 0.f;
  if (row_ok && hh == 0) {
    work[(size_t)bh * N + qrow] = dd;
    work[rows + (size_t)bh * N + qrow] = l2;
  }

  f32x16 acc[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db) acc[db] = f32x16{};

  const TileAddr<LY> ta(lane);
  int vo[LY::LPW];
  tile_load_offsets<LY>(wave, lane, vo);
  const uint32_t smem_lds = lds_addr(smem);
  auto issue = [&](int t) {
    const int k0 = t * BN;
    const int bytes = min(N - k0, BN) * LY::ROW;
    const uint32_t dst = smem_lds + (t & 1) * LY::STAGE + 1024 * wave * LY::LPW;
    load_lds_share(make_rsrc(Kh + (size_t)k0 * D, bytes), dst, vo);
    load_lds_share(make_rsrc(Vh + (size_t)k0 * D, bytes), dst + LY::TILE, vo);
  };

  const int kend = CAUSAL ? min(N, q0 + kBwdRows) : N;
  const int nt = (kend + BN - 1) / BN;
  issue(0);
  for (int t = 0; t < nt; ++t) {
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();  // tile t landed for every wave; every wave is done with tile t - 1
    if (t + 1 < nt) issue(t + 1);
    const char *ks = smem + (t & 1) * LY::STAGE;
    const char *vs = ks + LY::TILE;
    const int k0 = t * BN;

    // S^T and dP^T blocks of 32 keys x 32 queries: lane (l32, hh), register r
    // holds key k0 + 32 kb + 8 (r/4) + 4 hh + r%4 of query qrow.
    f32x16 s[NKB], dp[NKB];
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) {
#pragma unroll
      for (int cc = 0; cc < NCC; ++cc) {
        s[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ta.row(ks, kb, cc), qf[cc], cc == 0 ? f32x16{} : s[kb], 0, 0, 0);
        dp[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ta.row(vs, kb, cc), gf[cc], cc == 0 ? f32x16{} : dp[kb], 0, 0, 0);
        // Each step's two operand reads stay next to its MFMAs: hoisting every
        // read of the tile would spill at d = 128 (registers are full here).
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    // P = exp2(S c - L2) (masked: 0) and dS = P (dP - D), as bf16 B operands.
    bf16x8 dsb[NKB][2];
    auto probs = [&](auto edge_tag) {
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          float p = exp2_fast(fmaf(s[kb][r], c, -l2));
          if constexpr (decltype(edge_tag)::value) {
            const int key = k0 + 32 * kb + 8 * (r / 4) + 4 * hh + (r % 4);
            if (key >= N || (CAUSAL && key > qrow)) p = 0.f;
          }
          dsb[kb][r / 8][r % 8] = (bf16)(p * (dp[kb][r] - dd));
        }
    };
    if ((k0 + BN > N) || (CAUSAL && k0 + BN - 1 > qw))
      probs(std::true_type{});
    else
      probs(std::false_type{});
    // dQ^T += K^T dS^T.
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
      for (int mm = 0; mm < 2; ++mm)
#pragma unroll
        for (int db = 0; db < NDB; ++db)
          acc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ta.tr(ks, kb, mm, db), dsb[kb][mm], acc[db], 0, 0, 0);
  }

  // Lane (l32, hh) holds dQ^T[32 db + 8 g + 4 hh + e][qrow] in acc[db][4 g + e].
  if (row_ok) {
    bf16 *out = dQ + head + (size_t)qrow * D;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        bf16x4 v4;
#pragma unroll
        for (int e = 0; e < 4; ++e) v4[e] = (bf16)(acc[db][4 * g + e] * scale);
        *(bf16x4 *)(out + 32 * db + 8 * g + 4 * hh) = v4;
      }
  }
}

// dK = scale * dS^T Q and dV = P^T dO for 128 keys of one head. Eight waves:
// wave w owns keys 32 (w % 4) .. + 31 of the workgroup and query block w / 4
// (32 rows) of every 64-row tile, so two waves share a SIMD; K and V of the
// 128 keys stay in LDS for the whole loop and are read there as B operands,
// which keeps a wave's registers to its two accumulators. At the end the two
// waves of a key block add their partial dK, dV through LDS (block 0 + block
// 1, a fixed order).
template <int D, bool CAUSAL>
__global__ __launch_bounds__(512, 1) void fa_bwd_dkdv_bf16_kernel(
    const bf16 *__restrict__ Q, const bf16 *__restrict__ K, const bf16 *__restrict__ V,
    const bf16 *__restrict__ dO, const float *__restrict__ work, bf16 *__restrict__ dK,
    bf16 *__restrict__ dV, int N, int n_ktiles, int64_t rows, float c, float scale, int group) {
  constexpr int NW = 8;
  using LY = BfLayout<D, kBwdTile, NW>;   // streamed Q, dO tiles
  using LK = BfLayout<D, kBwdRows, NW>;   // the workgroup's K, V rows
  constexpr int BQ = kBwdTile;
  constexpr int NDB = D / 32;
  constexpr int NCC = D / 16;
  constexpr int KV = 2 * LK::TILE;                  // K then V
  constexpr int STAGE = 2 * LY::TILE + 2 * BQ * 4;  // Q tile, dO tile, L2, D
  constexpr int PART = 2 * NDB * 16 * 64 * 4;       // one wave's partial dK, dV
  constexpr int SMEM = (KV + 2 * STAGE > 4 * PART) ? KV + 2 * STAGE : 4 * PART;
  static_assert(SMEM <= 160 * 1024, "LDS budget of a CU");
  __shared__ __attribute__((aligned(1024))) char smem[SMEM];

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid / 64);
  const int lane = tid % 64;
  const int hh = lane / 32;
  const int kb = wave % 4;  // key block of this wave
  const int qb = wave / 4;  // query block of every tile

  // Key tiles in ascending order: when causal, the first ones see the most queries.
  int bh, kt;
  map_block(blockIdx.x, gridDim.x, n_ktiles, false, group, bh, kt);
  const size_t head = (size_t)bh * (size_t)N * D;
  const bf16 *Qh = Q + head;
  const bf16 *Gh = dO + head;
  const float *Dh = work + (size_t)bh * N;
  const float *L2h = work + rows + (size_t)bh * N;
  const int k0 = kt * kBwdRows;
  const int kw = k0 + kRowsPerWave * kb;  // first key of this wave
  const int krow = kw + lane % 32;

  const uint32_t smem_lds = lds_addr(smem);
  const char *ks = smem;
  const char *vs = smem + LK::TILE;
  {
    int vk[LK::LPW];
    tile_load_offsets<LK>(wave, lane, vk);
    const int bytes = min(N - k0, kBwdRows) * LK::ROW;
    const uint32_t dst = smem_lds + 1024 * wave * LK::LPW;
    load_lds_share(make_rsrc(K + head + (size_t)k0 * D, bytes), dst, vk);
    load_lds_share(make_rsrc(V + head + (size_t)k0 * D, bytes), dst + LK::TILE, vk);
  }

  f32x16 dk[NDB], dv[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db) {
    dk[db] = f32x16{};
    dv[db] = f32x16{};
  }

  const TileAddr<LY> ta(lane);
  int vo[LY::LPW];
  tile_load_offsets<LY>(wave, lane, vo);
  auto issue = [&](int t) {
    const int qa = t * BQ;
    const int n_ok = min(N - qa, BQ);
    const uint32_t dst = smem_lds + KV + (t & 1) * STAGE;
    load_lds_share(make_rsrc(Qh + (size_t)qa * D, n_ok * LY::ROW), dst + 1024 * wave * LY::LPW, vo);
    load_lds_share(make_rsrc(Gh + (size_t)qa * D, n_ok * LY::ROW), dst + LY::TILE + 1024 * wave * LY::LPW, vo);
    if (wave == 0) load_lds_4(make_rsrc(L2h + qa, n_ok * 4), dst + 2 * LY::TILE, 4 * lane);
    if (wave == 1) load_lds_4(make_rsrc(Dh + qa, n_ok * 4), dst + 2 * LY::TILE + BQ * 4, 4 * lane);
  };

  // Tile t: wait for it, start loading t + 1, and (unless every key of the
  // wave lies after every query of its block) compute this wave's block: S
  // and dP blocks of 32 queries x 32 keys (lane (l32, hh), register r holds
  // query qa + 8 (r/4) + 4 hh + r%4 of key krow), P and dS (EDGE: test every
  // element against N and the causal rule), dV^T += dO^T P, dK^T += Q^T dS.
  const int nt = (N + BQ - 1) / BQ;
  auto iteration = [&](int t, auto edge_tag) {
    constexpr bool EDGE = decltype(edge_tag)::value;
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();  // tile t (and K, V) landed for every wave; every wave is done with tile t - 1
    if (t + 1 < nt) issue(t + 1);
    const char *qs = smem + KV + (t & 1) * STAGE;
    const char *gs = qs + LY::TILE;
    const float *ls = (const float *)(gs + LY::TILE);
    const float *ds = ls + BQ;
    const int qa = t * BQ + 32 * qb;  // first query of this wave's block
    if (CAUSAL && EDGE && kw > qa + 31) return;  // every key of the wave after every query

    f32x16 s, dp;
    // At d = 64 each step's four operand reads stay next to its two MFMAs (the
    // fence keeps the compiler from hoisting every read of the block into
    // registers); at d = 128 the compiler's own order is faster (measured:
    // 1.5% on the whole backward at d = 128, 5% slower without the fence at
    // d = 64). The dV/dK products below are left to the compiler at both.
#pragma unroll
    for (int cc = 0; cc < NCC; ++cc) {
      s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ta.row(qs, qb, cc), ta.row(ks, kb, cc), cc == 0 ? f32x16{} : s, 0, 0, 0);
      dp = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ta.row(gs, qb, cc), ta.row(vs, kb, cc), cc == 0 ? f32x16{} : dp, 0, 0, 0);
      if constexpr (D == 64) __builtin_amdgcn_sched_barrier(0);
    }
    bf16x8 pb[2], dsb[2];
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const int qi = 32 * qb + 8 * g + 4 * hh;  // local query of registers 4g .. 4g + 3
      const f32x4 lq = *(const f32x4 *)(ls + qi);
      const f32x4 dq = *(const f32x4 *)(ds + qi);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int r = 4 * g + e;
        float p = exp2_fast(fmaf(s[r], c, -lq[e]));
        if constexpr (EDGE) {
          const int query = t * BQ + qi + e;
          if (query >= N || (CAUSAL && krow > query)) p = 0.f;
        }
        pb[r / 8][r % 8] = (bf16)p;
        dsb[r / 8][r % 8] = (bf16)(p * (dp[r] - dq[e]));
      }
    }
#pragma unroll
    for (int mm = 0; mm < 2; ++mm)
#pragma unroll
      for (int db = 0; db < NDB; ++db) {
        dv[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ta.tr(gs, qb, mm, db), pb[mm], dv[db], 0, 0, 0);
        dk[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ta.tr(qs, qb, mm, db), dsb[mm], dk[db], 0, 0, 0);
      }
  };

  // Three runs of tiles, so that the masked and unmasked forms are never live
  // together: the tiles that straddle the diagonal (causal: queries of the
  // workgroup's own 128 positions), the full tiles after them, and a ragged
  // last tile.
  const int t_first = CAUSAL ? k0 / BQ : 0;
  const int t_diag = CAUSAL ? min(nt, t_first + kBwdRows / BQ) : t_first;
  const int t_full = max(t_diag, N / BQ);
  issue(t_first);
  int t = t_first;
  for (; t < t_diag; ++t) iteration(t, std::true_type{});
  for (; t < t_full; ++t) iteration(t, std::false_type{});
  for (; t < nt; ++t) iteration(t, std::true_type{});

  // Merge the two query-block halves of each key block: qb = 1 waves park
  // their partials in LDS as [register][lane] floats, qb = 0 waves add them.
  __syncthreads();  // every wave is done with the K, V and tile LDS
  float *part = (float *)smem + (size_t)kb * (PART / 4);
  if (qb == 1) {
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        part[((2 * db) * 16 + r) * 64 + lane] = dk[db][r];
        part[((2 * db + 1) * 16 + r) * 64 + lane] = dv[db][r];
      }
  }
  __syncthreads();
  if (qb == 1 || krow >= N) return;
  // Lane (l32, hh) holds dV^T / dK^T[32 db + 8 g + 4 hh + e][krow] in [db][4 g + e].
  bf16 *ov = dV + head + (size_t)krow * D;
  bf16 *ok = dK + head + (size_t)krow * D;
#pragma unroll
  for (int db = 0; db < NDB; ++db)
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      bf16x4 a4, b4;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int r = 4 * g + e;
        const float kk = dk[db][r] + part[((2 * db) * 16 + r) * 64 + lane];
        const float vv = dv[db][r] + part[((2 * db + 1) * 16 + r) * 64 + lane];
        a4[e] = (bf16)vv;
        b4[e] = (bf16)(kk * scale);
      }
      *(bf16x4 *)(ov + 32 * db + 8 * g + 4 * hh) = a4;
      *(bf16x4 *)(ok + 32 * db + 8 * g + 4 * hh) = b4;
    }
}

// ---------------------------------------------------------------------------
// fp32 (v_mfma_f32_32x32x2_f32). A workgroup of four waves owns 32 query rows
// (dQ kernel) or 32 keys (dK/dV kernel) and its waves take every fourth
// 32-row tile of the other side, so each wave forms a partial gradient that
// the workgroup sums through LDS in wave order at the end. The workgroup's own
// rows stay in LDS (row stride D + 4 floats, so 16 rows read at one column hit
// distinct banks) and are read there as the shared operand of S and dP; the
// streamed tiles go straight from memory into VGPRs, once in row layout (lane
// l32 holds row l32, contraction over the head dimension) and once in the
// layout of the gradient product (lane (l32, hh) holds rows 8 (r/4) + 4 hh +
// r%4 at columns NDB l32 .. NDB l32 + NDB - 1, contraction over the rows). The
// product then yields column NDB i + db of the gradient in row i of block db.
constexpr int kF32Block = 32;  // rows per workgroup and per streamed tile (fp32)
constexpr int kF32BwdWaves = 4;

// scale * (sum over the waves' partials) into rows r0 .. r0 + 31 of `out`
// (rows at or past N skipped). `acc` holds this wave's partial in the layout
// the permuted-column products leave: lane (l32, hh), block db, register
// 4 g + e hold row l32, column NDB (8 g + 4 hh + e) + db. `part` is LDS of
// NW x 32 x (D + 4) floats; the caller has synchronised the workgroup before.
template <int D, int NW>
__device__ __forceinline__ void merge_store_f32(float *part, const f32x16 (&acc)[D / 32], int wave,
                                                int tid, float *out, int r0, int N, float scale) {
  constexpr int NDB = D / 32;
  constexpr int OS = D + 4;
  const int lane = tid % 64, l32 = lane % 32, hh = lane / 32;
  float *orow = part + (wave * kF32Block + l32) * OS;
#pragma unroll
  for (int g = 0; g < 4; ++g)
#pragma unroll
    for (int h = 0; h < NDB; ++h) {
      f32x4 v;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int idx = 4 * h + e;  // (column offset within the group) = e' NDB + db
        v[e] = acc[idx % NDB][4 * g + idx / NDB];
      }
      *(f32x4 *)(orow + NDB * (8 * g + 4 * hh) + 4 * h) = v;
    }
  __syncthreads();
  constexpr int C4 = D / 4;
  static_assert(kF32Block * C4 % (NW * 64) == 0, "merge must split evenly over the workgroup");
#pragma unroll
  for (int it = 0; it < kF32Block * C4 / (NW * 64); ++it) {
    const int idx = tid + NW * 64 * it;
    const int row = idx / C4, c4 = idx % C4;
    if (r0 + row >= N) continue;
    f32x4 sum = *(const f32x4 *)(part + row * OS + 4 * c4);
#pragma unroll
    for (int w = 1; w < NW; ++w) sum += *(const f32x4 *)(part + (w * kF32Block + row) * OS + 4 * c4);
    *(f32x4 *)(out + (size_t)(r0 + row) * D + 4 * c4) = sum * scale;
  }
}

// Rows r0 .. r0 + 31 of two row-major [N][D] fp32 arrays into LDS rows of
// D + 4 floats (rows at or past N as zeros).
template <int D, int NW>
__device__ __forceinline__ void stage_rows_f32(float *dst, const float *a, const float *b, int r0,
                                               int N, int tid) {
  constexpr int ROW = D * 4;
  constexpr int OS = D + 4;
  constexpr int C4 = D / 4;
  const int bytes = min(N - r0, kF32Block) * ROW;
  const __amdgpu_buffer_rsrc_t ra = make_rsrc(a + (size_t)r0 * D, bytes);
  const __amdgpu_buffer_rsrc_t rb = make_rsrc(b + (size_t)r0 * D, bytes);
#pragma unroll
  for (int it = 0; it < kF32Block * C4 / (NW * 64); ++it) {
    const int idx = tid + NW * 64 * it;
    const int row = idx / C4, c4 = idx % C4;
    *(f32x4 *)(dst + row * OS + 4 * c4) = F32Vec<4>::load(ra, row * ROW + 16 * c4);
    *(f32x4 *)(dst + (kF32Block + row) * OS + 4 * c4) = F32Vec<4>::load(rb, row * ROW + 16 * c4);
  }
}

// dQ = scale * dS K for 32 query rows of one head (fp32).
//  S^T = K Q^T, dP^T = V dO^T: K, V tiles in row layout as A operands, the
//  block's Q and dO rows from LDS as B operands; lane (l32, hh) then holds
//  keys 8 (r/4) + 4 hh + r%4 of query l32, whose L2 and D are lane scalars.
//  dQ^T += K^T dS^T with K in the gradient layout.
template <int D, bool CAUSAL>
__global__ __launch_bounds__(256, 1) void fa_bwd_dq_f32_kernel(
    const float *__restrict__ Q, const float *__restrict__ K, const float *__restrict__ V,
    const float *__restrict__ dO, const float *__restrict__ work, float *__restrict__ dQ, int N,
    int n_qblocks, int64_t rows, float c, float scale) {
  constexpr int NW = kF32BwdWaves;
  constexpr int BQ = kF32Block, BN = kF32Block;
  constexpr int HD = D / 2;
  constexpr int NDB = D / 32;
  constexpr int ROW = D * 4;
  constexpr int OS = D + 4;
  using VV = F32Vec<NDB>;
  typedef typename VV::type vvec;
  constexpr int OPND = 2 * BQ * OS;
  constexpr int PART = NW * BQ * OS;
  __shared__ __attribute__((aligned(16))) float smem[OPND > PART ? OPND : PART];

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid / 64);
  const int lane = tid % 64, l32 = lane % 32, hh = lane / 32;

  int bh, qb;
  map_block(blockIdx.x, gridDim.x, n_qblocks, CAUSAL, 0, bh, qb);
  const size_t head = (size_t)bh * (size_t)N * D;
  const float *Kh = K + head;
  const float *Vh = V + head;
  const int q0 = qb * BQ;
  const int qrow = q0 + l32;
  const bool row_ok = qrow < N;

  stage_rows_f32<D, NW>(smem, Q + head, dO + head, q0, N, tid);
  const float l2 = row_ok ? work[rows + (size_t)bh * N + qrow] : 0.f;
  const float dd = row_ok ? work[(size_t)bh * N + qrow] : 0.f;
  __syncthreads();
  const float *qs = smem + l32 * OS + hh * HD;
  const float *gs = smem + (BQ + l32) * OS + hh * HD;

  const int kend = CAUSAL ? min(N, q0 + BQ) : N;
  const int nt = (kend + BN - 1) / BN;

  f32x4 kf[HD / 4], vf[HD / 4];
  vvec kg[16];
  auto tile_rsrc = [&](const float *base, int t) {
    const int k0 = t * BN;
    return make_rsrc(base + (size_t)k0 * D, min(N - k0, BN) * ROW);
  };
  auto load_rows = [&](f32x4 (&dst)[HD / 4], const float *base, int t) {
    const __amdgpu_buffer_rsrc_t r = tile_rsrc(base, t);
#pragma unroll
    for (int j = 0; j < HD / 4; ++j) dst[j] = F32Vec<4>::load(r, l32 * ROW + hh * HD * 4 + 16 * j);
  };
  auto load_grad = [&](vvec (&dst)[16], const float *base, int t) {
    const __amdgpu_buffer_rsrc_t r = tile_rsrc(base, t);
#pragma unroll
    for (int i = 0; i < 16; ++i) dst[i] = VV::load(r, (8 * (i / 4) + 4 * hh + i % 4) * ROW + NDB * 4 * l32);
  };

  f32x16 acc[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db) acc[db] = f32x16{};

  if (wave < nt) {
    load_rows(kf, Kh, wave);
    load_rows(vf, Vh, wave);
  }
  for (int t = wave; t < nt; t += NW) {
    const int k0 = t * BN;
    const bool more = t + NW < nt;
    f32x16 s = f32x16{}, dp = f32x16{};
#pragma unroll
    for (int j = 0; j < HD / 4; ++j) {
      const f32x4 b = *(const f32x4 *)(qs + 4 * j);
#pragma unroll
      for (int e = 0; e < 4; ++e) s = __builtin_amdgcn_mfma_f32_32x32x2f32(kf[j][e], b[e], s, 0, 0, 0);
    }
    // The fences keep each load where the registers it fills have been freed.
    __builtin_amdgcn_sched_barrier(0);
    load_grad(kg, Kh, t);
#pragma unroll
    for (int j = 0; j < HD / 4; ++j) {
      const f32x4 b = *(const f32x4 *)(gs + 4 * j);
#pragma unroll
      for (int e = 0; e < 4; ++e) dp = __builtin_amdgcn_mfma_f32_32x32x2f32(vf[j][e], b[e], dp, 0, 0, 0);
    }
    __builtin_amdgcn_sched_barrier(0);
    if (more) load_rows(kf, Kh, t + NW);
    __builtin_amdgcn_sched_barrier(0);
    // dS^T = P^T o (dP^T - D); keys past N and (causal) after the query give P = 0.
    const bool edge = k0 + BN > N || (CAUSAL && k0 + BN > q0);
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      float p = exp2_fast(fmaf(s[r], c, -l2));
      if (edge) {
        const int key = k0 + 8 * (r / 4) + 4 * hh + r % 4;
        if (key >= N || (CAUSAL && key > qrow)) p = 0.f;
      }
      s[r] = p * (dp[r] - dd);
    }
#pragma unroll
    for (int r = 0; r < 16; ++r)
#pragma unroll
      for (int db = 0; db < NDB; ++db) acc[db] = __builtin_amdgcn_mfma_f32_32x32x2f32(kg[r][db], s[r], acc[db], 0, 0, 0);
    __builtin_amdgcn_sched_barrier(0);
    if (more) load_rows(vf, Vh, t + NW);
    // Keep the accumulators in AGPRs across iterations.
#pragma unroll
    for (int db = 0; db < NDB; ++db) asm volatile("" : "+a"(acc[db]));
  }

  __syncthreads();  // every wave is done with the Q, dO rows in LDS
  merge_store_f32<D, NW>(smem, acc, wave, tid, dQ + head, q0, N, scale);
}

// dK = scale * dS^T Q and dV = P^T dO for 32 keys of one head (fp32).
//  S = Q K^T, dP = dO V^T: Q, dO tiles in row layout as A operands, the
//  block's K and V rows from LDS as B operands; lane (l32, hh) then holds
//  queries 8 (r/4) + 4 hh + r%4 of key l32. dV^T += dO^T P and dK^T += Q^T dS
//  with dO and Q in the gradient layout.
template <int D, bool CAUSAL>
__global__ __launch_bounds__(256, 1) void fa_bwd_dkdv_f32_kernel(
    const float *__restrict__ Q, const float *__restrict__ K, const float *__restrict__ V,
    const float *__restrict__ dO, const float *__restrict__ work, float *__restrict__ dK,
    float *__restrict__ dV, int N, int n_kblocks, int64_t rows, float c, float scale) {
  constexpr int NW = kF32BwdWaves;
  constexpr int BQ = kF32Block, BK = kF32Block;
  constexpr int HD = D / 2;
  constexpr int NDB = D / 32;
  constexpr int ROW = D * 4;
  constexpr int OS = D + 4;
  using VV = F32Vec<NDB>;
  typedef typename VV::type vvec;
  constexpr int OPND = 2 * BK * OS + NW * 2 * BQ;  // K, V rows; per wave L2, D of its tile
  constexpr int PART = NW * BK * OS;
  __shared__ __attribute__((aligned(16))) float smem[OPND > PART ? OPND : PART];

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid / 64);
  const int lane = tid % 64, l32 = lane % 32, hh = lane / 32;

  // Key blocks in ascending order: when causal, the first ones see the most queries.
  int bh, kb;
  map_block(blockIdx.x, gridDim.x, n_kblocks, false, 0, bh, kb);
  const size_t head = (size_t)bh * (size_t)N * D;
  const float *Qh = Q + head;
  const float *Gh = dO + head;
  const float *Dh = work + (size_t)bh * N;
  const float *L2h = work + rows + (size_t)bh * N;
  const int k0 = kb * BK;
  const int krow = k0 + l32;

  stage_rows_f32<D, NW>(smem, K + head, V + head, k0, N, tid);
  __syncthreads();
  const float *ks = smem + l32 * OS + hh * HD;
  const float *vs = smem + (BK + l32) * OS + hh * HD;
  float *ld = smem + 2 * BK * OS + wave * 2 * BQ;  // [L2 of the tile's queries | their D]

  const int t_first = CAUSAL ? kb : 0;  // query tiles and key blocks have the same size
  const int nt = (N + BQ - 1) / BQ;

  f32x4 qf[HD / 4], gf[HD / 4];
  vvec gg[16], qg[16];
  auto tile_rsrc = [&](const float *base, int t) {
    const int qa = t * BQ;
    return make_rsrc(base + (size_t)qa * D, min(N - qa, BQ) * ROW);
  };
  auto load_rows = [&](f32x4 (&dst)[HD / 4], const float *base, int t) {
    const __amdgpu_buffer_rsrc_t r = tile_rsrc(base, t);
#pragma unroll
    for (int j = 0; j < HD / 4; ++j) dst[j] = F32Vec<4>::load(r, l32 * ROW + hh * HD * 4 + 16 * j);
  };
  auto load_grad = [&](vvec (&dst)[16], const float *base, int t) {
    const __amdgpu_buffer_rsrc_t r = tile_rsrc(base, t);
#pragma unroll
    for (int i = 0; i < 16; ++i) dst[i] = VV::load(r, (8 * (i / 4) + 4 * hh + i % 4) * ROW + NDB * 4 * l32);
  };

  f32x16 dk[NDB], dv[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db) {
    dk[db] = f32x16{};
    dv[db] = f32x16{};
  }

  if (t_first + wave < nt) {
    load_rows(qf, Qh, t_first + wave);
    load_rows(gf, Gh, t_first + wave);
  }
  for (int t = t_first + wave; t < nt; t += NW) {
    const int qa = t * BQ;
    const bool more = t + NW < nt;
    f32x16 s = f32x16{}, dp = f32x16{};
#pragma unroll
    for (int j = 0; j < HD / 4; ++j) {
      const f32x4 b = *(const f32x4 *)(ks + 4 * j);
#pragma unroll
      for (int e = 0; e < 4; ++e) s = __builtin_amdgcn_mfma_f32_32x32x2f32(qf[j][e], b[e], s, 0, 0, 0);
    }
    // The fences keep each load where the registers it fills have been freed.
    __builtin_amdgcn_sched_barrier(0);
    load_grad(gg, Gh, t);
    // Lane l32 + 32 hh fetches L2 (hh = 0) or D (hh = 1) of query qa + l32
    // (zero past N); the wave shares them through its LDS slot.
    const float lv = qa + l32 < N ? (hh ? Dh : L2h)[qa + l32] : 0.f;
#pragma unroll
    for (int j = 0; j < HD / 4; ++j) {
      const f32x4 b = *(const f32x4 *)(vs + 4 * j);
#pragma unroll
      for (int e = 0; e < 4; ++e) dp = __builtin_amdgcn_mfma_f32_32x32x2f32(gf[j][e], b[e], dp, 0, 0, 0);
    }
    __builtin_amdgcn_sched_barrier(0);
    load_grad(qg, Qh, t);
    __builtin_amdgcn_sched_barrier(0);
    ld[lane] = lv;  // a wave's LDS accesses complete in order: no barrier needed
    // Queries past N, keys past N and (causal) keys after the query give P = 0.
    const bool edge = qa + BQ > N || k0 + BK > N || (CAUSAL && qa == k0);
    f32x16 ds;
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const f32x4 l2v = *(const f32x4 *)(ld + 8 * g + 4 * hh);
      const f32x4 ddv = *(const f32x4 *)(ld + BQ + 8 * g + 4 * hh);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int r = 4 * g + e;
        float p = exp2_fast(fmaf(s[r], c, -l2v[e]));
        if (edge) {
          const int q = qa + 8 * g + 4 * hh + e;
          if (q >= N || krow >= N || (CAUSAL && krow > q)) p = 0.f;
        }
        s[r] = p;
        ds[r] = p * (dp[r] - ddv[e]);
      }
    }
#pragma unroll
    for (int r = 0; r < 16; ++r)
#pragma unroll
      for (int db = 0; db < NDB; ++db) dv[db] = __builtin_amdgcn_mfma_f32_32x32x2f32(gg[r][db], s[r], dv[db], 0, 0, 0);
    __builtin_amdgcn_sched_barrier(0);
    if (more) load_rows(qf, Qh, t + NW);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int r = 0; r < 16; ++r)
#pragma unroll
      for (int db = 0; db < NDB; ++db) dk[db] = __builtin_amdgcn_mfma_f32_32x32x2f32(qg[r][db], ds[r], dk[db], 0, 0, 0);
    __builtin_amdgcn_sched_barrier(0);
    if (more) load_rows(gf, Gh, t + NW);
    // Keep the accumulators in AGPRs across iterations (else the register
    // allocator shuttles them through VGPRs every tile).
#pragma unroll
    for (int db = 0; db < NDB; ++db) asm volatile("" : "+a"(dk[db]), "+a"(dv[db]));
  }

  __syncthreads();  // every wave is done with the K, V rows in LDS
  merge_store_f32<D, NW>(smem, dv, wave, tid, dV + head, k0, N, 1.f);
  __syncthreads();  // the dV partials are consumed
  merge_store_f32<D, NW>(smem, dk, wave, tid, dK + head, k0, N, scale);
}

template <int D, bool CAUSAL>
hipError_t launch_bwd_bf16(int64_t BH, int N, hipStream_t s, const void *Q, const void *K,
                           const void *V, const void *O, const float *L, const void *dO, void *dQ,
                           void *dK, void *dV, float *work, float c, float scale) {
  const int64_t rows = BH * N;
  const int ntiles = (N + kBwdRows - 1) / kBwdRows;
  // Both kernels stream two bf16 N x D matrices per head (K, V or Q, dO).
  const int group = head_group(BH, (int64_t)N * D * 2 * 2);
  hipLaunchKernelGGL((fa_bwd_dq_bf16_kernel<D, CAUSAL>), dim3((unsigned)(BH * ntiles)), dim3(256), 0, s,
                     (const bf16 *)Q, (const bf16 *)K, (const bf16 *)V, (const bf16 *)dO, (const bf16 *)O, L,
                     work, (bf16 *)dQ, N, ntiles, rows, c, scale, group);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((fa_bwd_dkdv_bf16_kernel<D, CAUSAL>), dim3((unsigned)(BH * ntiles)), dim3(512), 0, s,
                     (const bf16 *)Q, (const bf16 *)K, (const bf16 *)V, (const bf16 *)dO, work,
                     (bf16 *)dK, (bf16 *)dV, N, ntiles, rows, c, scale, group);
  return hipGetLastError();
}

template <int D, bool CAUSAL>
hipError_t launch_bwd_f32(int64_t BH, int N, hipStream_t s, const void *Q, const void *K,
                          const void *V, const void *O, const float *L, const void *dO, void *dQ,
                          void *dK, void *dV, float *work, float c, float scale) {
  const int64_t rows = BH * N;
  const int nb = (N + kF32Block - 1) / kF32Block;
  constexpr int prep_rows = 256 / (D / 4);
  hipLaunchKernelGGL((fa_bwd_prep_kernel<float, D>), dim3((unsigned)((rows + prep_rows - 1) / prep_rows)), dim3(256), 0, s,
                     (const float *)O, (const float *)dO, L, work, rows);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((fa_bwd_dq_f32_kernel<D, CAUSAL>), dim3((unsigned)(BH * nb)), dim3(64 * kF32BwdWaves), 0, s,
                     (const float *)Q, (const float *)K, (const float *)V, (const float *)dO, work,
                     (float *)dQ, N, nb, rows, c, scale);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((fa_bwd_dkdv_f32_kernel<D, CAUSAL>), dim3((unsigned)(BH * nb)), dim3(64 * kF32BwdWaves), 0, s,
                     (const float *)Q, (const float *)K, (const float *)V, (const float *)dO, work,
                     (float *)dK, (float *)dV, N, nb, rows, c, scale);
  return hipGetLastError();
}

bool overlaps(const void *a, size_t na, const void *b, size_t nb) {
  const uintptr_t x = (uintptr_t)a, y = (uintptr_t)b;
  return x < y + nb && y < x + na;
}


// Checks fa_bwd's arguments. `work` (2 * B * H * N floats of caller workspace)
// is checked only when `has_work`; the library's own workspace overlaps nothing.
fa_status_t bwd_validate(const void *Q, const void *K, const void *V, const void *O, const float *L,
                         const void *dO, void *dQ, void *dK, void *dV, const float *work, bool has_work,
                         int64_t B, int64_t H, int64_t N, int64_t d, float scale, int dtype) {
  if (!Q || !K || !V || !O || !L || !dO || !dQ || !dK || !dV || (has_work && !work))
    return FA_ERR_INVALID_ARGUMENT;
  if (B < 1 || H < 1 || N < 1) return FA_ERR_INVALID_ARGUMENT;
  if (!(scale > 0.f) || !isfinite((float)((double)scale * 1.4426950408889634074)))  // finite scale * log2(e)
    return FA_ERR_INVALID_ARGUMENT;
  if (dtype != FA_DTYPE_F32 && dtype != FA_DTYPE_BF16) return FA_ERR_INVALID_ARGUMENT;
  const bool bf = dtype == FA_DTYPE_BF16;
  // bf16: d = 64, 128 (the 8-wave dK/dV tile loads need 8 KiB tiles); fp32 also d = 32.
  if (d != 64 && d != 128 && !(d == 32 && !bf)) return FA_ERR_UNSUPPORTED;
  if (N > (int64_t)1 << 24) return FA_ERR_UNSUPPORTED;
  if (B > (int64_t)1 << 31 || H > (int64_t)1 << 31) return FA_ERR_UNSUPPORTED;  // B * H cannot overflow below
  const int64_t block_rows = bf ? kBwdRows : kF32Block;
  const int64_t ntiles = (N + block_rows - 1) / block_rows;
  if (B * H > ((int64_t)1 << 31) / ntiles - 1) return FA_ERR_UNSUPPORTED;
  if (B * H * N > ((int64_t)1 << 31) - 256) return FA_ERR_UNSUPPORTED;  // prep grid and row indices
  const size_t esize = bf ? 2 : 4;
  const size_t tbytes = (size_t)B * H * N * d * esize;
  const size_t lbytes = (size_t)B * H * N * sizeof(float);
  const void *ins[] = {Q, K, V, O, dO};
  void *outs[] = {dQ, dK, dV};
  for (void *o : outs) {
    for (const void *i : ins)
      if (overlaps(o, tbytes, i, tbytes)) return FA_ERR_INVALID_ARGUMENT;
    if (overlaps(o, tbytes, L, lbytes) || (has_work && overlaps(o, tbytes, work, 2 * lbytes)))
      return FA_ERR_INVALID_ARGUMENT;
  }
  if (overlaps(dQ, tbytes, dK, tbytes) || overlaps(dQ, tbytes, dV, tbytes) ||
      overlaps(dK, tbytes, dV, tbytes))
    return FA_ERR_INVALID_ARGUMENT;
  if (has_work) {
    for (const void *i : ins)
      if (overlaps(work, 2 * lbytes, i, tbytes)) return FA_ERR_INVALID_ARGUMENT;
    if (overlaps(work, 2 * lbytes, L, lbytes)) return FA_ERR_INVALID_ARGUMENT;
  }
  if (((uintptr_t)Q | (uintptr_t)K | (uintptr_t)V | (uintptr_t)O | (uintptr_t)L | (uintptr_t)dO |
       (uintptr_t)dQ | (uintptr_t)dK | (uintptr_t)dV | (has_work ? (uintptr_t)work : 0)) & 15)
    return FA_ERR_MISALIGNED;
  return FA_OK;
}

// Enqueues the kernels for validated arguments (bf16: dQ then dK/dV; fp32:
// preprocessing, dQ, dK/dV).
fa_status_t bwd_launch(const void *Q, const void *K, const void *V, const void *O, const float *L,
                       const void *dO, void *dQ, void *dK, void *dV, float *work, int64_t B, int64_t H,
                       int64_t N, int64_t d, int causal, float scale, void *stream, int dtype) {
  const bool bf = dtype == FA_DTYPE_BF16;
  const float c = (float)((double)scale * 1.4426950408889634074);  // scale * log2(e)
  hipStream_t s = (hipStream_t)stream;
  const int n = (int)N;
  const int64_t BH = B * H;
  hipError_t err;
  if (bf) {
    if (d == 64)
      err = causal ? launch_bwd_bf16<64, true>(BH, n, s, Q, K, V, O, L, dO, dQ, dK, dV, work, c, scale)
                   : launch_bwd_bf16<64, false>(BH, n, s, Q, K, V, O, L, dO, dQ, dK, dV, work, c, scale);
    else
      err = causal ? launch_bwd_bf16<128, true>(BH, n, s, Q, K, V, O, L, dO, dQ, dK, dV, work, c, scale)
                   : launch_bwd_bf16<128, false>(BH, n, s, Q, K, V, O, L, dO, dQ, dK, dV, work, c, scale);
  } else {
    if (d == 32)
      err = causal ? launch_bwd_f32<32, true>(BH, n, s, Q, K, V, O, L, dO, dQ, dK, dV, work, c, scale)
                   : launch_bwd_f32<32, false>(BH, n, s, Q, K, V, O, L, dO, dQ, dK, dV, work, c, scale);
    else if (d == 64)
      err = causal ? launch_bwd_f32<64, true>(BH, n, s, Q, K, V, O, L, dO, dQ, dK, dV, work, c, scale)
                   : launch_bwd_f32<64, false>(BH, n, s, Q, K, V, O, L, dO, dQ, dK, dV, work, c, scale);
    else
      err = causal ? launch_bwd_f32<128, true>(BH, n, s, Q, K, V, O, L, dO, dQ, dK, dV, work, c, scale)
                   : launch_bwd_f32<128, false>(BH, n, s, Q, K, V, O, L, dO, dQ, dK, dV, work, c, scale);
  }
  return err == hipSuccess ? FA_OK : FA_ERR_LAUNCH;
}

}  // namespace

// Workspace of the allocation-free entry point: one array per GPU, for the
// process's lifetime, shared by every fa_bwd_noalloc call on that GPU. In host
// code `scratch` names a host-side stand-in; the device address is fetched with
// hipGetSymbolAddress and used everywhere instead.
constexpr int64_t kBwdScratchFloats = (int64_t)1 << 21;  // 8 MiB: B * H * N <= 2^20 rows
static __device__ __align__(256) float scratch[kBwdScratchFloats];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mutex;
float *g_scratch_ptr[kMaxDevices];  // device address of `scratch` per device, once fetched

// The device address of `scratch` on the device of `stream` (fetched on the
// first call on that device, with that device current; the caller's current
// device is restored), or null on failure.
float *device_scratch(hipStream_t stream) {
  int dev = 0;
  if (stream_device(stream, &dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> lock(g_scratch_mutex);
  if (!g_scratch_ptr[dev]) {
    void *ptr = nullptr;
    const hipError_t e =
        on_device(dev, [&] { return hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) == hipSuccess && ptr; });
    if (e != hipSuccess) return nullptr;
    g_scratch_ptr[dev] = (float *)ptr;
  }
  return g_scratch_ptr[dev];
}

}  // namespace

extern "C" fa_status_t fa_bwd(const void *Q, const void *K, const void *V, const void *O,
                              const float *L, const void *dO, void *dQ, void *dK, void *dV,
                              float *work, int64_t B, int64_t H, int64_t N, int64_t d, int causal,
                              float scale, void *stream, int dtype) {
  const fa_status_t st = bwd_validate(Q, K, V, O, L, dO, dQ, dK, dV, work, true, B, H, N, d, scale, dtype);
  if (st != FA_OK) return st;
  return bwd_launch(Q, K, V, O, L, dO, dQ, dK, dV, work, B, H, N, d, causal, scale, stream, dtype);
}

extern "C" fa_status_t fa_bwd_noalloc(const void *Q, const void *K, const void *V, const void *O,
                                      const float *L, const void *dO, void *dQ, void *dK, void *dV,
                                      int64_t B, int64_t H, int64_t N, int64_t d, int causal,
                                      float scale, void *stream, int dtype) {
  if (B < 1 || H < 1 || N < 1) return FA_ERR_INVALID_ARGUMENT;
  // Each factor, then B * H, then the rows: no product below can overflow.
  if (B > kBwdScratchFloats || H > kBwdScratchFloats || N > kBwdScratchFloats || B * H > kBwdScratchFloats ||
      2 * B * H * N > kBwdScratchFloats)
    return FA_ERR_SCRATCH_LIMIT;
  const fa_status_t st = bwd_validate(Q, K, V, O, L, dO, dQ, dK, dV, nullptr, false, B, H, N, d, scale, dtype);
  if (st != FA_OK) return st;
  float *work = device_scratch((hipStream_t)stream);
  if (!work) return FA_ERR_LAUNCH;
  return bwd_launch(Q, K, V, O, L, dO, dQ, dK, dV, work, B, H, N, d, causal, scale, stream, dtype);
}
