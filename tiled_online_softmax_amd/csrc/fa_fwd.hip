// Tiled online-softmax attention forward pass for CDNA4 (gfx950, MI355X).
//
// Computes O = softmax(scale * Q K^T) V per head, optionally causal, and the
// per-row natural-log logsumexp L, without storing the N x N score matrix.
//
// The method: "FlashAttention-2 from PyTorch to Triton", section "What We Are
// Building" -- one workgroup per query tile, K/V tiles streamed past it, a
// running row maximum m, running row sum l and an unnormalised output
// accumulator that is rescaled by exp(m_old - m_new) on every key tile and
// divided by l once at the end; L = m + log l. The recurrence itself is the one
// derived in "Writing a FlashAttention kernel in Metal", sections "Online
// softmax", "One-query attention" and "Blockwise attention and causal
// masking"; the base-2 form with the guarded correction factor follows the
// softmax fragment of "Case Study: metal-flash-attention".
//
// gfx950 mapping (see the layout comments at each step):
//  * A workgroup of four wave64s owns 128 query rows; each wave owns 32 rows
//    and keeps its Q rows in VGPRs for the whole key loop.
//  * Scores are formed transposed, S^T = K Q^T, with v_mfma_f32_32x32x16_bf16
//    (bf16) or v_mfma_f32_32x32x2_f32 (fp32). In the result layout a lane holds
//    16 keys of ONE query, so the row maximum and row sum are 16 in-lane ops
//    plus one v_permlane32_swap between the two half-waves, and the running
//    state m, l is a per-lane scalar.
//  * The same registers, converted to bf16, are the B operand of the second
//    contraction O^T += V^T P^T with no data movement; V^T comes straight out
//    of LDS with ds_read_b64_tr_b16 (transposing 4-key x 16-column blocks).
//  * K/V tiles of 64 keys are staged through padded LDS rows; the global loads
//    of tile j+1 are in flight while tile j is computed.
//  * Scores are scaled into the base-2 domain (scale * log2 e folded into one
//    FMA) and exponentiated with v_exp_f32.
//  * Causal: key tiles wholly after the query tile are never loaded, 32-key
//    blocks wholly after a wave's rows are skipped by that wave, and the mask
//    is evaluated only on blocks that straddle the diagonal or the ragged end.
//  * The workgroup index is remapped so that the eight XCDs each own whole
//    heads (their L2 keeps that head's K/V), heaviest causal tiles first.

#include <hip/hip_runtime.h>

#include <math.h>
#include <stddef.h>
#include <stdint.h>

#include "fa.h"

namespace {

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;     // four wave64s
constexpr int kRowsPerWave = 32;  // query rows per wave (MFMA N dimension)
constexpr int kBlockM = 128;      // query rows per workgroup
constexpr int kNumXcd = 8;        // MI355X: 8 XCDs, workgroups dispatched round-robin
constexpr float kLn2 = 0.69314718055994530942f;

typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float log2_fast(float x) { return __builtin_amdgcn_logf(x); }

// Value held by the partner lane in the other half-wave (lane ^ 32), combined.
__device__ __forceinline__ float halves_max(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float halves_sum(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Workgroup index -> (head, query tile). Workgroups are dispatched to XCDs
// round-robin (bid % 8); renumber them so each XCD receives one contiguous
// run of the logical order, in its own dispatch order. The logical order is
// head-major; for causal attention query tiles run from the last (most key
// tiles) to the first within each head.
__device__ __forceinline__ void map_block(int bid, int nblocks, int n_qtiles, bool causal,
                                          int &bh, int &qt) {
  const int xcd = bid % kNumXcd;
  const int slot = bid / kNumXcd;
  const int base = nblocks / kNumXcd, extra = nblocks % kNumXcd;
  const int logical = xcd * base + min(xcd, extra) + slot;
  bh = logical / n_qtiles;
  const int t = logical % n_qtiles;
  qt = causal ? (n_qtiles - 1 - t) : t;
}

// ---------------------------------------------------------------------------
// bf16 kernel: Q, K, V, O bf16; S, P, m, l, O accumulation fp32; P rounded to
// bf16 (the element type of V) only as the operand of the second MFMA.
// ---------------------------------------------------------------------------
template <int D, bool CAUSAL>
__global__ __launch_bounds__(kThreads, 2) void fa_fwd_bf16_kernel(
    const bf16 *__restrict__ Q, const bf16 *__restrict__ K, const bf16 *__restrict__ V,
    bf16 *__restrict__ O, float *__restrict__ L, int N, int n_qtiles, float c) {
  constexpr int BN = 64;               // keys per LDS tile
  constexpr int KS = D + 8;            // K row stride in LDS (elements): 16 B pad
  constexpr int VS = D + 32;           // V row stride in LDS (elements): 64 B pad
  constexpr int CPR = D / 8;           // 16-byte chunks per row
  constexpr int PER_T = BN * CPR / kThreads;  // chunks of K (and of V) per thread
  static_assert(BN * CPR % kThreads == 0, "tile must split evenly over the workgroup");

  __shared__ __attribute__((aligned(16))) bf16 Ks[BN * KS];
  __shared__ __attribute__((aligned(16))) bf16 Vs[BN * VS];

  const int tid = threadIdx.x;
  const int wave = tid / 64, lane = tid % 64;
  const int l32 = lane % 32, hh = lane / 32;

  int bh, qt;
  map_block(blockIdx.x, gridDim.x, n_qtiles, CAUSAL, bh, qt);
  const size_t head = (size_t)bh * (size_t)N * D;
  const bf16 *Qh = Q + head;
  const bf16 *Kh = K + head;
  const bf16 *Vh = V + head;

  const int q0 = qt * kBlockM;
  const int qw = q0 + kRowsPerWave * wave;  // first query row of this wave
  const int qrow = qw + l32;                // the query row this lane carries

  // Q as the B operand of S^T = K Q^T: lane holds Q[qrow][16c + 8hh + 0..7].
  bf16x8 qf[D / 16];
#pragma unroll
  for (int cc = 0; cc < D / 16; ++cc) {
    if (qrow < N)
      qf[cc] = *(const bf16x8 *)(Qh + (size_t)qrow * D + 16 * cc + 8 * hh);
    else
      qf[cc] = bf16x8{};
  }

  f32x16 o[D / 32];
#pragma unroll
  for (int db = 0; db < D / 32; ++db) o[db] = f32x16{};
  float m = -INFINITY;  // running row maximum, base-2 scaled domain
  float lsum = 0.f;     // running row sum over this half-wave's keys

  const int kend = CAUSAL ? min(N, q0 + kBlockM) : N;
  const int ntiles = (kend + BN - 1) / BN;

  // Global -> register staging of one K/V tile (contiguous rows of the head).
  u32x4 kr[PER_T], vr[PER_T];
  auto gload = [&](int t) {
#pragma unroll
    for (int i = 0; i < PER_T; ++i) {
      const int idx = tid + kThreads * i;
      const int row = idx / CPR, ch = idx % CPR;
      const int key = t * BN + row;
      if (key < N) {
        kr[i] = *(const u32x4 *)(Kh + (size_t)key * D + 8 * ch);
        vr[i] = *(const u32x4 *)(Vh + (size_t)key * D + 8 * ch);
      } else {  // ragged end: zero rows (their scores are masked as well)
        kr[i] = u32x4{};
        vr[i] = u32x4{};
      }
    }
  };
  auto swrite = [&]() {
#pragma unroll
    for (int i = 0; i < PER_T; ++i) {
      const int idx = tid + kThreads * i;
      const int row = idx / CPR, ch = idx % CPR;
      *(u32x4 *)(&Ks[row * KS + 8 * ch]) = kr[i];
      *(u32x4 *)(&Vs[row * VS + 8 * ch]) = vr[i];
    }
  };

  gload(0);
  for (int t = 0; t < ntiles; ++t) {
    __syncthreads();  // every wave is done reading the previous tile
    swrite();
    __syncthreads();  // the tile is complete in LDS
    if (t + 1 < ntiles) gload(t + 1);

    if (qw >= N) continue;  // wave past the ragged end: loads and barriers only
    const int k0 = t * BN;

    // S^T blocks of 32 keys x 32 queries. Result layout: lane (l32, hh),
    // register r holds key 8(r/4) + 4hh + r%4 of the block, query qrow.
    f32x16 s[2];
    bool act[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      const int kb0 = k0 + 32 * kb;
      act[kb] = kb0 < N && (!CAUSAL || kb0 <= qw + kRowsPerWave - 1);
      s[kb] = f32x16{};
      if (act[kb]) {
#pragma unroll
        for (int cc = 0; cc < D / 16; ++cc) {
          // A operand: K[kb0 + l32][16cc + 8hh + 0..7]
          const bf16x8 a = *(const bf16x8 *)(&Ks[(32 * kb + l32) * KS + 16 * cc + 8 * hh]);
          s[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[cc], s[kb], 0, 0, 0);
        }
        const bool edge = (kb0 + 31 >= N) || (CAUSAL && kb0 + 31 > qw);
        if (edge) {
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int key = kb0 + 8 * (r / 4) + 4 * hh + (r % 4);
            if (key >= N || (CAUSAL && key > qrow)) s[kb][r] = -INFINITY;
          }
        }
      } else {
#pragma unroll
        for (int r = 0; r < 16; ++r) s[kb][r] = -INFINITY;
      }
    }

    // Row maximum over the tile, then the online-softmax update.
    float mx = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[kb][r]);
    mx = halves_max(mx);
    const float m_new = fmaxf(m, mx * c);
    // Guard: a row with no admissible key so far keeps a zero reference so
    // that no -inf - -inf appears (such rows have l == 0 and O == 0).
    const float m_ref = (m_new == -INFINITY) ? 0.f : m_new;
    const float alpha = exp2_fast(m - m_ref);
    m = m_new;

    float psum = 0.f;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float p = exp2_fast(fmaf(s[kb][r], c, -m_ref));
        s[kb][r] = p;
        psum += p;
      }
    lsum = fmaf(alpha, lsum, psum);
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int r = 0; r < 16; ++r) o[db][r] *= alpha;

    // O^T += V^T P^T. B operand (P^T, keys x queries) for key half mm of
    // block kb is registers 8mm..8mm+7 of s[kb], i.e. keys
    // 16mm + 8(t/4) + 4hh + t%4 for slot t; the A operand (V^T, d x keys)
    // must list the same keys: two transposing reads of 4 consecutive keys.
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      if (!act[kb]) continue;
#pragma unroll
      for (int mm = 0; mm < 2; ++mm) {
        bf16x8 pb;
#pragma unroll
        for (int t8 = 0; t8 < 8; ++t8) pb[t8] = (bf16)s[kb][8 * mm + t8];
        const int vrow = 32 * kb + 16 * mm + 4 * hh + (lane % 16) / 4;
        const int vcol = 16 * ((lane / 16) % 2) + 4 * (lane % 4);
#pragma unroll
        for (int db = 0; db < D / 32; ++db) {
          const bf16 *p0 = &Vs[vrow * VS + 32 * db + vcol];
          const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4 *)(p0));
          const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4 *)(p0 + 8 * VS));
          const bf16x8 a = __builtin_bit_cast(
              bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
          o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pb, o[db], 0, 0, 0);
        }
      }
    }
  }

  if (qw >= N) return;
  // Epilogue: one division by the row sum (both half-waves' keys), RNE to bf16.
  const float ltot = halves_sum(lsum);
  if (qrow < N) {
    const float inv = 1.f / ltot;
    bf16 *orow = O + head + (size_t)qrow * D;
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        bf16x4 v4;
#pragma unroll
        for (int e = 0; e < 4; ++e) v4[e] = (bf16)(o[db][4 * g + e] * inv);
        *(bf16x4 *)(orow + 32 * db + 8 * g + 4 * hh) = v4;
      }
    if (hh == 0) L[(size_t)bh * N + qrow] = (m + log2_fast(ltot)) * kLn2;
  }
}

// ---------------------------------------------------------------------------
// fp32 kernel: everything in fp32 (v_mfma_f32_32x32x2_f32); P is not rounded.
// Same work mapping and state layout as the bf16 kernel. The contraction over
// d is split between the half-waves as d = hh * D/2 + cc, so each lane reads
// contiguous runs of K and Q.
// ---------------------------------------------------------------------------
template <int D, bool CAUSAL>
__global__ __launch_bounds__(kThreads, 2) void fa_fwd_f32_kernel(
    const float *__restrict__ Q, const float *__restrict__ K, const float *__restrict__ V,
    float *__restrict__ O, float *__restrict__ L, int N, int n_qtiles, float c) {
  constexpr int BN = 32;      // keys per LDS tile
  constexpr int KS = D + 8;   // row strides in LDS (floats)
  constexpr int VS = D + 8;
  constexpr int CPR = D / 4;  // 16-byte chunks per row
  constexpr int PER_T = BN * CPR / kThreads;
  constexpr int HD = D / 2;
  static_assert(BN * CPR % kThreads == 0, "tile must split evenly over the workgroup");

  __shared__ __attribute__((aligned(16))) float Ks[BN * KS];
  __shared__ __attribute__((aligned(16))) float Vs[BN * VS];

  const int tid = threadIdx.x;
  const int wave = tid / 64, lane = tid % 64;
  const int l32 = lane % 32, hh = lane / 32;

  int bh, qt;
  map_block(blockIdx.x, gridDim.x, n_qtiles, CAUSAL, bh, qt);
  const size_t head = (size_t)bh * (size_t)N * D;
  const float *Qh = Q + head;
  const float *Kh = K + head;
  const float *Vh = V + head;

  const int q0 = qt * kBlockM;
  const int qw = q0 + kRowsPerWave * wave;
  const int qrow = qw + l32;

  // B operand of S^T = K Q^T for step cc: Q[qrow][hh * D/2 + cc].
  float qf[HD];
#pragma unroll
  for (int c4 = 0; c4 < HD / 4; ++c4) {
    f32x4 v = (qrow < N) ? *(const f32x4 *)(Qh + (size_t)qrow * D + hh * HD + 4 * c4) : f32x4{};
#pragma unroll
    for (int e = 0; e < 4; ++e) qf[4 * c4 + e] = v[e];
  }

  f32x16 o[D / 32];
#pragma unroll
  for (int db = 0; db < D / 32; ++db) o[db] = f32x16{};
  float m = -INFINITY, lsum = 0.f;

  const int kend = CAUSAL ? min(N, q0 + kBlockM) : N;
  const int ntiles = (kend + BN - 1) / BN;

  u32x4 kr[PER_T], vr[PER_T];
  auto gload = [&](int t) {
#pragma unroll
    for (int i = 0; i < PER_T; ++i) {
      const int idx = tid + kThreads * i;
      const int row = idx / CPR, ch = idx % CPR;
      const int key = t * BN + row;
      if (key < N) {
        kr[i] = *(const u32x4 *)(Kh + (size_t)key * D + 4 * ch);
        vr[i] = *(const u32x4 *)(Vh + (size_t)key * D + 4 * ch);
      } else {
        kr[i] = u32x4{};
        vr[i] = u32x4{};
      }
    }
  };
  auto swrite = [&]() {
#pragma unroll
    for (int i = 0; i < PER_T; ++i) {
      const int idx = tid + kThreads * i;
      const int row = idx / CPR, ch = idx % CPR;
      *(u32x4 *)(&Ks[row * KS + 4 * ch]) = kr[i];
      *(u32x4 *)(&Vs[row * VS + 4 * ch]) = vr[i];
    }
  };

  gload(0);
  for (int t = 0; t < ntiles; ++t) {
    __syncthreads();
    swrite();
    __syncthreads();
    if (t + 1 < ntiles) gload(t + 1);

    if (qw >= N) continue;
    const int k0 = t * BN;
    if (CAUSAL && k0 > qw + kRowsPerWave - 1) continue;  // block wholly after this wave's rows

    f32x16 s = f32x16{};
#pragma unroll
    for (int c4 = 0; c4 < HD / 4; ++c4) {
      const f32x4 a4 = *(const f32x4 *)(&Ks[l32 * KS + hh * HD + 4 * c4]);
#pragma unroll
      for (int e = 0; e < 4; ++e)
        s = __builtin_amdgcn_mfma_f32_32x32x2f32(a4[e], qf[4 * c4 + e], s, 0, 0, 0);
    }
    const bool edge = (k0 + 31 >= N) || (CAUSAL && k0 + 31 > qw);
    if (edge) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int key = k0 + 8 * (r / 4) + 4 * hh + (r % 4);
        if (key >= N || (CAUSAL && key > qrow)) s[r] = -INFINITY;
      }
    }

    float mx = -INFINITY;
#pragma unroll
    for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[r]);
    mx = halves_max(mx);
    const float m_new = fmaxf(m, mx * c);
    const float m_ref = (m_new == -INFINITY) ? 0.f : m_new;
    const float alpha = exp2_fast(m - m_ref);
    m = m_new;

    float psum = 0.f;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const float p = exp2_fast(fmaf(s[r], c, -m_ref));
      s[r] = p;
      psum += p;
    }
    lsum = fmaf(alpha, lsum, psum);
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int r = 0; r < 16; ++r) o[db][r] *= alpha;

    // O^T += V^T P^T, two keys per MFMA: key slot hh of step r is key
    // 8(r/4) + 4hh + r%4, whose P value is register r of this lane.
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int vrow = 8 * (r / 4) + 4 * hh + (r % 4);
#pragma unroll
      for (int db = 0; db < D / 32; ++db) {
        const float a = Vs[vrow * VS + 32 * db + l32];
        o[db] = __builtin_amdgcn_mfma_f32_32x32x2f32(a, s[r], o[db], 0, 0, 0);
      }
    }
  }

  if (qw >= N) return;
  const float ltot = halves_sum(lsum);
  if (qrow < N) {
    const float inv = 1.f / ltot;
    float *orow = O + head + (size_t)qrow * D;
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        f32x4 v4;
#pragma unroll
        for (int e = 0; e < 4; ++e) v4[e] = o[db][4 * g + e] * inv;
        *(f32x4 *)(orow + 32 * db + 8 * g + 4 * hh) = v4;
      }
    if (hh == 0) L[(size_t)bh * N + qrow] = (m + log2_fast(ltot)) * kLn2;
  }
}

template <typename Kern>
hipError_t launch(Kern kern, int nblocks, hipStream_t stream, const void *Q, const void *K,
                  const void *V, void *O, float *L, int N, int n_qtiles, float c) {
  void *args[] = {(void *)&Q, (void *)&K, (void *)&V, (void *)&O,
                  (void *)&L, (void *)&N, (void *)&n_qtiles, (void *)&c};
  return hipLaunchKernel((const void *)kern, dim3(nblocks), dim3(kThreads), args, 0, stream);
}

bool overlaps(const void *a, size_t na, const void *b, size_t nb) {
  const uintptr_t x = (uintptr_t)a, y = (uintptr_t)b;
  return x < y + nb && y < x + na;
}

}  // namespace

extern "C" fa_status_t fa_fwd(const void *Q, const void *K, const void *V, void *O, float *L,
                              int64_t B, int64_t H, int64_t N, int64_t d, int causal,
                              float scale, void *stream, int dtype) {
  if (!Q || !K || !V || !O || !L) return FA_ERR_INVALID_ARGUMENT;
  if (B < 1 || H < 1 || N < 1) return FA_ERR_INVALID_ARGUMENT;
  if (!(scale > 0.f) || !isfinite(scale)) return FA_ERR_INVALID_ARGUMENT;
  if (dtype != FA_DTYPE_F32 && dtype != FA_DTYPE_BF16) return FA_ERR_INVALID_ARGUMENT;
  const size_t esize = dtype == FA_DTYPE_BF16 ? 2 : 4;
  // Sizes: 32-bit row indices inside a head, grid size below 2^31.
  if (d != 64 && d != 128) return FA_ERR_UNSUPPORTED;
  if (N > (int64_t)1 << 24) return FA_ERR_UNSUPPORTED;
  const int64_t n_qtiles = (N + kBlockM - 1) / kBlockM;
  if (B * H > ((int64_t)1 << 31) / n_qtiles - 1) return FA_ERR_UNSUPPORTED;
  const size_t nelem = (size_t)B * (size_t)H * (size_t)N * (size_t)d;
  const size_t obytes = nelem * esize, lbytes = (size_t)B * H * N * sizeof(float);
  if (overlaps(O, obytes, Q, obytes) || overlaps(O, obytes, K, obytes) ||
      overlaps(O, obytes, V, obytes) || overlaps(O, obytes, L, lbytes) ||
      overlaps(L, lbytes, Q, obytes) || overlaps(L, lbytes, K, obytes) ||
      overlaps(L, lbytes, V, obytes))
    return FA_ERR_INVALID_ARGUMENT;
  if (((uintptr_t)Q | (uintptr_t)K | (uintptr_t)V | (uintptr_t)O | (uintptr_t)L) & 15)
    return FA_ERR_MISALIGNED;

  const int nblocks = (int)(B * H * n_qtiles);
  const float c = (float)((double)scale * 1.4426950408889634074);  // scale * log2(e)
  hipStream_t s = (hipStream_t)stream;
  const int n = (int)N, nq = (int)n_qtiles;
  hipError_t err;
  if (dtype == FA_DTYPE_BF16) {
    if (d == 64)
      err = causal ? launch(fa_fwd_bf16_kernel<64, true>, nblocks, s, Q, K, V, O, L, n, nq, c)
                   : launch(fa_fwd_bf16_kernel<64, false>, nblocks, s, Q, K, V, O, L, n, nq, c);
    else
      err = causal ? launch(fa_fwd_bf16_kernel<128, true>, nblocks, s, Q, K, V, O, L, n, nq, c)
                   : launch(fa_fwd_bf16_kernel<128, false>, nblocks, s, Q, K, V, O, L, n, nq, c);
  } else {
    if (d == 64)
      err = causal ? launch(fa_fwd_f32_kernel<64, true>, nblocks, s, Q, K, V, O, L, n, nq, c)
                   : launch(fa_fwd_f32_kernel<64, false>, nblocks, s, Q, K, V, O, L, n, nq, c);
    else
      err = causal ? launch(fa_fwd_f32_kernel<128, true>, nblocks, s, Q, K, V, O, L, n, nq, c)
                   : launch(fa_fwd_f32_kernel<128, false>, nblocks, s, Q, K, V, O, L, n, nq, c);
  }
  return err == hipSuccess ? FA_OK : FA_ERR_LAUNCH;
}

extern "C" const char *fa_status_string(int status) {
  switch (status) {
    case FA_OK: return "ok";
    case FA_ERR_INVALID_ARGUMENT: return "invalid argument";
    case FA_ERR_UNSUPPORTED: return "unsupported head dimension or size";
    case FA_ERR_MISALIGNED: return "buffer not 16-byte aligned";
    case FA_ERR_LAUNCH: return "kernel launch failed";
    default: return "unknown status";
  }
}

extern "C" int fa_version(void) { return 100; }
