// Device code of the tiled online-softmax attention forward pass (gfx950):
// the parameter block and the two kernel templates. Included by the library's
// forward source and, as text, compiled at run time by hipRTC for the
// shape-specialized entry point; it holds no host code.
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
//  * bf16: a workgroup of four wave64s owns 128 query rows; each wave owns 32
//    rows and keeps its Q rows in VGPRs for the whole key loop (grids too small
//    to fill the chip: 64 rows, two waves per 32 rows splitting the keys). fp32: a
//    workgroup owns 32 query rows and its waves split the key tiles, merging
//    their partial (m, l, O) through LDS at the end.
//  * Scores are formed transposed, S^T = K Q^T, with v_mfma_f32_32x32x16_bf16
//    (bf16) or v_mfma_f32_32x32x2_f32 (fp32). In the result layout a lane holds
//    16 keys of ONE query, so the row maximum and row sum are 16 in-lane ops
//    plus one v_permlane32_swap between the two half-waves, and the running
//    state m, l is a per-lane scalar.
//  * The same registers, converted to bf16, are the B operand of the second
//    contraction O^T += V^T P^T with no data movement; V^T comes straight out
//    of LDS with ds_read_b64_tr_b16 (transposing 4-key x 16-column blocks).
//  * bf16: K/V tiles of 64 keys are copied global -> LDS (XOR-swizzled rows),
//    K two tiles and V one tile ahead of their use. fp32: each wave loads its
//    32-key K/V operands straight into VGPRs, the next tile's loads in flight
//    while the current tile is computed.
//  * Scores are scaled into the base-2 domain (scale * log2 e folded into one
//    FMA) and exponentiated with v_exp_f32.
//  * Causal: key tiles wholly after the query tile are never loaded, 32-key
//    blocks wholly after a wave's rows are skipped by that wave, and the mask
//    is evaluated only on blocks that straddle the diagonal or the ragged end.
//  * The workgroup index is remapped so that the eight XCDs each own whole
//    heads (their L2 keeps that head's K/V) and take them a few at a time
//    (the heads whose K and V total at most 8 MiB), heaviest causal tiles
//    first.
//
// Shape specialization: when FA_SPEC_NQ is defined (hipRTC builds), the row
// counts, the batch and head counts and the strides of a contiguous
// [B][H][N][d] layout are compile-time constants (FA_SPEC_B, FA_SPEC_H,
// FA_SPEC_NQ, FA_SPEC_NK) instead of parameter-block fields; the kernels are
// otherwise the same.
#ifndef FA_FWD_KERNELS_H_
#define FA_FWD_KERNELS_H_

#include "fa_device.h"

#include <type_traits>

namespace {

// ---------------------------------------------------------------------------
// bf16 kernel: Q, K, V, O bf16; S, P, m, l, O accumulation fp32; P rounded to
// bf16 (the element type of V) only as the operand of the second MFMA.
//
// LDS: two stages, each holding one K tile and one V tile of BN keys. Tiles are
// written by buffer_load_dwordx4 ... lds (global -> LDS without VGPRs, 1 KiB
// per wave instruction, lane l writing bytes [16l, 16l+16)); rows past N read
// as zero through the buffer range check. Inside a row the 16-byte chunks are
// XOR-permuted so that both read patterns are free of bank conflicts:
//  * K (ds_read_b128, lanes = 32 consecutive keys, same chunk): chunk c of
//    row r sits in slot c ^ swz_k(r), with swz_k spreading 16 consecutive rows
//    over the 16 slots of a 256-byte bank line;
//  * V (ds_read_b64_tr_b16, a 16-lane group reads 4 consecutive rows x 32
//    bytes and its partner group the next 32 bytes): slot c ^ swz_v(r) with
//    swz_v(r) = 4 * (row index within the group of 4) so the 4 x 4 chunks of
//    a group pair land in 16 distinct slots.
//
// Software pipeline (per wave, iteration j):
//   phase 1: MFMAs of S(j+1) = K(j+1) Q^T   |  VALU: P(j) = exp2(S(j) c - m) to bf16, its row sum
//            and, only if some row's sum reached 2^8 (a row maximum grew past the
//            reference plus the slack; rare, since a moved reference sits 64 above
//            the maximum): the row maximum of S(j), the moved reference, O and l
//            rescaled, P(j) and its sum formed again
//   phase 2: MFMAs of O += V(j)^T P(j)^T     |  VALU: mask of S(j+1) (edge tiles)
// K runs one tile ahead of V: iteration j reads K(j+1) and V(j); the loads
// issued at its start fill K(j+2) and V(j+1), so every load has a whole
// iteration to land before the barrier that publishes it.
// ---------------------------------------------------------------------------

// One call's operands. Q, O are B x H x Nq x d, K, V are B x H x Nk x d, all
// with unit stride along d; strides are in elements (batch, head, row). L is
// B x H x Nq fp32 with its own strides. The host validates that every row
// starts 16-byte aligned and that a row stride times the element size is at
// most 2^24 bytes, so a tile of up to 64 rows spans less than 2^30 bytes (the
// buffer-offset range used below, with 2^30 marking a load as out of range).
struct FwdParams {
  const void *Q, *K, *V;
  void *O;
  float *L;
  int64_t q_b, q_h, k_b, k_h, v_b, v_h, o_b, o_h, l_b, l_h;
  int q_r, k_r, v_r, o_r, l_r;
  int H, Nq, Nk, n_qtiles;
  int head_group;  // heads an XCD works on at a time (map_block)
  float c;         // scale * log2(e)
};

// The sizes and strides a kernel works with: the parameter block's fields, or,
// in a shape-specialized build, compile-time constants of a contiguous
// [B][H][N][d] layout. BM is the kernel's query rows per workgroup.
template <int D, int BM>
struct Shape {
#if defined(FA_SPEC_NQ)
  static constexpr int B = FA_SPEC_B, H = FA_SPEC_H, Nq = FA_SPEC_NQ, Nk = FA_SPEC_NK;
  static constexpr int n_qtiles = (Nq + BM - 1) / BM;
  static constexpr int q_r = D, k_r = D, v_r = D, o_r = D, l_r = 1;
  static constexpr int64_t q_h = (int64_t)Nq * D, k_h = (int64_t)Nk * D, v_h = k_h, o_h = q_h, l_h = Nq;
  static constexpr int64_t q_b = H * q_h, k_b = H * k_h, v_b = k_b, o_b = q_b, l_b = H * l_h;
  int group;
  __device__ explicit Shape(const FwdParams &p) : group(p.head_group) {}
  // Workgroup -> (batch * head, query tile); the grid size is a constant too.
  __device__ void place(bool causal, int &bh, int &qt) const {
    map_block(blockIdx.x, B * H * n_qtiles, n_qtiles, causal, group, bh, qt);
  }
#else
  int H, Nq, Nk, n_qtiles, group;
  int q_r, k_r, v_r, o_r, l_r;
  int64_t q_h, k_h, v_h, o_h, l_h, q_b, k_b, v_b, o_b, l_b;
  __device__ explicit Shape(const FwdParams &p)
      : H(p.H), Nq(p.Nq), Nk(p.Nk), n_qtiles(p.n_qtiles), group(p.head_group), q_r(p.q_r), k_r(p.k_r),
        v_r(p.v_r), o_r(p.o_r), l_r(p.l_r), q_h(p.q_h), k_h(p.k_h), v_h(p.v_h), o_h(p.o_h), l_h(p.l_h), q_b(p.q_b), k_b(p.k_b),
        v_b(p.v_b), o_b(p.o_b), l_b(p.l_b) {}
  __device__ void place(bool causal, int &bh, int &qt) const {
    map_block(blockIdx.x, gridDim.x, n_qtiles, causal, group, bh, qt);
  }
#endif
};

// Buffer offset that always fails the range check (reads as zero).
constexpr int kOutOfRange = 1 << 30;

// Rows of a reference maximum may lag the true running maximum by up to this
// much (base-2 exponent) before the accumulators are rescaled: weights stay
// below 2^8, and O/l and m + log2 l do not depend on the reference chosen.
constexpr float kRescaleSlack = 8.0f;

// bf16 kernel: a reference that moves is set this far above the row maximum
// (base-2 exponent), so a row rescales only once its maximum has grown by more
// than 64 + 8 since the reference last moved (with wide logits it otherwise
// grows past the slack on most tiles). The weights stay below 2^8 as above; the
// row's leading weights are about 2^-64, normal in fp32 and bf16. A weight
// underflows to zero only for a key more than 62 below the row maximum, a
// relative weight below 2^-62 per key (below 2^-38 for 2^24 keys).
constexpr float kReferenceLead = 64.0f;

// D < 32 (d = 16) runs on the layout of D = 32: the missing columns of the K
// and V tiles are filled with zeros by out-of-range loads, Q's with zeros, and
// the extra output columns are not stored.
//
// Key split KS > 1 (for grids too small to occupy every compute unit): the
// waves form NW / KS groups of 32 query rows, and wave ks of a group takes the
// 32-key blocks ks, ks + KS, ... of every tile; all waves still load and share
// the same LDS tiles. Each wave keeps its own (m, l, O) over its keys, and at
// the end the other waves of a group hand theirs to wave 0 of the group through
// LDS, which merges them by the rule that combines two key blocks (rescale each
// by exp2 of its reference maximum minus the larger one, then add).
template <int D, bool CAUSAL, int NW, int BN, int KS = 1>
__global__ __launch_bounds__(NW * 64, NW == 4 ? 2 : 1) void fa_fwd_bf16_kernel(const FwdParams p) {
  constexpr int DP = D < 32 ? 32 : D;    // head dimension of the tile layout
  using LY = BfLayout<DP, BN, NW>;
  constexpr int NKB = BN / 32;           // 32-key MFMA blocks per tile
  static_assert(NW % KS == 0 && NKB % KS == 0, "the key split divides the waves and the blocks of a tile");
  constexpr int NKW = NKB / KS;          // 32-key blocks per tile of one wave
  constexpr int BM = kRowsPerWave * (NW / KS);  // query rows per workgroup
  constexpr int NDB = DP / 32;           // 32-column blocks of the output
  constexpr int NCC = DP / 16;           // 16-wide steps of the score contraction
  __shared__ __attribute__((aligned(1024))) char smem[2 * LY::STAGE];

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid / 64);  // uniform: keep it in an SGPR
  const int lane = tid % 64;
  const int l32 = lane % 32, hh = lane / 32;
  const Shape<D, BM> sh(p);
  const int Nq = sh.Nq, Nk = sh.Nk;
  const float c = p.c;

  int bh, qt;
  sh.place(CAUSAL, bh, qt);
  const int b = bh / sh.H, h = bh - b * sh.H;
  const bf16 *Qh = (const bf16 *)p.Q + b * sh.q_b + h * sh.q_h;
  const bf16 *Kh = (const bf16 *)p.K + b * sh.k_b + h * sh.k_h;
  const bf16 *Vh = (const bf16 *)p.V + b * sh.v_b + h * sh.v_h;

  const int q0 = qt * BM;
  const int ks = KS == 1 ? 0 : wave % KS;         // this wave's share of the key blocks
  const int qw = q0 + kRowsPerWave * (wave / KS);  // first query row of this wave
  const int qrow = qw + l32;                // the query row this lane carries
  const bool wave_live = qw < Nq;           // wave has rows to compute (uniform)

  // Per-lane byte offsets (within a tile) of this wave's share of the tile loads:
  // LDS slot p = 1024 * gi + 16 * lane holds chunk (slot ^ swz(row)) of row p / ROW.
  // Load i adds 1024 i through its instruction offset, so it is taken out here.
  // Chunks past the D columns of a row (d = 16) read out of range: zeros.
  const int krs = 2 * sh.k_r, vrs = 2 * sh.v_r;  // row strides in bytes
  int kvo[LY::LPW], vvo[LY::LPW];
#pragma unroll
  for (int i = 0; i < LY::LPW; ++i) {
    const int sl = 64 * (wave * LY::LPW + i) + lane;  // 16-byte slot index in the tile
    const int r = sl / LY::CPR, j = sl % LY::CPR;
    const int jk = j ^ LY::swz_k(r), jv = j ^ LY::swz_v(r);
    kvo[i] = (16 * jk < 2 * D ? r * krs + 16 * jk : kOutOfRange) - 1024 * i;
    vvo[i] = (16 * jv < 2 * D ? r * vrs + 16 * jv : kOutOfRange) - 1024 * i;
  }
  const uint32_t smem_lds = lds_addr(smem);
  // Range of a tile: its last row ends the buffer, so rows past Nk read as zero.
  auto issue_k = [&](int t) {
    const int k0 = t * BN;
    const __amdgpu_buffer_rsrc_t rs =
        make_rsrc(Kh + (size_t)k0 * sh.k_r, (min(Nk - k0, BN) - 1) * krs + 2 * D);
    const uint32_t dst = smem_lds + (t & 1) * LY::STAGE + 1024 * wave * LY::LPW;
    load_lds_share(rs, dst, kvo);
  };
  auto issue_v = [&](int t) {
    const int k0 = t * BN;
    const __amdgpu_buffer_rsrc_t rs =
        make_rsrc(Vh + (size_t)k0 * sh.v_r, (min(Nk - k0, BN) - 1) * vrs + 2 * D);
    const uint32_t dst = smem_lds + (t & 1) * LY::STAGE + LY::TILE + 1024 * wave * LY::LPW;
    load_lds_share(rs, dst, vvo);
  };

  // K reads (A operand of S^T = K Q^T): row 32kb + l32, chunk 2cc + hh; the
  // chunk index only flips bits 5..7 of the byte address. Both swizzles repeat
  // every 32 rows, so the wave's first block (32 ks rows in) is a plain offset.
  const int kbase = (32 * ks + l32) * LY::ROW + 16 * (hh ^ LY::swz_k(l32));
  // V transposing reads: 16-lane group g reads rows 4hh + (lane%16)/4 (+8u, +16mm,
  // +32kb) and columns 32db + 16(g%2) + 4(lane%4); in slot terms the column block
  // db is XORed with swz_v(row)/4.
  const int vrow = 4 * hh + (lane % 16) / 4;
  const int vchunk = 2 * ((lane / 16) % 2) + (lane % 4) / 2;  // chunk within a 32-column block
  const int vbase = (32 * ks + vrow) * LY::ROW + 16 * (vchunk ^ LY::swz_v(vrow)) + 8 * (lane % 2);

  // Q as the B operand of S^T = K Q^T: lane holds Q[qrow][16cc + 8hh + 0..7]
  // (zeros past row Nq or column D).
  bf16x8 qf[NCC];
#pragma unroll
  for (int cc = 0; cc < NCC; ++cc) {
    if (qrow < Nq && 16 * cc + 8 * hh < D)
      qf[cc] = *(const bf16x8 *)(Qh + (size_t)qrow * sh.q_r + 16 * cc + 8 * hh);
    else
      qf[cc] = bf16x8{};
  }

  f32x16 o[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db) o[db] = f32x16{};
  float m = -INFINITY;  // reference row maximum (base-2 scaled domain)
  float lsum = 0.f;     // row sum relative to m over this half-wave's keys

  const int kend = CAUSAL ? min(Nk, q0 + BM) : Nk;
  const int nt = (kend + BN - 1) / BN;
  // Leading tiles that need no mask for any row of the workgroup.
  const int nfull = CAUSAL ? min((q0 + 1) / BN, Nk / BN) : Nk / BN;

  // First key of this wave's block kb (of NKW) in tile t.
  auto block_key = [&](int t, int kb) { return t * BN + 32 * (KS * kb + ks); };
  // Is this wave's block kb of tile t needed by the wave? (always, off the edge)
  auto block_live = [&](int t, int kb) {
    const int kb0 = block_key(t, kb);
    return kb0 < Nk && (!CAUSAL || kb0 <= qw + kRowsPerWave - 1);
  };

  // S^T blocks of 32 keys x 32 queries for tile t. Result layout: lane (l32, hh),
  // register r holds key 8(r/4) + 4hh + r%4 of the block, query qrow.
  auto scores = [&](int t, f32x16 (&s)[NKW], auto edge_tag) {
    constexpr bool EDGE = decltype(edge_tag)::value;
    const char *kt = smem + (t & 1) * LY::STAGE;
#pragma unroll
    for (int kb = 0; kb < NKW; ++kb) {
      if (EDGE && !block_live(t, kb)) {
#pragma unroll
        for (int r = 0; r < 16; ++r) s[kb][r] = -INFINITY;
        continue;
      }
#pragma unroll
      for (int cc = 0; cc < NCC; ++cc) {
        const bf16x8 a = *(const bf16x8 *)(kt + 32 * KS * kb * LY::ROW + (kbase ^ (32 * cc)));
        s[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[cc], cc == 0 ? f32x16{} : s[kb], 0, 0, 0);
      }
    }
  };
  auto mask = [&](int t, f32x16 (&s)[NKW]) {
#pragma unroll
    for (int kb = 0; kb < NKW; ++kb) {
      const int kb0 = block_key(t, kb);
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int key = kb0 + 8 * (r / 4) + 4 * hh + (r % 4);
        const bool bad = key >= Nk || (CAUSAL && key > qrow);
        s[kb][r] = bad ? -INFINITY : s[kb][r];
      }
    }
  };
  auto rowmax = [&](const f32x16 (&s)[NKW]) {
    float mx = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < NKW; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[kb][r]);
    return halves_max(mx);
  };
  // Move the reference maximum only when some row of the wave grew past the
  // slack (always on the first tile, where m = -inf), to the new maximum plus
  // the lead; rows that did not grow get alpha = 1.
  auto update_ref = [&](float mx) {
    const float mc = mx * c;
    const bool grow = mc > m + kRescaleSlack;
    if (__builtin_amdgcn_ballot_w64(grow)) {
      const float m_new = grow ? mc + kReferenceLead : m;
      const float alpha = exp2_fast(m - m_new);  // 0 while m is still -inf
      lsum *= alpha;
#pragma unroll
      for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) o[db][r] *= alpha;
      m = m_new;
    }
  };
  // P = exp2(S c - m) in bf16 as the B operand (P^T) of the second MFMA: key
  // half mm of block kb is registers 8mm..8mm+7 of s[kb]. The scores stay as
  // they are, in case the reference has to move and P be formed again.
  auto exponentiate = [&](const f32x16 (&s)[NKW], bf16x8 (&pb)[NKW][2]) {
    const float mref = (m == -INFINITY) ? 0.f : m;  // no -inf - -inf
#pragma unroll
    for (int kb = 0; kb < NKW; ++kb)
#pragma unroll
      for (int mm = 0; mm < 2; ++mm)
#pragma unroll
        for (int t8 = 0; t8 < 8; ++t8) pb[kb][mm][t8] = (bf16)exp2_fast(fmaf(s[kb][8 * mm + t8], c, -mref));
  };
  // Adds to `acc` the row sum of the weights as they enter the second MFMA: the
  // bf16 values of P, two per v_dot2_f32_bf16 against (1, 1). Dividing by this
  // sum makes each output row an exact convex combination of the value rows
  // under the rounded weights (the rounding of a weight then cancels between
  // numerator and denominator when one key dominates a row).
  auto rowsum_into = [&](const bf16x8 (&pb)[NKW][2], float acc) {
    const bf16x2 one = {(bf16)1.f, (bf16)1.f};
#pragma unroll
    for (int kb = 0; kb < NKW; ++kb)
#pragma unroll
      for (int mm = 0; mm < 2; ++mm)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const bf16x2 w = {pb[kb][mm][2 * i], pb[kb][mm][2 * i + 1]};
          acc = __builtin_amdgcn_fdot2_f32_bf16(w, one, acc, false);
        }
    return acc;
  };
  // O^T += V^T P^T for tile t. The A operand (V^T) lists the keys of P's slots
  // 16mm + 8(t/4) + 4hh + t%4 via two transposing reads of 4 consecutive keys.
  auto accumulate = [&](int t, const bf16x8 (&pb)[NKW][2], auto edge_tag) {
    constexpr bool EDGE = decltype(edge_tag)::value;
    const char *vs = smem + (t & 1) * LY::STAGE + LY::TILE;
#pragma unroll
    for (int kb = 0; kb < NKW; ++kb) {
      if (EDGE && !block_live(t, kb)) continue;
#pragma unroll
      for (int mm = 0; mm < 2; ++mm) {
        const int roff = (32 * KS * kb + 16 * mm) * LY::ROW;
#pragma unroll
        for (int db = 0; db < NDB; ++db) {
          const char *p0 = vs + roff + (vbase ^ (64 * db));
          const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4 *)(p0));
          const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4 *)(p0 + 8 * LY::ROW));
          const bf16x8 a = __builtin_bit_cast(
              bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
          o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pb[kb][mm], o[db], 0, 0, 0);
        }
      }
    }
  };
  // The weights of a tile and their row sum, added to l. The row maximum is
  // taken only when the reference may have to move: a row whose maximum grew
  // past the reference plus the slack has a weight above 2^8, so the sum of
  // its lane's weights reaches 2^8 (or is not finite). Then the wave takes the
  // tile's row maxima, moves the references of the rows that grew (rescaling
  // O and l) and forms P again; a lane whose sum reached 2^8 without a weight
  // above 2^8 keeps its reference and gets the same P. Either way every weight
  // that enters O and l is at most 2^8 (to the rounding of exp2 there), as when
  // the maximum is taken on every tile.
  auto weigh = [&](const f32x16 (&s)[NKW], bf16x8 (&pb)[NKW][2]) {
    exponentiate(s, pb);
    float ts = rowsum_into(pb, 0.f);
    if (__builtin_amdgcn_ballot_w64(!(ts < 256.f))) {
      update_ref(rowmax(s));
      exponentiate(s, pb);
      ts = rowsum_into(pb, 0.f);
    }
    lsum += ts;
  };
  // All of this wave's loads issued so far have landed; after the barrier, so
  // have every wave's, and every wave is done with the previous iteration.
  auto publish = [&]() {
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
  };

  // Iteration t: loads for K(t+2), V(t+1); S(t+1) next to P(t); O += V(t) P(t).
  // The steady-state form (both tiles full, a next tile exists) is straight-line
  // code; the generic form, used for the few tiles at the diagonal or the
  // ragged end, tests its conditions at run time (all uniform).
  auto iteration_full = [&](int t, f32x16 (&s_cur)[NKW], f32x16 (&s_nxt)[NKW]) {
    publish();
    if (t + 2 < nt) issue_k(t + 2);
    issue_v(t + 1);
    bf16x8 pb[NKW][2];
    scores(t + 1, s_nxt, std::false_type{});
    weigh(s_cur, pb);
    accumulate(t, pb, std::false_type{});
  };
  auto iteration_edge = [&](int t, f32x16 (&s_cur)[NKW], f32x16 (&s_nxt)[NKW]) {
    const bool has_next = t + 1 < nt;
    publish();
    if (t + 2 < nt) issue_k(t + 2);
    if (has_next) issue_v(t + 1);
    bf16x8 pb[NKW][2];
    if (has_next) scores(t + 1, s_nxt, std::true_type{});
    weigh(s_cur, pb);
    accumulate(t, pb, std::true_type{});
    if (has_next && t + 1 >= nfull) mask(t + 1, s_nxt);
  };

  f32x16 sa[NKW], sb[NKW];
  // Prologue: K(0), V(0), K(1) in flight; S(0) and its reference maximum.
  issue_k(0);
  issue_v(0);
  if (nt > 1) issue_k(1);
  publish();
  // Waves whose rows all lie past Nq (only in the last query tile of a ragged
  // sequence) run the same code on zero Q rows and store nothing: no branch
  // around the loop, so the Q loads are known complete before it.
  // Tile 0 is computed for every block (the mask removes dead ones), so every
  // path through here has consumed Q before the loop.
  scores(0, sa, std::false_type{});
  if (nfull == 0) mask(0, sa);
  update_ref(rowmax(sa));

  int t = 0;
  // Steady state, two iterations per trip so that S(t) and S(t+1) swap
  // registers without copies: both tiles after t are full tiles.
  // Not unrolled even when a specialized build knows the trip count (the body is
  // large; a fully unrolled loop only grows the instruction footprint).
#pragma nounroll
  for (; t + 2 < nfull; t += 2) {
    iteration_full(t, sa, sb);
    iteration_full(t + 1, sb, sa);
  }
#pragma nounroll
  for (; t < nt; t += 2) {
    iteration_edge(t, sa, sb);
    if (t + 1 < nt) iteration_edge(t + 1, sb, sa);
  }

  if constexpr (KS > 1) {
    // Hand-over area: for wave (group g, share j >= 1), NDB x 4 f32x4 of O per
    // lane (lane-contiguous, conflict-free), then m and l per lane. The tiles
    // are dead: no loads are in flight after the last iteration.
    constexpr int SLOT = (16 * NDB + 2) * 64;  // floats per handing wave
    static_assert((NW / KS) * (KS - 1) * SLOT * 4 <= 2 * LY::STAGE, "hand-over fits in the tile buffers");
    float *xs = (float *)smem;
    const int g = wave / KS;
    __syncthreads();  // every wave is done reading the tiles
    if (ks != 0) {
      float *slot = xs + (g * (KS - 1) + ks - 1) * SLOT;
#pragma unroll
      for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
          f32x4 v;
#pragma unroll
          for (int e = 0; e < 4; ++e) v[e] = o[db][4 * q4 + e];
          *(f32x4 *)(slot + 4 * ((4 * db + q4) * 64 + lane)) = v;
        }
      slot[16 * NDB * 64 + lane] = m;
      slot[16 * NDB * 64 + 64 + lane] = lsum;
    }
    __syncthreads();
    if (ks != 0) return;
    // Share 0 has a live key in every tile it visits (the tile's first key is
    // at or before every row of the group), so m is finite; a share that saw
    // no live key has m = -inf and weight exp2(-inf) = 0.
    float mt = m;
#pragma unroll
    for (int j = 1; j < KS; ++j) mt = fmaxf(mt, xs[(g * (KS - 1) + j - 1) * SLOT + 16 * NDB * 64 + lane]);
    const float f0 = exp2_fast(m - mt);
    lsum *= f0;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int r = 0; r < 16; ++r) o[db][r] *= f0;
#pragma unroll
    for (int j = 1; j < KS; ++j) {
      const float *slot = xs + (g * (KS - 1) + j - 1) * SLOT;
      const float fj = exp2_fast(slot[16 * NDB * 64 + lane] - mt);
      lsum = fmaf(slot[16 * NDB * 64 + 64 + lane], fj, lsum);
#pragma unroll
      for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
          const f32x4 v = *(const f32x4 *)(slot + 4 * ((4 * db + q4) * 64 + lane));
#pragma unroll
          for (int e = 0; e < 4; ++e) o[db][4 * q4 + e] = fmaf(v[e], fj, o[db][4 * q4 + e]);
        }
    }
    m = mt;
  }

  if (!wave_live) return;
  // Epilogue: one division by the row sum (both half-waves' keys), RNE to bf16.
  const float ltot = halves_sum(lsum);
  if (qrow < Nq) {
    const float inv = 1.f / ltot;
    bf16 *orow = (bf16 *)p.O + b * sh.o_b + h * sh.o_h + (size_t)qrow * sh.o_r;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        if (D < DP && 8 * g + 4 * hh >= D) continue;  // padding columns (d = 16)
        bf16x4 v4;
#pragma unroll
        for (int e = 0; e < 4; ++e) v4[e] = (bf16)(o[db][4 * g + e] * inv);
        *(bf16x4 *)(orow + 32 * db + 8 * g + 4 * hh) = v4;
      }
    if (hh == 0) p.L[b * sh.l_b + h * sh.l_h + (size_t)qrow * sh.l_r] = (m + log2_fast(ltot)) * kLn2;
  }
}

// ---------------------------------------------------------------------------
// fp32 kernel: everything in fp32 (v_mfma_f32_32x32x2_f32); P is not rounded.
//
// Work mapping: one workgroup per (head, block of 32 query rows). Its NW waves
// all carry the same 32 rows and split the block's 32-key tiles round-robin
// (wave w takes tiles w, w + NW, ...), each with its own running m, l and
// accumulator; the NW partial states are merged through LDS at the end with
// the same rescaling rule that merges two key blocks (the recurrence is
// associative over key blocks). This fills the GPU with 32-row blocks where a
// 128-row tile would leave most CUs idle (8 heads x 1024 rows is 256
// workgroups here, 64 with 128-row tiles), and no LDS or barrier is needed in
// the key loop: every wave reads its K and V operands straight from global
// memory (L2) into VGPRs with range-checked buffer loads, the next tile's
// loads in flight while the current tile is computed.
//
// Operand layouts (lane = 32 hh + l32):
//  * S^T = K Q^T, step s (< D/2): A = K[key l32][hh D/2 + s], B = Q[row l32][hh
//    D/2 + s], so each lane reads D/2 contiguous floats of one K row and keeps
//    D/2 floats of its Q row.
//  * O^T += V^T P^T: the 32x32 output blocks db < D/32 hold columns NDB i + db
//    (row i of the block), so at step r the A operands of all blocks are the
//    NDB consecutive floats V[key][NDB l32 ..], one vector load, and the B
//    operand is register r of the scores (key 8(r/4) + 4hh + r%4), as in the
//    bf16 kernel. In the result a lane holds 4 NDB consecutive output columns
//    per group r/4.
// ---------------------------------------------------------------------------
constexpr int kF32Rows = 32;  // query rows per workgroup (fp32 kernel)
constexpr int kF32Keys = 32;  // keys per tile (fp32 kernel)

// Two workgroups of four waves per CU at d = 64 (at most 256 VGPRs a wave, so
// the MFMA accumulators stay in VGPRs and are rescaled in place).
//
// D = 16 keeps the 32-row output blocks: lanes l32 >= 16 read V columns past
// the row (or zeros past the tile) into output rows that are never stored.
template <int D, bool CAUSAL, int NW>
__global__ __launch_bounds__(NW * 64, (NW == 4 && D == 64) ? 2 : 1) void fa_fwd_f32_kernel(const FwdParams p) {
  constexpr int BN = kF32Keys;
  constexpr int DP = D < 32 ? 32 : D;  // columns of the output blocks
  constexpr int HD = D / 2;            // contraction steps of S^T per tile
  constexpr int NDB = DP / 32;         // 32-row blocks of O^T
  constexpr int OS = DP + 4;           // row stride (floats) of the merge buffer
  using VV = F32Vec<NDB>;
  typedef typename VV::type vvec;

  __shared__ __attribute__((aligned(16))) float Os[NW][kF32Rows * OS];
  __shared__ float Ms[NW][kF32Rows], Ls[NW][kF32Rows];

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid / 64);
  const int lane = tid % 64, l32 = lane % 32, hh = lane / 32;
  const Shape<D, kF32Rows> sh(p);
  const int Nq = sh.Nq, Nk = sh.Nk;
  const float c = p.c;

  int bh, qb;
  sh.place(CAUSAL, bh, qb);
  const int b = bh / sh.H, h = bh - b * sh.H;
  const float *Kh = (const float *)p.K + b * sh.k_b + h * sh.k_h;
  const float *Vh = (const float *)p.V + b * sh.v_b + h * sh.v_h;
  const int qrs = 4 * sh.q_r, krs = 4 * sh.k_r, vrs = 4 * sh.v_r;  // row strides in bytes
  const int q0 = qb * kF32Rows;
  const int qrow = q0 + l32;

  // Q rows of the block (rows past Nq read as zero; the range ends with the last row).
  float qf[HD];
  {
    const __amdgpu_buffer_rsrc_t rq = make_rsrc((const float *)p.Q + b * sh.q_b + h * sh.q_h + (size_t)q0 * sh.q_r,
                                                (min(Nq - q0, kF32Rows) - 1) * qrs + 4 * D);
#pragma unroll
    for (int j = 0; j < HD / 4; ++j) {
      const f32x4 w = F32Vec<4>::load(rq, l32 * qrs + hh * HD * 4 + 16 * j);
#pragma unroll
      for (int e = 0; e < 4; ++e) qf[4 * j + e] = w[e];
    }
  }

  const int kend = CAUSAL ? min(Nk, q0 + kF32Rows) : Nk;
  const int nt = (kend + BN - 1) / BN;

  f32x4 kf[HD / 4];  // K operand of one tile
  vvec vf[16];       // V operands of one tile, one vector per MFMA step
  auto load_k = [&](int t) {
    const int k0 = t * BN;
    const __amdgpu_buffer_rsrc_t rk = make_rsrc(Kh + (size_t)k0 * sh.k_r, (min(Nk - k0, BN) - 1) * krs + 4 * D);
#pragma unroll
    for (int j = 0; j < HD / 4; ++j) kf[j] = F32Vec<4>::load(rk, l32 * krs + hh * HD * 4 + 16 * j);
  };
  auto load_v = [&](int t) {
    const int k0 = t * BN;
    const __amdgpu_buffer_rsrc_t rv = make_rsrc(Vh + (size_t)k0 * sh.v_r, (min(Nk - k0, BN) - 1) * vrs + 4 * D);
#pragma unroll
    for (int r = 0; r < 16; ++r)
      vf[r] = VV::load(rv, (8 * (r / 4) + 4 * hh + r % 4) * vrs + NDB * 4 * l32);
  };

  f32x16 o[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db) o[db] = f32x16{};
  float m = -INFINITY, lsum = 0.f;  // m: reference row maximum in the base-2 domain

  if (wave < nt) {
    load_k(wave);
    load_v(wave);
  }
#pragma nounroll
  for (int t = wave; t < nt; t += NW) {
    const int k0 = t * BN;
    const bool more = t + NW < nt;
    f32x16 s = f32x16{};
#pragma unroll
    for (int j = 0; j < HD / 4; ++j)
#pragma unroll
      for (int e = 0; e < 4; ++e) s = __builtin_amdgcn_mfma_f32_32x32x2f32(kf[j][e], qf[4 * j + e], s, 0, 0, 0);
    if (more) load_k(t + NW);

    // Ragged end and the causal diagonal tile (k0 == q0) only.
    if (k0 + BN > Nk || (CAUSAL && k0 + BN > q0)) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int key = k0 + 8 * (r / 4) + 4 * hh + r % 4;
        if (key >= Nk || (CAUSAL && key > qrow)) s[r] = -INFINITY;
      }
    }
    float mx = -INFINITY;
#pragma unroll
    for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[r]);
    mx = halves_max(mx) * c;
    // The reference m moves (and O, l are rescaled) only when some row of the
    // wave exceeds it by more than the slack.
    const bool grow = mx > m + kRescaleSlack;
    if (__builtin_amdgcn_ballot_w64(grow)) {
      const float m_new = grow ? mx : m;
      const float alpha = exp2_fast(m - m_new);  // 0 while m is still -inf
      lsum *= alpha;
#pragma unroll
      for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) o[db][r] *= alpha;
      m = m_new;
    }
    const float m_ref = (m == -INFINITY) ? 0.f : m;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      s[r] = exp2_fast(fmaf(s[r], c, -m_ref));
      lsum += s[r];
    }
#pragma unroll
    for (int r = 0; r < 16; ++r)
#pragma unroll
      for (int db = 0; db < NDB; ++db) o[db] = __builtin_amdgcn_mfma_f32_32x32x2f32(vf[r][db], s[r], o[db], 0, 0, 0);
    if (more) load_v(t + NW);
  }

  // Merge the NW partial states of each row: M = max_w m_w, weights 2^(m_w - M).
  const float lw = halves_sum(lsum);
  if (hh == 0) {
    Ms[wave][l32] = m;
    Ls[wave][l32] = lw;
  }
  __syncthreads();
  float mtot = -INFINITY;
#pragma unroll
  for (int w = 0; w < NW; ++w) mtot = fmaxf(mtot, Ms[w][l32]);
  const float f = exp2_fast(m - mtot);  // 0 for a wave that saw no key tile
  {
    float *orow = &Os[wave][l32 * OS];
#pragma unroll
    for (int g = 0; g < 4; ++g)
#pragma unroll
      for (int h = 0; h < NDB; ++h) {
        // floats 4h .. 4h+3 of the 4 NDB consecutive columns of group g
        f32x4 v;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int idx = 4 * h + e;  // (r % 4) * NDB + db
          v[e] = o[idx % NDB][4 * g + idx / NDB] * f;
        }
        *(f32x4 *)(orow + NDB * (8 * g + 4 * hh) + 4 * h) = v;
      }
  }
  __syncthreads();
  // Sum the partial outputs, divide once by the merged row sum, store the D
  // columns.
  constexpr int C4 = D / 4;
  float *Ob = (float *)p.O + b * sh.o_b + h * sh.o_h;
  float *Lb = p.L + b * sh.l_b + h * sh.l_h;
#pragma unroll
  for (int it = 0; it < (kF32Rows * C4 + NW * 64 - 1) / (NW * 64); ++it) {
    const int idx = tid + NW * 64 * it;
    const int row = idx / C4, c4 = idx % C4;
    if (row >= kF32Rows || q0 + row >= Nq) continue;
    float mrow = -INFINITY;
#pragma unroll
    for (int w = 0; w < NW; ++w) mrow = fmaxf(mrow, Ms[w][row]);
    float lrow = 0.f;
    f32x4 acc = f32x4{};
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      lrow = fmaf(Ls[w][row], exp2_fast(Ms[w][row] - mrow), lrow);
      acc += *(const f32x4 *)(&Os[w][row * OS + 4 * c4]);
    }
    const float inv = 1.f / lrow;
    *(f32x4 *)(Ob + (size_t)(q0 + row) * sh.o_r + 4 * c4) = acc * inv;
    if (c4 == 0) Lb[(size_t)(q0 + row) * sh.l_r] = (mrow + log2_fast(lrow)) * kLn2;
  }
}

}  // namespace

#endif  // FA_FWD_KERNELS_H_
