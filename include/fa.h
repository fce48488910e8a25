/*
 * fa.h -- C ABI of the tiled online-softmax attention forward and backward
 * passes (gfx950).
 *
 * The operation is exact scaled-dot-product attention with the per-row
 * logsumexp, as defined in "Writing a FlashAttention kernel in Metal"
 * (section "Standard attention": S = scale * Q K^T, P = row softmax of S,
 * O = P V; section "Blockwise attention and causal masking": with causal
 * masking a query attends only to keys at or before its own position) and in
 * "FlashAttention-2 from PyTorch to Triton" (section "What We Are Building":
 * L_i = m_i + log l_i, the natural-log logsumexp of row i of the scaled
 * scores). It is computed by the tiled online-softmax recurrence (running row
 * maximum, running row sum and an unnormalised output accumulator, divided by
 * the sum once at the end), so the N x N score matrix is never stored.
 *
 * This header is plain C. It needs no HIP or torch header.
 */
#ifndef FA_H_
#define FA_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Status codes. FA_OK is zero; every other value is an error. */
typedef enum {
  FA_OK = 0,
  FA_ERR_INVALID_ARGUMENT = 1, /* null pointer, B/H/N < 1, scale <= 0 or scale*log2(e) not finite in fp32, bad dtype */
  FA_ERR_UNSUPPORTED = 2,      /* head dimension not supported by the entry point, or a size too large */
  FA_ERR_MISALIGNED = 3,       /* a buffer not 16-byte aligned */
  FA_ERR_LAUNCH = 4,           /* the HIP runtime refused the kernel launch */
  FA_ERR_JIT = 5,              /* run-time compilation or loading of a specialized kernel failed */
  FA_ERR_SCRATCH_LIMIT = 6     /* fa_bwd_noalloc: the problem needs more than its static workspace */
} fa_status_t;

/* Element type of Q, K, V and O. */
typedef enum {
  FA_DTYPE_F32 = 0, /* IEEE binary32; all arithmetic in fp32 */
  FA_DTYPE_BF16 = 1 /* bfloat16 inputs and output; fp32 scores, softmax state and accumulation */
} fa_dtype_t;

/*
 * fa_fwd -- attention forward pass over B*H independent heads.
 *
 *   Q, K, V  device pointers, contiguous row-major [B][H][N][d] of `dtype`.
 *   O        device pointer, contiguous [B][H][N][d] of `dtype`; written.
 *            O[b][h][i][:] = sum_j P[i][j] V[b][h][j][:], rounded to nearest
 *            even when dtype is bf16. Must not overlap Q, K, V or L.
 *   L        device pointer, contiguous [B][H][N] fp32; written with the
 *            natural-log logsumexp of each row of scaled scores.
 *   B, H, N  batch, heads, sequence length (queries and keys share positions
 *            0..N-1). Each >= 1. N need not be a multiple of any tile size.
 *   d        head dimension: 16, 32, 64 or 128.
 *   causal   0: every query sees every key. Non-zero: query i sees keys j <= i.
 *   scale    multiplier of Q K^T (usually 1/sqrt(d)); > 0, with scale * log2(e) finite in fp32.
 *   stream   hipStream_t to enqueue on (NULL = the null stream).
 *   dtype    an fa_dtype_t value.
 *
 * Ownership: the caller owns all five buffers; the library allocates no
 * memory and keeps no state between calls. The call is asynchronous: it
 * returns once the kernel is enqueued, and the results are valid after the
 * caller synchronises the stream. Arguments are validated synchronously,
 * before any device work, in the order of the status list above; on an error
 * nothing is enqueued and O, L are untouched. Faults inside the kernel (for
 * example a pointer that is not device memory) surface at the caller's next
 * synchronisation, not here. Calls on different streams may run
 * concurrently; they share no state. Repeated calls with the same arguments
 * and data give bitwise identical results; with bf16, a head's result can
 * differ in the last bits between launches with different B, H or N, because
 * small grids split each tile's keys between two waves (a different
 * summation order, within the same error bound).
 *
 * Value range (finite inputs; NaN and infinities propagate): with bf16 the
 * output accumulators hold between about 2^-64 |v| and 2^8 N |v| (the softmax
 * reference of a row sits up to 64 above its running maximum), so O keeps
 * its relative precision for value magnitudes from about 2^-76 (through fp32
 * denormals) up to 2^120 / N; below that O degrades in relative terms
 * while its absolute error stays below the values' magnitude. fp32 keeps the
 * reference at the row maximum: accumulators between |v| and 2^8 N |v|.
 */
fa_status_t fa_fwd(const void *Q, const void *K, const void *V, void *O, float *L,
                   int64_t B, int64_t H, int64_t N, int64_t d, int causal, float scale,
                   void *stream, int dtype);

/*
 * fa_fwd_strided -- the forward pass of fa_fwd for the general layout of the
 * kernel in "FlashAttention-2 from PyTorch to Triton" (section "The Triton
 * Kernel"): separate query and key counts and arbitrary strides.
 *
 *   Q, O     device pointers to B x H x Nq x d arrays of `dtype`.
 *   K, V     device pointers to B x H x Nk x d arrays of `dtype`.
 *   L        device pointer to a B x H x Nq fp32 array; written as in fa_fwd.
 *   x_strides  (x = q, k, v, o, l) host arrays of three element strides:
 *            batch, head, row. The stride along d is 1. Zero batch or head
 *            strides broadcast an input (for example one K, V head shared by
 *            all query heads).
 *   Nq, Nk   query rows and key rows, each >= 1 and <= 2^24.
 *   causal   0: every query sees every key. Non-zero: query i sees keys
 *            j <= i, positions counted from 0 in both (the mask is aligned at
 *            the top-left corner of the Nq x Nk score matrix, as in that
 *            page's kernel), so every query sees at least key 0.
 *   B, H, d, scale, stream, dtype: as for fa_fwd.
 *
 * Requirements, checked before any device work:
 *   - all strides >= 0 and <= 2^40; the row stride of Q, K, V and O >= d
 *     (else FA_ERR_INVALID_ARGUMENT);
 *   - O and L are laid out without two elements at one address, and neither
 *     overlaps the byte range of any other operand (else
 *     FA_ERR_INVALID_ARGUMENT);
 *   - a row stride times the element size <= 2^24 bytes, the L row stride
 *     < 2^31 (else FA_ERR_UNSUPPORTED);
 *   - Q, K, V, O 16-byte aligned and their strides multiples of 16 bytes; L
 *     4-byte aligned (else FA_ERR_MISALIGNED).
 * Ownership, asynchrony and error behaviour as for fa_fwd. With contiguous
 * strides and Nq = Nk = N the results equal fa_fwd's.
 */
fa_status_t fa_fwd_strided(const void *Q, const void *K, const void *V, void *O, float *L,
                           int64_t B, int64_t H, int64_t Nq, int64_t Nk, int64_t d,
                           const int64_t *q_strides, const int64_t *k_strides,
                           const int64_t *v_strides, const int64_t *o_strides,
                           const int64_t *l_strides, int causal, float scale, void *stream,
                           int dtype);

/*
 * fa_fwd_specialized -- fa_fwd with the kernel compiled at run time for this
 * exact shape: the sizes B, H, N (and the contiguous strides they imply)
 * become compile-time constants, in the manner of the per-shape function
 * constants of "Case Study: metal-flash-attention" (its sections on compiling
 * a kernel per problem shape). Same arguments, semantics and validation as
 * fa_fwd; the results agree with fa_fwd's within the fa_fwd tolerances.
 *
 * The first call for a (device, dtype, d, causal, B, H, N) compiles the
 * forward kernel source embedded in the library with hipRTC (for gfx950, with
 * the flags of the library's own build; about a second) and loads it on the
 * stream's device (the current device for the null stream; the caller's
 * current device is restored); later calls reuse it. Loaded kernels are kept until the
 * process ends. The cache is guarded by a mutex, so concurrent calls from
 * several threads are safe; a call that compiles blocks its thread meanwhile.
 * Returns FA_ERR_JIT if compiling or loading fails (nothing is enqueued).
 */
fa_status_t fa_fwd_specialized(const void *Q, const void *K, const void *V, void *O, float *L,
                               int64_t B, int64_t H, int64_t N, int64_t d, int causal, float scale,
                               void *stream, int dtype);

/*
 * fa_jit_code_object -- compile the kernel fa_fwd_specialized would load for
 * (dtype, d, causal, B, H, N) and return its code object (an AMDGPU ELF for
 * gfx950), without touching any GPU: for inspection or for callers that keep
 * compiled kernels themselves.
 *
 *   buffer   host memory receiving the code object, or NULL to ask for its size.
 *   size     in: the capacity of buffer; out: the code object's size in bytes.
 * Returns FA_ERR_INVALID_ARGUMENT if size is NULL or the capacity is too small
 * (*size then holds the size needed), FA_ERR_UNSUPPORTED / FA_ERR_INVALID_ARGUMENT
 * for sizes and types fa_fwd rejects, FA_ERR_JIT if compilation fails.
 */
fa_status_t fa_jit_code_object(int dtype, int64_t d, int causal, int64_t B, int64_t H, int64_t N,
                               void *buffer, size_t *size);

/*
 * fa_bwd -- attention backward pass over B*H independent heads: the gradients
 * of a loss with respect to Q, K and V, given its gradient dO with respect to
 * O, for the same function fa_fwd computes. L is treated as an auxiliary
 * output of the forward pass (not differentiated). The probabilities are
 * recomputed from L as P = exp(S - L) ("FlashAttention-2 from PyTorch to
 * Triton", section "What We Are Building"), so nothing N x N is stored, and
 * the work is split into a dQ kernel and a dK/dV kernel that each own their
 * outputs (as "Case Study: metal-flash-attention" describes for that
 * project's backward pass).
 *
 *   Q, K, V  the forward inputs: device, contiguous [B][H][N][d] of `dtype`.
 *   O, L     the forward outputs of fa_fwd for these inputs (same layouts).
 *   dO       device, contiguous [B][H][N][d] of `dtype`: gradient w.r.t. O.
 *   dQ,dK,dV device, contiguous [B][H][N][d] of `dtype`; written, rounded to
 *            nearest even when bf16. They must not overlap each other, the
 *            inputs or `work`.
 *   work     device workspace of 2*B*H*N floats, overwritten (per row: the
 *            sum over c of dO*O, then L * log2 e). Owned by the caller; its
 *            contents after the call carry no meaning.
 *   B,H,N, causal, scale, stream: as for fa_fwd.
 *   d        64 or 128; with FA_DTYPE_F32 also 32. Other values return
 *            FA_ERR_UNSUPPORTED.
 *   dtype    FA_DTYPE_BF16 or FA_DTYPE_F32 (all of Q, K, V, O, dO and the
 *            gradients in that type).
 *
 * dS = P o (dP - D) with dP = dO V^T and D_i = sum_c dO[i][c] O[i][c];
 * dQ = scale dS K, dK = scale dS^T Q, dV = P^T dO; accumulation in fp32. For
 * bf16, P and dS are rounded to bf16 as MFMA operands; for fp32 every operand
 * stays fp32. Each gradient element is summed in a fixed order, so repeated
 * calls give bitwise identical results. Ownership, asynchrony and validation as
 * for fa_fwd: the library allocates no memory; on an error nothing is
 * enqueued and the outputs are untouched.
 */
fa_status_t fa_bwd(const void *Q, const void *K, const void *V, const void *O, const float *L,
                   const void *dO, void *dQ, void *dK, void *dV, float *work,
                   int64_t B, int64_t H, int64_t N, int64_t d, int causal, float scale,
                   void *stream, int dtype);

/*
 * fa_bwd_noalloc -- fa_bwd for callers that cannot allocate device memory
 * (code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc): the same kernels and results, without the `work` argument. The
 * 2*B*H*N-float workspace is a static array inside the library, one per GPU,
 * held until the process ends: at most 2^21 floats (8 MiB), so
 * B*H*N <= 2^20 rows (else FA_ERR_SCRATCH_LIMIT, nothing enqueued). The call
 * allocates nothing, on the host or the device. Every call on one GPU (the
 * stream's device; the current device for the null stream) uses that GPU's
 * array; each call rewrites every entry it reads (per row: the sum over c
 * of dO*O, then L * log2 e) before reading it, so nothing carries over between
 * calls, but calls that overlap in time on one GPU (different streams, or
 * several host threads) race on the array and must be serialized by the
 * caller. FA_ERR_LAUNCH if the array's device address cannot be obtained.
 * Every other argument, requirement and status as for fa_bwd.
 */
fa_status_t fa_bwd_noalloc(const void *Q, const void *K, const void *V, const void *O, const float *L,
                           const void *dO, void *dQ, void *dK, void *dV,
                           int64_t B, int64_t H, int64_t N, int64_t d, int causal, float scale,
                           void *stream, int dtype);

/* Static, human-readable name of a status code (never NULL). */
const char *fa_status_string(int status);

/* Library version as major * 10000 + minor * 100 + patch. */
int fa_version(void);

#ifdef __cplusplus
}
#endif

#endif /* FA_H_ */
