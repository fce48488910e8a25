// Tiled online-softmax attention forward pass for CDNA4 (gfx950, MI355X):
// the host side of libfa.so's forward entry points. The kernels and the method
// they implement are described in fa_fwd_kernels.h. Here:
//  * fa_fwd (contiguous [B][H][N][d]) and fa_fwd_strided (separate query and
//    key counts, per-tensor strides) validate their arguments and fill one
//    parameter block for the same kernels;
//  * fa_fwd_specialized compiles those kernels again at run time (hipRTC) with
//    the sizes as constants, and caches the loaded code per device and shape;
//  * fa_jit_code_object returns such a code object without a GPU.

#include <hip/hip_runtime.h>

#include <math.h>
#include <stddef.h>
#include <stdint.h>
#include <string.h>

#include <hip/hiprtc.h>

#include <algorithm>
#include <map>
#include <mutex>
#include <string>
#include <tuple>
#include <type_traits>
#include <vector>

#include "fa.h"
#include "fa_fwd_kernels.h"
#include "fa_jit_source.inc"

namespace {

hipError_t launch(const void *kern, int64_t nblocks, int threads, hipStream_t stream, FwdParams p) {
  void *args[] = {(void *)&p};
  return hipLaunchKernel(kern, dim3((unsigned)nblocks), dim3(threads), args, 0, stream);
}

// Tile configuration of the bf16 kernel: waves per workgroup (32 query rows
// each) and keys per LDS tile.
#ifndef FA_BF16_NW
#define FA_BF16_NW 4
#endif
#ifndef FA_BF16_BN
#define FA_BF16_BN 64
#endif
constexpr int kBf16Waves = FA_BF16_NW;
constexpr int kBf16Keys = FA_BF16_BN;

constexpr int kBf16Rows = kRowsPerWave * kBf16Waves;  // query rows per workgroup

// Compute units of the MI355X (gfx950).
constexpr int64_t kComputeUnits = 256;

// Key split of the bf16 kernel for small grids: the kernel runs with its waves
// paired over the key blocks of each tile (64 query rows per workgroup, twice
// the workgroups, half the keys per wave) when one workgroup per 128 query rows
// gives at most 3/4 of a workgroup per compute unit, or, when causal, at most
// 3/2: causal workgroups differ in length (a query tile sees the keys up to
// its diagonal), and while the grid fits in one round of two per compute unit
// the longest one sets the time, which the split halves.
constexpr int kBf16SmallGridSplit = 2;
bool bf16_small_grid(int64_t BH, int64_t Nq, bool causal) {
  const int64_t wgs = BH * ((Nq + kBf16Rows - 1) / kBf16Rows);
  return causal ? 2 * wgs <= 3 * kComputeUnits : 4 * wgs <= 3 * kComputeUnits;
}
int64_t bf16_rows(int64_t BH, int64_t Nq, bool causal) {
  return bf16_small_grid(BH, Nq, causal) ? kBf16Rows / kBf16SmallGridSplit : kBf16Rows;
}

template <int D, bool CAUSAL>
hipError_t launch_bf16(int64_t BH, hipStream_t s, FwdParams p) {
  p.head_group = head_group(BH, (int64_t)p.Nk * D * 2 * 2);
  if (bf16_small_grid(BH, p.Nq, CAUSAL)) {
    constexpr int rows = kBf16Rows / kBf16SmallGridSplit;
    p.n_qtiles = (p.Nq + rows - 1) / rows;
    const void *kern = (const void *)&fa_fwd_bf16_kernel<D, CAUSAL, kBf16Waves, kBf16Keys, kBf16SmallGridSplit>;
    return launch(kern, BH * p.n_qtiles, 64 * kBf16Waves, s, p);
  }
  p.n_qtiles = (p.Nq + kBf16Rows - 1) / kBf16Rows;
  const void *kern = (const void *)&fa_fwd_bf16_kernel<D, CAUSAL, kBf16Waves, kBf16Keys>;
  return launch(kern, BH * p.n_qtiles, 64 * kBf16Waves, s, p);
}

// Waves per workgroup of the fp32 kernel (each takes every NW-th key tile).
#ifndef FA_F32_NW
#define FA_F32_NW 4
#endif
constexpr int kF32Waves = FA_F32_NW;

template <int D, bool CAUSAL>
hipError_t launch_f32(int64_t BH, hipStream_t s, FwdParams p) {
  p.head_group = head_group(BH, (int64_t)p.Nk * D * 4 * 2);
  p.n_qtiles = (p.Nq + kF32Rows - 1) / kF32Rows;
  const void *kern = (const void *)&fa_fwd_f32_kernel<D, CAUSAL, kF32Waves>;
  return launch(kern, BH * p.n_qtiles, 64 * kF32Waves, s, p);
}

// Enqueue the kernel for (dtype, d, causal); the arguments are validated.
hipError_t dispatch(int dtype, int64_t d, bool causal, int64_t BH, hipStream_t s, const FwdParams &p) {
#define FA_CASE(DD)                                                                              \
  case DD:                                                                                       \
    if (dtype == FA_DTYPE_BF16)                                                                  \
      return causal ? launch_bf16<DD, true>(BH, s, p) : launch_bf16<DD, false>(BH, s, p);        \
    return causal ? launch_f32<DD, true>(BH, s, p) : launch_f32<DD, false>(BH, s, p);
  switch (d) {
    FA_CASE(16)
    FA_CASE(32)
    FA_CASE(64)
    FA_CASE(128)
    default:
      return hipErrorInvalidValue;
  }
#undef FA_CASE
}

bool overlaps(const void *a, size_t na, const void *b, size_t nb) {
  const uintptr_t x = (uintptr_t)a, y = (uintptr_t)b;
  return x < y + nb && y < x + na;
}


bool supported_head_dim(int64_t d) { return d == 16 || d == 32 || d == 64 || d == 128; }

// Row counts up to 2^24 keep every row index in 32 bits; the grid stays below 2^31.
// B and H are bounded first, so that B * H cannot overflow.
bool supported_sizes(int dtype, int64_t B, int64_t H, int64_t Nq, int64_t Nk) {
  if (Nq > (int64_t)1 << 24 || Nk > (int64_t)1 << 24) return false;
  if (B > (int64_t)1 << 31 || H > (int64_t)1 << 31) return false;
  const int64_t block_rows = dtype == FA_DTYPE_BF16 ? kBf16Rows : kF32Rows;
  const int64_t n_qtiles = (Nq + block_rows - 1) / block_rows;
  return B * H <= ((int64_t)1 << 31) / n_qtiles - 1;
}

// Byte range [lo, hi) covered by a B x H x rows x inner array with element
// strides st (batch, head, row) and unit stride inside a row.
struct Span {
  uintptr_t lo, hi;
};
// Elements from the first to one past the last element of the array, or
// false if that count (times the element size) does not fit in 2^62.
bool element_extent(int64_t B, int64_t H, int64_t rows, int64_t inner, const int64_t st[3], size_t esize,
                    int64_t *extent) {
  const int64_t ext[3] = {B, H, rows};
  int64_t total = inner;
  for (int i = 0; i < 3; ++i) {
    int64_t step;
    if (__builtin_mul_overflow(ext[i] - 1, st[i], &step) || __builtin_add_overflow(total, step, &total))
      return false;
  }
  int64_t bytes;
  if (__builtin_mul_overflow(total, (int64_t)esize, &bytes) || bytes > ((int64_t)1 << 62)) return false;
  *extent = total;
  return true;
}
Span tensor_span(const void *base, int64_t B, int64_t H, int64_t rows, int64_t inner, const int64_t st[3],
                 size_t esize) {
  int64_t extent = 0;
  element_extent(B, H, rows, inner, st, esize, &extent);  // checked by the caller
  return {(uintptr_t)base, (uintptr_t)base + (uintptr_t)extent * esize};
}
bool spans_overlap(Span a, Span b) { return a.lo < b.hi && b.lo < a.hi; }

// No two elements share an address: taken in increasing stride order, every
// dimension of extent > 1 steps over the whole span of the ones inside it.
bool non_overlapping(int64_t B, int64_t H, int64_t rows, int64_t inner, const int64_t st[3]) {
  int64_t ext[3] = {B, H, rows}, str[3] = {st[0], st[1], st[2]};
  for (int i = 0; i < 3; ++i)  // sort the three dimensions by stride
    for (int j = i + 1; j < 3; ++j)
      if (str[j] < str[i]) {
        int64_t t = str[i];
        str[i] = str[j];
        str[j] = t;
        t = ext[i];
        ext[i] = ext[j];
        ext[j] = t;
      }
  int64_t span = inner;
  for (int i = 0; i < 3; ++i) {
    if (ext[i] == 1) continue;
    if (str[i] < span) return false;
    int64_t step;
    if (__builtin_mul_overflow(ext[i] - 1, str[i], &step) || __builtin_add_overflow(span, step, &span))
      return false;
  }
  return true;
}

fa_status_t launch_checked(int dtype, int64_t d, int causal, int64_t BH, void *stream, const FwdParams &p) {
  const hipError_t err = dispatch(dtype, d, causal != 0, BH, (hipStream_t)stream, p);
  return err == hipSuccess ? FA_OK : FA_ERR_LAUNCH;
}

float log2e_scale(float scale) { return (float)((double)scale * 1.4426950408889634074); }



// Checks of fa_fwd and fa_fwd_specialized (contiguous [B][H][N][d] operands).
fa_status_t validate_contiguous(const void *Q, const void *K, const void *V, const void *O, const float *L,
                                int64_t B, int64_t H, int64_t N, int64_t d, float scale, int dtype) {
  if (!Q || !K || !V || !O || !L) return FA_ERR_INVALID_ARGUMENT;
  if (B < 1 || H < 1 || N < 1) return FA_ERR_INVALID_ARGUMENT;
  if (!(scale > 0.f) || !isfinite(log2e_scale(scale))) return FA_ERR_INVALID_ARGUMENT;  // finite scale * log2(e)
  if (dtype != FA_DTYPE_F32 && dtype != FA_DTYPE_BF16) return FA_ERR_INVALID_ARGUMENT;
  const size_t esize = dtype == FA_DTYPE_BF16 ? 2 : 4;
  if (!supported_head_dim(d)) return FA_ERR_UNSUPPORTED;
  if (!supported_sizes(dtype, B, H, N, N)) return FA_ERR_UNSUPPORTED;
  const size_t nelem = (size_t)B * (size_t)H * (size_t)N * (size_t)d;
  const size_t obytes = nelem * esize, lbytes = (size_t)B * H * N * sizeof(float);
  if (overlaps(O, obytes, Q, obytes) || overlaps(O, obytes, K, obytes) ||
      overlaps(O, obytes, V, obytes) || overlaps(O, obytes, L, lbytes) ||
      overlaps(L, lbytes, Q, obytes) || overlaps(L, lbytes, K, obytes) ||
      overlaps(L, lbytes, V, obytes))
    return FA_ERR_INVALID_ARGUMENT;
  if (((uintptr_t)Q | (uintptr_t)K | (uintptr_t)V | (uintptr_t)O | (uintptr_t)L) & 15)
    return FA_ERR_MISALIGNED;
  return FA_OK;
}

FwdParams contiguous_params(const void *Q, const void *K, const void *V, void *O, float *L, int64_t H,
                            int64_t N, int64_t d, float scale) {
  FwdParams p{};
  p.Q = Q;
  p.K = K;
  p.V = V;
  p.O = O;
  p.L = L;
  p.q_h = p.k_h = p.v_h = p.o_h = N * d;
  p.q_b = p.k_b = p.v_b = p.o_b = H * N * d;
  p.q_r = p.k_r = p.v_r = p.o_r = (int)d;
  p.l_b = H * N;
  p.l_h = N;
  p.l_r = 1;
  p.H = (int)H;
  p.Nq = p.Nk = (int)N;
  p.c = log2e_scale(scale);
  return p;
}

// ---------------------------------------------------------------------------
// Shape specialization at run time (hipRTC). The embedded device headers are
// compiled for one (dtype, d, causal, B, H, N) with those sizes as constants
// (FA_SPEC_*, see fa_fwd_kernels.h), with the flags of the ahead-of-time build,
// and the code object is loaded once per device and kept for the process.

// Query rows per workgroup and threads per workgroup of the kernel that
// launch_bf16 / launch_f32 pick for this shape.
int64_t block_rows(int dtype, int64_t BH, int64_t N, bool causal) {
  return dtype == FA_DTYPE_BF16 ? bf16_rows(BH, N, causal) : kF32Rows;
}
int block_threads(int dtype) { return 64 * (dtype == FA_DTYPE_BF16 ? kBf16Waves : kF32Waves); }

std::string kernel_expression(int dtype, int64_t d, int causal, int64_t BH, int64_t N) {
  const std::string c = causal ? "true" : "false";
  if (dtype == FA_DTYPE_BF16)
    return "fa_fwd_bf16_kernel<" + std::to_string(d) + ", " + c + ", " + std::to_string(kBf16Waves) + ", " +
           std::to_string(kBf16Keys) + ", " +
           std::to_string(bf16_small_grid(BH, N, causal != 0) ? kBf16SmallGridSplit : 1) + ">";
  return "fa_fwd_f32_kernel<" + std::to_string(d) + ", " + c + ", " + std::to_string(kF32Waves) + ">";
}

// Compiles the kernel for one shape; on success *code holds the code object and
// *name the kernel's symbol in it.
fa_status_t jit_compile(int dtype, int64_t d, int causal, int64_t B, int64_t H, int64_t N, std::string *code,
                        std::string *name) {
  hiprtcProgram prog;
  if (hiprtcCreateProgram(&prog, "#include \"fa_fwd_kernels.h\"\n", "fa_fwd_specialized.hip", kJitNumSources,
                          kJitSources, kJitSourceNames) != HIPRTC_SUCCESS)
    return FA_ERR_JIT;
  const std::string expr = kernel_expression(dtype, d, causal, B * H, N);
  const std::vector<std::string> opts = {
      "--offload-arch=gfx950", "-O3", "-std=c++17",
      "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
      "-DFA_SPEC_B=" + std::to_string(B), "-DFA_SPEC_H=" + std::to_string(H),
      "-DFA_SPEC_NQ=" + std::to_string(N), "-DFA_SPEC_NK=" + std::to_string(N)};
  std::vector<const char *> argv;
  for (const std::string &o : opts) argv.push_back(o.c_str());
  fa_status_t st = FA_ERR_JIT;
  const char *lowered = nullptr;
  size_t size = 0;
  if (hiprtcAddNameExpression(prog, expr.c_str()) == HIPRTC_SUCCESS &&
      hiprtcCompileProgram(prog, (int)argv.size(), argv.data()) == HIPRTC_SUCCESS &&
      hiprtcGetLoweredName(prog, expr.c_str(), &lowered) == HIPRTC_SUCCESS &&
      hiprtcGetCodeSize(prog, &size) == HIPRTC_SUCCESS && size > 0) {
    code->assign(size, '\0');
    *name = lowered;
    if (hiprtcGetCode(prog, &(*code)[0]) == HIPRTC_SUCCESS) st = FA_OK;
  }
  hiprtcDestroyProgram(&prog);
  return st;
}

struct JitKernel {
  hipModule_t module;
  hipFunction_t function;
};
std::mutex g_jit_mutex;
// (device, dtype, d, causal, B, H, N) -> loaded kernel; entries live until the process ends.
std::map<std::tuple<int, int, int64_t, int, int64_t, int64_t, int64_t>, JitKernel> g_jit_kernels;

}  // namespace

extern "C" fa_status_t fa_fwd(const void *Q, const void *K, const void *V, void *O, float *L,
                              int64_t B, int64_t H, int64_t N, int64_t d, int causal,
                              float scale, void *stream, int dtype) {
  const fa_status_t st = validate_contiguous(Q, K, V, O, L, B, H, N, d, scale, dtype);
  if (st != FA_OK) return st;
  return launch_checked(dtype, d, causal, B * H, stream, contiguous_params(Q, K, V, O, L, H, N, d, scale));
}

extern "C" fa_status_t fa_fwd_specialized(const void *Q, const void *K, const void *V, void *O, float *L,
                                          int64_t B, int64_t H, int64_t N, int64_t d, int causal,
                                          float scale, void *stream, int dtype) {
  const fa_status_t st = validate_contiguous(Q, K, V, O, L, B, H, N, d, scale, dtype);
  if (st != FA_OK) return st;
  int device = 0;
  if (stream_device((hipStream_t)stream, &device) != hipSuccess) return FA_ERR_LAUNCH;
  JitKernel kern;
  {
    std::lock_guard<std::mutex> lock(g_jit_mutex);
    const auto key = std::make_tuple(device, dtype, d, causal != 0 ? 1 : 0, B, H, N);
    auto it = g_jit_kernels.find(key);
    if (it == g_jit_kernels.end()) {
      std::string code, name;
      const fa_status_t cs = jit_compile(dtype, d, causal != 0, B, H, N, &code, &name);
      if (cs != FA_OK) return cs;
      // Loaded on the stream's device, made current for the load.
      JitKernel k{};
      const hipError_t e = on_device(device, [&] {
        if (hipModuleLoadData(&k.module, code.data()) != hipSuccess) return false;
        if (hipModuleGetFunction(&k.function, k.module, name.c_str()) != hipSuccess) {
          (void)hipModuleUnload(k.module);  // already failing: the unload's status adds nothing
          return false;
        }
        return true;
      });
      if (e != hipSuccess) return FA_ERR_JIT;
      it = g_jit_kernels.emplace(key, k).first;
    }
    kern = it->second;
  }
  FwdParams p = contiguous_params(Q, K, V, O, L, H, N, d, scale);
  const int64_t rows = block_rows(dtype, B * H, N, causal != 0);
  p.n_qtiles = (int)((N + rows - 1) / rows);
  p.head_group = head_group(B * H, N * d * (dtype == FA_DTYPE_BF16 ? 2 : 4) * 2);
  void *args[] = {(void *)&p};
  const hipError_t err = hipModuleLaunchKernel(kern.function, (unsigned)(B * H * p.n_qtiles), 1, 1,
                                               (unsigned)block_threads(dtype), 1, 1, 0, (hipStream_t)stream,
                                               args, nullptr);
  return err == hipSuccess ? FA_OK : FA_ERR_LAUNCH;
}

extern "C" fa_status_t fa_jit_code_object(int dtype, int64_t d, int causal, int64_t B, int64_t H, int64_t N,
                                          void *buffer, size_t *size) {
  if (!size) return FA_ERR_INVALID_ARGUMENT;
  if (B < 1 || H < 1 || N < 1) return FA_ERR_INVALID_ARGUMENT;
  if (dtype != FA_DTYPE_F32 && dtype != FA_DTYPE_BF16) return FA_ERR_INVALID_ARGUMENT;
  if (!supported_head_dim(d)) return FA_ERR_UNSUPPORTED;
  if (!supported_sizes(dtype, B, H, N, N)) return FA_ERR_UNSUPPORTED;
  std::string code, name;
  const fa_status_t st = jit_compile(dtype, d, causal != 0, B, H, N, &code, &name);
  if (st != FA_OK) return st;
  if (buffer) {
    if (*size < code.size()) {
      *size = code.size();
      return FA_ERR_INVALID_ARGUMENT;
    }
    memcpy(buffer, code.data(), code.size());
  }
  *size = code.size();
  return FA_OK;
}

extern "C" fa_status_t fa_fwd_strided(const void *Q, const void *K, const void *V, void *O, float *L,
                                      int64_t B, int64_t H, int64_t Nq, int64_t Nk, int64_t d,
                                      const int64_t *q_strides, const int64_t *k_strides,
                                      const int64_t *v_strides, const int64_t *o_strides,
                                      const int64_t *l_strides, int causal, float scale, void *stream,
                                      int dtype) {
  if (!Q || !K || !V || !O || !L || !q_strides || !k_strides || !v_strides || !o_strides || !l_strides)
    return FA_ERR_INVALID_ARGUMENT;
  if (B < 1 || H < 1 || Nq < 1 || Nk < 1 || d < 1) return FA_ERR_INVALID_ARGUMENT;
  if (!(scale > 0.f) || !isfinite(log2e_scale(scale))) return FA_ERR_INVALID_ARGUMENT;  // finite scale * log2(e)
  if (dtype != FA_DTYPE_F32 && dtype != FA_DTYPE_BF16) return FA_ERR_INVALID_ARGUMENT;
  const int64_t *ts[4] = {q_strides, k_strides, v_strides, o_strides};
  for (const int64_t *st : ts)
    for (int i = 0; i < 3; ++i)
      if (st[i] < 0 || st[i] > ((int64_t)1 << 40)) return FA_ERR_INVALID_ARGUMENT;
  for (int i = 0; i < 3; ++i)
    if (l_strides[i] < 0 || l_strides[i] > ((int64_t)1 << 40)) return FA_ERR_INVALID_ARGUMENT;
  for (const int64_t *st : ts)
    if (st[2] < d) return FA_ERR_INVALID_ARGUMENT;  // rows of a tensor do not overlap
  if (!non_overlapping(B, H, Nq, d, o_strides) || !non_overlapping(B, H, Nq, 1, l_strides))
    return FA_ERR_INVALID_ARGUMENT;
  const size_t esize = dtype == FA_DTYPE_BF16 ? 2 : 4;
  {
    int64_t extent;
    if (!element_extent(B, H, Nq, d, q_strides, esize, &extent) ||
        !element_extent(B, H, Nk, d, k_strides, esize, &extent) ||
        !element_extent(B, H, Nk, d, v_strides, esize, &extent) ||
        !element_extent(B, H, Nq, d, o_strides, esize, &extent) ||
        !element_extent(B, H, Nq, 1, l_strides, sizeof(float), &extent))
      return FA_ERR_INVALID_ARGUMENT;  // an array spans more than 2^62 bytes
  }
  if (!supported_head_dim(d)) return FA_ERR_UNSUPPORTED;
  if (!supported_sizes(dtype, B, H, Nq, Nk)) return FA_ERR_UNSUPPORTED;
  for (const int64_t *st : ts)
    if (st[2] * (int64_t)esize > ((int64_t)1 << 24)) return FA_ERR_UNSUPPORTED;
  if (l_strides[2] > ((int64_t)1 << 31) - 1) return FA_ERR_UNSUPPORTED;
  const Span sq = tensor_span(Q, B, H, Nq, d, q_strides, esize);
  const Span sk = tensor_span(K, B, H, Nk, d, k_strides, esize);
  const Span sv = tensor_span(V, B, H, Nk, d, v_strides, esize);
  const Span so = tensor_span(O, B, H, Nq, d, o_strides, esize);
  const Span sl = tensor_span(L, B, H, Nq, 1, l_strides, sizeof(float));
  if (spans_overlap(so, sq) || spans_overlap(so, sk) || spans_overlap(so, sv) || spans_overlap(so, sl) ||
      spans_overlap(sl, sq) || spans_overlap(sl, sk) || spans_overlap(sl, sv))
    return FA_ERR_INVALID_ARGUMENT;
  const int64_t emask = 16 / (int64_t)esize - 1;  // element strides keep 16-byte row alignment
  if (((uintptr_t)Q | (uintptr_t)K | (uintptr_t)V | (uintptr_t)O) & 15) return FA_ERR_MISALIGNED;
  if ((uintptr_t)L & 3) return FA_ERR_MISALIGNED;
  for (const int64_t *st : ts)
    if ((st[0] | st[1] | st[2]) & emask) return FA_ERR_MISALIGNED;

  FwdParams p{};
  p.Q = Q;
  p.K = K;
  p.V = V;
  p.O = O;
  p.L = L;
  p.q_b = q_strides[0];
  p.q_h = q_strides[1];
  p.q_r = (int)q_strides[2];
  p.k_b = k_strides[0];
  p.k_h = k_strides[1];
  p.k_r = (int)k_strides[2];
  p.v_b = v_strides[0];
  p.v_h = v_strides[1];
  p.v_r = (int)v_strides[2];
  p.o_b = o_strides[0];
  p.o_h = o_strides[1];
  p.o_r = (int)o_strides[2];
  p.l_b = l_strides[0];
  p.l_h = l_strides[1];
  p.l_r = (int)l_strides[2];
  p.H = (int)H;
  p.Nq = (int)Nq;
  p.Nk = (int)Nk;
  p.c = log2e_scale(scale);
  return launch_checked(dtype, d, causal, B * H, stream, p);
}

extern "C" const char *fa_status_string(int status) {
  switch (status) {
    case FA_OK: return "ok";
    case FA_ERR_INVALID_ARGUMENT: return "invalid argument";
    case FA_ERR_UNSUPPORTED: return "unsupported head dimension or size";
    case FA_ERR_MISALIGNED: return "buffer not 16-byte aligned";
    case FA_ERR_LAUNCH: return "kernel launch failed";
    case FA_ERR_JIT: return "run-time compilation of a specialized kernel failed";
    case FA_ERR_SCRATCH_LIMIT: return "problem larger than the static workspace of fa_bwd_noalloc";
    default: return "unknown status";
  }
}

extern "C" int fa_version(void) { return 100; }
