// Device-side helpers shared by the forward and backward kernels of libfa.so
// (gfx950). Internal to the library: included only by its .hip sources.
#ifndef FA_DEVICE_H_
#define FA_DEVICE_H_

#if defined(__HIPCC_RTC__)
// Run-time compilation (hipRTC) provides the HIP device builtins but not the C
// headers: the fixed-width types and INFINITY come from the compiler itself.
typedef __UINT32_TYPE__ uint32_t;
typedef __INT64_TYPE__ int64_t;
typedef __UINTPTR_TYPE__ uintptr_t;
#define INFINITY (__builtin_inff())
#else
#include <hip/hip_runtime.h>

#include <math.h>
#include <stddef.h>
#include <stdint.h>
#endif

namespace {

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kRowsPerWave = 32;  // query rows per wave (MFMA N dimension)
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

// Workgroup index -> (head, query tile). Workgroups are dispatched to the
// eight XCDs round-robin (XCD = bid % 8, in order bid / 8 within an XCD).
// When the heads split evenly over the XCDs, XCD x takes heads
// [x*hpx, (x+1)*hpx), so each head's K/V stays in one XCD's L2, and works on
// them `group` heads at a time (group divides hpx; 0 or any other value: all
// hpx at once): the heads of one group, ordered by query tile, all heads at
// one tile before the next, then the next group. Otherwise the whole grid is
// ordered by query tile. For causal attention the tiles run from the last
// query tile (most key tiles) to the first, so the longest workgroups start
// first and the short ones fill the tail.
__device__ __forceinline__ void map_block(int bid, int nblocks, int n_qtiles, bool causal, int group,
                                          int &bh, int &qt) {
  const int n_heads = nblocks / n_qtiles;
  int t;
  if (n_heads % kNumXcd == 0) {
    const int hpx = n_heads / kNumXcd;
    const int g = (group > 0 && hpx % group == 0) ? group : hpx;
    const int xcd = bid % kNumXcd, slot = bid / kNumXcd;
    const int per = g * n_qtiles;  // workgroups of one group
    const int grp = slot / per, r = slot - grp * per;
    t = r / g;
    bh = xcd * hpx + grp * g + r % g;
  } else {
    t = bid / n_heads;
    bh = bid % n_heads;
  }
  qt = causal ? (n_qtiles - 1 - t) : t;
}

#if !defined(__HIPCC_RTC__)
// Host side of map_block: the heads each XCD works on at a time, the largest
// divisor of the XCD's heads whose streamed tiles (tile_bytes per head: K and V
// in the forward and the dQ kernel, Q and dO in the dK/dV kernel) total at most
// 8 MiB, at least one head; 0 (no grouping) when the heads do not split evenly
// over the XCDs. An XCD's L2 is 4 MB: with all of an XCD's heads at once the
// causal workloads read their tiles from HBM 4-7 times over; with groups of
// 8 MiB the concurrent workgroups of a group share its tiles closely enough in
// time (groups of 4 MiB fetch less but run slower).
inline int head_group(int64_t BH, int64_t tile_bytes) {
  constexpr int64_t kGroupBytes = (int64_t)8 << 20;
  if (BH < kNumXcd || BH % kNumXcd != 0) return 0;
  const int64_t hpx = BH / kNumXcd;
  const int64_t fit = kGroupBytes / (tile_bytes > 0 ? tile_bytes : 1);
  int64_t g = hpx < 4096 ? hpx : 4096;
  if (g > fit) g = fit > 0 ? fit : 1;
  while (hpx % g != 0) --g;
  return (int)g;
}

// The device a launch on `stream` runs on: the stream's own device, or the
// current device for the null stream.
inline hipError_t stream_device(hipStream_t stream, int *device) {
  if (!stream) return hipGetDevice(device);
  return hipStreamGetDevice(stream, device);
}

// Runs f() with `device` current and restores the caller's current device;
// hipErrorUnknown if f fails, else the first error of switching devices.
template <typename F>
hipError_t on_device(int device, F f) {
  int cur = 0;
  hipError_t e = hipGetDevice(&cur);
  if (e != hipSuccess) return e;
  if (cur != device && (e = hipSetDevice(device)) != hipSuccess) return e;
  const bool ok = f();
  if (cur != device && (e = hipSetDevice(cur)) != hipSuccess) return e;
  return ok ? hipSuccess : hipErrorUnknown;
}
#endif

// Layout of a bf16 tile of BN rows x D columns staged in LDS (rows of K, V, Q
// or dO). Rows are written by LDS DMA in 1 KiB wave instructions; inside a row
// the 16-byte chunks are XOR-permuted by one of three row functions, chosen per
// tile by how it is read:
//  * swz_k, for ds_read_b128 of 32 consecutive rows at one chunk: spreads 16
//    consecutive rows over the 16 slots of a 256-byte bank line;
//  * swz_v, for ds_read_b64_tr_b16 (a 16-lane group reads 4 consecutive rows x
//    32 bytes and its partner group the next 32 bytes): 4 * (row index within
//    the group of 4), so the 4 x 4 chunks of a group pair land in 16 slots;
//  * swz_b, for tiles read both ways (d = 64 and 128 only): the row's position
//    within its group of 4 sets chunk bits 2-3 (d = 128; at d = 64, where two
//    rows share a bank line, its bit 1 sets chunk bit 2) and the group's index
//    modulo 4 sets chunk bits 0-1, so both patterns fill each 256-byte bank
//    line once per pass (swz_k leaves the transposing reads 4-way conflicted
//    at d = 128 and 2-way at d = 64).
template <int D, int BN, int NW>
struct BfLayout {
  static constexpr int CPR = D / 8;                // 16-byte chunks per row
  static constexpr int RPB = 16 / CPR;             // rows per 256-byte bank line
  static constexpr int ROW = D * 2;                // bytes per row
  static constexpr int TILE = BN * ROW;            // bytes per K (or V) tile
  static constexpr int STAGE = 2 * TILE;           // K tile then V tile
  static constexpr int LOADS = TILE / 1024;        // wave instructions per tile matrix
  static constexpr int LPW = LOADS / NW;           // ... per wave
  static_assert(LOADS % NW == 0, "tile loads must split evenly over the waves");
  static_assert(BN % 32 == 0, "key tile is a multiple of the 32-key MFMA block");
  __device__ static constexpr int swz_k(int r) { return (r / RPB) & (CPR - 1); }
  __device__ static constexpr int swz_v(int r) { return 4 * ((r / RPB) & (4 / RPB - 1)); }
  __device__ static constexpr int swz_b(int r) {
    return CPR == 16 ? 4 * (r & 3) + ((r >> 2) & 3) : 4 * ((r >> 1) & 1) + ((r >> 2) & 3);
  }
};

typedef __attribute__((address_space(3))) void lds_void;

// LDS byte address of a pointer into a __shared__ array.
__device__ __forceinline__ uint32_t lds_addr(const void *p) {
  return (uint32_t)(uintptr_t)(const lds_void *)p;
}

// Buffer resource over `bytes` bytes at `base` (raw, unswizzled; reads past the
// end return zero).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void *base, int bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, bytes, 0x00020000);
}

// One wave's share of a tile matrix, LPW x buffer_load_dwordx4 ... lds: load i
// moves 16 bytes per lane from rsrc + vo[i] + 1024 i into LDS at byte address
// `lds` (via M0) + 1024 i + 16 * lane. The instruction offset (1024 i) is added
// to both the buffer offset, inside the range check, and the LDS address, so
// M0 is written once per share. Written as inline assembly so that the
// compiler does not treat every later LDS read as possibly aliasing these
// asynchronous writes (it would wait for the next tile's loads before reading
// the current one); the kernel publishes the data itself with s_waitcnt
// vmcnt(0) and a workgroup barrier. M0 is used by nothing else here.
// On GFX9-family GPUs an LDS DMA must not read M0 in the instruction right
// after the SALU write of M0: without the wait state (s_nop 0) the load can
// still see the previous M0 and land in the previous share's slots.
// The host compilation pass of the kernel templates never calls it.
template <int LPW>
__device__ __forceinline__ void load_lds_share(__amdgpu_buffer_rsrc_t rsrc, uint32_t lds, const int (&vo)[LPW]) {
#if defined(__HIP_DEVICE_COMPILE__)
  static_assert(LPW == 1 || LPW == 2 || LPW == 4, "one wave issues 1, 2 or 4 loads per tile matrix");
  if constexpr (LPW == 1)
    asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\t"
                 "buffer_load_dwordx4 %1, %2, 0 offen lds"
                 :
                 : "s"(lds), "v"(vo[0]), "s"(rsrc)
                 : "memory", "m0");
  else if constexpr (LPW == 4)
    asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\t"
                 "buffer_load_dwordx4 %1, %5, 0 offen lds\n\t"
                 "buffer_load_dwordx4 %2, %5, 0 offen offset:1024 lds\n\t"
                 "buffer_load_dwordx4 %3, %5, 0 offen offset:2048 lds\n\t"
                 "buffer_load_dwordx4 %4, %5, 0 offen offset:3072 lds"
                 :
                 : "s"(lds), "v"(vo[0]), "v"(vo[1]), "v"(vo[2]), "v"(vo[3]), "s"(rsrc)
                 : "memory", "m0");
  else
    asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\t"
                 "buffer_load_dwordx4 %1, %3, 0 offen lds\n\t"
                 "buffer_load_dwordx4 %2, %3, 0 offen offset:1024 lds"
                 :
                 : "s"(lds), "v"(vo[0]), "v"(vo[1]), "s"(rsrc)
                 : "memory", "m0");
#else
  (void)rsrc, (void)lds, (void)vo;
#endif
}

// N_ consecutive floats at byte offset `off` of a buffer resource, one
// range-checked load (zeros past the end).
template <int N_>
struct F32Vec;
template <>
struct F32Vec<1> {
  typedef float type __attribute__((ext_vector_type(1)));
  __device__ static type load(__amdgpu_buffer_rsrc_t r, int off) {
    type v;
    v[0] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(r, off, 0, 0));
    return v;
  }
};
template <>
struct F32Vec<2> {
  typedef float type __attribute__((ext_vector_type(2)));
  __device__ static type load(__amdgpu_buffer_rsrc_t r, int off) {
    return __builtin_bit_cast(type, __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, 0));
  }
};
template <>
struct F32Vec<4> {
  typedef f32x4 type;
  __device__ static type load(__amdgpu_buffer_rsrc_t r, int off) {
    return __builtin_bit_cast(type, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
  }
};

}  // namespace

#endif  // FA_DEVICE_H_
