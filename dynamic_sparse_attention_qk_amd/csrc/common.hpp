// Shared device-side definitions of the gfx950 sparse-attention kernels.
//
// MFMA operand/result layouts used throughout (wave64, checked on gfx950):
//   v_mfma_f32_32x32x16_bf16  D[32x32] += A[32x16] * B[16x32]
//     lane l supplies A[l%32][8*(l/32) + e] and B[8*(l/32) + e][l%32], e = 0..7;
//     lane l receives D[8*(e/4) + 4*(l/32) + e%4][l%32], e = 0..15.
//   v_mfma_f32_32x32x2_f32    same output layout; lane l supplies A[l%32][l/32]
//     and B[l/32][l%32].
// The k index inside one MFMA may be permuted freely as long as A and B use
// the same permutation; the kernels exploit that to feed softmax results
// straight from accumulators into the next product.
#pragma once

#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <stdint.h>

namespace dsa {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint16_t bf16_t;  // bf16 storage (bit pattern)

constexpr int kBlock = 64;      // KV block size (tokens)
constexpr int kMaxHeads = 128;  // capacity of the per-head table passed by value
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// Per-head kept-block counts, passed by value in the kernel arguments.
// Row (b, h, g) of a kept-block list starts at
//   b * NG * ksum + NG * kofs[h] + g * k[h].
struct HeadTable {
  int32_t k[kMaxHeads];
  int32_t kofs[kMaxHeads + 1];
  int32_t ksum;
};

__device__ __forceinline__ int64_t row_base(const HeadTable& ht, int b, int h, int ng) {
  return (int64_t)b * ng * ht.ksum + (int64_t)ng * ht.kofs[h];
}

__device__ __forceinline__ int lane_id() { return threadIdx.x & 63; }

// Number of set bits of m held by lanes below this one.
__device__ __forceinline__ int mask_rank(uint64_t m) {
  return __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
}

__device__ __forceinline__ float bf16_to_f32(bf16_t v) {
  return __uint_as_float(((uint32_t)v) << 16);
}

// Order-preserving map of an fp32 score to uint32 (larger score -> larger
// key); -0.0 is folded onto +0.0 first so that IEEE-equal scores tie.
__device__ __forceinline__ uint32_t score_key(float s) {
  uint32_t b = __float_as_uint(s);
  if (b == 0x80000000u) b = 0u;
  return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}

// The block score: tau * (qhat . khat) as a fixed fma chain over r, shared by
// the materialising and the streaming kernels so their scores are bit-equal.
template <int R>
__device__ __forceinline__ float score_dot(const float* __restrict__ qh, const float* __restrict__ kh, float tau) {
  float acc = 0.f;
#pragma unroll
  for (int r = 0; r < R; ++r) acc = __builtin_fmaf(qh[r], kh[r], acc);
  return acc * tau;
}

__device__ __forceinline__ f32x16 mfma32(const bf16x8& a, const bf16x8& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// fp16 operands: used where one operand is a softmax probability or its
// gradient (rounded from fp32) so that rounding stays 8x below bf16's.
__device__ __forceinline__ f32x16 mfma32h(const f16x8& a, const f16x8& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
}

// 16x16x32 fp16: lane l supplies A[l%16][8*(l/16) + e] and B[8*(l/16) + e][l%16],
// e = 0..7, and receives D[4*(l/16) + e][l%16], e = 0..3.
__device__ __forceinline__ f32x4 mfma16h(const f16x8& a, const f16x8& b, const f32x4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ f32x16 mfma32_f32(float a, float b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, 0, 0, 0);
}


__device__ __forceinline__ f16x8 pack_f16(const f32x16& x, int c) {
  f16x8 r;
#pragma unroll
  for (int e = 0; e < 8; ++e) r[e] = (_Float16)x[8 * c + e];
  return r;
}


// Exact conversion of 8 bf16 values (one 16-byte register) to fp16: every
// bf16 value of magnitude in [2^-14, 65504] is representable in fp16.
__device__ __forceinline__ uint4 bf16x8_to_f16x8(const uint4& v) {
  uint4 r;
  const uint32_t* w = reinterpret_cast<const uint32_t*>(&v);
  uint32_t* o = reinterpret_cast<uint32_t*>(&r);
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const float lo = __uint_as_float(w[q] << 16), hi = __uint_as_float(w[q] & 0xFFFF0000u);
    o[q] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_pkrtz(lo, hi));
  }
  return r;
}



// 16-byte global load / store helpers.
__device__ __forceinline__ uint4 ldg16(const void* p) { return *reinterpret_cast<const uint4*>(p); }



// ---------------------------------------------------------------- LDS tiles filled by DMA
// A 64 x D 16-bit tile is stored row-major without padding (row = 2*D bytes)
// with its 16-byte chunks XOR-swizzled per row: physical chunk p of row r holds
// logical chunk p ^ tile_swz<D>(r).  gfx950's LDS serves 64 banks (256 bytes)
// per cycle; the swizzle puts each hardware pass of every access pattern of
// the kernels on distinct 16-byte bank groups:
//   - 8 or 16 consecutive rows read at one logical chunk (128-bit reads),
//   - 4 consecutive rows x 4 chunks, 4 rows x 2 chunks and 8 rows x 2 chunks
//     at aligned positions (the lane groups of transpose reads feeding 32x32
//     and 16x16 MFMAs).
// For D = 128 (256-byte rows) the row bits r3 r2 r1 r0 map to r1 r0 (r2^r3) r2,
// the one map among those measured with no conflict in any of the four
// patterns (the plain reordering r1 r0 r2 r3 costs the 16x16 operand reads of
// the dK/dV kernel one extra pass in two); for D = 64 two rows share a
// 256-byte window, r0 picks the half, and the 3-bit chunk map is r1 (r2^r3) r2.
typedef __attribute__((address_space(3))) void lds_void;
typedef short i16x4 __attribute__((ext_vector_type(4)));

template <int D>
__device__ __forceinline__ int tile_swz(int r) {
  if constexpr (D == 128) {
    const int r2 = (r >> 2) & 1, r3 = (r >> 3) & 1;
    return ((r & 3) << 2) | ((r2 ^ r3) << 1) | r2;
  } else {
    const int r1 = (r >> 1) & 1, r2 = (r >> 2) & 1, r3 = (r >> 3) & 1;
    return (r1 << 2) | ((r2 ^ r3) << 1) | r2;
  }
}

// Byte offset of logical chunk q of row r.
template <int D>
__device__ __forceinline__ int tile_off(int r, int q) { return r * (2 * D) + 16 * (q ^ tile_swz<D>(r)); }

// Issue the global->LDS copies of one 64 x D tile (rows of D contiguous 16-bit
// values starting at src) into the LDS tile at lds_base; the NW waves of the
// workgroup share the D/8 one-kilobyte copies.  Completion is awaited with
// wait_vmem() before the workgroup barrier that publishes the tile.
template <int D, int NW>
__device__ __forceinline__ void dma_tile(const uint16_t* __restrict__ src, char* lds_base, int wave, int lane) {
  constexpr int RB = 2 * D;            // bytes per row
  constexpr int RPI = 1024 / RB;       // rows per 1 KB copy
  static_assert((D / 8) % NW == 0, "each wave issues the same number of copies");
  const int rin = (lane * 16) / RB;    // row within the copy
  const int p = ((lane * 16) % RB) / 16;
#pragma unroll
  for (int i = 0; i < D / 8 / NW; ++i) {
    const int j = wave + i * NW;
    const int r = j * RPI + rin;
    // uniform base + 32-bit per-lane byte offset (the scalar-base addressing form)
    uint32_t off = (uint32_t)(2 * (r * D + 8 * (p ^ tile_swz<D>(r))));
    asm volatile("" : "+v"(off));  // keeps the offset 32-bit at the load (not widened once outside a loop)
    const void* g = reinterpret_cast<const char*>(src) + off;
    __builtin_amdgcn_global_load_lds(g, (lds_void*)(lds_base + j * 1024), 16, 0, 0);
  }
}

// A list entry read through the vector memory path (a per-lane address the
// compiler cannot prove uniform), for reads issued steps ahead of their use:
// a scalar load in flight would force every LDS operand wait of the step to
// drain the whole LDS/scalar counter, while a vector load is counted with the
// tile copies, which each step drains anyway.  Take readfirstlane at the use.
__device__ __forceinline__ int32_t ldv_i32(const int32_t* __restrict__ p) {
  int32_t z;
  asm volatile("v_mov_b32 %0, 0" : "=v"(z));
  return p[z];
}

__device__ __forceinline__ void wait_vmem() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }



// 4-byte-per-lane DMA of 64 consecutive floats (one wave) into LDS.
__device__ __forceinline__ void dma_row64_f32(const float* __restrict__ src, char* lds, int lane) {
  // 4 * lane, recomputed at each use (a loop-invariant copy would hold a register)
  uint32_t off;
  asm volatile("v_mbcnt_lo_u32_b32 %0, -1, 0\n\tv_mbcnt_hi_u32_b32 %0, -1, %0\n\tv_lshlrev_b32 %0, 2, %0" : "=v"(off));
  __builtin_amdgcn_global_load_lds(reinterpret_cast<const char*>(src) + off, (lds_void*)lds, 4, 0, 0);
}

// Transpose read (ds_read_b64_tr_b16): within each 16-lane group, lane i
// receives element i%4 of the 8-byte chunks addressed by lanes 4e + i/4 of the
// group, e = 0..3.  If lane L addresses row (r0 + L/4), columns c0 + 4*(L%4),
// lane i receives column c0 + i of rows r0..r0+3.
__device__ __forceinline__ i16x4 lds_read_tr16(const char* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) i16x4*)(p));
}

__device__ __forceinline__ f16x8 join_f16(i16x4 a, i16x4 b) {
  typedef short i16x8 __attribute__((ext_vector_type(8)));
  i16x8 v = {a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
  return __builtin_bit_cast(f16x8, v);
}



// Workgroups are dispatched round-robin over the 8 XCDs (each with its own
// L2).  Map the hardware id w (of n) to a logical index such that every XCD
// runs one contiguous range of the logical order -- neighbouring query groups,
// which share most kept blocks, then meet in the same L2.  (Interleaving
// 64-item runs across the XCDs measured slower on the 57.6k-token workload.)
constexpr uint32_t kXcds = 8;
// Work-balanced variant for kernels whose tasks (ordered (b, h, item)) cost
// different amounts per head: the host cuts the task list into kXcds
// contiguous ranges of about equal work; workgroup w runs task start[x] + w / 8
// of XCD x = w % 8, or exits at once when that is past the range.  The grid is
// 8 x the longest range.  With equal work per task this is xcd_remap.
// Workgroup w runs on XCD w % 8.  Tasks are numbered run by run ((b, h) pairs), `items` per run, and
// split over the XCDs in one of two ways:
//  - contiguous (items == 0 in the struct): XCD x runs tasks [start[x], start[x+1]), eight ranges of
//    equal estimated work; each XCD then works through a few heads of its own;
//  - head-synchronous (items > 0): every run is cut into eight contiguous parts of equal count and XCD
//    x takes part x of every run, runs in order, so all XCDs work on the same head at a time.
// Both keep contiguous groups (or blocks) of one head on each XCD, which is what its L2 reuses.  The
// host picks head-synchronous when eight heads' K and V (or Q and dO) would not fit the 256 MB MALL.
struct XcdSplit {
  int32_t start[kXcds + 1];
  int32_t items;  // head-synchronous: tasks per run (0: contiguous ranges)
  int32_t runs;   // head-synchronous: B * H
};

__device__ __forceinline__ int64_t xcd_task(const XcdSplit& sp, uint32_t w) {
  const int32_t x = (int32_t)(w % kXcds), i = (int32_t)(w / kXcds);
  if (sp.items == 0) {
    const int64_t t = (int64_t)sp.start[x] + i;
    return t < sp.start[x + 1] ? t : -1;
  }
  const int32_t lo = (int32_t)((int64_t)x * sp.items / kXcds);
  const int32_t len = (int32_t)((int64_t)(x + 1) * sp.items / kXcds) - lo;
  if (len <= 0) return -1;
  const int32_t run = i / len;
  if (run >= sp.runs) return -1;
  return (int64_t)run * sp.items + lo + i % len;
}

// Host: the split of the B*H*items tasks, a task of head h costing k_h * scale + overhead; head_bytes is
// what one (b, h) run streams (K and V, or Q and dO), which decides the mode.  grid covers the largest part.
// MI355X's Infinity Cache (MALL), shared by the XCDs
constexpr double kMallBytes = 256.0 * 1024 * 1024;
// Phases of the attention kernels when one head's K and V (or Q and dO) fill more than half the MALL:
// segments of every list in sequence.  Measured at 520k tokens (one pass / 4 / 8 phases, ms): forward
// 688 / 578 / 542, dQ 677 / 600 / 569, dK/dV 828 / 793 / 825.
constexpr int kMallPhasesKV = 8;   // kernels streaming K and V tiles (forward, dQ)
constexpr int kMallPhasesQdO = 4;  // the kernel streaming Q and dO tiles (dK/dV)

inline XcdSplit make_xcd_split(int B, int H, int items, const HeadTable& ht, double scale, double overhead,
                               double head_bytes, unsigned* grid) {
  XcdSplit sp;
  if (kXcds * head_bytes > kMallBytes) {
    sp.items = items;
    sp.runs = B * H;
    for (uint32_t i = 0; i <= kXcds; ++i) sp.start[i] = 0;
    *grid = kXcds * (unsigned)((items + kXcds - 1) / kXcds) * (unsigned)(B * H);
    return sp;
  }
  sp.items = 0;
  sp.runs = 0;
  double total = 0.0;
  for (int h = 0; h < H; ++h) total += (double)B * items * (ht.k[h] * scale + overhead);
  sp.start[0] = 0;
  uint32_t x = 1;
  double cum = 0.0;
  int64_t t = 0;
  for (int b = 0; b < B; ++b)
    for (int h = 0; h < H; ++h) {
      const double wt = ht.k[h] * scale + overhead;
      while (x < kXcds && cum + items * wt >= total * x / kXcds) {
        int64_t m = (int64_t)std::ceil((total * x / kXcds - cum) / wt);
        m = m < 0 ? 0 : (m > items ? items : m);
        sp.start[x++] = (int32_t)(t + m);
      }
      cum += items * wt;
      t += items;
    }
  while (x <= kXcds) sp.start[x++] = (int32_t)t;
  int32_t longest = 0;
  for (uint32_t i = 0; i < kXcds; ++i) longest = std::max(longest, sp.start[i + 1] - sp.start[i]);
  *grid = kXcds * (unsigned)longest;
  return sp;
}

// The XCD parts as segments [first, last) of the task range: the contiguous ranges, or one per (run, XCD).
__device__ __forceinline__ void xcd_segment(const XcdSplit& sp, int s, int32_t& first, int32_t& last) {
  if (sp.items == 0) {
    first = sp.start[s];
    last = sp.start[s + 1];
    return;
  }
  const int x = s % kXcds, run = s / kXcds;
  first = run * sp.items + (int32_t)((int64_t)x * sp.items / kXcds);
  last = run * sp.items + (int32_t)((int64_t)(x + 1) * sp.items / kXcds);
}

__device__ __forceinline__ uint32_t xcd_remap(uint32_t w, uint32_t n) {
  const uint32_t q = n / kXcds, r = n % kXcds;
  const uint32_t x = w % kXcds, i = w / kXcds;
  return (x < r ? x * (q + 1) : r * (q + 1) + (x - r) * q) + i;
}

// bf16 -> fp16 shadow copy (exact for |x| in [2^-14, 65504]); 8 values per thread step.
namespace {
__global__ __launch_bounds__(256) void cvt_bf16_f16_kernel(const uint4* __restrict__ src, uint4* __restrict__ dst,
                                                           int64_t n16) {
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n16; i += (int64_t)gridDim.x * 256)
    dst[i] = bf16x8_to_f16x8(src[i]);
}
}  // namespace

inline hipError_t launch_cvt_f16(const void* src, void* dst, int64_t elems, hipStream_t st) {
  const int64_t n16 = elems / 8;
  const int64_t nwg = (n16 + 255) / 256;
  hipLaunchKernelGGL(cvt_bf16_f16_kernel, dim3((unsigned)(nwg < 8192 ? nwg : 8192)), dim3(256), 0, st,
                     static_cast<const uint4*>(src), static_cast<uint4*>(dst), n16);
  return hipGetLastError();
}

// Max / sum of v over the lane pair (l, l ^ 32), by v_permlane32_swap (no LDS
// round trip): the two results of the swap hold v of both lanes of the pair.
__device__ __forceinline__ float wave_max_pair(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float wave_sum_pair(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Sum of the 8 fp16 values of x, accumulated in fp32 onto acc (v_dot2 with ones).
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ float sum_f16x8(const f16x8& x, float acc) {
#pragma unroll
  for (int i = 0; i < 4; ++i) acc = __builtin_amdgcn_fdot2(f16x2{x[2 * i], x[2 * i + 1]}, f16x2{1, 1}, acc, false);
  return acc;
}

}  // namespace dsa
