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

// hi + lo bf16 split of 8 fp32 values (two MFMA operands): hi = the upper 16 bits of each value (rounded
// toward zero: one byte permute per pair), lo = the exact remainder x - hi rounded to the nearest bf16 (one
// packed conversion per pair).  hi + lo carries 16 significant bits, in fp32's exponent range.
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ void split_bf16x8(const float (&x)[8], bf16x8& hi, bf16x8& lo) {
  uint32_t h[4], l[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const uint32_t a = __float_as_uint(x[2 * q]), b = __float_as_uint(x[2 * q + 1]);
    h[q] = __builtin_amdgcn_perm(b, a, 0x07060302u);  // [a.bits 16-31, b.bits 16-31]
    const f32x2 r = {x[2 * q] - __uint_as_float(a & 0xFFFF0000u), x[2 * q + 1] - __uint_as_float(b & 0xFFFF0000u)};
    l[q] = __builtin_bit_cast(uint32_t, __builtin_convertvector(r, bf16x2));
  }
  hi = __builtin_bit_cast(bf16x8, h);
  lo = __builtin_bit_cast(bf16x8, l);
}

// 16x16x32 bf16: the same operand and result layout as the fp16 one.
__device__ __forceinline__ f32x4 mfma16b(const bf16x8& a, const bf16x8& b, const f32x4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
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
__device__ __forceinline__ bf16x8 join_bf16(i16x4 a, i16x4 b) {
  typedef short i16x8 __attribute__((ext_vector_type(8)));
  i16x8 v = {a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
  return __builtin_bit_cast(bf16x8, v);
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

// ---------------------------------------------------------------- scaled fp16 copies of bf16 tensors
//
// The products with a probability or its gradient run on fp16 MFMA, whose operands span [2^-24, 65504]
// only (normal from 2^-14), while bf16 spans fp32's range: activations of any magnitude, and gradients
// dO that are typically 1e-6..1e-8 in training.  Each (b, h) slice of a tensor is therefore copied to fp16
// multiplied by a power of two 2^e chosen from the slice's largest magnitude, so that it lands in
// [2^a, 2^(a+1)); the kernels undo the scales exactly (ldexp) on their fp32 results.  Power-of-two scaling
// is exact for every value that stays normal in fp16.  The targets a per tensor:
//   Q, K:  14  -- the widest range fp16 allows: values down to 2^-28 of the slice's largest stay normal;
//   V:      3  -- and dO: 2, so that |dO.V^T - D| <= 2 d max|dO| max|V| < 2^(1+7+3+4) = 2^15 for d <= 128
//              (|D| = |dO.O| <= d max|dO| max|V|: O is a convex combination of V rows), i.e. dS = P (dP - D)
//              and its fp16 hi part stay below 2^15.
// The exponent table [4][B*H] (Q, K, V, dO) is written once per call and read by the attention kernels.
constexpr int kExpTargetQK = 14;
constexpr int kExpTargetV = 3;
constexpr int kExpTargetDO = 2;
constexpr int kAmaxChunks = 32;  // partial maxima per (tensor, b, h) slice
enum { kTQ = 0, kTK = 1, kTV = 2, kTDO = 3 };

// The scale exponent for a slice whose largest |bf16| has the bit pattern amax (sign cleared): 2^e * amax
// lies in [2^target, 2^(target+1)).  An all-zero slice keeps e = 0; bf16 subnormals are treated as 2^-126;
// e is clamped to [-100, 100] (slices beyond that lose resolution, as they would in any fp16 copy).
__host__ __device__ __forceinline__ int scale_exponent(uint32_t amax, int target) {
  if (amax == 0u) return 0;
  const int E = (int)(amax >> 7);  // biased exponent of a bf16 (0 for subnormals)
  const int e = target - ((E < 1 ? 1 : E) - 127);
  return e < -100 ? -100 : (e > 100 ? 100 : e);
}

// Up to four bf16 tensors [B*H, n_per_bh] whose per-slice maxima are wanted (null: skipped).
struct AmaxSrc {
  const uint16_t* t[4];
};

namespace {
// Partial maxima of |x| per (tensor, b*h, chunk): part[(t * BH + bh) * kAmaxChunks + chunk] (bf16 bit
// patterns with the sign cleared, which order like the magnitudes).  Grid (kAmaxChunks, BH, 4).
__global__ __launch_bounds__(256) void amax_kernel(AmaxSrc src, uint32_t* __restrict__ part, int64_t n_per_bh,
                                                   int BH) {
  __shared__ uint32_t wmax[4];
  const int t = blockIdx.z, bh = blockIdx.y, chunk = blockIdx.x;
  if (!src.t[t]) return;  // uniform over the workgroup
  const int64_t n16 = n_per_bh / 8;
  const int64_t lo = n16 * chunk / kAmaxChunks, hi = n16 * (chunk + 1) / kAmaxChunks;
  const uint4* p = reinterpret_cast<const uint4*>(src.t[t] + (int64_t)bh * n_per_bh);
  auto amax8 = [](const uint4& v) {
    const uint32_t w[4] = {v.x & 0x7FFF7FFFu, v.y & 0x7FFF7FFFu, v.z & 0x7FFF7FFFu, v.w & 0x7FFF7FFFu};
    uint32_t r = 0;
#pragma unroll
    for (int q = 0; q < 4; ++q) r = max(r, max(w[q] & 0xFFFFu, w[q] >> 16));
    return r;
  };
  uint32_t m = 0;
  int64_t i = lo + threadIdx.x;
  for (; i + 3 * 256 < hi; i += 4 * 256) {  // four loads in flight per thread
    uint4 v[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) v[u] = p[i + u * 256];
#pragma unroll
    for (int u = 0; u < 4; ++u) m = max(m, amax8(v[u]));
  }
  for (; i < hi; i += 256) m = max(m, amax8(p[i]));
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) m = max(m, (uint32_t)__shfl_xor((int)m, off));
  if ((threadIdx.x & 63) == 0) wmax[threadIdx.x >> 6] = m;
  __syncthreads();
  if (threadIdx.x == 0)
    part[((int64_t)t * BH + bh) * kAmaxChunks + chunk] = max(max(wmax[0], wmax[1]), max(wmax[2], wmax[3]));
}
}  // namespace

inline hipError_t launch_amax(const AmaxSrc& src, uint32_t* part, int64_t n_per_bh, int BH, hipStream_t st) {
  hipLaunchKernelGGL(amax_kernel, dim3(kAmaxChunks, BH, 4), dim3(256), 0, st, src, part, n_per_bh, BH);
  return hipGetLastError();
}

// The exponent of slice (t, bh) from its partial maxima.
__device__ __forceinline__ int slice_exponent(const uint32_t* __restrict__ part, int t, int bh, int BH, int target) {
  const uint32_t* pp = part + ((int64_t)t * BH + bh) * kAmaxChunks;
  uint32_t m = 0;
#pragma unroll 8
  for (int c = 0; c < kAmaxChunks; ++c) m = max(m, pp[c]);
  return scale_exponent(m, target);
}

// 8 bf16 values (one 16-byte register) times 2^e, rounded to fp16 (nearest even; exact while the scaled
// value is a normal fp16 number, which the exponent choice makes true for the slice's larger values).
__device__ __forceinline__ uint4 bf16x8_to_f16x8_scaled(const uint4& v, int e) {
  uint4 r;
  const uint32_t* w = reinterpret_cast<const uint32_t*>(&v);
  uint32_t* o = reinterpret_cast<uint32_t*>(&r);
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const float lo = __builtin_ldexpf(__uint_as_float(w[q] << 16), e);
    const float hi = __builtin_ldexpf(__uint_as_float(w[q] & 0xFFFF0000u), e);
    const _Float16 a = (_Float16)lo, b = (_Float16)hi;
    o[q] = (uint32_t)__builtin_bit_cast(uint16_t, a) | ((uint32_t)__builtin_bit_cast(uint16_t, b) << 16);
  }
  return r;
}

namespace {
// Scaled fp16 copy of one bf16 tensor [B*H, n_per_bh] (tensor slot t of the exponent table).  Grid
// (chunks, BH); the first workgroup of each slice also writes its exponent to ex[t * BH + bh].
__global__ __launch_bounds__(256) void cvt_scaled_kernel(const uint16_t* __restrict__ src, uint16_t* __restrict__ dst,
                                                         const uint32_t* __restrict__ part, int32_t* __restrict__ ex,
                                                         int t, int target, int64_t n_per_bh, int BH) {
  const int bh = blockIdx.y;
  const int e = slice_exponent(part, t, bh, BH, target);
  if (blockIdx.x == 0 && threadIdx.x == 0) ex[t * BH + bh] = e;
  const int64_t n16 = n_per_bh / 8;
  const int64_t lo = n16 * blockIdx.x / gridDim.x, hi = n16 * (blockIdx.x + 1) / gridDim.x;
  const uint4* s = reinterpret_cast<const uint4*>(src + (int64_t)bh * n_per_bh);
  uint4* d = reinterpret_cast<uint4*>(dst + (int64_t)bh * n_per_bh);
  for (int64_t i = lo + threadIdx.x; i < hi; i += 256) d[i] = bf16x8_to_f16x8_scaled(s[i], e);
}
}  // namespace

// The forward's V: per-slice maxima, then the scaled copy and its exponent (slot kTV of ex).
inline hipError_t launch_cvt_scaled_v(const void* V, uint16_t* V16, uint32_t* part, int32_t* ex, int64_t n_per_bh,
                                      int BH, hipStream_t st) {
  AmaxSrc a = {{nullptr, nullptr, static_cast<const uint16_t*>(V), nullptr}};
  hipError_t e = launch_amax(a, part, n_per_bh, BH, st);
  if (e != hipSuccess) return e;
  const int64_t per = n_per_bh / 8 / 256;  // 256-thread passes per slice
  const unsigned chunks = (unsigned)std::max<int64_t>(1, std::min<int64_t>(64, per / 4));
  hipLaunchKernelGGL(cvt_scaled_kernel, dim3(chunks, BH), dim3(256), 0, st, static_cast<const uint16_t*>(V), V16,
                     part, ex, (int)kTV, kExpTargetV, n_per_bh, BH);
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
