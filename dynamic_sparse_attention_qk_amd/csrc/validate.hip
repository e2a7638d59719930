// List checks of the debug build (DSA_DEBUG).
//
// The attention kernels take the kept-block lists and the reverse index as
// given; a release build clamps every id it reads into range, so a corrupt
// list gives wrong results but never an access out of bounds.  A debug build
// runs these checks before the attention launches instead and turns a bad
// list into an error.  What a valid list is follows from how selection writes
// it: each (b, h, g) row holds its kept block ids in strictly ascending order,
// all in [0, NB) (with per-row counts in [1, k_h]: the first cnt entries, the
// rest -1);
// rev_ptr of each (b, h) starts at 0 and never decreases, and each block's
// reverse list holds strictly ascending group ids in [0, NG).
//
// The first failure found (by any thread) is recorded in err[0..3]: a code,
// the row or (b, h, block) index, the position in the list and the value.
#include "launch.hpp"

namespace dsa {

namespace {

__device__ __forceinline__ void report(uint32_t* err, uint32_t code, int64_t where, int64_t pos, int64_t value) {
  if (atomicCAS(&err[0], 0u, code) == 0u) {
    err[1] = (uint32_t)where;
    err[2] = (uint32_t)pos;
    err[3] = (uint32_t)value;
  }
}

// one thread per (b, h, g) row
__global__ __launch_bounds__(256) void check_kept_kernel(const int32_t* __restrict__ idx,
                                                         const int32_t* __restrict__ cnt, HeadTable ht, int NG,
                                                         int NB, int B, int H, uint32_t* err) {
  const int64_t row = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (row >= (int64_t)B * H * NG) return;
  const int g = (int)(row % NG);
  const int64_t bh = row / NG;
  const int h = (int)(bh % H), b = (int)(bh / H);
  const int k = ht.k[h];
  const int n = cnt ? cnt[row] : k;
  if (n < 1 || n > k) {
    report(err, kListBadCount, row, -1, n);
    return;
  }
  const int32_t* r = idx + row_base(ht, b, h, NG) + (int64_t)g * k;
  int32_t prev = -1;
  for (int p = 0; p < k; ++p) {
    const int32_t v = r[p];
    if (p < n) {
      if (v < 0 || v >= NB) { report(err, kListOutOfRange, row, p, v); return; }
      if (v <= prev) { report(err, kListNotAscending, row, p, v); return; }
      prev = v;
    } else if (v != -1) {
      report(err, kListBadPadding, row, p, v);
      return;
    }
  }
}

// one thread per (b, h, block)
__global__ __launch_bounds__(256) void check_rev_kernel(const int32_t* __restrict__ rev_ptr,
                                                        const int32_t* __restrict__ rev_idx, HeadTable ht, int NG,
                                                        int NB, int B, int H, uint32_t* err) {
  const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (t >= (int64_t)B * H * NB) return;
  const int j = (int)(t % NB);
  const int64_t bh = t / NB;
  const int h = (int)(bh % H), b = (int)(bh / H);
  const int32_t* rp = rev_ptr + bh * (NB + 1);
  const int64_t cap = (int64_t)NG * ht.k[h];
  if (j == 0 && rp[0] != 0) { report(err, kRevBadPointer, t, 0, rp[0]); return; }
  const int32_t s0 = rp[j], s1 = rp[j + 1];
  if (s1 < s0 || s0 < 0 || s1 > cap) { report(err, kRevBadPointer, t, j + 1, s1); return; }
  const int32_t* list = rev_idx + row_base(ht, b, h, NG) + s0;
  int32_t prev = -1;
  for (int32_t i = 0; i < s1 - s0; ++i) {
    const int32_t v = list[i];
    if (v < 0 || v >= NG) { report(err, kRevOutOfRange, t, i, v); return; }
    if (v <= prev) { report(err, kRevNotAscending, t, i, v); return; }
    prev = v;
  }
}

}  // namespace

hipError_t launch_check_lists(const Shape& s, const HeadTable& ht, const int32_t* idx, const int32_t* cnt,
                              const int32_t* rev_ptr, const int32_t* rev_idx, uint32_t* err, hipStream_t st) {
  if (idx) {
    const int64_t rows = (int64_t)s.B * s.H * s.NG;
    hipLaunchKernelGGL(check_kept_kernel, dim3((unsigned)((rows + 255) / 256)), dim3(256), 0, st, idx, cnt, ht, s.NG,
                       s.NB, s.B, s.H, err);
  }
  if (rev_ptr && rev_idx) {
    const int64_t n = (int64_t)s.B * s.H * s.NB;
    hipLaunchKernelGGL(check_rev_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st, rev_ptr, rev_idx, ht,
                       s.NG, s.NB, s.B, s.H, err);
  }
  return hipGetLastError();
}

}  // namespace dsa
