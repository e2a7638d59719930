// Critical KV block selection and the reverse (block -> groups) index.
//
// DSV (gist.science explainer, hi edition) technical summary §2.A: the
// low-rank estimates pick the critical KV per query group; §2.B: the top-k
// selection is fused with the low-rank product so the O(S^2) score matrix need
// not exist (memory O(S*k)).
//
// topk_select: one wave64 per (b, h, g) row.  The row's NB scores are held as
// order-preserving uint32 keys in registers (KPL per lane, j = lane + 64*t).
// The k-th largest key T is found by a 32-step bisection whose counts are
// wave ballots; then every key > T and the lowest-index keys == T (as many as
// still needed) are emitted in ascending j order by ballot/rank compaction.
// In streaming mode the scores are computed in-kernel from qhat (registers) and
// khat chunks staged in LDS (shared by the 4 rows of a workgroup) with the
// same fma chain as block_scores, so both modes select identically.
//
// reverse index: count per block (integer atomics), exclusive scan, scatter,
// then each block's segment is put in ascending group order through an LDS
// bitmap -- a deterministic result for any atomic order.
#include "launch.hpp"

namespace dsa {

namespace {

constexpr int kSelThreads = 256;  // 4 rows per workgroup

template <int KPL>
__device__ __forceinline__ uint32_t wave_count_ge(const uint32_t (&key)[KPL], uint32_t cand) {
  uint32_t c = 0;
#pragma unroll
  for (int t = 0; t < KPL; ++t) c += (uint32_t)__popcll(__ballot(key[t] >= cand));
  return c;
}

// The score whose order-preserving key is k (inverse of score_key; -0.0 comes back as +0.0).
__device__ __forceinline__ float key_score(uint32_t k) {
  return __uint_as_float((k & 0x80000000u) ? (k & 0x7FFFFFFFu) : ~k);
}

template <int KPL>
__device__ __forceinline__ float wave_mass_ge(const uint32_t (&key)[KPL], const float (&e)[KPL], uint32_t cand) {
  float m = 0.f;
#pragma unroll
  for (int t = 0; t < KPL; ++t) m += key[t] >= cand ? e[t] : 0.f;
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) m += __shfl_xor(m, off);
  return m;
}

// COVER: the row keeps the shortest run of blocks, in score order, whose estimated attention mass (the
// softmax of the row's block scores) reaches `coverage` of the total, at most k_h; the count goes to
// cnt[b,h,g] and the row's unused slots get -1.
// diag_group > 0: the blocks holding the row's own diag_group query tokens are kept first (their keys are
// raised above every score; in COVER mode their real masses still count).
template <int KPL, int R, bool STREAM, bool COVER>
__global__ __launch_bounds__(kSelThreads) void topk_select_kernel(const float* __restrict__ scores,
                                                                   const float* __restrict__ qhat,
                                                                   const float* __restrict__ khat,
                                                                   int32_t* __restrict__ idx,
                                                                   int32_t* __restrict__ cnt,
                                                                   float* __restrict__ dump, HeadTable ht, int NG,
                                                                   int NB, int H, float tau, float coverage,
                                                                   int diag_group) {
  constexpr int CH = KPL < 4 ? KPL : (R > 32 ? 2 : 4);  // 64-block chunks of khat staged per LDS round
  __shared__ float sk[STREAM ? 64 * CH : 1][R + 1];
  const int b = blockIdx.z, h = blockIdx.y;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int g = blockIdx.x * 4 + wave;
  const bool valid = g < NG;
  const size_t bh = (size_t)b * H + h;
  uint32_t key[KPL];

  if constexpr (!STREAM) {
    const float* srow = scores + (bh * NG + (valid ? g : 0)) * (size_t)NB;
#pragma unroll
    for (int t = 0; t < KPL; ++t) {
      const int j = lane + 64 * t;
      key[t] = (valid && j < NB) ? score_key(srow[j]) : 0u;
    }
  } else {
    float q[R];
    const float* qrow = qhat + (bh * NG + (valid ? g : 0)) * (size_t)R;
#pragma unroll
    for (int r = 0; r < R; r += 4) {
      float4 v = *reinterpret_cast<const float4*>(qrow + r);
      q[r] = v.x; q[r + 1] = v.y; q[r + 2] = v.z; q[r + 3] = v.w;
    }
    const float* kbh = khat + bh * (size_t)NB * R;
    float* drow = dump ? dump + (bh * NG + (valid ? g : 0)) * (size_t)NB : nullptr;
#pragma unroll
    for (int t0 = 0; t0 < KPL; t0 += CH) {
      __syncthreads();
      for (int e = threadIdx.x; e < 64 * CH * R; e += kSelThreads) {
        const int jr = e / R, r = e % R;
        const int j = 64 * t0 + jr;
        sk[jr][r] = (j < NB) ? kbh[(size_t)j * R + r] : 0.f;
      }
      __syncthreads();
#pragma unroll
      for (int c = 0; c < CH; ++c) {
        const int t = t0 + c;
        const int j = lane + 64 * t;
        if (valid && j < NB) {
          const float s = score_dot<R>(q, &sk[64 * c + lane][0], tau);
          key[t] = score_key(s);
          if (drow) drow[j] = s;
        } else {
          key[t] = 0u;
        }
      }
    }
  }
  if (!valid) return;  // wave-uniform; all barriers are behind us

  const int kcap = ht.k[h];
  // forced blocks [d0, d1): the ones that hold this group's tokens
  const int d0 = diag_group ? g * diag_group / kBlock : 0, d1 = diag_group ? (g + 1) * diag_group / kBlock : 0;
  int k = kcap;
  uint32_t T = 0, need = 0;
  bool counted = true;  // T and need still to be found by the count bisection for k
  if constexpr (COVER) {
    // masses e_j = exp(s_j - s_max) (0 for the padding keys, which are 0), total Z = M(0)
    uint32_t kmax = 0;
#pragma unroll
    for (int t = 0; t < KPL; ++t) kmax = max(kmax, key[t]);
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) kmax = max(kmax, (uint32_t)__shfl_xor((int)kmax, off));
    const float smax = key_score(kmax);
    float e[KPL];
#pragma unroll
    for (int t = 0; t < KPL; ++t) {
      e[t] = key[t] ? expf(key_score(key[t]) - smax) : 0.f;
      const int j = lane + 64 * t;
      if (j >= d0 && j < d1) key[t] = 0xFFFFFFFFu;  // forced: above every real score (their masses stay)
    }
    const float target = coverage * wave_mass_ge<KPL>(key, e, 0u);
    // T = max{x : M(x) >= target}, M(x) = mass of the keys >= x (non-increasing in x)
#pragma unroll 1
    for (int bit = 31; bit >= 0; --bit) {
      const uint32_t cand = T | (1u << bit);
      if (wave_mass_ge<KPL>(key, e, cand) >= target) T = cand;
    }
    const bool top = T == 0xFFFFFFFFu;
    const uint32_t n_gt = top ? 0u : wave_count_ge<KPL>(key, T + 1u);
    const uint32_t n_eq = wave_count_ge<KPL>(key, T) - n_gt;
    const float m_gt = top ? 0.f : wave_mass_ge<KPL>(key, e, T + 1u);
    // the keys equal to T share one mass; take them, lowest id first, until the target is reached
    const float e_t = expf(key_score(T) - smax);
    // smallest m >= 1 (at most n_eq) with m_gt + m e_t >= target: start near the quotient, then step
    uint32_t m = 1;
    if (top) {
      m = n_eq;  // the forced blocks alone reach the target: all of them, nothing else
    } else {
      if (e_t > 0.f) m = (uint32_t)fminf(fmaxf((target - m_gt) / e_t - 1.f, 1.f), (float)n_eq);
      while (m > 1 && m_gt + (float)(m - 1) * e_t >= target) --m;
      while (m < n_eq && m_gt + (float)m * e_t < target) ++m;
    }
    if ((int)(n_gt + m) <= kcap) {
      k = (int)(n_gt + m);
      need = m;
      counted = false;
    }
  }
  if (counted) {
    if constexpr (!COVER) {
#pragma unroll
      for (int t = 0; t < KPL; ++t) {
        const int j = lane + 64 * t;
        if (j >= d0 && j < d1) key[t] = 0xFFFFFFFFu;  // forced: above every real score
      }
    }
    // Bisection for T = max{x : #(key >= x) >= k}; keys of real scores are > 0.
    T = 0;
#pragma unroll 1
    for (int bit = 31; bit >= 0; --bit) {
      const uint32_t cand = T | (1u << bit);
      if (wave_count_ge<KPL>(key, cand) >= (uint32_t)k) T = cand;
    }
    const uint32_t n_gt = (T == 0xFFFFFFFFu) ? 0u : wave_count_ge<KPL>(key, T + 1u);
    need = (uint32_t)k - n_gt;  // equal keys to take, lowest index first
  }

  int32_t* out = idx + row_base(ht, b, h, NG) + (int64_t)g * kcap;
  if constexpr (COVER) {
    for (int p = k + lane; p < kcap; p += 64) out[p] = -1;
    if (lane == 0) cnt[bh * NG + g] = k;
  }
  uint32_t pos = 0, eq_seen = 0;
#pragma unroll
  for (int t = 0; t < KPL; ++t) {
    const bool gt = key[t] > T;
    const bool eq = key[t] == T;
    const uint64_t beq = __ballot(eq);
    const bool sel = gt || (eq && eq_seen + (uint32_t)mask_rank(beq) < need);
    const uint64_t bsel = __ballot(sel);
    if (sel) out[pos + mask_rank(bsel)] = lane + 64 * t;
    pos += (uint32_t)__popcll(bsel);
    eq_seen += (uint32_t)__popcll(beq);
  }
}

template <int KPL, int R, bool COVER>
void select_launch_c(const Shape& s, const float* scores, const float* qhat, const float* khat, int32_t* idx,
                     int32_t* cnt, float* dump, const HeadTable& ht, float tau, float coverage, int diag,
                     hipStream_t st) {
  dim3 grid((s.NG + 3) / 4, s.H, s.B);
  if (scores)
    hipLaunchKernelGGL((topk_select_kernel<KPL, R, false, COVER>), grid, dim3(kSelThreads), 0, st, scores, qhat, khat,
                       idx, cnt, dump, ht, s.NG, s.NB, s.H, tau, coverage, diag);
  else
    hipLaunchKernelGGL((topk_select_kernel<KPL, R, true, COVER>), grid, dim3(kSelThreads), 0, st, scores, qhat, khat,
                       idx, cnt, dump, ht, s.NG, s.NB, s.H, tau, coverage, diag);
}

template <int KPL, int R>
hipError_t select_launch(const Shape& s, const float* scores, const float* qhat, const float* khat, int32_t* idx,
                         int32_t* cnt, float* dump, const HeadTable& ht, float tau, float coverage, int diag,
                         hipStream_t st) {
  if (cnt)
    select_launch_c<KPL, R, true>(s, scores, qhat, khat, idx, cnt, dump, ht, tau, coverage, diag, st);
  else
    select_launch_c<KPL, R, false>(s, scores, qhat, khat, idx, cnt, dump, ht, tau, coverage, diag, st);
  return hipGetLastError();
}

template <int KPL>
hipError_t select_dispatch_r(const Shape& s, const float* scores, const float* qhat, const float* khat,
                             int32_t* idx, int32_t* cnt, float* dump, const HeadTable& ht, float tau, float coverage,
                             int diag, hipStream_t st) {
  if (scores)  // the rank only matters when streaming
    return select_launch<KPL, 8>(s, scores, qhat, khat, idx, cnt, dump, ht, tau, coverage, diag, st);
  switch (s.R) {
    case 8: return select_launch<KPL, 8>(s, scores, qhat, khat, idx, cnt, dump, ht, tau, coverage, diag, st);
    case 16: return select_launch<KPL, 16>(s, scores, qhat, khat, idx, cnt, dump, ht, tau, coverage, diag, st);
    case 32: return select_launch<KPL, 32>(s, scores, qhat, khat, idx, cnt, dump, ht, tau, coverage, diag, st);
    case 64: return select_launch<KPL, 64>(s, scores, qhat, khat, idx, cnt, dump, ht, tau, coverage, diag, st);
    default: return hipErrorInvalidValue;
  }
}

// ---------------------------------------------------------------- reverse index

__global__ void fill_i32_kernel(int32_t* __restrict__ p, int64_t n, int32_t v) {
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x)
    p[i] = v;
}

__global__ __launch_bounds__(256) void rev_count_kernel(const int32_t* __restrict__ idx, int32_t* __restrict__ cnt,
                                                        HeadTable ht, int NG, int NB, int H) {
  const int b = blockIdx.z, h = blockIdx.y;
  const int64_t n = (int64_t)NG * ht.k[h];
  const int32_t* src = idx + row_base(ht, b, h, NG);
  int32_t* c = cnt + ((size_t)b * H + h) * NB;
  for (int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x; e < n; e += (int64_t)gridDim.x * 256) {
    const int32_t j = src[e];
    if ((uint32_t)j < (uint32_t)NB) atomicAdd(&c[j], 1);  // ids are valid by construction; never index out of range
  }
}

// One workgroup per (b, h): exclusive scan of NB counts into rev_ptr, and the
// counts are replaced by the segment starts (scatter cursors).
__global__ __launch_bounds__(256) void rev_scan_kernel(int32_t* __restrict__ cnt, int32_t* __restrict__ rev_ptr,
                                                       int NB, int H) {
  __shared__ int32_t part[256];
  const int b = blockIdx.z, h = blockIdx.y;
  int32_t* c = cnt + ((size_t)b * H + h) * NB;
  int32_t* rp = rev_ptr + ((size_t)b * H + h) * (NB + 1);
  const int per = (NB + 255) / 256;
  const int j0 = threadIdx.x * per;
  int32_t local = 0;
  for (int j = j0; j < j0 + per && j < NB; ++j) local += c[j];
  part[threadIdx.x] = local;
  __syncthreads();
  for (int off = 1; off < 256; off <<= 1) {  // Hillis-Steele inclusive scan
    const int32_t v = threadIdx.x >= off ? part[threadIdx.x - off] : 0;
    __syncthreads();
    part[threadIdx.x] += v;
    __syncthreads();
  }
  int32_t run = part[threadIdx.x] - local;
  for (int j = j0; j < j0 + per && j < NB; ++j) {
    const int32_t cj = c[j];
    rp[j] = run;
    c[j] = run;
    run += cj;
  }
  if (threadIdx.x == 255) rp[NB] = part[255];
}

__global__ __launch_bounds__(256) void rev_scatter_kernel(const int32_t* __restrict__ idx, int32_t* __restrict__ cur,
                                                          int32_t* __restrict__ tmp, HeadTable ht, int NG, int NB,
                                                          int H) {
  const int b = blockIdx.z, h = blockIdx.y;
  const int k = ht.k[h];
  const int64_t n = (int64_t)NG * k;
  const int64_t base = row_base(ht, b, h, NG);
  int32_t* c = cur + ((size_t)b * H + h) * NB;
  for (int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x; e < n; e += (int64_t)gridDim.x * 256) {
    const int32_t j = idx[base + e];
    if ((uint32_t)j >= (uint32_t)NB) continue;
    const int32_t pos = atomicAdd(&c[j], 1);
    tmp[base + pos] = (int32_t)(e / k);
  }
}

constexpr int kMaxGroupWords = 256;  // NG <= 8192

// One wave per (b, h, j): rebuild the segment in ascending group order.
__global__ __launch_bounds__(256) void rev_sort_kernel(const int32_t* __restrict__ tmp,
                                                       const int32_t* __restrict__ rev_ptr,
                                                       int32_t* __restrict__ rev_idx, HeadTable ht, int NG, int NB,
                                                       int H) {
  __shared__ uint32_t bm[4][kMaxGroupWords];
  const int b = blockIdx.z, h = blockIdx.y;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int j = blockIdx.x * 4 + wave;
  const bool valid = j < NB;
  const int words = (NG + 31) / 32;
  for (int w = lane; w < words; w += 64) bm[wave][w] = 0u;
  __syncthreads();
  const int64_t base = row_base(ht, b, h, NG);
  const int32_t* rp = rev_ptr + ((size_t)b * H + h) * (NB + 1);
  const int32_t s0 = valid ? rp[j] : 0, s1 = valid ? rp[j + 1] : 0;
  for (int32_t e = s0 + lane; e < s1; e += 64) {
    const int32_t g = tmp[base + e];
    if ((uint32_t)g < (uint32_t)NG) atomicOr(&bm[wave][g >> 5], 1u << (g & 31));
  }
  __syncthreads();
  if (!valid) return;
  int32_t* out = rev_idx + base + s0;
  int32_t run = 0;
  for (int w0 = 0; w0 < words; w0 += 64) {
    const int w = w0 + lane;
    uint32_t bits = w < words ? bm[wave][w] : 0u;
    const int pc = __popc(bits);
    int incl = pc;  // inclusive scan over the wave
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const int v = __shfl_up(incl, off);
      if (lane >= off) incl += v;
    }
    int o = run + incl - pc;
    while (bits) {
      const int bit = __ffs(bits) - 1;
      out[o++] = w * 32 + bit;
      bits &= bits - 1u;
    }
    run += __shfl(incl, 63);
  }
}

}  // namespace

hipError_t launch_topk_select(const Shape& s, const float* scores, const float* qhat, const float* khat, int32_t* idx,
                              float* dump, const HeadTable& ht, float tau, int kmax, hipStream_t st, int32_t* cnt,
                              float coverage, int diag_group) {
  const int diag = diag_group;
  (void)kmax;
  const int kpl = (s.NB + 63) / 64;
  if (kpl <= 1) return select_dispatch_r<1>(s, scores, qhat, khat, idx, cnt, dump, ht, tau, coverage, diag, st);
  if (kpl <= 2) return select_dispatch_r<2>(s, scores, qhat, khat, idx, cnt, dump, ht, tau, coverage, diag, st);
  if (kpl <= 4) return select_dispatch_r<4>(s, scores, qhat, khat, idx, cnt, dump, ht, tau, coverage, diag, st);
  if (kpl <= 8) return select_dispatch_r<8>(s, scores, qhat, khat, idx, cnt, dump, ht, tau, coverage, diag, st);
  if (kpl <= 16) return select_dispatch_r<16>(s, scores, qhat, khat, idx, cnt, dump, ht, tau, coverage, diag, st);
  if (kpl <= 32) return select_dispatch_r<32>(s, scores, qhat, khat, idx, cnt, dump, ht, tau, coverage, diag, st);
  if (kpl <= 64) return select_dispatch_r<64>(s, scores, qhat, khat, idx, cnt, dump, ht, tau, coverage, diag, st);
  if (kpl <= 128) return select_dispatch_r<128>(s, scores, qhat, khat, idx, cnt, dump, ht, tau, coverage, diag, st);
  return hipErrorInvalidValue;
}

hipError_t launch_reverse_index(const Shape& s, const int32_t* idx, int32_t* rev_ptr, int32_t* rev_idx,
                                int32_t* counters, int32_t* scratch, const HeadTable& ht, int kmax, hipStream_t st) {
  const int64_t ncnt = (int64_t)s.B * s.H * s.NB;
  hipLaunchKernelGGL(fill_i32_kernel, dim3((unsigned)((ncnt + 255) / 256 < 4096 ? (ncnt + 255) / 256 : 4096)), dim3(256),
                     0, st, counters, ncnt, 0);
  const int64_t per_bh = (int64_t)s.NG * kmax;
  const unsigned gx = (unsigned)((per_bh + 255) / 256 < 8192 ? (per_bh + 255) / 256 : 8192);
  hipLaunchKernelGGL(rev_count_kernel, dim3(gx, s.H, s.B), dim3(256), 0, st, idx, counters, ht, s.NG, s.NB, s.H);
  hipLaunchKernelGGL(rev_scan_kernel, dim3(1, s.H, s.B), dim3(256), 0, st, counters, rev_ptr, s.NB, s.H);
  hipLaunchKernelGGL(rev_scatter_kernel, dim3(gx, s.H, s.B), dim3(256), 0, st, idx, counters, scratch, ht, s.NG, s.NB,
                     s.H);
  hipLaunchKernelGGL(rev_sort_kernel, dim3((s.NB + 3) / 4, s.H, s.B), dim3(256), 0, st, scratch, rev_ptr, rev_idx, ht,
                     s.NG, s.NB, s.H);
  return hipGetLastError();
}

}  // namespace dsa
