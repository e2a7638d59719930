// Critical KV block selection and the reverse (block -> groups) index.
//
// DSV (gist.science explainer, hi edition) technical summary §2.A: the
// low-rank estimates pick the critical KV per query group; §2.B: the top-k
// selection is fused with the low-rank product so the O(S^2) score matrix need
// not exist (memory O(S*k)).
//
// select_kernel: a workgroup handles 32 consecutive rows (query groups) of one
// (b, h), one wave per row at a time.  A row's NB scores are held as
// order-preserving uint32 keys in registers (KPL per lane, j = lane + 64*t).
// The k-th largest key T is found by a radix select over a 256-bin histogram
// in LDS: the first level's buckets split the row's own key range [min, max]
// in 256 equal parts, each further level splits the one bucket that holds the
// k-th largest key, until a bucket is one key value (at most four levels).
// Every key > T and the lowest-index keys == T (as many as still needed) are
// then emitted in ascending j order by ballot/rank compaction.  In streaming
// mode the scores are computed in-kernel from qhat (registers) and khat chunks
// staged in LDS (shared by the workgroup's rows of one pass) with the same fma
// chain as block_scores, so both modes select identically.  Selection by
// coverage keeps its 32-step bisection on the cumulative mass.
//
// Reverse index without atomics on global memory: each workgroup also builds,
// in LDS, the membership bitmap of its 32 rows (bit g%32 of word j: row g kept
// block j) and writes it once.  Then per (b, h): count the set bits of each
// block's words, scan the counts into rev_ptr, and write each block's groups in
// ascending order from its words -- deterministic by construction.
#include "launch.hpp"

namespace dsa {

namespace {

constexpr int kRowsPerWg = 32;  // rows (query groups) per workgroup: one bitmap word per block

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

__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v = max(v, (uint32_t)__shfl_xor((int)v, off));
  return v;
}
__device__ __forceinline__ uint32_t wave_min_u32(uint32_t v) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v = min(v, (uint32_t)__shfl_xor((int)v, off));
  return v;
}

__device__ __forceinline__ void lds_wait() { asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory"); }

// The k-th largest key of the row (1 <= k <= number of real keys) and how many keys exceed it, by radix
// select over the wave's 256-bin LDS histogram hist.  Keys 0 are padding (below every real key: the key of
// any real score, even -inf, is above 0).  Each level histograms the keys inside [lo, hi] -- the range
// known to hold the answer -- by (key - lo) >> s, s the smallest shift that leaves at most 256 buckets, and
// narrows [lo, hi] to the bucket that holds the k-th largest; with s = 0 the bucket is a single key.
template <int KPL>
__device__ __forceinline__ void radix_kth(const uint32_t (&key)[KPL], uint32_t k, uint32_t* hist, int lane,
                                          uint32_t& T, uint32_t& n_gt) {
  uint32_t kmax = 0, kmin = 0xFFFFFFFFu;
#pragma unroll
  for (int t = 0; t < KPL; ++t) {
    kmax = max(kmax, key[t]);
    kmin = min(kmin, key[t] ? key[t] : 0xFFFFFFFFu);
  }
  uint32_t lo = wave_min_u32(kmin), hi = wave_max_u32(kmax);
  uint32_t above = 0;  // keys > hi
#pragma unroll 1
  for (int level = 0; level < 5; ++level) {
    const uint32_t width = hi - lo;
    const int s = width < 256u ? 0 : (32 - __clz(width)) - 8;
    reinterpret_cast<uint4*>(hist)[lane] = make_uint4(0u, 0u, 0u, 0u);
#pragma unroll
    for (int t = 0; t < KPL; ++t)
      if (key[t] >= lo && key[t] <= hi) atomicAdd(&hist[(key[t] - lo) >> s], 1u);
    lds_wait();
    const uint4 hv = reinterpret_cast<const uint4*>(hist)[lane];  // buckets 4 lane .. 4 lane + 3
    const uint32_t c = hv.x + hv.y + hv.z + hv.w;
    uint32_t suf = c;  // keys in this lane's buckets and all higher ones
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const uint32_t v = (uint32_t)__shfl_down((int)suf, off);
      if (lane + off < 64) suf += v;
    }
    lds_wait();  // every lane has read the histogram before the next level clears it
    const uint32_t want = k - above;  // rank of the answer among the keys in [lo, hi]
    uint32_t base = suf - c;          // keys in higher lanes' buckets
    int found = -1;
    uint32_t above_b = 0;
    const uint32_t h[4] = {hv.x, hv.y, hv.z, hv.w};
#pragma unroll
    for (int i = 3; i >= 0; --i) {
      if (found < 0 && base < want && want <= base + h[i]) {
        found = i;
        above_b = base;
      }
      base += h[i];
    }
    const uint64_t m = __ballot(found >= 0);
    if (m == 0) break;  // cannot happen while [lo, hi] holds the answer; keeps the lane index defined
    const int src = (int)__builtin_ctzll(m);
    const uint32_t b = 4u * (uint32_t)src + (uint32_t)__shfl(found, src);
    above += (uint32_t)__shfl((int)above_b, src);
    const uint32_t nlo = lo + (b << s);
    const uint32_t span = (s == 0) ? 0u : ((1u << s) - 1u);
    hi = (hi - nlo) <= span ? hi : nlo + span;
    lo = nlo;
    if (s == 0) break;
  }
  T = lo;
  n_gt = above;
}

// COVER: the row keeps the shortest run of blocks, in score order, whose estimated attention mass (the
// softmax of the row's block scores) reaches `coverage` of the total, at most k_h; the count goes to
// cnt[b,h,g] and the row's unused slots get -1.
// diag_group > 0: the blocks holding the row's own diag_group query tokens are kept first (their keys are
// raised above every score; in COVER mode their real masses still count).
// The workgroup (NWV waves) handles rows 32 x blockIdx.x .. + 31 of (b, h) = (blockIdx.z, blockIdx.y) and
// writes their membership bitmap bits[((b*H + h) * W + blockIdx.x) * NB + j] (W = ceil(NG / 32)).
template <int KPL, int R, bool STREAM, bool COVER, int NWV>
__global__ __launch_bounds__(NWV * 64) void select_kernel(const float* __restrict__ scores,
                                                          const float* __restrict__ qhat,
                                                          const float* __restrict__ khat,
                                                          int32_t* __restrict__ idx, int32_t* __restrict__ cnt,
                                                          uint32_t* __restrict__ bits, float* __restrict__ dump,
                                                          HeadTable ht, int NG, int NB, int H, float tau,
                                                          float coverage, int diag_group) {
  constexpr int CH = KPL < 4 ? KPL : (R > 32 ? 2 : 4);  // 64-block chunks of khat staged per LDS round
  constexpr int NT = NWV * 64;
  __shared__ float sk[STREAM ? 64 * CH : 1][R + 1];
  __shared__ __attribute__((aligned(16))) uint32_t hist[COVER ? 1 : NWV][256];
  extern __shared__ uint32_t bm[];  // NB words: the membership bitmap of the workgroup's 32 rows
  const int b = blockIdx.z, h = blockIdx.y;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const size_t bh = (size_t)b * H + h;
  const int kcap = ht.k[h];
  for (int j = threadIdx.x; j < NB; j += NT) bm[j] = 0u;
  __syncthreads();

#pragma unroll 1
  for (int pass = 0; pass < kRowsPerWg / NWV; ++pass) {
    const int g = blockIdx.x * kRowsPerWg + pass * NWV + wave;
    const bool valid = g < NG;
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
        for (int e = threadIdx.x; e < 64 * CH * R; e += NT) {
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
    if (!valid) continue;  // wave-uniform; no barrier below until the next pass

    // forced blocks [d0, d1): the ones that hold this group's tokens
    const int d0 = diag_group ? g * diag_group / kBlock : 0, d1 = diag_group ? (g + 1) * diag_group / kBlock : 0;
    int k = kcap;
    uint32_t T = 0, need = 0;
    if constexpr (COVER) {
      bool counted = true;  // T and need still to be found by the count bisection for k
      // masses e_j = exp(s_j - s_max) (0 for the padding keys, which are 0), total Z = M(0)
      uint32_t kmax = 0;
#pragma unroll
      for (int t = 0; t < KPL; ++t) kmax = max(kmax, key[t]);
      kmax = wave_max_u32(kmax);
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
      if (counted) {
        // Bisection for T = max{x : #(key >= x) >= k}; keys of real scores are > 0.
        T = 0;
#pragma unroll 1
        for (int bit = 31; bit >= 0; --bit) {
          const uint32_t cand = T | (1u << bit);
          if (wave_count_ge<KPL>(key, cand) >= (uint32_t)k) T = cand;
        }
        const uint32_t n_gt2 = (T == 0xFFFFFFFFu) ? 0u : wave_count_ge<KPL>(key, T + 1u);
        need = (uint32_t)k - n_gt2;  // equal keys to take, lowest index first
      }
    } else {
#pragma unroll
      for (int t = 0; t < KPL; ++t) {
        const int j = lane + 64 * t;
        if (j >= d0 && j < d1) key[t] = 0xFFFFFFFFu;  // forced: above every real score
      }
      uint32_t n_gt = 0;
      radix_kth<KPL>(key, (uint32_t)k, hist[COVER ? 0 : wave], lane, T, n_gt);
      need = (uint32_t)k - n_gt;  // equal keys to take, lowest index first
    }

    int32_t* out = idx + row_base(ht, b, h, NG) + (int64_t)g * kcap;
    if constexpr (COVER) {
      for (int p = k + lane; p < kcap; p += 64) out[p] = -1;
      if (lane == 0) cnt[bh * NG + g] = k;
    }
    const uint32_t gbit = 1u << (g & 31);
    uint32_t pos = 0, eq_seen = 0;
#pragma unroll
    for (int t = 0; t < KPL; ++t) {
      const bool gt = key[t] > T;
      const bool eq = key[t] == T;
      const uint64_t beq = __ballot(eq);
      const bool sel = gt || (eq && eq_seen + (uint32_t)mask_rank(beq) < need);
      const uint64_t bsel = __ballot(sel);
      if (sel) {
        out[pos + mask_rank(bsel)] = lane + 64 * t;
        atomicOr(&bm[lane + 64 * t], gbit);
      }
      pos += (uint32_t)__popcll(bsel);
      eq_seen += (uint32_t)__popcll(beq);
    }
  }
  __syncthreads();
  const int W = (NG + kRowsPerWg - 1) / kRowsPerWg;
  uint32_t* dst = bits + (bh * W + blockIdx.x) * (size_t)NB;
  for (int j = threadIdx.x; j < NB; j += NT) dst[j] = bm[j];
}

template <int KPL, int R, bool COVER>
void select_launch_c(const Shape& s, const float* scores, const float* qhat, const float* khat, int32_t* idx,
                     int32_t* cnt, uint32_t* bits, float* dump, const HeadTable& ht, float tau, float coverage,
                     int diag, hipStream_t st) {
  // eight waves while the keys leave room for two per SIMD, four beyond
  constexpr int NWV = KPL <= 32 ? 8 : 4;
  dim3 grid((s.NG + kRowsPerWg - 1) / kRowsPerWg, s.H, s.B);
  const size_t lds = (size_t)s.NB * sizeof(uint32_t);
  if (scores)
    hipLaunchKernelGGL((select_kernel<KPL, R, false, COVER, NWV>), grid, dim3(NWV * 64), lds, st, scores, qhat, khat,
                       idx, cnt, bits, dump, ht, s.NG, s.NB, s.H, tau, coverage, diag);
  else
    hipLaunchKernelGGL((select_kernel<KPL, R, true, COVER, NWV>), grid, dim3(NWV * 64), lds, st, scores, qhat, khat,
                       idx, cnt, bits, dump, ht, s.NG, s.NB, s.H, tau, coverage, diag);
}

template <int KPL, int R>
hipError_t select_launch(const Shape& s, const float* scores, const float* qhat, const float* khat, int32_t* idx,
                         int32_t* cnt, uint32_t* bits, float* dump, const HeadTable& ht, float tau, float coverage,
                         int diag, hipStream_t st) {
  if (cnt)
    select_launch_c<KPL, R, true>(s, scores, qhat, khat, idx, cnt, bits, dump, ht, tau, coverage, diag, st);
  else
    select_launch_c<KPL, R, false>(s, scores, qhat, khat, idx, cnt, bits, dump, ht, tau, coverage, diag, st);
  return hipGetLastError();
}

template <int KPL>
hipError_t select_dispatch_r(const Shape& s, const float* scores, const float* qhat, const float* khat,
                             int32_t* idx, int32_t* cnt, uint32_t* bits, float* dump, const HeadTable& ht, float tau,
                             float coverage, int diag, hipStream_t st) {
  if (scores)  // the rank only matters when streaming
    return select_launch<KPL, 8>(s, scores, qhat, khat, idx, cnt, bits, dump, ht, tau, coverage, diag, st);
  switch (s.R) {
    case 8: return select_launch<KPL, 8>(s, scores, qhat, khat, idx, cnt, bits, dump, ht, tau, coverage, diag, st);
    case 16: return select_launch<KPL, 16>(s, scores, qhat, khat, idx, cnt, bits, dump, ht, tau, coverage, diag, st);
    case 32: return select_launch<KPL, 32>(s, scores, qhat, khat, idx, cnt, bits, dump, ht, tau, coverage, diag, st);
    case 64: return select_launch<KPL, 64>(s, scores, qhat, khat, idx, cnt, bits, dump, ht, tau, coverage, diag, st);
    default: return hipErrorInvalidValue;
  }
}

// ---------------------------------------------------------------- reverse index from the bitmaps

// counts[bh * NB + j] = number of groups that kept block j (the set bits of its W words).
__global__ __launch_bounds__(256) void rev_count_kernel(const uint32_t* __restrict__ bits, int32_t* __restrict__ counts,
                                                        int NB, int W) {
  const int j = blockIdx.x * 256 + threadIdx.x;
  const size_t bh = blockIdx.y;
  if (j >= NB) return;
  const uint32_t* col = bits + bh * (size_t)W * NB + j;
  int32_t c = 0;
  for (int w = 0; w < W; ++w) c += __popc(col[(size_t)w * NB]);
  counts[bh * NB + j] = c;
}

// One workgroup per (b, h): exclusive scan of the NB counts into rev_ptr [B*H, NB + 1].
__global__ __launch_bounds__(256) void rev_scan_kernel(const int32_t* __restrict__ counts,
                                                       int32_t* __restrict__ rev_ptr, int NB) {
  __shared__ int32_t part[256];
  const size_t bh = blockIdx.x;
  const int32_t* c = counts + bh * NB;
  int32_t* rp = rev_ptr + bh * (NB + 1);
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
    rp[j] = run;
    run += c[j];
  }
  if (threadIdx.x == 255) rp[NB] = part[255];
}

// rev_idx: block j's groups in ascending order (the set bits of its words, word by word), at its offset.
__global__ __launch_bounds__(256) void rev_write_kernel(const uint32_t* __restrict__ bits,
                                                        const int32_t* __restrict__ rev_ptr,
                                                        int32_t* __restrict__ rev_idx, HeadTable ht, int NG, int NB,
                                                        int W, int H) {
  const int j = blockIdx.x * 256 + threadIdx.x;
  const int bhi = blockIdx.y;
  if (j >= NB) return;
  const int b = bhi / H, h = bhi % H;
  const uint32_t* col = bits + (size_t)bhi * W * NB + j;
  int32_t* out = rev_idx + row_base(ht, b, h, NG) + rev_ptr[(size_t)bhi * (NB + 1) + j];
  int32_t pos = 0;
  for (int w = 0; w < W; ++w) {
    uint32_t m = col[(size_t)w * NB];
    while (m) {
      out[pos++] = 32 * w + __builtin_ctz(m);
      m &= m - 1u;
    }
  }
}

}  // namespace

hipError_t launch_select(const Shape& s, const float* scores, const float* qhat, const float* khat, int32_t* idx,
                         float* dump, const HeadTable& ht, float tau, int kmax, int32_t* rev_ptr, int32_t* rev_idx,
                         int32_t* counts, uint32_t* bits, hipStream_t st, int32_t* cnt, float coverage,
                         int diag_group) {
  (void)kmax;
  const int diag = diag_group;
  const int kpl = (s.NB + 63) / 64;
  hipError_t e;
  if (kpl <= 1) e = select_dispatch_r<1>(s, scores, qhat, khat, idx, cnt, bits, dump, ht, tau, coverage, diag, st);
  else if (kpl <= 2) e = select_dispatch_r<2>(s, scores, qhat, khat, idx, cnt, bits, dump, ht, tau, coverage, diag, st);
  else if (kpl <= 4) e = select_dispatch_r<4>(s, scores, qhat, khat, idx, cnt, bits, dump, ht, tau, coverage, diag, st);
  else if (kpl <= 8) e = select_dispatch_r<8>(s, scores, qhat, khat, idx, cnt, bits, dump, ht, tau, coverage, diag, st);
  else if (kpl <= 16) e = select_dispatch_r<16>(s, scores, qhat, khat, idx, cnt, bits, dump, ht, tau, coverage, diag, st);
  else if (kpl <= 32) e = select_dispatch_r<32>(s, scores, qhat, khat, idx, cnt, bits, dump, ht, tau, coverage, diag, st);
  else if (kpl <= 64) e = select_dispatch_r<64>(s, scores, qhat, khat, idx, cnt, bits, dump, ht, tau, coverage, diag, st);
  else if (kpl <= 128) e = select_dispatch_r<128>(s, scores, qhat, khat, idx, cnt, bits, dump, ht, tau, coverage, diag, st);
  else return hipErrorInvalidValue;
  if (e != hipSuccess) return e;
  const int W = (s.NG + kRowsPerWg - 1) / kRowsPerWg;
  const dim3 gcol((s.NB + 255) / 256, s.B * s.H);
  hipLaunchKernelGGL(rev_count_kernel, gcol, dim3(256), 0, st, bits, counts, s.NB, W);
  hipLaunchKernelGGL(rev_scan_kernel, dim3(s.B * s.H), dim3(256), 0, st, counts, rev_ptr, s.NB);
  hipLaunchKernelGGL(rev_write_kernel, gcol, dim3(256), 0, st, bits, rev_ptr, rev_idx, ht, s.NG, s.NB, W, s.H);
  return hipGetLastError();
}

}  // namespace dsa
