// Critical KV block selection and the reverse (block -> groups) index.
//
// DSV (gist.science explainer, hi edition) technical summary §2.A: the
// low-rank estimates pick the critical KV per query group; §2.B: the top-k
// selection is fused with the low-rank product so the O(S^2) score matrix need
// not exist (memory O(S*k)).
//
// A workgroup (8 waves) handles 32 consecutive rows (query groups) of one
// (b, h), one row per wave at a time.  A row's NB scores are held in registers
// (KPL per lane, block j = lane + 64 t).  The k-th largest score T comes from
// a radix select over 256-bin LDS histograms: the first level bins the scores
// linearly over the row's [min, max], finding the bucket that holds T; a
// bucket of at most 64 scores is gathered one per lane and ranked exactly, a
// fuller one is split further over the order-preserving uint32 keys of its
// range.  Every score > T and the lowest-index scores == T (as many as still
// needed) are emitted in ascending j order by ballot/rank compaction.
//
// select_scores_kernel reads a materialised score matrix (coalesced rows, the
// next row prefetched while the current one is selected).
// select_stream_kernel computes the scores itself: each thread keeps one
// k-hat row in registers (the next one in flight), takes the q-hat rows of
// the workgroup's 8 current query groups as wave-uniform (scalar) operands,
// and writes 8 scores per block into a double-buffered LDS tile from which
// each wave reads its own row's keys -- the same fma chain as block_scores,
// so both kernels select identically.
// Selection by coverage keeps a 32-step bisection on the cumulative mass.
//
// Reverse index without atomics on global memory: each workgroup also builds,
// in LDS, the membership bitmap of its 32 rows (bit g%32 of word j: row g kept
// block j) and writes it once.  Then per (b, h): count the set bits of each
// block's words, then per 64 blocks sum the counts before them and scan their
// own into rev_ptr, and write each block's groups in ascending order from its
// words -- deterministic by construction.
#include "launch.hpp"

namespace dsa {

namespace {

constexpr int kRowsPerWg = 32;  // rows (query groups) per workgroup: one bitmap word per block
constexpr int kHistWords = 256 + 64;  // 256 bins + one discard bin per lane (never read)

// Waves per workgroup (rows selected at once): eight while a row's keys and the selection's temporaries fit
// the registers of two waves per SIMD, four beyond (a wave may then use the whole register file).
template <int KPL, bool STREAM, bool COVER>
constexpr int sel_waves() { return KPL <= 32 ? 8 : COVER ? 4 : (STREAM || KPL <= 64) ? 8 : 4; }

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


// DPP lane moves (GFX9 encodings): row_shr:n shifts within each 16-lane row (lanes shifted in read 0 with
// bound_ctrl); row_bcast:15 / :31 pass lane 15 / 31 of a row to the rows selected by the row mask.
template <int CTRL, int ROW_MASK, bool BOUND_ZERO>
__device__ __forceinline__ uint32_t dpp(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, ROW_MASK, 0xf, BOUND_ZERO);
}

// Inclusive prefix sum over the 64 lanes.
__device__ __forceinline__ uint32_t wave_incl_sum(uint32_t v) {
  v += dpp<0x111, 0xf, true>(v);   // row_shr:1
  v += dpp<0x112, 0xf, true>(v);   // row_shr:2
  v += dpp<0x114, 0xf, true>(v);   // row_shr:4
  v += dpp<0x118, 0xf, true>(v);   // row_shr:8
  v += dpp<0x142, 0xa, false>(v);  // row_bcast:15 into rows 1 and 3
  v += dpp<0x143, 0xc, false>(v);  // row_bcast:31 into rows 2 and 3
  return v;
}

// Maximum over the 64 lanes (0 is the identity: keys are unsigned), as a wave-uniform value.
__device__ __forceinline__ uint32_t wave_max_key(uint32_t v) {
  v = max(v, dpp<0x111, 0xf, true>(v));
  v = max(v, dpp<0x112, 0xf, true>(v));
  v = max(v, dpp<0x114, 0xf, true>(v));
  v = max(v, dpp<0x118, 0xf, true>(v));
  v = max(v, dpp<0x142, 0xa, false>(v));
  v = max(v, dpp<0x143, 0xc, false>(v));
  return (uint32_t)__builtin_amdgcn_readlane((int)v, 63);
}

__device__ __forceinline__ uint32_t readlane(uint32_t v, int l) {
  return (uint32_t)__builtin_amdgcn_readlane((int)v, l);
}

__device__ __forceinline__ void lds_wait() { asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory"); }

// In the loops over a row's keys (unrolled: the keys live in registers), every 8 keys: no instruction is
// scheduled across, so the per-key temporaries (compare masks, addresses) of one group are dead before the
// next group starts instead of all KPL sets being live at once.
#define DSA_KEY_GROUP_FENCE(t) \
  if (((t) & 7) == 7) __builtin_amdgcn_sched_barrier(0)

// A copy of a lane-varying value that the compiler cannot see through: taken at the top of each pass over
// rows, it keeps the per-key values derived from it (block ids lane + 64 t, their bounds masks) from being
// hoisted out of the pass loop and held, KPL of each, for the whole kernel.
__device__ __forceinline__ int opaque(int v) {
  asm volatile("" : "+v"(v));
  return v;
}
// The same for a float: per-key values recomputed from it in a later loop (a score's bin) are then not merged
// with the earlier loop's and kept live in between.
__device__ __forceinline__ float opaque_f(float v) {
  asm volatile("" : "+v"(v));
  return v;
}

// Float min / max over the 64 lanes (NaN lanes are ignored by fminf / fmaxf), as wave-uniform values.
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ float dppf(float v, float identity) {
  return __int_as_float(
      __builtin_amdgcn_update_dpp(__float_as_int(identity), __float_as_int(v), CTRL, ROW_MASK, 0xf, false));
}
__device__ __forceinline__ float wave_min_f(float v) {
  const float I = __builtin_inff();
  v = fminf(v, dppf<0x111, 0xf>(v, I));
  v = fminf(v, dppf<0x112, 0xf>(v, I));
  v = fminf(v, dppf<0x114, 0xf>(v, I));
  v = fminf(v, dppf<0x118, 0xf>(v, I));
  v = fminf(v, dppf<0x142, 0xa>(v, I));
  v = fminf(v, dppf<0x143, 0xc>(v, I));
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 63));
}
__device__ __forceinline__ float wave_max_f(float v) {
  const float I = -__builtin_inff();
  v = fmaxf(v, dppf<0x111, 0xf>(v, I));
  v = fmaxf(v, dppf<0x112, 0xf>(v, I));
  v = fmaxf(v, dppf<0x114, 0xf>(v, I));
  v = fmaxf(v, dppf<0x118, 0xf>(v, I));
  v = fmaxf(v, dppf<0x142, 0xa>(v, I));
  v = fmaxf(v, dppf<0x143, 0xc>(v, I));
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 63));
}

// Sum over the 64 lanes as a wave-uniform value: an inclusive prefix sum by DPP (a fixed order, so the same
// inputs always give the same bits), read at lane 63.
__device__ __forceinline__ float wave_sum_f(float v) {
  v += dppf<0x111, 0xf>(v, 0.f);
  v += dppf<0x112, 0xf>(v, 0.f);
  v += dppf<0x114, 0xf>(v, 0.f);
  v += dppf<0x118, 0xf>(v, 0.f);
  v += dppf<0x142, 0xa>(v, 0.f);
  v += dppf<0x143, 0xc>(v, 0.f);
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 63));
}

// Mass of the row's keys >= cand (e: each key's mass, 0 for padding).
template <int KPL>
__device__ __forceinline__ float wave_mass_ge(const uint32_t (&key)[KPL], const float (&e)[KPL], uint32_t cand) {
  float m = 0.f;
#pragma unroll
  for (int t = 0; t < KPL; ++t) m += key[t] >= cand ? e[t] : 0.f;
  return wave_sum_f(m);
}

// The bucket of this wave's 256-bin histogram (just filled) that holds the want-th largest counted key:
// its index b, the keys in higher buckets (above) and its own count (cnt).
struct Bucket {
  uint32_t b, above, cnt;
  bool found;
};
__device__ __forceinline__ Bucket pick_bucket(const uint32_t* hist, int lane, uint32_t want) {
  lds_wait();
  const uint4 hv = reinterpret_cast<const uint4*>(hist)[lane];  // buckets 4 lane .. 4 lane + 3
  const uint32_t c = hv.x + hv.y + hv.z + hv.w;
  const uint32_t incl = wave_incl_sum(c);
  const uint32_t total = readlane(incl, 63);
  uint32_t base = total - incl;  // keys in higher lanes' buckets
  int found = -1;
  uint32_t above_b = 0, cnt_b = 0;
  const uint32_t h[4] = {hv.x, hv.y, hv.z, hv.w};
#pragma unroll
  for (int i = 3; i >= 0; --i) {
    if (found < 0 && base < want && want <= base + h[i]) {
      found = i;
      above_b = base;
      cnt_b = h[i];
    }
    base += h[i];
  }
  const uint64_t m = __ballot(found >= 0);
  const int src = m ? (int)__builtin_ctzll(m) : 0;  // exactly one lane holds the bucket
  Bucket r;
  r.b = 4u * (uint32_t)src + readlane((uint32_t)found, src);
  r.above = readlane(above_b, src);
  r.cnt = readlane(cnt_b, src);
  r.found = m != 0;  // always, while the counted keys hold the answer
  return r;
}

// The (at most 64) values val(t) of the keys with in(t), one per lane in ascending t order, written to the
// first 64 words of buf (the histogram's, already read); returns how many (capped at 64).
template <int KPL, class In, class Val>
__device__ __forceinline__ uint32_t gather64(uint32_t* buf, int lane, In in, Val val) {
  uint32_t nc = 0;
#pragma unroll
  for (int t = 0; t < KPL; ++t) {
    const bool i = in(t);
    const uint64_t mi = __ballot(i);
    const uint32_t p = nc + (uint32_t)mask_rank(mi);
    if (i && p < 64u) buf[p] = val(t);
    nc += (uint32_t)__popcll(mi);
    DSA_KEY_GROUP_FENCE(t);
  }
  lds_wait();
  return min(nc, 64u);
}

// Key-space radix select of the want-th largest among the keys keyof(t) in [lo, hi] (above: keys of the row
// greater than hi).  Keys 0 are padding (below every real key: the key of any real score, even -inf, is
// above 0).  Each level histograms the keys inside [lo, hi] by (key - lo) >> s, s the smallest shift that
// leaves at most 256 buckets, and narrows [lo, hi] to the bucket holding the answer.  Once that bucket is one
// key value the answer is known; once it holds at most 64 keys they are gathered one per lane and T is the
// smallest with fewer than want of them above it.  T = the answer, n_gt = #keys > T, n_eq = #keys == T.
template <int KPL, class KeyOf>
__device__ __forceinline__ void kth_in_key_range(KeyOf keyof, uint32_t lo, uint32_t hi, uint32_t above,
                                                 uint32_t want, uint32_t* hist, int lane, uint32_t& T,
                                                 uint32_t& n_gt, uint32_t& n_eq) {
#pragma unroll 1
  for (int level = 0; level < 4; ++level) {
    const uint32_t width = hi - lo;
    const int s = width < 256u ? 0 : (32 - __clz(width)) - 8;
    const int ln = opaque(lane);
    reinterpret_cast<uint4*>(hist)[lane] = make_uint4(0u, 0u, 0u, 0u);
#pragma unroll
    for (int t = 0; t < KPL; ++t) {
      const uint32_t d = keyof(t, ln) - lo;
      const uint32_t bin = d <= width ? (d >> s) : 256u + (uint32_t)lane;
      __hip_atomic_fetch_add(&hist[bin], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
      DSA_KEY_GROUP_FENCE(t);
    }
    const Bucket bk = pick_bucket(hist, lane, want);
    above += bk.above;
    want -= bk.above;
    const uint32_t nlo = lo + (bk.b << s);
    const uint32_t span = (s == 0) ? 0u : ((1u << s) - 1u);
    hi = (hi - nlo) <= span ? hi : nlo + span;
    lo = nlo;
    if (s == 0 || !bk.found) {  // the bucket is one key value (!found cannot happen; keeps T a real key)
      T = lo;
      n_gt = above;
      n_eq = bk.cnt;
      return;
    }
    if (bk.cnt <= 64u) break;
  }
  const uint32_t width = hi - lo;
  const int ln = opaque(lane);
  const uint32_t nc = gather64<KPL>(hist, lane, [&](int t) { return keyof(t, ln) - lo <= width; },
                                    [&](int t) { return keyof(t, ln); });
  const bool real = (uint32_t)lane < nc;
  const uint32_t c = real ? hist[lane] : 0u;
  uint32_t gt = 0;
#pragma unroll 1
  for (uint32_t j = 0; j < nc; ++j) gt += readlane(c, (int)j) > c ? 1u : 0u;
  T = ~wave_max_key(real && gt < want ? ~c : 0u);
  n_gt = above + (uint32_t)__popcll(__ballot(real && c > T));
  n_eq = (uint32_t)__popcll(__ballot(real && c == T));
  lds_wait();  // every lane has read its candidate before the words are written again
}

// The k-th largest of a row held as keys (coverage selection): 1 <= k <= number of real keys.
template <int KPL>
__device__ __forceinline__ void kth_largest_keys(const uint32_t (&key)[KPL], uint32_t k, uint32_t* hist, int lane,
                                                 uint32_t& T, uint32_t& n_gt, uint32_t& n_eq) {
  uint32_t kmax = 0, nkmin = 0;  // nkmin: max of ~key over the real keys
#pragma unroll
  for (int t = 0; t < KPL; ++t) {
    kmax = max(kmax, key[t]);
    nkmin = max(nkmin, key[t] ? ~key[t] : 0u);
  }
  kth_in_key_range<KPL>([&](int t, int) { return key[t]; }, ~wave_max_key(nkmin), wave_max_key(kmax), 0u, k,
                        hist, lane, T, n_gt, n_eq);
}

// The k-th largest of a row held as scores (top-k selection): NaN marks padding (never counted), +inf the
// forced blocks (above every real score); mn, mx: the least and greatest real score (+inf excluded).
// The first level bins the scores linearly over [mn, mx] (256 bins; a monotone map, so each bin is a range
// of scores), which spreads a row's values far more evenly than bins of their bit patterns; a bucket of at
// most 64 scores is ranked directly, a fuller one goes on in key space over its own range.
template <int KPL>
__device__ __forceinline__ void kth_largest_scores(const float (&sc)[KPL], float mn, float mx, uint32_t k, int NB,
                                                   uint32_t* hist, int lane, float& T, uint32_t& n_gt,
                                                   uint32_t& n_eq) {
  // a real score: block lane + 64 t < NB, tested by index with a lane copy of each loop's own (see opaque)
  auto keyof = [&](int t, int ln) { return ln + 64 * t < NB ? score_key(sc[t]) : 0u; };
  uint32_t above = 0, want = k, lo, hi;
  const float range = mx - mn;
  if (range > 0.f && range < __builtin_inff()) {
    const float inv = fminf(256.f / range, 1e30f);
    auto bin = [](float s, float m0, float iv) {
      return (uint32_t)__builtin_amdgcn_fmed3f((s - m0) * iv, 0.f, 255.f);
    };
    constexpr bool KEEP = KPL <= 32;  // short rows keep each score's bin (256 + lane: padding) for the gather
    uint32_t bn[KEEP ? KPL : 1];
    const int lane1 = opaque(lane);
    reinterpret_cast<uint4*>(hist)[lane] = make_uint4(0u, 0u, 0u, 0u);
#pragma unroll
    for (int t = 0; t < KPL; ++t) {
      const uint32_t bi = lane1 + 64 * t < NB ? bin(sc[t], mn, inv) : 256u + (uint32_t)lane;
      if constexpr (KEEP) bn[t] = bi;
      __hip_atomic_fetch_add(&hist[bi], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
      DSA_KEY_GROUP_FENCE(t);
    }
    const Bucket bk = pick_bucket(hist, lane, want);
    above = bk.above;
    want -= bk.above;
    const float mn2 = opaque_f(mn), inv2 = opaque_f(inv);
    const int lane2 = opaque(lane);
    auto in = [&](int t) {
      if constexpr (KEEP) return bn[t] == bk.b;
      else return lane2 + 64 * t < NB && bin(sc[t], mn2, inv2) == bk.b;
    };
    if (bk.cnt <= 64u && bk.found) {
      const uint32_t nc = gather64<KPL>(hist, lane, in, [&](int t) { return __float_as_uint(sc[t]); });
      const bool real = (uint32_t)lane < nc;
      const float c = real ? __uint_as_float(hist[lane]) : -__builtin_inff();
      uint32_t gt = 0;
#pragma unroll 1
      for (uint32_t j = 0; j < nc; ++j)
        gt += __int_as_float(__builtin_amdgcn_readlane(__float_as_int(c), (int)j)) > c ? 1u : 0u;
      T = wave_min_f(real && gt < want ? c : __builtin_inff());
      n_gt = above + (uint32_t)__popcll(__ballot(real && c > T));
      n_eq = (uint32_t)__popcll(__ballot(real && c == T));
      lds_wait();
      return;
    }
    // the bucket's own key range
    float blo = __builtin_inff(), bhi = -__builtin_inff();
#pragma unroll
    for (int t = 0; t < KPL; ++t) {
      if (in(t)) {
        blo = fminf(blo, sc[t]);
        bhi = fmaxf(bhi, sc[t]);
      }
    }
    lo = score_key(wave_min_f(blo));
    hi = score_key(wave_max_f(bhi));
  } else {  // every real score equal (or a range past fp32): key space over all real keys
    uint32_t kmax = 0, nkmin = 0;
    const int ln = opaque(lane);
#pragma unroll
    for (int t = 0; t < KPL; ++t) {
      const uint32_t kk = keyof(t, ln);
      kmax = max(kmax, kk);
      nkmin = max(nkmin, kk ? ~kk : 0u);
    }
    lo = ~wave_max_key(nkmin);
    hi = wave_max_key(kmax);
  }
  uint32_t Tk;
  kth_in_key_range<KPL>(keyof, lo, hi, above, want, hist, lane, Tk, n_gt, n_eq);
  T = key_score(Tk);
}

// Selects row g of (b, h) by coverage from its keys (padding 0) and writes its kept ids (ascending), its
// count and its bits in the workgroup's membership bitmap bm: the row keeps the shortest run of blocks, in
// score order, whose estimated attention mass (the softmax of the row's block scores) reaches `coverage` of
// the total, at most k_h; the count goes to cnt[b,h,g] and the row's unused slots get -1.
// diag_group > 0: the blocks holding the row's own diag_group query tokens are kept first (their keys are
// raised above every score; their real masses still count).
template <int KPL>
__device__ __forceinline__ void select_row_cover(uint32_t (&key)[KPL], int b, int h, int g, int NG,
                                                 const HeadTable& ht, float coverage, int diag_group,
                                                 int32_t* __restrict__ idx, int32_t* __restrict__ cnt,
                                                 uint32_t* hist, uint32_t* bm, int lane, size_t bh) {
  const int kcap = ht.k[h];
  const int d0 = diag_group ? g * diag_group / kBlock : 0, d1 = diag_group ? (g + 1) * diag_group / kBlock : 0;
  int k = kcap;
  uint32_t T = 0, need = 0, n_eq = 0;
  bool counted = true;  // T and need still to be found for the k_h largest
  // masses e_j = exp(s_j - s_max) (0 for the padding keys, which are 0), total Z = M(0)
  uint32_t kmax = 0;
#pragma unroll
  for (int t = 0; t < KPL; ++t) kmax = max(kmax, key[t]);
  kmax = wave_max_key(kmax);
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
  const uint32_t neq = wave_count_ge<KPL>(key, T) - n_gt;
  const float m_gt = top ? 0.f : wave_mass_ge<KPL>(key, e, T + 1u);
  // the keys equal to T share one mass; take them, lowest id first, until the target is reached
  const float e_t = expf(key_score(T) - smax);
  // smallest m >= 1 (at most neq) with m_gt + m e_t >= target: start near the quotient, then step
  uint32_t m = 1;
  if (top) {
    m = neq;  // the forced blocks alone reach the target: all of them, nothing else
  } else {
    if (e_t > 0.f) m = (uint32_t)fminf(fmaxf((target - m_gt) / e_t - 1.f, 1.f), (float)neq);
    while (m > 1 && m_gt + (float)(m - 1) * e_t >= target) --m;
    while (m < neq && m_gt + (float)m * e_t < target) ++m;
  }
  if ((int)(n_gt + m) <= kcap) {
    k = (int)(n_gt + m);
    need = m;
    n_eq = neq;
    counted = false;
  }
  if (counted) {
    uint32_t gt2 = 0;
    kth_largest_keys<KPL>(key, (uint32_t)k, hist, lane, T, gt2, n_eq);
    need = (uint32_t)k - gt2;
  }

  int32_t* out = idx + row_base(ht, b, h, NG) + (int64_t)g * kcap;
  for (int p = k + lane; p < kcap; p += 64) out[p] = -1;
  if (lane == 0) cnt[bh * NG + g] = k;
  const uint32_t gbit = 1u << (g & 31);
  uint32_t pos = 0, eq_seen = 0;
#pragma unroll
  for (int t = 0; t < KPL; ++t) {
    const bool gt = key[t] > T;
    const bool eq = key[t] == T;
    const uint64_t beq = __ballot(eq);
    const bool sel = gt || (eq && eq_seen + (uint32_t)mask_rank(beq) < need);
    const uint64_t bsel = __ballot(sel);
    const uint32_t p = pos + (uint32_t)mask_rank(bsel);
    if (sel && p < (uint32_t)k) {
      out[p] = lane + 64 * t;
      atomicOr(&bm[lane + 64 * t], gbit);
    }
    pos += (uint32_t)__popcll(bsel);
    eq_seen += (uint32_t)__popcll(beq);
    DSA_KEY_GROUP_FENCE(t);
  }
}

// Selects the k_h largest of row g of (b, h) from its scores (NaN padding) and writes its kept ids
// (ascending) and its bits in the workgroup's membership bitmap bm.  Ties at the k-th score go to the lower
// block ids.  diag_group > 0: the blocks holding the row's own diag_group query tokens are kept first (their
// scores are raised to +inf, above every real score).
template <int KPL>
__device__ __forceinline__ void select_row_topk(float (&sc)[KPL], int b, int h, int g, int NG, int NB,
                                                const HeadTable& ht, int diag_group, int32_t* __restrict__ idx,
                                                uint32_t* hist, uint32_t* bm, int lane) {
  const int k = ht.k[h];
  float mn = __builtin_inff(), mx = -__builtin_inff();
#pragma unroll
  for (int t = 0; t < KPL; ++t) {
    mn = fminf(mn, sc[t]);
    mx = fmaxf(mx, sc[t]);
  }
  mn = wave_min_f(mn);
  mx = wave_max_f(mx);
  if (diag_group) {  // forced blocks [d0, d1): the ones that hold this group's tokens
    const int d0 = g * diag_group / kBlock, d1 = (g + 1) * diag_group / kBlock;
#pragma unroll
    for (int t = 0; t < KPL; ++t) {
      const int j = lane + 64 * t;
      if (j >= d0 && j < d1) sc[t] = __builtin_inff();
    }
  }
  float T;
  uint32_t n_gt = 0, n_eq = 0;
  kth_largest_scores<KPL>(sc, mn, mx, (uint32_t)k, NB, hist, lane, T, n_gt, n_eq);
  const uint32_t need = (uint32_t)k - n_gt;  // scores equal to T to keep, lowest id first

  int32_t* out = idx + row_base(ht, b, h, NG) + (int64_t)g * k;
  const uint32_t gbit = 1u << (g & 31);
  uint32_t pos = 0;
  if (need == n_eq) {  // every score equal to T is kept
#pragma unroll
    for (int t = 0; t < KPL; ++t) {
      const bool sel = sc[t] >= T;
      const uint64_t bsel = __ballot(sel);
      const uint32_t p = pos + (uint32_t)mask_rank(bsel);
      if (sel && p < (uint32_t)k) {
        out[p] = lane + 64 * t;
        atomicOr(&bm[lane + 64 * t], gbit);
      }
      pos += (uint32_t)__popcll(bsel);
      DSA_KEY_GROUP_FENCE(t);
    }
  } else {
    uint32_t eq_seen = 0;
#pragma unroll
    for (int t = 0; t < KPL; ++t) {
      const bool gt = sc[t] > T;
      const bool eq = sc[t] == T;
      const uint64_t beq = __ballot(eq);
      const bool sel = gt || (eq && eq_seen + (uint32_t)mask_rank(beq) < need);
      const uint64_t bsel = __ballot(sel);
      const uint32_t p = pos + (uint32_t)mask_rank(bsel);
      if (sel && p < (uint32_t)k) {
        out[p] = lane + 64 * t;
        atomicOr(&bm[lane + 64 * t], gbit);
      }
      pos += (uint32_t)__popcll(bsel);
      eq_seen += (uint32_t)__popcll(beq);
      DSA_KEY_GROUP_FENCE(t);
    }
  }
}

// One row: top-k from its scores, or coverage from its keys.
template <int KPL, bool COVER>
__device__ __forceinline__ void select_row(float (&sc)[KPL], int b, int h, int g, int NG, int NB, const HeadTable& ht,
                                           float coverage, int diag_group, int32_t* __restrict__ idx,
                                           int32_t* __restrict__ cnt, uint32_t* hist, uint32_t* bm, int lane,
                                           size_t bh) {
  if constexpr (COVER) {
    uint32_t key[KPL];
#pragma unroll
    for (int t = 0; t < KPL; ++t) key[t] = sc[t] == sc[t] ? score_key(sc[t]) : 0u;
    select_row_cover<KPL>(key, b, h, g, NG, ht, coverage, diag_group, idx, cnt, hist, bm, lane, bh);
  } else {
    select_row_topk<KPL>(sc, b, h, g, NG, NB, ht, diag_group, idx, hist, bm, lane);
  }
}

// Rows 32 x blockIdx.x .. + 31 of (b, h) = (blockIdx.z, blockIdx.y) from the score matrix; writes their
// membership bitmap bits[((b*H + h) * W + blockIdx.x) * NB + j] (W = ceil(NG / 32)).
template <int KPL, bool COVER, int NWV = sel_waves<KPL, false, COVER>()>
__global__ __launch_bounds__(NWV * 64) void select_scores_kernel(const float* __restrict__ scores,
                                                                    int32_t* __restrict__ idx,
                                                                    int32_t* __restrict__ cnt,
                                                                    uint32_t* __restrict__ bits, HeadTable ht, int NG,
                                                                    int NB, int H, float coverage, int diag_group) {
  constexpr bool PREFETCH = KPL <= 32;  // the next row's scores in flight while this one is selected
  constexpr int NT = NWV * 64;
  __shared__ __attribute__((aligned(16))) uint32_t hist[NWV][kHistWords];
  extern __shared__ uint32_t bm[];  // NB words: the membership bitmap of the workgroup's 32 rows
  const int b = blockIdx.z, h = blockIdx.y;
  const int lane0 = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const size_t bh = (size_t)b * H + h;
  for (int j = threadIdx.x; j < NB; j += NT) bm[j] = 0u;
  __syncthreads();

  const float* sbh = scores + bh * NG * (size_t)NB;
  float nxt[PREFETCH ? KPL : 1];
  auto load = [&](int g, float* dst, int lane) {
    const float* srow = sbh + (size_t)(g < NG ? g : 0) * NB;
#pragma unroll
    for (int t = 0; t < KPL; ++t) {
      const int j = lane + 64 * t;
      dst[t] = j < NB ? srow[j] : __builtin_nanf("");
    }
  };
  const int g0 = blockIdx.x * kRowsPerWg + wave;
  if constexpr (PREFETCH) load(g0, nxt, lane0);
#pragma unroll 1
  for (int pass = 0; pass < kRowsPerWg / NWV; ++pass) {
    const int g = g0 + pass * NWV;
    if (g >= NG) break;  // later passes of this wave are past the end too
    const int lane = opaque(lane0);
    float sc[KPL];  // the row's scores, NaN past NB
    if constexpr (PREFETCH) {
#pragma unroll
      for (int t = 0; t < KPL; ++t) sc[t] = nxt[t];
      if (pass + 1 < kRowsPerWg / NWV && g + NWV < NG) load(g + NWV, nxt, lane);
    } else {
      load(g, sc, lane);
    }
    select_row<KPL, COVER>(sc, b, h, g, NG, NB, ht, coverage, diag_group, idx, cnt, hist[wave], bm, lane, bh);
  }
  __syncthreads();
  const int W = (NG + kRowsPerWg - 1) / kRowsPerWg;
  uint32_t* dst = bits + (bh * W + blockIdx.x) * (size_t)NB;
  for (int j = threadIdx.x; j < NB; j += NT) dst[j] = bm[j];
}

// The same selection with the scores computed in-kernel: score(g, j) = tau * (qhat[g] . khat[j]) by
// score_dot's fma chain.  Per pass the NWV waves select NWV rows; the blocks go by in chunks of CB = min(64 NWV,
// 64 KPL): thread i scores block c CB + i against the NWV rows (q-hat values wave-uniform), writes the scores
// into the LDS tile kt[c & 1][row][i], and after the chunk's barrier each wave takes its row's CB scores.
// dump (if not null) receives the scores [B, H, NG, NB].
template <int KPL, int R, bool COVER, int NWV = sel_waves<KPL, true, COVER>()>
__global__ __launch_bounds__(NWV * 64) void select_stream_kernel(const float* __restrict__ qhat,
                                                                    const float* __restrict__ khat,
                                                                    int32_t* __restrict__ idx,
                                                                    int32_t* __restrict__ cnt,
                                                                    uint32_t* __restrict__ bits,
                                                                    float* __restrict__ dump, HeadTable ht, int NG,
                                                                    int NB, int H, float tau, float coverage,
                                                                    int diag_group, int zero) {
  constexpr int NT = NWV * 64;
  constexpr int CB = KPL >= NWV ? NT : 64 * KPL;  // blocks per chunk
  constexpr int KPC = CB / 64;                    // keys per lane per chunk
  constexpr int NC = KPL / KPC;                   // chunks per row
  constexpr int PASSES = kRowsPerWg / NWV;
  constexpr int NIT = PASSES * NC;
  __shared__ __attribute__((aligned(16))) uint32_t hist[NWV][kHistWords];
  __shared__ float kt[2][NWV][CB];
  extern __shared__ uint32_t bm[];
  const int b = blockIdx.z, h = blockIdx.y;
  const int wave = threadIdx.x >> 6;
  const int tid0 = threadIdx.x;
  const size_t bh = (size_t)b * H + h;
  for (int j = tid0; j < NB; j += NT) bm[j] = 0u;

  const float* qbh = qhat + bh * (size_t)NG * R;
  const float* kbh = khat + bh * (size_t)NB * R;
  float* dbh = dump ? dump + bh * (size_t)NG * NB : nullptr;
  const int gbase = blockIdx.x * kRowsPerWg;
  // k-hat row of block it's chunk for this thread (zeros past NB; threads >= CB score nothing)
  auto load_k = [&](int it, float (&kr)[R], int tid) {
    const int j = (it % NC) * CB + tid;
    if (tid < CB && j < NB) {
#pragma unroll
      for (int r = 0; r < R; r += 4) {
        const float4 v = *reinterpret_cast<const float4*>(kbh + (size_t)j * R + r);
        kr[r] = v.x; kr[r + 1] = v.y; kr[r + 2] = v.z; kr[r + 3] = v.w;
      }
    } else {
#pragma unroll
      for (int r = 0; r < R; ++r) kr[r] = 0.f;
    }
  };
  float kr[R], kn[R];  // this chunk's k-hat row and the next chunk's, in flight during this chunk's fmas
  load_k(0, kr, tid0);
  float sc[KPL];  // the wave's current row, NaN past NB
#pragma unroll 1
  for (int pass = 0; pass < PASSES; ++pass) {
    const int g0 = gbase + pass * NWV;
    const int tid = opaque(tid0), lane = tid & 63;
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      const int it = pass * NC + c;
      const int j = c * CB + tid;
      if (it + 1 < NIT) load_k(it + 1, kn, tid);
      float sk[NWV];
#pragma unroll
      for (int w = 0; w < NWV; ++w) {
        // rows past the end score row NG - 1 and select nothing; zero (always 0) makes each chunk's q-hat
        // loads distinct, so they are issued per chunk instead of all 8 rows' values being held across chunks
        const int g = min(g0 + w, NG - 1) + zero * (c + 1);
        const float s = score_dot<R>(qbh + (size_t)g * R, kr, tau);
        sk[w] = (tid < CB && j < NB) ? s : __builtin_nanf("");
        if (dbh && tid < CB && j < NB && g0 + w < NG) dbh[(size_t)(g0 + w) * NB + j] = s;
      }
      if (tid < CB) {
#pragma unroll
        for (int w = 0; w < NWV; ++w) kt[it & 1][w][tid] = sk[w];
      }
      __syncthreads();  // the chunk's scores are in the tile; the tile of chunk it - 1 is free again
#pragma unroll
      for (int q = 0; q < KPC; ++q) sc[c * KPC + q] = kt[it & 1][wave][lane + 64 * q];
#pragma unroll
      for (int r = 0; r < R; ++r) kr[r] = kn[r];
    }
    const int g = g0 + wave;
    if (g < NG)
      select_row<KPL, COVER>(sc, b, h, g, NG, NB, ht, coverage, diag_group, idx, cnt, hist[wave], bm, lane, bh);
  }
  __syncthreads();
  const int W = (NG + kRowsPerWg - 1) / kRowsPerWg;
  uint32_t* dst = bits + (bh * W + blockIdx.x) * (size_t)NB;
  for (int j = tid0; j < NB; j += NT) dst[j] = bm[j];
}

template <int KPL, bool COVER>
hipError_t select_launch_c(const Shape& s, const float* scores, const float* qhat, const float* khat, int32_t* idx,
                           int32_t* cnt, uint32_t* bits, float* dump, const HeadTable& ht, float tau, float coverage,
                           int diag, hipStream_t st) {
  dim3 grid((s.NG + kRowsPerWg - 1) / kRowsPerWg, s.H, s.B);
  const size_t lds = (size_t)s.NB * sizeof(uint32_t);
  if (scores) {
    hipLaunchKernelGGL((select_scores_kernel<KPL, COVER>), grid, dim3(sel_waves<KPL, false, COVER>() * 64), lds, st,
                       scores, idx, cnt, bits, ht, s.NG, s.NB, s.H, coverage, diag);
    return hipGetLastError();
  }
  switch (s.R) {
#define DSA_SEL_STREAM(RR)                                                                                \
  case RR:                                                                                                \
    hipLaunchKernelGGL((select_stream_kernel<KPL, RR, COVER>), grid, dim3(sel_waves<KPL, true, COVER>() * 64), \
                       lds, st, qhat, khat, idx, cnt, bits, dump, ht, s.NG, s.NB, s.H, tau, coverage, diag, 0);  \
    break;
    DSA_SEL_STREAM(8)
    DSA_SEL_STREAM(16)
    DSA_SEL_STREAM(32)
    DSA_SEL_STREAM(64)
#undef DSA_SEL_STREAM
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <int KPL>
hipError_t select_dispatch(const Shape& s, const float* scores, const float* qhat, const float* khat, int32_t* idx,
                           int32_t* cnt, uint32_t* bits, float* dump, const HeadTable& ht, float tau, float coverage,
                           int diag, hipStream_t st) {
  if (cnt) return select_launch_c<KPL, true>(s, scores, qhat, khat, idx, cnt, bits, dump, ht, tau, coverage, diag, st);
  return select_launch_c<KPL, false>(s, scores, qhat, khat, idx, cnt, bits, dump, ht, tau, coverage, diag, st);
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

// rev_ptr and rev_idx: block j's groups in ascending order, at its offset.  A workgroup takes 64 consecutive
// blocks of one (b, h): it sums the counts of all blocks before them (its list offset) and scans its own 64
// (writing their rev_ptr entries; the last workgroup also writes the total), copies their W bitmap words into
// LDS (coalesced rows, transposed by the padded stride), then each wave writes whole lists, one block at a
// time -- lane l holds words l, l + 64, ..., a wave prefix sum of their bit counts gives each lane its place
// in the list, and the lanes' stores land in one short span.
constexpr int kRevBlocks = 64;
constexpr int kRevWaves = 8;
__global__ __launch_bounds__(kRevWaves * 64) void rev_write_kernel(const uint32_t* __restrict__ bits,
                                                                   const int32_t* __restrict__ counts,
                                                                   int32_t* __restrict__ rev_ptr,
                                                                   int32_t* __restrict__ rev_idx, HeadTable ht,
                                                                   int NG, int NB, int W, int H) {
  extern __shared__ uint32_t tile[];  // [W][kRevBlocks + 1]
  __shared__ int32_t part[kRevWaves];
  __shared__ int32_t ofs[kRevBlocks + 1];
  const int j0 = blockIdx.x * kRevBlocks;
  const int bhi = blockIdx.y;
  const int b = bhi / H, h = bhi % H;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int32_t* cnt = counts + (size_t)bhi * NB;
  int32_t* rp = rev_ptr + (size_t)bhi * (NB + 1);
  // entries of the blocks before j0
  int32_t before = 0;
  for (int j = threadIdx.x; j < j0; j += kRevWaves * 64) before += cnt[j];
  before = (int32_t)readlane(wave_incl_sum((uint32_t)before), 63);
  if (lane == 0) part[wave] = before;
  const uint32_t* src = bits + (size_t)bhi * W * NB;
  for (int e = threadIdx.x; e < W * kRevBlocks; e += kRevWaves * 64) {
    const int w = e / kRevBlocks, jj = e % kRevBlocks;
    tile[w * (kRevBlocks + 1) + jj] = j0 + jj < NB ? src[(size_t)w * NB + j0 + jj] : 0u;
  }
  __syncthreads();
  if (wave == 0) {
    int32_t base = 0;
#pragma unroll
    for (int i = 0; i < kRevWaves; ++i) base += part[i];
    const int32_t c = j0 + lane < NB ? cnt[j0 + lane] : 0;
    const int32_t incl = (int32_t)wave_incl_sum((uint32_t)c);
    ofs[lane] = base + incl - c;
    if (j0 + lane < NB) rp[j0 + lane] = base + incl - c;
    if (lane == 63) {
      ofs[64] = base + incl;
      if (j0 + kRevBlocks >= NB) rp[NB] = base + incl;
    }
  }
  __syncthreads();
  int32_t* out0 = rev_idx + row_base(ht, b, h, NG);
  for (int jj = wave; jj < kRevBlocks && j0 + jj < NB; jj += kRevWaves) {
    int32_t* out = out0 + ofs[jj];
    uint32_t off = 0;
    for (int w0 = 0; w0 < W; w0 += 64) {
      const int w = w0 + lane;
      uint32_t m = w < W ? tile[w * (kRevBlocks + 1) + jj] : 0u;
      const uint32_t c = (uint32_t)__popc(m);
      const uint32_t incl = wave_incl_sum(c);
      uint32_t pos = off + incl - c;
      while (m) {
        out[pos++] = 32 * w + __builtin_ctz(m);
        m &= m - 1u;
      }
      off += readlane(incl, 63);
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
  if (kpl <= 1) e = select_dispatch<1>(s, scores, qhat, khat, idx, cnt, bits, dump, ht, tau, coverage, diag, st);
  else if (kpl <= 2) e = select_dispatch<2>(s, scores, qhat, khat, idx, cnt, bits, dump, ht, tau, coverage, diag, st);
  else if (kpl <= 4) e = select_dispatch<4>(s, scores, qhat, khat, idx, cnt, bits, dump, ht, tau, coverage, diag, st);
  else if (kpl <= 8) e = select_dispatch<8>(s, scores, qhat, khat, idx, cnt, bits, dump, ht, tau, coverage, diag, st);
  else if (kpl <= 16) e = select_dispatch<16>(s, scores, qhat, khat, idx, cnt, bits, dump, ht, tau, coverage, diag, st);
  else if (kpl <= 32) e = select_dispatch<32>(s, scores, qhat, khat, idx, cnt, bits, dump, ht, tau, coverage, diag, st);
  else if (kpl <= 64) e = select_dispatch<64>(s, scores, qhat, khat, idx, cnt, bits, dump, ht, tau, coverage, diag, st);
  else if (kpl <= 128) e = select_dispatch<128>(s, scores, qhat, khat, idx, cnt, bits, dump, ht, tau, coverage, diag, st);
  else return hipErrorInvalidValue;
  if (e != hipSuccess) return e;
  const int W = (s.NG + kRowsPerWg - 1) / kRowsPerWg;
  const dim3 gcol((s.NB + 255) / 256, s.B * s.H);
  hipLaunchKernelGGL(rev_count_kernel, gcol, dim3(256), 0, st, bits, counts, s.NB, W);
  const size_t tile = (size_t)W * (kRevBlocks + 1) * sizeof(uint32_t);
  hipLaunchKernelGGL(rev_write_kernel, dim3((s.NB + kRevBlocks - 1) / kRevBlocks, s.B * s.H), dim3(kRevWaves * 64),
                     tile, st, bits, counts, rev_ptr, rev_idx, ht, s.NG, s.NB, W, s.H);
  return hipGetLastError();
}

}  // namespace dsa
