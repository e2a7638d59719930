// Sparse attention backward over the kept KV blocks, deterministic (no atomics).
//
// The pages present DSV as a training system (gist.science explainer, hi
// edition, technical summary §2 and §3); the gradient is the standard one of
// softmax attention restricted to each group's kept keys, the selection held
// fixed.  With P = exp(tau Q K^T - LSE) recomputed from the forward's LSE:
//   D_i = dO_i . O_i,  dP = dO V^T,  dS = P (dP - D),
//   dV_j = sum_g P^T dO_g,  dK_j = tau sum_g dS^T Q_g,  dQ_g = tau sum_j dS K_j.
//
// bwd_pre computes D and -LSE*log2(e) and the scaled fp16 copies of K (and of V
// when the forward's copy is not reused), each (b, h) slice multiplied by a
// power of two (common.hpp).
//
// bwd_dq: one workgroup per (b, h, group) over the group's kept blocks; waves
// = 32-row tile x key half, partial dQ of the two halves summed at the end.  Its
// products run on fp16 MFMA: K and V tiles from the scaled copies, the wave's own
// Q and dO rows converted in registers with a power of two from the wave's
// largest magnitude, dS rounded once to fp16.
// bwd_dkdv: one workgroup per (b, h, KV block) over the block's reverse list;
// each wave owns 32 keys and half of every 64-row query tile, dK/dV in
// registers.  Its products run on bf16 MFMA straight from the bf16 inputs (bf16
// spans fp32's range: no scaling), with P (for dV) and dS (for dK) each split
// into a bf16 hi + lo pair: 16 significant bits.
// Tiles are DMA-loaded into XOR-swizzled LDS (no register staging or conversion
// in the loops) and transposed operands read with ds_read_b64_tr_b16.
#include "launch.hpp"

namespace dsa {

namespace {

// D_i = sum_c dO_ic O_ic, nl2_i = -LSE_i * log2(e), and the scaled fp16 copies of K (and of V unless the
// forward's copy is reused), in one pass over the rows of one (b, h) slice per grid row; one 16-lane slice
// per row (D = 128) or 8 (D = 64), 8 columns per lane.  The slice's exponents come from the partial maxima;
// its first workgroup records them in ex.
template <int D>
__global__ __launch_bounds__(256) void bwd_pre_kernel(const bf16_t* __restrict__ K, const bf16_t* __restrict__ V,
                                                      const bf16_t* __restrict__ dO, const float* __restrict__ O,
                                                      const float* __restrict__ LSE, float* __restrict__ Dvec,
                                                      float* __restrict__ nl2, uint16_t* __restrict__ K16,
                                                      uint16_t* __restrict__ V16, const uint32_t* __restrict__ part,
                                                      int32_t* __restrict__ ex, int N, int BH, int convert_v) {
  constexpr int LPR = D / 8;           // lanes per row
  constexpr int RPB = 256 / LPR;       // rows per workgroup pass
  const int bh = blockIdx.y;
  const int eK = slice_exponent(part, kTK, bh, BH, kExpTargetQK);
  const int eV = convert_v ? slice_exponent(part, kTV, bh, BH, kExpTargetV) : 0;
  if (blockIdx.x == 0 && threadIdx.x == 0) {
    ex[kTK * BH + bh] = eK;
    if (convert_v) ex[kTV * BH + bh] = eV;
  }
  const int sub = threadIdx.x % LPR;
  const int64_t r0 = (int64_t)bh * N + (int64_t)N * blockIdx.x / gridDim.x;
  const int64_t r1 = (int64_t)bh * N + (int64_t)N * (blockIdx.x + 1) / gridDim.x;
  // two rows per thread per pass (the second RPB rows further), so that both rows' loads are in flight together
  for (int64_t row = r0 + threadIdx.x / LPR; row < r1; row += 2 * RPB) {
    const bool two = row + RPB < r1;  // uniform over the row's LPR lanes
    const int64_t at[2] = {row * D + 8 * sub, (row + (two ? RPB : 0)) * D + 8 * sub};
    uint4 k[2], v[2], d[2];
    float4 o[2][2];
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      k[u] = ldg16(K + at[u]);
      if (convert_v) v[u] = ldg16(V + at[u]);
      d[u] = ldg16(dO + at[u]);
      o[u][0] = *reinterpret_cast<const float4*>(O + at[u]);
      o[u][1] = *reinterpret_cast<const float4*>(O + at[u] + 4);
    }
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      if (u == 1 && !two) break;
      *reinterpret_cast<uint4*>(K16 + at[u]) = bf16x8_to_f16x8_scaled(k[u], eK);
      if (convert_v) *reinterpret_cast<uint4*>(V16 + at[u]) = bf16x8_to_f16x8_scaled(v[u], eV);
    }
    float s[2];
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const uint32_t* w = reinterpret_cast<const uint32_t*>(&d[u]);
      const float4 o0 = o[u][0], o1 = o[u][1];
      s[u] = __uint_as_float(w[0] << 16) * o0.x + __uint_as_float(w[0] & 0xFFFF0000u) * o0.y +
             __uint_as_float(w[1] << 16) * o0.z + __uint_as_float(w[1] & 0xFFFF0000u) * o0.w +
             __uint_as_float(w[2] << 16) * o1.x + __uint_as_float(w[2] & 0xFFFF0000u) * o1.y +
             __uint_as_float(w[3] << 16) * o1.z + __uint_as_float(w[3] & 0xFFFF0000u) * o1.w;
#pragma unroll
      for (int off = 1; off < LPR; off <<= 1) s[u] += __shfl_xor(s[u], off);
    }
    if (sub == 0) {
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        if (u == 1 && !two) break;
        const int64_t r = row + u * RPB;
        Dvec[r] = s[u];
        nl2[r] = -LSE[r] * kLog2e;
      }
    }
  }
}

// Largest |bf16| (bit pattern, sign cleared) among the 8 values of each of n registers, over the wave.
template <int n>
__device__ __forceinline__ uint32_t wave_amax_bf16(const uint4 (&v)[n]) {
  uint32_t m = 0;
#pragma unroll
  for (int t = 0; t < n; ++t) {
    const uint32_t w[4] = {v[t].x & 0x7FFF7FFFu, v[t].y & 0x7FFF7FFFu, v[t].z & 0x7FFF7FFFu, v[t].w & 0x7FFF7FFFu};
#pragma unroll
    for (int q = 0; q < 4; ++q) m = max(m, max(w[q] & 0xFFFFu, w[q] >> 16));
  }
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) m = max(m, (uint32_t)__shfl_xor((int)m, off));
  return m;
}

// ---------------------------------------------------------------- dQ

// kLists false: dense attention (no lists; list position t is block t).
// kMerge: phase `phase` of n_phase launches in sequence, each over one segment of every row's list (for
// heads whose K and V fill more than half the MALL); launches after the first add into the stored dQ.
template <int D, int G, bool kLists, bool kMerge>
__global__ __launch_bounds__(G * 4, 2) void bwd_dq_kernel(const bf16_t* __restrict__ Q,
                                                          const uint16_t* __restrict__ K16,
                                                          const uint16_t* __restrict__ V16,
                                                          const bf16_t* __restrict__ dO,
                                                          const float* __restrict__ NL2, const float* __restrict__ Dvec,
                                                          const int32_t* __restrict__ idx,
                                                          const int32_t* __restrict__ cnt, float* __restrict__ dQ,
                                                          const int32_t* __restrict__ ex, HeadTable ht, XcdSplit sp,
                                                          int N, int H, int B, float tau, int n_phase, int phase) {
  constexpr int NRT = G / 32;
  constexpr int NW = 2 * NRT;
  constexpr int RB = 2 * D;
  constexpr int TILE = 64 * RB;
  constexpr int OBUF = D * 128;  // one wave's dQ partial: 64 lanes x D/2 floats
  __shared__ __attribute__((aligned(1024))) char st0[2 * TILE];
  __shared__ __attribute__((aligned(1024))) char st1[2 * TILE];
  static_assert(NRT * OBUF <= 4 * TILE, "merge buffers must fit in the stages");

  const int NG = N / G;
  const int64_t task = xcd_task(sp, blockIdx.x);
  if (task < 0) return;
  const uint32_t L = (uint32_t)task;
  const int g = L % NG, h = (L / NG) % H, b = L / (NG * H);
  // blocks of this row: cnt (if given, clamped to [1, k_h]) or k_h; rows are k_h entries apart
  const int kfull = (kLists && cnt) ? min(max(cnt[((size_t)b * H + h) * NG + g], 1), ht.k[h]) : ht.k[h];
  const int kbeg = kMerge ? phase * kfull / n_phase : 0;  // this phase's segment of the list
  const int k = kMerge ? (phase + 1) * kfull / n_phase - kbeg : kfull;
  const int NB = N / kBlock;
  const int32_t* irow = kLists ? idx + row_base(ht, b, h, NG) + (int64_t)g * ht.k[h] + kbeg : nullptr;
  const size_t bh = (size_t)b * H + h;
  const uint16_t* Kbh = K16 + bh * (size_t)N * D;
  const uint16_t* Vbh = V16 + bh * (size_t)N * D;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int l32 = lane & 31, hh = lane >> 5;
  const int rt = wave % NRT, kh = wave / NRT;
  const size_t qrow = bh * N + (size_t)g * G + rt * 32 + l32;
  if (kMerge && k == 0) {  // an empty segment (uniform over the workgroup, before any barrier)
    if (phase == 0 && kh == 0) {
      float* orow = dQ + qrow * D;
#pragma unroll
      for (int c = 0; c < D / 32; ++c)
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4)
          *reinterpret_cast<float4*>(orow + 32 * c + 8 * q4 + 4 * hh) = make_float4(0.f, 0.f, 0.f, 0.f);
    }
    return;
  }
  // block of list position min(t, k-1); ids are valid by contract, clamped so a bad list cannot read out of bounds
  auto block_id = [&](int t) {
    if constexpr (kLists) return min(max(irow[min(t, k - 1)], 0), NB - 1);
    else return kbeg + min(t, k - 1);
  };

  // The wave's Q and dO rows (B operands of S^T and dP^T) as fp16, each multiplied by the power of two that
  // puts the wave's largest magnitude in the target range (the two key-half waves of a row tile read the
  // same rows and find the same exponents).  K16, V16 carry their slices' 2^eK, 2^eV.  So S^T accumulates
  // 2^(eQ+eK) S, dP and D (scaled here) 2^(eO+eV), dQ^T 2^(eO+eV+eK) dQ^T / tau.
  f16x8 qreg[D / 16], oreg[D / 16];
  int eQ, eO;
  {
    uint4 qraw[D / 16], oraw[D / 16];
#pragma unroll
    for (int t = 0; t < D / 16; ++t) {
      qraw[t] = ldg16(Q + qrow * D + 16 * t + 8 * hh);
      oraw[t] = ldg16(dO + qrow * D + 16 * t + 8 * hh);
    }
    eQ = scale_exponent(wave_amax_bf16(qraw), kExpTargetQK);
    eO = scale_exponent(wave_amax_bf16(oraw), kExpTargetDO);
#pragma unroll
    for (int t = 0; t < D / 16; ++t) {
      qreg[t] = __builtin_bit_cast(f16x8, bf16x8_to_f16x8_scaled(qraw[t], eQ));
      oreg[t] = __builtin_bit_cast(f16x8, bf16x8_to_f16x8_scaled(oraw[t], eO));
    }
  }
  const int BHn = B * H;
  const int eK = ex[kTK * BHn + bh], eV = ex[kTV * BHn + bh];
  const float scale_log2 = __builtin_ldexpf(tau * kLog2e, -(eQ + eK));
  const float nl2 = NL2[qrow];
  const float dvec = __builtin_ldexpf(Dvec[qrow], eO + eV);

  int kofs[D / 16];  // K and V rows (keys of this half) as A operands
#pragma unroll
  for (int c = 0; c < D / 16; ++c) kofs[c] = tile_off<D>(32 * kh + l32, 2 * c + hh);
  const int li = lane & 15, g16 = lane >> 4;
  const int rl = 4 * hh + (li >> 2);
  int tofs[D / 32][2];  // transpose reads of K (K^T as the A operand of dQ^T)
#pragma unroll
  for (int c = 0; c < D / 32; ++c)
#pragma unroll
    for (int r = 0; r < 2; ++r)
      tofs[c][r] = tile_off<D>(32 * kh + 8 * r + rl, 4 * c + 2 * (g16 & 1) + ((li & 3) >> 1)) + 8 * (li & 1);

  f32x16 acc[D / 32];
#pragma unroll
  for (int c = 0; c < D / 32; ++c) acc[c] = f32x16{};

  auto fetch = [&](int j, char* dst) {
    dma_tile<D, NW>(Kbh + (size_t)j * kBlock * D, dst, wave, lane);
    dma_tile<D, NW>(Vbh + (size_t)j * kBlock * D, dst + TILE, wave, lane);
  };
  // block ids read ahead: at step t, id_n = block of t+1 and id_pf = block of t+2 are in registers
  int id_n, id_pf;
  auto step = [&](int t, const char* cur, char* nxt) {
    wait_vmem();
    __syncthreads();
    if (t + 1 < k) fetch(id_n, nxt);
    id_n = id_pf;
    id_pf = block_id(t + 3);
    // S^T and dP^T: rows = this half's 32 keys, columns = the wave's 32 queries
    // S first, then dP with the exponentials of S beside its MFMAs
    f32x16 s = f32x16{}, dp = f32x16{};
#pragma unroll
    for (int c = 0; c < D / 16; ++c) s = mfma32h(*reinterpret_cast<const f16x8*>(cur + kofs[c]), qreg[c], s);
    __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
#pragma unroll
    for (int i = 0; i < D / 16 - 2; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    }
    __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
    __builtin_amdgcn_sched_barrier(0);
    float pe[16];
#pragma unroll
    for (int e = 0; e < 16; ++e) pe[e] = __builtin_amdgcn_exp2f(__builtin_fmaf(s[e], scale_log2, nl2));
#pragma unroll
    for (int c = 0; c < D / 16; ++c) dp = mfma32h(*reinterpret_cast<const f16x8*>(cur + TILE + kofs[c]), oreg[c], dp);
    // K^T operands of dQ^T, read under the dP MFMAs
    f16x8 kt[D / 32][2];
#pragma unroll
    for (int c = 0; c < D / 32; ++c) {
      const char* t0 = cur + tofs[c][0];
      const char* t1 = cur + tofs[c][1];
      kt[c][0] = join_f16(lds_read_tr16(t0), lds_read_tr16(t1));
      kt[c][1] = join_f16(lds_read_tr16(t0 + 16 * RB), lds_read_tr16(t1 + 16 * RB));
    }
    __builtin_amdgcn_sched_group_barrier(0x100, 4, 1);
#pragma unroll
    for (int i = 0; i < D / 16 - 2; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 1);
      __builtin_amdgcn_sched_group_barrier(0x002, 4, 1);
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 1);
    }
    __builtin_amdgcn_sched_group_barrier(0x008, 2, 1);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int e = 0; e < 16; ++e) dp[e] = pe[e] * (dp[e] - dvec);
    const f16x8 d0 = pack_f16(dp, 0), d1 = pack_f16(dp, 1);
    // dQ^T[c][i] += K^T[c][m] dS^T[m][i]
#pragma unroll
    for (int c = 0; c < D / 32; ++c) {
      acc[c] = mfma32h(kt[c][0], d0, acc[c]);
      acc[c] = mfma32h(kt[c][1], d1, acc[c]);
    }
  };

  fetch(block_id(0), st0);
  id_n = block_id(1);
  id_pf = block_id(2);
  for (int t = 0; t < k; t += 2) {
    step(t, st0, st1);
    if (t + 1 < k) step(t + 1, st1, st0);
  }

  // sum the two key halves of each row tile
  __syncthreads();
  float* mb = reinterpret_cast<float*>((rt < 2 ? st0 : st1) + (rt & 1) * OBUF);
  if (kh == 1) {
#pragma unroll
    for (int c = 0; c < D / 32; ++c)
#pragma unroll
      for (int e = 0; e < 16; ++e) mb[(c * 16 + e) * 64 + lane] = acc[c][e];
  }
  __syncthreads();
  if (kh == 0) {
    float* orow = dQ + qrow * D;
#pragma unroll
    for (int c = 0; c < D / 32; ++c)
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        float* op = orow + 32 * c + 8 * q4 + 4 * hh;
        float4 prev = make_float4(0.f, 0.f, 0.f, 0.f);
        if (kMerge && phase > 0) prev = *reinterpret_cast<const float4*>(op);
        float v[4];
#pragma unroll
        for (int r = 0; r < 4; ++r)
          v[r] = __builtin_ldexpf((acc[c][4 * q4 + r] + mb[(c * 16 + 4 * q4 + r) * 64 + lane]) * tau, -(eO + eV + eK));
        *reinterpret_cast<float4*>(op) = make_float4(prev.x + v[0], prev.y + v[1], prev.z + v[2], prev.w + v[3]);
      }
  }
}

// ---------------------------------------------------------------- dK, dV

// Order of the dK/dV tasks within each XCD segment (a contiguous range, or an
// XCD's part of one (b, h) run): the blocks whose reverse list is longer than
// half the head's mean first, the rest after, each in task order (so
// neighbouring blocks still run together).  The workgroups that start last
// then have short lists, which trims the tail of the launch.  One workgroup
// per segment; a stable partition by block-wide prefix counts.
__global__ __launch_bounds__(256) void dkdv_order_kernel(const int32_t* __restrict__ rev_ptr,
                                                         int32_t* __restrict__ order, HeadTable ht, XcdSplit sp,
                                                         int NB, int NG, int H) {
  __shared__ int wsum[4];
  __shared__ int run[2];
  int32_t t0, t1;
  xcd_segment(sp, blockIdx.x, t0, t1);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  auto is_long = [&](int32_t t) {
    const int32_t bh = t / NB, j = t % NB, h = bh % H;
    const int32_t* rp = rev_ptr + (int64_t)bh * (NB + 1);
    const int32_t len = rp[j + 1] - rp[j];
    return 2LL * len * NB > (long long)NG * ht.k[h];  // len > NG k_h / (2 NB)
  };
  // block-wide exclusive prefix of flag over the 256 threads; returns the block total
  auto block_scan = [&](int flag, int& prefix) {
    const uint64_t m = __ballot(flag);
    const int below = __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0));
    if (lane == 0) wsum[wave] = __popcll(m);
    __syncthreads();
    int base = 0, total = 0;
    for (int w = 0; w < 4; ++w) {
      base += w < wave ? wsum[w] : 0;
      total += wsum[w];
    }
    __syncthreads();
    prefix = base + below;
    return total;
  };
  // pass 1: number of long tasks in the range
  int nlong = 0;
  for (int32_t c = t0; c < t1; c += 256) {
    const int32_t t = c + (int32_t)threadIdx.x;
    int pre;
    nlong += block_scan(t < t1 && is_long(t), pre);
  }
  // pass 2: stable partition
  if (threadIdx.x == 0) { run[0] = 0; run[1] = 0; }
  __syncthreads();
  for (int32_t c = t0; c < t1; c += 256) {
    const int32_t t = c + (int32_t)threadIdx.x;
    const bool valid = t < t1;
    const bool lg = valid && is_long(t);
    int pl, ps;
    const int nl = block_scan(lg, pl);
    const int ns = block_scan(valid && !lg, ps);
    if (valid) order[lg ? t0 + run[0] + pl : t0 + nlong + run[1] + ps] = t;
    __syncthreads();
    if (threadIdx.x == 0) { run[0] += nl; run[1] += ns; }
    __syncthreads();
  }
}

// kLists false: dense attention (no reverse lists or order; every block has all NG groups).
//
// Wave w = (kh, qh) owns keys 32*kh..32*kh+31 of the block and query rows
// 32*qh..32*qh+31 of every 64-row tile, on 16x16x32 MFMAs over two 16-key
// halves: each operand read from LDS feeds both halves (half the LDS bytes per
// MFMA of a wave with 16 keys), and the two query halves' dK, dV partials are
// summed once at the end.  S starts from -LSE/tau and dP from -D, so
// P = exp2(S tau log2 e) and dS = P dP need no per-row values afterwards.
// kMerge: phase `phase` of n_phase launches in sequence, each over one segment of every reverse list
// (for heads whose Q and dO fill more than half the MALL); launches after the first add into dK, dV.
template <int D, int G, bool kLists, bool kMerge>
__global__ __launch_bounds__(256, 2) void bwd_dkdv_kernel(const bf16_t* __restrict__ Q,
                                                          const bf16_t* __restrict__ K,
                                                          const bf16_t* __restrict__ V,
                                                          const bf16_t* __restrict__ dO,
                                                          const float* __restrict__ NL2,
                                                          const float* __restrict__ Dvec,
                                                          const int32_t* __restrict__ rev_ptr,
                                                          const int32_t* __restrict__ rev_idx,
                                                          const int32_t* __restrict__ order, float* __restrict__ dK,
                                                          float* __restrict__ dV, HeadTable ht, XcdSplit sp, int N,
                                                          int H, int NB, int B, float tau, int n_phase, int phase) {
  constexpr int NW = 4;
  constexpr int RB = 2 * D;
  constexpr int TILE = 64 * RB;
  constexpr int STAGE = 2 * TILE + 512;  // Q tile, dO tile, -LSE*log2e row, D row
  constexpr int SUB = G / 64;            // 64-row query tiles per group
  constexpr int NT = D / 32;             // 32-wide steps of the head dimension (S, dP)
  constexpr int NC = D / 16;             // 16-wide column tiles of dK, dV
  constexpr int XBUF = 2 * NC * 4 * 64 * 4;  // one wave's partial of one tensor
  static_assert(2 * XBUF <= STAGE, "the partials of one key half must fit in one stage");
  __shared__ __attribute__((aligned(1024))) char st0[STAGE];
  __shared__ __attribute__((aligned(1024))) char st1[STAGE];

  const int64_t slot = xcd_task(sp, blockIdx.x);
  if (slot < 0) return;
  const int32_t n_tasks = NB * H * B;
  // a permutation of the range (the identity for dense attention); clamped
  const uint32_t L = kLists ? (uint32_t)min(max(order[slot], 0), n_tasks - 1) : (uint32_t)slot;
  const int j = L % NB, h = (L / NB) % H, b = L / (NB * H);
  const int NG = N / G;
  const size_t bh = (size_t)b * H + h;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int l16 = lane & 15, q4 = lane >> 4;
  const int kh = wave & 1, qh = wave >> 1;
  const int32_t total = NG * ht.k[h];  // size of the (b, h) region of the reverse list
  const float scale_log2 = tau * kLog2e;
  const float inv_scale = 1.0f / scale_log2;
  int32_t s0 = 0, s1 = NG;
  const int32_t* rlist = nullptr;
  if constexpr (kLists) {
    const int32_t* rp = rev_ptr + bh * (NB + 1);
    s0 = min(max(rp[j], 0), total);
    s1 = min(max(rp[j + 1], s0), total);
  }
  if constexpr (kMerge) {  // this phase's segment of the list
    const int32_t len = s1 - s0, base = s0;
    s0 = base + (int32_t)((int64_t)phase * len / n_phase);
    s1 = base + (int32_t)((int64_t)(phase + 1) * len / n_phase);
    if (phase > 0 && s1 == s0) return;  // nothing to add (uniform over the workgroup, before any barrier)
  }
  if constexpr (kLists) rlist = rev_idx + row_base(ht, b, h, NG) + s0;
  const int iters = (s1 - s0) * SUB;

  // this wave's keys as B operands (half kk: keys 32*kh + 16*kk + l16): K for
  // S = Q K^T, V for dP = dO V^T
  bf16x8 kreg[2][NT], vreg[2][NT];
#pragma unroll
  for (int kk = 0; kk < 2; ++kk) {
    const size_t key = bh * N + (size_t)j * kBlock + 32 * kh + 16 * kk + l16;
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      kreg[kk][t] = __builtin_bit_cast(bf16x8, ldg16(K + key * D + 32 * t + 8 * q4));
      vreg[kk][t] = __builtin_bit_cast(bf16x8, ldg16(V + key * D + 32 * t + 8 * q4));
    }
  }
  // A operands of S and dP: query row 32*qh + 16*qq + l16, logical chunk 4t + q4,
  // at byte offset (abase ^ 64t) + 16*qq*RB (the swizzle permutes chunks within
  // a row and repeats every 16 rows)
  const int abase = tile_off<D>(32 * qh + l16, q4);
  // transpose reads (B operands of dV, dK): lane i of 16-lane group q4 reads row
  // 32*qh + 4*q4 + i/4 (+16), columns 16c + 4*(i%4), at (tbase ^ 32c)
  const int tbase = tile_off<D>(32 * qh + 4 * q4 + (l16 >> 2), (l16 & 3) >> 1) + 8 * (l16 & 1);

  f32x4 dk[2][NC], dv[2][NC];
#pragma unroll
  for (int kk = 0; kk < 2; ++kk)
#pragma unroll
    for (int c = 0; c < NC; ++c) { dk[kk][c] = f32x4{}; dv[kk][c] = f32x4{}; }

  // group of query tile min(it, iters-1) (needs iters > 0), read ahead as a
  // vector load; clamped when used: never out of bounds
  auto group_of = [&](int it) {
    if constexpr (kLists) return ldv_i32(rlist + min(it, iters - 1) / SUB);
    else return s0 + min(it, iters - 1) / SUB;
  };
  // groups read ahead: at step it, g_n = group of tile it+1 and g_pf = group of tile it+2 are in registers
  int g_n = 0, g_pf = 0;
  auto fetch = [&](int it, int graw, char* dst) {
    const int g = min(max(__builtin_amdgcn_readfirstlane(graw), 0), NG - 1);
    const size_t row0 = bh * N + (size_t)g * G + (size_t)(it % SUB) * 64;
    dma_tile<D, NW>(Q + row0 * D, dst, wave, lane);
    dma_tile<D, NW>(dO + row0 * D, dst + TILE, wave, lane);
    if (wave == 0) dma_row64_f32(NL2 + row0, dst + 2 * TILE, lane);
    if (wave == 1) dma_row64_f32(Dvec + row0, dst + 2 * TILE + 256, lane);
  };
  auto step = [&](int it, const char* cur, char* nxt) {
    wait_vmem();
    __syncthreads();  // tile it is in LDS and every wave is done with tile it-1
    if (it + 1 < iters) fetch(it + 1, g_n, nxt);
    g_n = g_pf;
    g_pf = group_of(it + 3);
    // offsets recomputed per step (kept out of registers across the loop)
    int ab = abase, tb = tbase;
    asm volatile("" : "+v"(ab), "+v"(tb));
    // S[kk][qq], dP[kk][qq]: element e of lane l is query 32*qh + 16*qq + 4*q4 + e,
    // key 32*kh + 16*kk + l16
    const float* nrow = reinterpret_cast<const float*>(cur + 2 * TILE) + 32 * qh + 4 * q4;
    const float* drow = reinterpret_cast<const float*>(cur + 2 * TILE + 256) + 32 * qh + 4 * q4;
    f32x4 s[2][2], dp[2][2];
#pragma unroll
    for (int qq = 0; qq < 2; ++qq) {
      const f32x4 n4 = *reinterpret_cast<const f32x4*>(nrow + 16 * qq);
      const f32x4 d4 = *reinterpret_cast<const f32x4*>(drow + 16 * qq);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        s[0][qq][e] = s[1][qq][e] = n4[e] * inv_scale;
        dp[0][qq][e] = dp[1][qq][e] = -d4[e];
      }
    }
#pragma unroll
    for (int qq = 0; qq < 2; ++qq)
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        const bf16x8 a = *reinterpret_cast<const bf16x8*>(cur + 16 * qq * RB + (ab ^ (64 * t)));
        s[0][qq] = mfma16b(a, kreg[0][t], s[0][qq]);
        s[1][qq] = mfma16b(a, kreg[1][t], s[1][qq]);
      }
#pragma unroll
    for (int qq = 0; qq < 2; ++qq)
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        const bf16x8 a = *reinterpret_cast<const bf16x8*>(cur + TILE + 16 * qq * RB + (ab ^ (64 * t)));
        dp[0][qq] = mfma16b(a, vreg[0][t], dp[0][qq]);
        dp[1][qq] = mfma16b(a, vreg[1][t], dp[1][qq]);
      }
    // P = exp2(S tau log2 e), dS = P (dP - D); A operands per key half kk:
    // element e' <-> query 32*qh + 16*(e'/4) + 4*q4 + e'%4
    // P and dS each enter their products as a bf16 hi + lo pair (16 significant bits, fp32's range): dV sums
    // P against dO and dK sums a cancelling dS against clustered Q, and one 11-bit rounding of either
    // (fp16, 2^-12 relative) left errors of a few 1e-2 on gradients of magnitude 100-200
    bf16x8 ph[2], pl[2], dh[2], dl[2];
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      float pv[8], dsv[8];
#pragma unroll
      for (int qq = 0; qq < 2; ++qq)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          pv[4 * qq + e] = __builtin_amdgcn_exp2f(s[kk][qq][e] * scale_log2);
          dsv[4 * qq + e] = pv[4 * qq + e] * dp[kk][qq][e];
        }
      split_bf16x8(pv, ph[kk], pl[kk]);
      split_bf16x8(dsv, dh[kk], dl[kk]);
    }
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      const char* o = cur + TILE + (tb ^ (32 * c));
      const bf16x8 ob = join_bf16(lds_read_tr16(o), lds_read_tr16(o + 16 * RB));
      const char* q = cur + (tb ^ (32 * c));
      const bf16x8 qb = join_bf16(lds_read_tr16(q), lds_read_tr16(q + 16 * RB));
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) {
        dv[kk][c] = mfma16b(ph[kk], ob, dv[kk][c]);
        dv[kk][c] = mfma16b(pl[kk], ob, dv[kk][c]);
        dk[kk][c] = mfma16b(dh[kk], qb, dk[kk][c]);
        dk[kk][c] = mfma16b(dl[kk], qb, dk[kk][c]);
      }
    }
    // (no scheduling groups: at this register load the compiler's own order is faster, 9.33 vs 9.71 ms)
  };

  if (iters > 0) {
    fetch(0, group_of(0), st0);
    g_n = group_of(1);
    g_pf = group_of(2);
  }
  for (int it = 0; it < iters; it += 2) {
    step(it, st0, st1);
    if (it + 1 < iters) step(it + 1, st1, st0);
  }

  // sum the two query halves: the qh = 1 wave parks its dK partial, the qh = 0
  // wave its dV partial, in the stage of their key half; each then stores one
  __syncthreads();
  float* xb = reinterpret_cast<float*>(kh ? st1 : st0);
  float* park = xb + (qh ? 0 : XBUF / 4);
#pragma unroll
  for (int kk = 0; kk < 2; ++kk)
#pragma unroll
    for (int c = 0; c < NC; ++c)
#pragma unroll
      for (int e = 0; e < 4; ++e) park[((kk * NC + c) * 4 + e) * 64 + lane] = qh ? dk[kk][c][e] : dv[kk][c][e];
  __syncthreads();
  const float* other = xb + (qh ? XBUF / 4 : 0);
  float* out = qh ? dV : dK;
  const float mul = qh ? 1.0f : tau;
  // accumulator element e of column tile c, half kk: key 32*kh + 16*kk + 4*q4 + e, column 16c + l16
  const size_t key0 = bh * N + (size_t)j * kBlock + 32 * kh + 4 * q4;
#pragma unroll
  for (int kk = 0; kk < 2; ++kk)
#pragma unroll
    for (int c = 0; c < NC; ++c)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float own = qh ? dv[kk][c][e] : dk[kk][c][e];
        float* op = out + (key0 + 16 * kk + e) * D + 16 * c + l16;
        const float prev = (kMerge && phase > 0) ? *op : 0.0f;
        *op = prev + (own + other[((kk * NC + c) * 4 + e) * 64 + lane]) * mul;
      }
}

template <int D>
hipError_t pre_launch(const Shape& s, const bf16_t* K, const bf16_t* V, const float* O, const bf16_t* dO,
                      const float* LSE, const BwdWork& w, bool v_from_fwd, hipStream_t st) {
  const int BH = s.B * s.H;
  const int64_t n_per_bh = (int64_t)s.N * D;
  AmaxSrc a = {{nullptr, K, v_from_fwd ? nullptr : V, nullptr}};
  hipError_t e = launch_amax(a, w.part, n_per_bh, BH, st);
  if (e != hipSuccess) return e;
  constexpr int RPB = 256 / (D / 8);
  const int64_t passes = ((int64_t)s.N + RPB - 1) / RPB;  // workgroup passes over one slice's rows
  const unsigned chunks = (unsigned)std::max<int64_t>(1, std::min<int64_t>(256, passes / 4));
  hipLaunchKernelGGL(bwd_pre_kernel<D>, dim3(chunks, BH), dim3(256), 0, st, K, V, dO, O, LSE, w.Dvec, w.nl2, w.K16,
                     w.V16, w.part, w.ex, s.N, BH, v_from_fwd ? 0 : 1);
  return hipGetLastError();
}

template <int D, int G>
hipError_t dkdv_launch(const Shape& s, const BwdWork& w, const bf16_t* Q, const bf16_t* K, const bf16_t* V,
                       const bf16_t* dO, const int32_t* rev_ptr, const int32_t* rev_idx, float* dK, float* dV,
                       const HeadTable& ht, hipStream_t st) {
  const float tau = 1.0f / sqrtf((float)D);
  // a KV block costs its reverse-list length, NG * k_h / NB on average, + 1; a head streams its Q and dO
  unsigned nwg = 0;
  const double head_bytes = 4.0 * s.N * D;  // one head's Q and dO (16-bit)
  const int nph = head_bytes > 0.5 * kMallBytes ? kMallPhasesQdO : 1;  // phases over segments of every list
  const XcdSplit sp = make_xcd_split(s.B, s.H, s.NB, ht, (double)s.NG / s.NB / nph, 1.0, head_bytes, &nwg);
  const unsigned nseg = sp.items ? kXcds * (unsigned)sp.runs : kXcds;
  // dense (no reverse lists): every block has all NG groups and the order is the identity
  if (rev_ptr)
    hipLaunchKernelGGL(dkdv_order_kernel, dim3(nseg), dim3(256), 0, st, rev_ptr, w.order, ht, sp, s.NB, s.NG, s.H);
  if (nph > 1) {
    auto kern = rev_ptr ? bwd_dkdv_kernel<D, G, true, true> : bwd_dkdv_kernel<D, G, false, true>;
    for (int ph = 0; ph < nph; ++ph)
      hipLaunchKernelGGL(kern, dim3(nwg), dim3(256), 0, st, Q, K, V, dO, w.nl2, w.Dvec, rev_ptr, rev_idx, w.order,
                         dK, dV, ht, sp, s.N, s.H, s.NB, s.B, tau, nph, ph);
    return hipGetLastError();
  }
  auto kern = rev_ptr ? bwd_dkdv_kernel<D, G, true, false> : bwd_dkdv_kernel<D, G, false, false>;
  hipLaunchKernelGGL(kern, dim3(nwg), dim3(256), 0, st, Q, K, V, dO, w.nl2, w.Dvec, rev_ptr, rev_idx, w.order, dK,
                     dV, ht, sp, s.N, s.H, s.NB, s.B, tau, 1, -1);
  return hipGetLastError();
}

template <int D, int G>
hipError_t dq_launch(const Shape& s, const BwdWork& w, const bf16_t* Q, const bf16_t* dO, const int32_t* idx,
                     const int32_t* cnt, float* dQ, const HeadTable& ht, hipStream_t st) {
  const float tau = 1.0f / sqrtf((float)D);
  unsigned nwg = 0;
  const double head_bytes = 4.0 * s.N * D;  // one head's K and V (their fp16 copies)
  if (head_bytes > 0.5 * kMallBytes) {  // phases over segments of every list, each streaming ~1/kMallPhasesKV
    const XcdSplit sp = make_xcd_split(s.B, s.H, s.NG, ht, 1.0 / kMallPhasesKV, 1.0, head_bytes, &nwg);
    auto kern = idx ? bwd_dq_kernel<D, G, true, true> : bwd_dq_kernel<D, G, false, true>;
    for (int ph = 0; ph < kMallPhasesKV; ++ph)
      hipLaunchKernelGGL(kern, dim3(nwg), dim3(G * 4), 0, st, Q, w.K16, w.V16, dO, w.nl2, w.Dvec, idx, cnt, dQ, w.ex,
                         ht, sp, s.N, s.H, s.B, tau, kMallPhasesKV, ph);
    return hipGetLastError();
  }
  const XcdSplit sp = make_xcd_split(s.B, s.H, s.NG, ht, 1.0, 1.0, head_bytes, &nwg);  // a group costs k_h + 1
  auto kern = idx ? bwd_dq_kernel<D, G, true, false> : bwd_dq_kernel<D, G, false, false>;
  hipLaunchKernelGGL(kern, dim3(nwg), dim3(G * 4), 0, st, Q, w.K16, w.V16, dO, w.nl2, w.Dvec, idx, cnt, dQ, w.ex, ht,
                     sp, s.N, s.H, s.B, tau, 1, -1);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_bwd_pre(const Shape& s, const void* Q, const void* K, const void* V, const float* O,
                          const void* dO, const float* LSE, const BwdWork& w, bool v_from_fwd, hipStream_t st) {
  (void)Q;
  const bf16_t* k = static_cast<const bf16_t*>(K);
  const bf16_t* v = static_cast<const bf16_t*>(V);
  const bf16_t* o = static_cast<const bf16_t*>(dO);
  return s.D == 64 ? pre_launch<64>(s, k, v, O, o, LSE, w, v_from_fwd, st)
                   : pre_launch<128>(s, k, v, O, o, LSE, w, v_from_fwd, st);
}

hipError_t launch_bwd_dkdv(const Shape& s, const BwdWork& w, const void* Q, const void* K, const void* V,
                           const void* dO, const int32_t* rev_ptr, const int32_t* rev_idx, float* dK, float* dV,
                           const HeadTable& ht, hipStream_t st) {
  const bf16_t* q = static_cast<const bf16_t*>(Q);
  const bf16_t* k = static_cast<const bf16_t*>(K);
  const bf16_t* v = static_cast<const bf16_t*>(V);
  const bf16_t* o = static_cast<const bf16_t*>(dO);
  if (s.D == 64)
    return s.G == 64 ? dkdv_launch<64, 64>(s, w, q, k, v, o, rev_ptr, rev_idx, dK, dV, ht, st)
                     : dkdv_launch<64, 128>(s, w, q, k, v, o, rev_ptr, rev_idx, dK, dV, ht, st);
  return s.G == 64 ? dkdv_launch<128, 64>(s, w, q, k, v, o, rev_ptr, rev_idx, dK, dV, ht, st)
                   : dkdv_launch<128, 128>(s, w, q, k, v, o, rev_ptr, rev_idx, dK, dV, ht, st);
}

hipError_t launch_bwd_dq(const Shape& s, const BwdWork& w, const void* Q, const void* dO, const int32_t* idx,
                         float* dQ, const HeadTable& ht, hipStream_t st, const int32_t* cnt) {
  const bf16_t* q = static_cast<const bf16_t*>(Q);
  const bf16_t* o = static_cast<const bf16_t*>(dO);
  if (s.D == 64)
    return s.G == 64 ? dq_launch<64, 64>(s, w, q, o, idx, cnt, dQ, ht, st)
                     : dq_launch<64, 128>(s, w, q, o, idx, cnt, dQ, ht, st);
  return s.G == 64 ? dq_launch<128, 64>(s, w, q, o, idx, cnt, dQ, ht, st)
                   : dq_launch<128, 128>(s, w, q, o, idx, cnt, dQ, ht, st);
}

}  // namespace dsa
