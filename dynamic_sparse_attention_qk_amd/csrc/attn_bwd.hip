// Sparse attention backward over the kept KV blocks, deterministic (no atomics).
//
// The pages present DSV as a training system (gist.science explainer, hi
// edition, technical summary §2 and §3); the gradient is the standard one of
// softmax attention restricted to each group's kept keys, the selection held
// fixed.  With P = exp(tau Q K^T - LSE) recomputed from the forward's LSE:
//   D_i = dO_i . O_i,  dP = dO V^T,  dS = P (dP - D),
//   dV_j = sum_g P^T dO_g,  dK_j = tau sum_g dS^T Q_g,  dQ_g = tau sum_j dS K_j.
//
// bwd_pre computes D.  bwd_dkdv runs one workgroup per (b, h, KV block) over
// the groups of the block's reverse list; each of its 2 waves owns 32 keys and
// keeps dK/dV in registers.  bwd_dq runs one workgroup per (b, h, group) over
// the group's kept blocks; each wave owns 32 query rows.  Operands whose
// contraction index is the row index in memory (Q and dO in dkdv, K in dq) are
// staged transposed in LDS so every MFMA operand is a contiguous LDS read.
#include "launch.hpp"

namespace dsa {

namespace {

// D_i = sum_c dO_ic O_ic; one 16-lane slice per row, 8 columns per lane.
template <int D>
__global__ __launch_bounds__(256) void bwd_pre_kernel(const bf16_t* __restrict__ dO, const float* __restrict__ O,
                                                      float* __restrict__ Dvec, int64_t rows) {
  constexpr int LPR = D / 8;           // lanes per row
  constexpr int RPB = 256 / LPR;       // rows per workgroup pass
  const int sub = threadIdx.x % LPR;
  for (int64_t row = (int64_t)blockIdx.x * RPB + threadIdx.x / LPR; row < rows; row += (int64_t)gridDim.x * RPB) {
    const uint4 d = ldg16(dO + row * D + 8 * sub);
    const float4 o0 = *reinterpret_cast<const float4*>(O + row * D + 8 * sub);
    const float4 o1 = *reinterpret_cast<const float4*>(O + row * D + 8 * sub + 4);
    const uint32_t* w = reinterpret_cast<const uint32_t*>(&d);
    float s = __uint_as_float(w[0] << 16) * o0.x + __uint_as_float(w[0] & 0xFFFF0000u) * o0.y +
              __uint_as_float(w[1] << 16) * o0.z + __uint_as_float(w[1] & 0xFFFF0000u) * o0.w +
              __uint_as_float(w[2] << 16) * o1.x + __uint_as_float(w[2] & 0xFFFF0000u) * o1.y +
              __uint_as_float(w[3] << 16) * o1.z + __uint_as_float(w[3] & 0xFFFF0000u) * o1.w;
#pragma unroll
    for (int off = 1; off < LPR; off <<= 1) s += __shfl_xor(s, off);
    if (sub == 0) Dvec[row] = s;
  }
}

template <int D, int G>
__global__ __launch_bounds__(128) void bwd_dkdv_kernel(const bf16_t* __restrict__ Q, const bf16_t* __restrict__ K,
                                                       const bf16_t* __restrict__ V, const bf16_t* __restrict__ dO,
                                                       const float* __restrict__ LSE, const float* __restrict__ Dvec,
                                                       const int32_t* __restrict__ rev_ptr,
                                                       const int32_t* __restrict__ rev_idx, float* __restrict__ dK,
                                                       float* __restrict__ dV, HeadTable ht, int N, int H, int NB,
                                                       int B, float scale_log2, float tau) {
  constexpr int NT = 128;
  constexpr int LD = kRowLd<D>;   // row-major tiles
  constexpr int TLD = kColLd;     // transposed tiles
  constexpr int SUB = G / 64;     // 64-row query sub-tiles per group
  __shared__ __attribute__((aligned(16))) bf16_t sQ[64 * LD];
  __shared__ __attribute__((aligned(16))) bf16_t sdO[64 * LD];
  __shared__ __attribute__((aligned(16))) uint16_t sQt[D * TLD];   // fp16
  __shared__ __attribute__((aligned(16))) uint16_t sdOt[D * TLD];  // fp16
  __shared__ __attribute__((aligned(16))) float sL[64];
  __shared__ __attribute__((aligned(16))) float sD[64];

  const uint32_t L = xcd_remap(blockIdx.x, (uint32_t)(NB * H * B));
  const int j = L % NB, h = (L / NB) % H, b = L / (NB * H);
  const int NG = N / G;
  const size_t bh = (size_t)b * H + h;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int l32 = lane & 31, hh = lane >> 5;
  const int32_t* rp = rev_ptr + bh * (NB + 1);
  const int32_t total = NG * ht.k[h];  // size of the (b, h) region of the reverse list
  const int32_t s0 = min(max(rp[j], 0), total), s1 = min(max(rp[j + 1], s0), total);
  const int32_t* rlist = rev_idx + row_base(ht, b, h, NG) + s0;
  const int iters = (s1 - s0) * SUB;

  // the wave's 32 keys as B operands (K for S = Q K^T, V for dP = dO V^T)
  bf16x8 kreg[D / 16], vreg[D / 16];
  {
    const size_t key = bh * N + (size_t)j * kBlock + 32 * wave + l32;
    const bf16_t* kp = K + key * D + 8 * hh;
    const bf16_t* vp = V + key * D + 8 * hh;
#pragma unroll
    for (int t = 0; t < D / 16; ++t) {
      kreg[t] = *reinterpret_cast<const bf16x8*>(kp + 16 * t);
      vreg[t] = *reinterpret_cast<const bf16x8*>(vp + 16 * t);
    }
  }
  f32x16 dk[D / 32], dv[D / 32];
#pragma unroll
  for (int c = 0; c < D / 32; ++c) { dk[c] = f32x16{}; dv[c] = f32x16{}; }

  TileMover<D, NT> mq, mo;
  float lse_pre = 0.f, d_pre = 0.f;
  auto fetch = [&](int it) {
    const int g = min(max(rlist[it / SUB], 0), NG - 1);  // valid by contract; never read out of bounds
    const size_t row0 = bh * N + (size_t)g * G + (size_t)(it % SUB) * 64;
    mq.load(Q + row0 * D);
    mo.load(dO + row0 * D);
    if (threadIdx.x < 64) {
      lse_pre = LSE[row0 + threadIdx.x] * kLog2e;
      d_pre = Dvec[row0 + threadIdx.x];
    }
  };
  if (iters > 0) fetch(0);

  for (int it = 0; it < iters; ++it) {
    __syncthreads();
    mq.store_rows(sQ);
    mq.store_cols_f16(sQt);
    mo.store_rows(sdO);
    mo.store_cols_f16(sdOt);
    if (threadIdx.x < 64) { sL[threadIdx.x] = lse_pre; sD[threadIdx.x] = d_pre; }
    __syncthreads();
    if (it + 1 < iters) fetch(it + 1);

    // S[i][m] and dP[i][m] for the 64 queries (two 32-row tiles) x the wave's 32 keys
    f32x16 s[2], dp[2];
#pragma unroll
    for (int qt = 0; qt < 2; ++qt) {
      s[qt] = f32x16{};
      dp[qt] = f32x16{};
#pragma unroll
      for (int c = 0; c < D / 16; ++c) {
        const bf16x8 aq = *reinterpret_cast<const bf16x8*>(&sQ[(32 * qt + l32) * LD + 16 * c + 8 * hh]);
        const bf16x8 ao = *reinterpret_cast<const bf16x8*>(&sdO[(32 * qt + l32) * LD + 16 * c + 8 * hh]);
        s[qt] = mfma32(aq, kreg[c], s[qt]);
        dp[qt] = mfma32(ao, vreg[c], dp[qt]);
      }
    }
    // P and dS; accumulator element e of tile qt is query 32*qt + 8*(e/4) + 4*hh + e%4
#pragma unroll
    for (int qt = 0; qt < 2; ++qt)
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        const float4 l4 = *reinterpret_cast<const float4*>(&sL[32 * qt + 8 * q4 + 4 * hh]);
        const float4 d4 = *reinterpret_cast<const float4*>(&sD[32 * qt + 8 * q4 + 4 * hh]);
        const float lv[4] = {l4.x, l4.y, l4.z, l4.w};
        const float dvv[4] = {d4.x, d4.y, d4.z, d4.w};
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int e = 4 * q4 + r;
          const float p = __builtin_amdgcn_exp2f(__builtin_fmaf(s[qt][e], scale_log2, -lv[r]));
          s[qt][e] = p;
          dp[qt][e] = p * (dp[qt][e] - dvv[r]);
        }
      }
    // dV[m][c] += P^T dO, dK[m][c] += dS^T Q  (A from accumulators, B transposed tiles)
#pragma unroll
    for (int qc = 0; qc < 4; ++qc) {
      // dK sums dS (which cancels across queries) against Q of clustered rows: its
      // operand is split hi + lo so fp16 rounding of dS does not reach the result.
      const f16x8 pa = pack_f16(s[qc >> 1], qc & 1);
      f16x8 da, da_lo;
      pack_f16_split(dp[qc >> 1], qc & 1, da, da_lo);
#pragma unroll
      for (int c = 0; c < D / 32; ++c) {
        dv[c] = mfma32h(pa, lds_pair_b64_h(&sdOt[(32 * c + l32) * TLD + 16 * qc + 4 * hh]), dv[c]);
        const f16x8 qb = lds_pair_b64_h(&sQt[(32 * c + l32) * TLD + 16 * qc + 4 * hh]);
        dk[c] = mfma32h(da, qb, dk[c]);
        dk[c] = mfma32h(da_lo, qb, dk[c]);
      }
    }
  }

  // accumulator element e: key 8*(e/4) + 4*hh + e%4 of the wave's 32, column 32*c + l32
  const size_t key0 = bh * N + (size_t)j * kBlock + 32 * wave;
#pragma unroll
  for (int c = 0; c < D / 32; ++c)
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const size_t key = key0 + 8 * (e / 4) + 4 * hh + (e % 4);
      dK[key * D + 32 * c + l32] = dk[c][e] * tau;
      dV[key * D + 32 * c + l32] = dv[c][e];
    }
}

template <int D, int G>
__global__ __launch_bounds__(G * 2) void bwd_dq_kernel(const bf16_t* __restrict__ Q, const bf16_t* __restrict__ K,
                                                       const bf16_t* __restrict__ V, const bf16_t* __restrict__ dO,
                                                       const float* __restrict__ LSE, const float* __restrict__ Dvec,
                                                       const int32_t* __restrict__ idx, float* __restrict__ dQ,
                                                       HeadTable ht, int N, int H, int B, float scale_log2, float tau) {
  constexpr int NT = G * 2;
  constexpr int LD = kRowLd<D>;
  constexpr int TLD = kColLd;
  __shared__ __attribute__((aligned(16))) bf16_t sK[64 * LD];
  __shared__ __attribute__((aligned(16))) bf16_t sV[64 * LD];
  __shared__ __attribute__((aligned(16))) uint16_t sKt[D * TLD];  // fp16

  const int NG = N / G;
  const uint32_t L = xcd_remap(blockIdx.x, (uint32_t)(NG * H * B));
  const int g = L % NG, h = (L / NG) % H, b = L / (NG * H);
  const int k = ht.k[h];
  const int32_t* irow = idx + row_base(ht, b, h, NG) + (int64_t)g * k;
  const size_t bh = (size_t)b * H + h;
  const bf16_t* Kbh = K + bh * (size_t)N * D;
  const bf16_t* Vbh = V + bh * (size_t)N * D;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int l32 = lane & 31, hh = lane >> 5;
  const size_t qrow = bh * N + (size_t)g * G + wave * 32 + l32;

  bf16x8 qreg[D / 16], oreg[D / 16];
  {
    const bf16_t* qp = Q + qrow * D + 8 * hh;
    const bf16_t* op = dO + qrow * D + 8 * hh;
#pragma unroll
    for (int t = 0; t < D / 16; ++t) {
      qreg[t] = *reinterpret_cast<const bf16x8*>(qp + 16 * t);
      oreg[t] = *reinterpret_cast<const bf16x8*>(op + 16 * t);
    }
  }
  const float lse2 = LSE[qrow] * kLog2e;
  const float dvec = Dvec[qrow];

  f32x16 acc[D / 32];
#pragma unroll
  for (int c = 0; c < D / 32; ++c) acc[c] = f32x16{};

  const int NB = N / kBlock;
  auto block_id = [&](int t) { return min(max(irow[t], 0), NB - 1); };
  TileMover<D, NT> mk, mv;
  {
    const int j = block_id(0);
    mk.load(Kbh + (size_t)j * kBlock * D);
    mv.load(Vbh + (size_t)j * kBlock * D);
  }
  for (int t = 0; t < k; ++t) {
    __syncthreads();
    mk.store_rows(sK);
    mk.store_cols_f16(sKt);
    mv.store_rows(sV);
    __syncthreads();
    if (t + 1 < k) {
      const int j = block_id(t + 1);
      mk.load(Kbh + (size_t)j * kBlock * D);
      mv.load(Vbh + (size_t)j * kBlock * D);
    }
    // S^T and dP^T: rows = the block's keys (two 32-key tiles), columns = the wave's queries
    f32x16 s[2], dp[2];
#pragma unroll
    for (int kt = 0; kt < 2; ++kt) {
      s[kt] = f32x16{};
      dp[kt] = f32x16{};
#pragma unroll
      for (int c = 0; c < D / 16; ++c) {
        const bf16x8 ak = *reinterpret_cast<const bf16x8*>(&sK[(32 * kt + l32) * LD + 16 * c + 8 * hh]);
        const bf16x8 av = *reinterpret_cast<const bf16x8*>(&sV[(32 * kt + l32) * LD + 16 * c + 8 * hh]);
        s[kt] = mfma32(ak, qreg[c], s[kt]);
        dp[kt] = mfma32(av, oreg[c], dp[kt]);
      }
    }
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const float p = __builtin_amdgcn_exp2f(__builtin_fmaf(s[kt][e], scale_log2, -lse2));
        dp[kt][e] = p * (dp[kt][e] - dvec);
      }
    // dQ^T[c][i] += K^T[c][m] dS^T[m][i]
#pragma unroll
    for (int kc = 0; kc < 4; ++kc) {
      const f16x8 db = pack_f16(dp[kc >> 1], kc & 1);
#pragma unroll
      for (int c = 0; c < D / 32; ++c)
        acc[c] = mfma32h(lds_pair_b64_h(&sKt[(32 * c + l32) * TLD + 16 * kc + 4 * hh]), db, acc[c]);
    }
  }

  float* orow = dQ + qrow * D;
#pragma unroll
  for (int c = 0; c < D / 32; ++c)
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4) {
      float4 v = make_float4(acc[c][4 * q4] * tau, acc[c][4 * q4 + 1] * tau, acc[c][4 * q4 + 2] * tau,
                             acc[c][4 * q4 + 3] * tau);
      *reinterpret_cast<float4*>(orow + 32 * c + 8 * q4 + 4 * hh) = v;
    }
}

template <int D>
hipError_t pre_launch(const Shape& s, const float* O, const bf16_t* dO, float* Dvec, hipStream_t st) {
  const int64_t rows = (int64_t)s.B * s.H * s.N;
  constexpr int RPB = 256 / (D / 8);
  const int64_t nwg = (rows + RPB - 1) / RPB;
  hipLaunchKernelGGL(bwd_pre_kernel<D>, dim3((unsigned)(nwg < 65536 ? nwg : 65536)), dim3(256), 0, st, dO, O, Dvec,
                     rows);
  return hipGetLastError();
}

template <int D, int G>
hipError_t dkdv_launch(const Shape& s, const bf16_t* Q, const bf16_t* K, const bf16_t* V, const bf16_t* dO,
                       const float* LSE, const float* Dvec, const int32_t* rev_ptr, const int32_t* rev_idx, float* dK,
                       float* dV, const HeadTable& ht, hipStream_t st) {
  const float tau = 1.0f / sqrtf((float)D);
  hipLaunchKernelGGL((bwd_dkdv_kernel<D, G>), dim3((unsigned)(s.NB * s.H * s.B)), dim3(128), 0, st, Q, K, V, dO, LSE,
                     Dvec, rev_ptr, rev_idx, dK, dV, ht, s.N, s.H, s.NB, s.B, tau * kLog2e, tau);
  return hipGetLastError();
}

template <int D, int G>
hipError_t dq_launch(const Shape& s, const bf16_t* Q, const bf16_t* K, const bf16_t* V, const bf16_t* dO,
                     const float* LSE, const float* Dvec, const int32_t* idx, float* dQ, const HeadTable& ht,
                     hipStream_t st) {
  const float tau = 1.0f / sqrtf((float)D);
  hipLaunchKernelGGL((bwd_dq_kernel<D, G>), dim3((unsigned)(s.NG * s.H * s.B)), dim3(G * 2), 0, st, Q, K, V, dO, LSE,
                     Dvec, idx, dQ, ht, s.N, s.H, s.B, tau * kLog2e, tau);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_bwd_pre(const Shape& s, const float* O, const void* dO, float* Dvec, hipStream_t st) {
  const bf16_t* o = static_cast<const bf16_t*>(dO);
  return s.D == 64 ? pre_launch<64>(s, O, o, Dvec, st) : pre_launch<128>(s, O, o, Dvec, st);
}

hipError_t launch_bwd_dkdv(const Shape& s, const void* Q, const void* K, const void* V, const void* dO,
                           const float* LSE, const float* Dvec, const int32_t* rev_ptr, const int32_t* rev_idx,
                           float* dK, float* dV, const HeadTable& ht, hipStream_t st) {
  const bf16_t* q = static_cast<const bf16_t*>(Q);
  const bf16_t* k = static_cast<const bf16_t*>(K);
  const bf16_t* v = static_cast<const bf16_t*>(V);
  const bf16_t* o = static_cast<const bf16_t*>(dO);
  if (s.D == 64)
    return s.G == 64 ? dkdv_launch<64, 64>(s, q, k, v, o, LSE, Dvec, rev_ptr, rev_idx, dK, dV, ht, st)
                     : dkdv_launch<64, 128>(s, q, k, v, o, LSE, Dvec, rev_ptr, rev_idx, dK, dV, ht, st);
  return s.G == 64 ? dkdv_launch<128, 64>(s, q, k, v, o, LSE, Dvec, rev_ptr, rev_idx, dK, dV, ht, st)
                   : dkdv_launch<128, 128>(s, q, k, v, o, LSE, Dvec, rev_ptr, rev_idx, dK, dV, ht, st);
}

hipError_t launch_bwd_dq(const Shape& s, const void* Q, const void* K, const void* V, const void* dO,
                         const float* LSE, const float* Dvec, const int32_t* idx, float* dQ, const HeadTable& ht,
                         hipStream_t st) {
  const bf16_t* q = static_cast<const bf16_t*>(Q);
  const bf16_t* k = static_cast<const bf16_t*>(K);
  const bf16_t* v = static_cast<const bf16_t*>(V);
  const bf16_t* o = static_cast<const bf16_t*>(dO);
  if (s.D == 64)
    return s.G == 64 ? dq_launch<64, 64>(s, q, k, v, o, LSE, Dvec, idx, dQ, ht, st)
                     : dq_launch<64, 128>(s, q, k, v, o, LSE, Dvec, idx, dQ, ht, st);
  return s.G == 64 ? dq_launch<128, 64>(s, q, k, v, o, LSE, Dvec, idx, dQ, ht, st)
                   : dq_launch<128, 128>(s, q, k, v, o, LSE, Dvec, idx, dQ, ht, st);
}

}  // namespace dsa
