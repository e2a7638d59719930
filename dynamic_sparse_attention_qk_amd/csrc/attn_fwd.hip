// Sparse attention forward over the kept KV blocks.
//
// DSV (gist.science explainer, hi edition) technical summary §2.A stage 2:
// only the critical subset of KV pairs is computed; §2.B query grouping: a
// whole query group shares one kept-block list, which gives dense, coalesced
// tiles for the matrix cores.
//
// One workgroup per (b, h, query group); G/32 waves, each owning 32 query rows.
// For every kept block the 64 x d K tile (row-major) and V tile (transposed,
// V^T[c][m]) are staged in LDS; the next block's tiles are prefetched into
// registers while the current one is computed.  Per wave and block:
//   S^T = K Q^T     (A = K rows from LDS, B = the wave's Q rows in registers)
//   online softmax in the exp2 domain; each lane owns one query row, so row
//   statistics need one cross-lane step (lane l and l^32)
//   O^T += V^T P^T  (A = V^T from LDS, B = P packed from the S accumulators)
// O^T accumulators keep lane <-> query, so the per-row rescale is lane-local.
#include "launch.hpp"

namespace dsa {

namespace {

template <int D, int G>
__global__ __launch_bounds__(G * 2) void attn_fwd_bf16_kernel(const bf16_t* __restrict__ Q,
                                                              const bf16_t* __restrict__ K,
                                                              const bf16_t* __restrict__ V,
                                                              const int32_t* __restrict__ idx, float* __restrict__ O,
                                                              float* __restrict__ LSE, HeadTable ht, int N, int H,
                                                              int B, float scale_log2) {
  constexpr int NT = G * 2;      // G/32 waves
  constexpr int KLD = kRowLd<D>;
  constexpr int VLD = kColLd;
  __shared__ __attribute__((aligned(16))) bf16_t sK[64 * KLD];
  __shared__ __attribute__((aligned(16))) uint16_t sVt[D * VLD];  // fp16

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
  const int qrow = g * G + wave * 32 + l32;

  bf16x8 qreg[D / 16];
  {
    const bf16_t* qp = Q + (bh * N + qrow) * (size_t)D + 8 * hh;
#pragma unroll
    for (int t = 0; t < D / 16; ++t) qreg[t] = *reinterpret_cast<const bf16x8*>(qp + 16 * t);
  }

  const int NB = N / kBlock;
  // block ids are valid by contract; clamping keeps a bad list from reading out of bounds
  auto block_id = [&](int t) { return min(max(irow[t], 0), NB - 1); };
  TileMover<D, NT> kt, vt;
  {
    const int j = block_id(0);
    kt.load(Kbh + (size_t)j * kBlock * D);
    vt.load(Vbh + (size_t)j * kBlock * D);
  }

  float m_run = -INFINITY, l_run = 0.f;
  f32x16 oacc[D / 32];
#pragma unroll
  for (int c = 0; c < D / 32; ++c) oacc[c] = f32x16{};

  for (int t = 0; t < k; ++t) {
    __syncthreads();
    kt.store_rows(sK);
    vt.store_cols_f16(sVt);
    __syncthreads();
    if (t + 1 < k) {
      const int j = block_id(t + 1);
      kt.load(Kbh + (size_t)j * kBlock * D);
      vt.load(Vbh + (size_t)j * kBlock * D);
    }
    // S^T tiles: keys 0..31 and 32..63 of the block against the wave's 32 queries
    f32x16 s0 = f32x16{}, s1 = f32x16{};
#pragma unroll
    for (int c = 0; c < D / 16; ++c) {
      const bf16x8 a0 = *reinterpret_cast<const bf16x8*>(&sK[l32 * KLD + 16 * c + 8 * hh]);
      const bf16x8 a1 = *reinterpret_cast<const bf16x8*>(&sK[(32 + l32) * KLD + 16 * c + 8 * hh]);
      s0 = mfma32(a0, qreg[c], s0);
      s1 = mfma32(a1, qreg[c], s1);
    }
    float mx = s0[0];
#pragma unroll
    for (int e = 0; e < 16; ++e) mx = fmaxf(mx, fmaxf(s0[e], s1[e]));
    mx = wave_max_pair(mx) * scale_log2;
    const float m_new = fmaxf(m_run, mx);
    const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
    float rs = 0.f;
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      s0[e] = __builtin_amdgcn_exp2f(__builtin_fmaf(s0[e], scale_log2, -m_new));
      s1[e] = __builtin_amdgcn_exp2f(__builtin_fmaf(s1[e], scale_log2, -m_new));
      rs += s0[e] + s1[e];
    }
    l_run = l_run * alpha + rs;
    m_run = m_new;
#pragma unroll
    for (int c = 0; c < D / 32; ++c) oacc[c] *= alpha;
    const f16x8 p0 = pack_f16(s0, 0), p1 = pack_f16(s0, 1), p2 = pack_f16(s1, 0), p3 = pack_f16(s1, 1);
#pragma unroll
    for (int c = 0; c < D / 32; ++c) {
      const uint16_t* vrow = &sVt[(32 * c + l32) * VLD + 4 * hh];
      oacc[c] = mfma32h(lds_pair_b64_h(vrow + 0), p0, oacc[c]);
      oacc[c] = mfma32h(lds_pair_b64_h(vrow + 16), p1, oacc[c]);
      oacc[c] = mfma32h(lds_pair_b64_h(vrow + 32), p2, oacc[c]);
      oacc[c] = mfma32h(lds_pair_b64_h(vrow + 48), p3, oacc[c]);
    }
  }

  const float l_tot = l_run + __shfl_xor(l_run, 32);
  const float inv = 1.0f / l_tot;
  float* orow = O + (bh * N + qrow) * (size_t)D;
#pragma unroll
  for (int c = 0; c < D / 32; ++c)
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4) {
      float4 v = make_float4(oacc[c][4 * q4] * inv, oacc[c][4 * q4 + 1] * inv, oacc[c][4 * q4 + 2] * inv,
                             oacc[c][4 * q4 + 3] * inv);
      *reinterpret_cast<float4*>(orow + 32 * c + 8 * q4 + 4 * hh) = v;
    }
  if (hh == 0) LSE[bh * N + qrow] = (m_run + __log2f(l_tot)) * kLn2;
}

// fp32 operands: v_mfma_f32_32x32x2_f32, K and V row-major in LDS.
template <int D, int G>
__global__ __launch_bounds__(G * 2) void attn_fwd_f32_kernel(const float* __restrict__ Q, const float* __restrict__ K,
                                                             const float* __restrict__ V,
                                                             const int32_t* __restrict__ idx, float* __restrict__ O,
                                                             float* __restrict__ LSE, HeadTable ht, int N, int H,
                                                             int B, float scale_log2) {
  constexpr int NT = G * 2;
  constexpr int LD = D + 1;
  __shared__ float sK[64 * LD];
  __shared__ float sV[64 * LD];

  const int NG = N / G;
  const uint32_t L = xcd_remap(blockIdx.x, (uint32_t)(NG * H * B));
  const int g = L % NG, h = (L / NG) % H, b = L / (NG * H);
  const int k = ht.k[h];
  const int32_t* irow = idx + row_base(ht, b, h, NG) + (int64_t)g * k;
  const size_t bh = (size_t)b * H + h;
  const float* Kbh = K + bh * (size_t)N * D;
  const float* Vbh = V + bh * (size_t)N * D;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int l32 = lane & 31, hh = lane >> 5;
  const int qrow = g * G + wave * 32 + l32;

  float qreg[D / 2];
  {
    const float* qp = Q + (bh * N + qrow) * (size_t)D + hh;
#pragma unroll
    for (int t = 0; t < D / 2; ++t) qreg[t] = qp[2 * t];
  }

  float m_run = -INFINITY, l_run = 0.f;
  f32x16 oacc[D / 32];
#pragma unroll
  for (int c = 0; c < D / 32; ++c) oacc[c] = f32x16{};

  const int NB = N / kBlock;
  for (int t = 0; t < k; ++t) {
    const int j = min(max(irow[t], 0), NB - 1);
    __syncthreads();
    for (int e = threadIdx.x; e < 64 * D; e += NT) {
      const int m = e / D, c = e % D;
      sK[m * LD + c] = Kbh[((size_t)j * kBlock + m) * D + c];
      sV[m * LD + c] = Vbh[((size_t)j * kBlock + m) * D + c];
    }
    __syncthreads();
    f32x16 s0 = f32x16{}, s1 = f32x16{};
#pragma unroll
    for (int c = 0; c < D / 2; ++c) {
      s0 = mfma32_f32(sK[l32 * LD + 2 * c + hh], qreg[c], s0);
      s1 = mfma32_f32(sK[(32 + l32) * LD + 2 * c + hh], qreg[c], s1);
    }
    float mx = s0[0];
#pragma unroll
    for (int e = 0; e < 16; ++e) mx = fmaxf(mx, fmaxf(s0[e], s1[e]));
    mx = wave_max_pair(mx) * scale_log2;
    const float m_new = fmaxf(m_run, mx);
    const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
    float rs = 0.f;
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      s0[e] = __builtin_amdgcn_exp2f(__builtin_fmaf(s0[e], scale_log2, -m_new));
      s1[e] = __builtin_amdgcn_exp2f(__builtin_fmaf(s1[e], scale_log2, -m_new));
      rs += s0[e] + s1[e];
    }
    l_run = l_run * alpha + rs;
    m_run = m_new;
#pragma unroll
    for (int c = 0; c < D / 32; ++c) oacc[c] *= alpha;
    // O^T[c][i] += sum over 2-key chunks: lane half hh supplies key 8*(e/4) + 4*hh + e%4 (+32 for s1)
#pragma unroll
    for (int c = 0; c < D / 32; ++c)
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int m = 8 * (e / 4) + 4 * hh + (e % 4);
        oacc[c] = mfma32_f32(sV[m * LD + 32 * c + l32], s0[e], oacc[c]);
        oacc[c] = mfma32_f32(sV[(32 + m) * LD + 32 * c + l32], s1[e], oacc[c]);
      }
  }

  const float l_tot = l_run + __shfl_xor(l_run, 32);
  const float inv = 1.0f / l_tot;
  float* orow = O + (bh * N + qrow) * (size_t)D;
#pragma unroll
  for (int c = 0; c < D / 32; ++c)
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4) {
      float4 v = make_float4(oacc[c][4 * q4] * inv, oacc[c][4 * q4 + 1] * inv, oacc[c][4 * q4 + 2] * inv,
                             oacc[c][4 * q4 + 3] * inv);
      *reinterpret_cast<float4*>(orow + 32 * c + 8 * q4 + 4 * hh) = v;
    }
  if (hh == 0) LSE[bh * N + qrow] = (m_run + __log2f(l_tot)) * kLn2;
}

template <int D, int G>
hipError_t fwd_launch(const Shape& s, const void* Q, const void* K, const void* V, const int32_t* idx, float* O,
                      float* LSE, const HeadTable& ht, hipStream_t st) {
  const float scale_log2 = (1.0f / sqrtf((float)D)) * kLog2e;
  dim3 grid((unsigned)(s.NG * s.H * s.B));
  if (s.bf16)
    hipLaunchKernelGGL((attn_fwd_bf16_kernel<D, G>), grid, dim3(G * 2), 0, st, static_cast<const bf16_t*>(Q),
                       static_cast<const bf16_t*>(K), static_cast<const bf16_t*>(V), idx, O, LSE, ht, s.N, s.H,
                       s.B, scale_log2);
  else
    hipLaunchKernelGGL((attn_fwd_f32_kernel<D, G>), grid, dim3(G * 2), 0, st, static_cast<const float*>(Q),
                       static_cast<const float*>(K), static_cast<const float*>(V), idx, O, LSE, ht, s.N, s.H,
                       s.B, scale_log2);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_attn_fwd(const Shape& s, const void* Q, const void* K, const void* V, const int32_t* idx, float* O,
                           float* LSE, const HeadTable& ht, hipStream_t st) {
  if (s.D == 64) return s.G == 64 ? fwd_launch<64, 64>(s, Q, K, V, idx, O, LSE, ht, st) : fwd_launch<64, 128>(s, Q, K, V, idx, O, LSE, ht, st);
  if (s.D == 128) return s.G == 64 ? fwd_launch<128, 64>(s, Q, K, V, idx, O, LSE, ht, st) : fwd_launch<128, 128>(s, Q, K, V, idx, O, LSE, ht, st);
  return hipErrorInvalidValue;
}

}  // namespace dsa
