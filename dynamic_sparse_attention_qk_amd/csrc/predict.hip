// Low-rank sparsity predictor: pooled proxy query / block key projection and
// block scores.  DSV (gist.science explainer, hi edition) technical summary
// §2.A: per-head predictors W^Q_lr, W^K_lr estimate QK^T through an r << d
// projection; §2.B query grouping: one proxy per query group.
//
// pool_project is bound by HBM: it streams Q (or K) once, 16-byte coalesced,
// and writes r floats per group.  block_scores writes NG x NB fp32 scores per
// (b, h) with coalesced rows.
#include "launch.hpp"

namespace dsa {

namespace {

constexpr int kPoolThreads = 256;
constexpr int kPoolGroupsPerWG = 8;  // 2 rounds of 4 waves

template <typename T, int D, int R>
__global__ __launch_bounds__(kPoolThreads) void pool_project_kernel(const T* __restrict__ X,
                                                                     const float* __restrict__ W,
                                                                     float* __restrict__ out,
                                                                     float* __restrict__ mean_out, int N, int P,
                                                                     int H) {
  constexpr int VE = 16 / sizeof(T);  // elements per 16-byte vector
  constexpr int VR = D / VE;          // vectors per row
  constexpr int RP = 64 / VR;         // rows covered by one wave-wide load
  constexpr int PARTS = 64 / R;       // lanes sharing one output column in the projection
  __shared__ float sW[D * R];
  __shared__ float smean[4][D];

  const int b = blockIdx.z, h = blockIdx.y;
  const int npool = N / P;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const float* Wh = W + (size_t)h * D * R;
  for (int i = threadIdx.x * 4; i < D * R; i += kPoolThreads * 4)
    *reinterpret_cast<float4*>(&sW[i]) = *reinterpret_cast<const float4*>(&Wh[i]);

  const size_t bh = (size_t)b * H + h;
  const T* Xbh = X + bh * (size_t)N * D;
  float* obh = out + bh * (size_t)npool * R;
  const int cv = lane % VR, r0 = lane / VR;
  const float inv = 1.0f / (float)P;

  for (int round = 0; round < kPoolGroupsPerWG; round += 4) {
    const int g = blockIdx.x * kPoolGroupsPerWG + round + wave;
    const bool valid = g < npool;
    if (valid) {
      float acc[VE];
#pragma unroll
      for (int e = 0; e < VE; ++e) acc[e] = 0.f;
      const T* base = Xbh + (size_t)g * P * D + cv * VE;
#pragma unroll 8
      for (int row = r0; row < P; row += RP) {
        uint4 v = ldg16(base + (size_t)row * D);
        if constexpr (sizeof(T) == 2) {
          const uint32_t* w = reinterpret_cast<const uint32_t*>(&v);
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            acc[2 * q] += __uint_as_float(w[q] << 16);
            acc[2 * q + 1] += __uint_as_float(w[q] & 0xFFFF0000u);
          }
        } else {
          const float* f = reinterpret_cast<const float*>(&v);
#pragma unroll
          for (int q = 0; q < 4; ++q) acc[q] += f[q];
        }
      }
#pragma unroll
      for (int off = VR; off < 64; off <<= 1)
#pragma unroll
        for (int e = 0; e < VE; ++e) acc[e] += __shfl_xor(acc[e], off);
      if (r0 == 0) {
#pragma unroll
        for (int e = 0; e < VE; ++e) smean[wave][cv * VE + e] = acc[e] * inv;
        if (mean_out) {
          float* mo = mean_out + (bh * npool + g) * D + cv * VE;
#pragma unroll
          for (int e = 0; e < VE; e += 4)
            *reinterpret_cast<float4*>(mo + e) = make_float4(acc[e] * inv, acc[e + 1] * inv, acc[e + 2] * inv,
                                                             acc[e + 3] * inv);
        }
      }
    }
    __syncthreads();
    if (valid) {
      const int rr = lane % R, part = lane / R;
      constexpr int CSPAN = D / PARTS;
      float s = 0.f;
#pragma unroll 8
      for (int c = part * CSPAN; c < (part + 1) * CSPAN; ++c) s = __builtin_fmaf(smean[wave][c], sW[c * R + rr], s);
#pragma unroll
      for (int off = R; off < 64; off <<= 1) s += __shfl_xor(s, off);
      if (part == 0) obh[(size_t)g * R + rr] = s;
    }
    __syncthreads();
  }
}

constexpr int kScoreRows = 32;   // query groups per workgroup
constexpr int kScoreCols = 256;  // KV blocks per workgroup, one per thread

// scores[b,h,g,j] for a 32 x 256 tile: the 32 q-hat rows sit in LDS (read as
// broadcasts), each thread keeps its k-hat row in registers and writes one
// coalesced column of the tile.  score_dot's fixed fma chain makes the values
// bit-identical to the ones the streamed selection recomputes.
template <int R>
__global__ __launch_bounds__(kScoreCols) void block_scores_kernel(const float* __restrict__ qhat,
                                                                   const float* __restrict__ khat,
                                                                   float* __restrict__ scores, int NG, int NB,
                                                                   float tau) {
  __shared__ float sq[kScoreRows][R];
  const int ncx = (NB + kScoreCols - 1) / kScoreCols;
  const size_t bh = (size_t)blockIdx.z * gridDim.y + blockIdx.y;
  const int g0 = (blockIdx.x / ncx) * kScoreRows;
  const int j = (blockIdx.x % ncx) * kScoreCols + threadIdx.x;
  const float* qbh = qhat + bh * (size_t)NG * R;
  const float* kbh = khat + bh * (size_t)NB * R;
  float* sbh = scores + bh * (size_t)NG * NB;
  for (int t = threadIdx.x; t < kScoreRows * R; t += kScoreCols) {
    const int row = t / R, r = t % R;
    sq[row][r] = (g0 + row < NG) ? qbh[(size_t)(g0 + row) * R + r] : 0.f;
  }
  float kr[R];
  if (j < NB) {
#pragma unroll
    for (int r = 0; r < R; r += 4) {
      const float4 v = *reinterpret_cast<const float4*>(kbh + (size_t)j * R + r);
      kr[r] = v.x;
      kr[r + 1] = v.y;
      kr[r + 2] = v.z;
      kr[r + 3] = v.w;
    }
  }
  __syncthreads();
  if (j >= NB) return;
  const int rows = min(kScoreRows, NG - g0);
  for (int row = 0; row < rows; ++row) sbh[(size_t)(g0 + row) * NB + j] = score_dot<R>(sq[row], kr, tau);
}

template <typename T, int D>
hipError_t pool_dispatch_r(const Shape& s, const T* X, const float* W, float* out, float* mean_out, int pool,
                           hipStream_t st) {
  const int npool = s.N / pool;
  dim3 grid((npool + kPoolGroupsPerWG - 1) / kPoolGroupsPerWG, s.H, s.B);
  dim3 blk(kPoolThreads);
  switch (s.R) {
    case 8: hipLaunchKernelGGL((pool_project_kernel<T, D, 8>), grid, blk, 0, st, X, W, out, mean_out, s.N, pool, s.H); break;
    case 16: hipLaunchKernelGGL((pool_project_kernel<T, D, 16>), grid, blk, 0, st, X, W, out, mean_out, s.N, pool, s.H); break;
    case 32: hipLaunchKernelGGL((pool_project_kernel<T, D, 32>), grid, blk, 0, st, X, W, out, mean_out, s.N, pool, s.H); break;
    case 64: hipLaunchKernelGGL((pool_project_kernel<T, D, 64>), grid, blk, 0, st, X, W, out, mean_out, s.N, pool, s.H); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_pool_project(const Shape& s, const void* X, const float* W, float* out, int pool,
                               hipStream_t st, float* mean_out) {
  if (s.bf16) {
    const bf16_t* x = static_cast<const bf16_t*>(X);
    return s.D == 64 ? pool_dispatch_r<bf16_t, 64>(s, x, W, out, mean_out, pool, st)
                     : pool_dispatch_r<bf16_t, 128>(s, x, W, out, mean_out, pool, st);
  }
  const float* x = static_cast<const float*>(X);
  return s.D == 64 ? pool_dispatch_r<float, 64>(s, x, W, out, mean_out, pool, st)
                   : pool_dispatch_r<float, 128>(s, x, W, out, mean_out, pool, st);
}

hipError_t launch_block_scores(const Shape& s, const float* qhat, const float* khat, float* scores, float tau,
                               hipStream_t st) {
  dim3 grid((unsigned)(((s.NB + kScoreCols - 1) / kScoreCols) * ((s.NG + kScoreRows - 1) / kScoreRows)), s.H, s.B);
  switch (s.R) {
    case 8: hipLaunchKernelGGL(block_scores_kernel<8>, grid, dim3(kScoreCols), 0, st, qhat, khat, scores, s.NG, s.NB, tau); break;
    case 16: hipLaunchKernelGGL(block_scores_kernel<16>, grid, dim3(kScoreCols), 0, st, qhat, khat, scores, s.NG, s.NB, tau); break;
    case 32: hipLaunchKernelGGL(block_scores_kernel<32>, grid, dim3(kScoreCols), 0, st, qhat, khat, scores, s.NG, s.NB, tau); break;
    case 64: hipLaunchKernelGGL(block_scores_kernel<64>, grid, dim3(kScoreCols), 0, st, qhat, khat, scores, s.NG, s.NB, tau); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace dsa
