// Stage-1 training of the low-rank predictor: loss and gradient with respect
// to W_q and W_k.  DSV (gist.science explainers, hi and nl editions) technical
// summary §2.A, stage 1: the per-head predictors are trained next to the full
// attention of normal training, by a loss that keeps the relative magnitude of
// the estimated scores.
//
// Per (b, h), with qbar/kbar the group/block means of Q/K, qhat = qbar W_q,
// khat = kbar W_k:
//   diff[g, j] = tau (qhat_g . khat_j - qbar_g . kbar_j)   (block score minus
//                the mean of tau Q K^T over the G x 64 tile)
//   E[g, j]    = diff[g, j] - mean_j diff[g, j]            (row-centred)
//   L          = mean over (b, g, j) of E^2                (per head)
//   dW_q = 2 tau / (B NG NB) sum_b qbar^T (E khat),  dW_k = 2 tau / (B NG NB) sum_b kbar^T (E^T qhat)
//
// Seven launches, all deterministic (fixed summation orders, no atomics):
//   pool_project_kernel (predict.hip) x2 with mean output: qbar, qhat; kbar, khat   HBM: reads Q, K once
//   pred_diff_kernel: diff, 32 x 256 tiles, one column per thread                   ALU (d + r fma per entry)
//   pred_rows_kernel: four rows per wave: centre E in place, row sums of E^2, Y = E khat
//   pred_cols_kernel: 64 columns per workgroup: Z = E^T qhat
//   pred_wgrad_kernel: the d x r outer-product sums over 16 row ranges per (head, W_q or W_k)
//   pred_wreduce_kernel: the 16 partials added in order, scaled; the loss
#include "launch.hpp"

namespace dsa {

namespace {

constexpr int kDiffRows = 32;   // query groups per workgroup
constexpr int kDiffCols = 256;  // KV blocks per workgroup, one per thread

// diff for a 32 x 256 tile: the rows' [qhat | qbar] sit in LDS (broadcast reads); each thread owns one
// column j and walks its [khat | -kbar] in chunks of 32 values, accumulating all 32 rows in registers.
template <int D, int R>
__global__ __launch_bounds__(kDiffCols) void pred_diff_kernel(const float* __restrict__ qbar,
                                                               const float* __restrict__ kbar,
                                                               const float* __restrict__ qhat,
                                                               const float* __restrict__ khat,
                                                               float* __restrict__ diff, int NG, int NB, float tau) {
  constexpr int L = R + D;
  constexpr int CH = R < 32 ? R : 32;  // chunk of the concatenated dimension (divides R and D)
  __shared__ float su[kDiffRows][L];
  const int ncx = (NB + kDiffCols - 1) / kDiffCols;
  const size_t bh = (size_t)blockIdx.z * gridDim.y + blockIdx.y;
  const int g0 = (blockIdx.x / ncx) * kDiffRows;
  const int j = (blockIdx.x % ncx) * kDiffCols + threadIdx.x;
  for (int t = threadIdx.x; t < kDiffRows * L; t += kDiffCols) {
    const int row = t / L, c = t % L, g = g0 + row;
    float v = 0.f;
    if (g < NG) v = c < R ? qhat[(bh * NG + g) * R + c] : qbar[(bh * NG + g) * D + (c - R)];
    su[row][c] = v;
  }
  __syncthreads();
  if (j >= NB) return;
  const float* kh = khat + (bh * NB + j) * R;
  const float* kb = kbar + (bh * NB + j) * D;
  float acc[kDiffRows];
#pragma unroll
  for (int row = 0; row < kDiffRows; ++row) acc[row] = 0.f;
  for (int c0 = 0; c0 < L; c0 += CH) {
    float v[CH];
#pragma unroll
    for (int c = 0; c < CH; c += 4) {
      const bool hat = c0 < R;
      const float4 x = *reinterpret_cast<const float4*>(hat ? kh + c0 + c : kb + (c0 - R) + c);
      const float sg = hat ? 1.f : -1.f;
      v[c] = sg * x.x, v[c + 1] = sg * x.y, v[c + 2] = sg * x.z, v[c + 3] = sg * x.w;
    }
#pragma unroll
    for (int row = 0; row < kDiffRows; ++row)
#pragma unroll
      for (int c = 0; c < CH; ++c) acc[row] = __builtin_fmaf(su[row][c0 + c], v[c], acc[row]);
  }
  const int rows = min(kDiffRows, NG - g0);
  for (int row = 0; row < rows; ++row) diff[(bh * NG + g0 + row) * NB + j] = acc[row] * tau;
}

__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) x += __shfl_xor(x, off);
  return x;
}

constexpr int kRowsPerWave = 4;

// Each wave takes 4 consecutive (b, h, g) rows of one (b, h) (NG is a multiple of 4 only when it is; a
// row beyond the (b, h) is skipped): E = diff - row mean (in place), lrow = sum_j E^2,
// Y_g = sum_j E_gj khat_j.  The four rows share every khat load.
template <int R>
__global__ __launch_bounds__(256) void pred_rows_kernel(float* __restrict__ E, const float* __restrict__ khat,
                                                        float* __restrict__ Y, float* __restrict__ lrow, int BH,
                                                        int NG, int NB) {
  constexpr int W = kRowsPerWave;
  const int lane = threadIdx.x & 63;
  const int per_bh = (NG + W - 1) / W;  // waves per (b, h)
  const int64_t wv = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (wv >= (int64_t)BH * per_bh) return;
  const int64_t bh = wv / per_bh;
  const int g0 = (int)(wv % per_bh) * W;
  const int nr = min(W, NG - g0);
  float* e0 = E + (bh * NG + g0) * NB;
  const float* kbh = khat + bh * NB * R;
  float mu[W];
#pragma unroll
  for (int i = 0; i < W; ++i) {
    float s = 0.f;
    if (i < nr)
      for (int j = lane; j < NB; j += 64) s += e0[(int64_t)i * NB + j];
    mu[i] = wave_sum(s) / (float)NB;
  }
  float y[W][R];
  float l[W];
#pragma unroll
  for (int i = 0; i < W; ++i) {
    l[i] = 0.f;
#pragma unroll
    for (int r = 0; r < R; ++r) y[i][r] = 0.f;
  }
  for (int j = lane; j < NB; j += 64) {
    float e[W];
#pragma unroll
    for (int i = 0; i < W; ++i) {
      e[i] = 0.f;
      if (i < nr) {
        e[i] = e0[(int64_t)i * NB + j] - mu[i];
        e0[(int64_t)i * NB + j] = e[i];
      }
      l[i] = __builtin_fmaf(e[i], e[i], l[i]);
    }
    const float* kh = kbh + (int64_t)j * R;
#pragma unroll
    for (int r = 0; r < R; r += 4) {
      const float4 x = *reinterpret_cast<const float4*>(kh + r);
#pragma unroll
      for (int i = 0; i < W; ++i) {
        y[i][r] = __builtin_fmaf(e[i], x.x, y[i][r]);
        y[i][r + 1] = __builtin_fmaf(e[i], x.y, y[i][r + 1]);
        y[i][r + 2] = __builtin_fmaf(e[i], x.z, y[i][r + 2]);
        y[i][r + 3] = __builtin_fmaf(e[i], x.w, y[i][r + 3]);
      }
    }
  }
#pragma unroll
  for (int i = 0; i < W; ++i) {
    const float li = wave_sum(l[i]);
    float out = 0.f;
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const float t = wave_sum(y[i][r]);
      if (lane == r) out = t;
    }
    if (i < nr) {
      if (lane < R) Y[(bh * NG + g0 + i) * R + lane] = out;
      if (lane == 0) lrow[bh * NG + g0 + i] = li;
    }
  }
}

// Z_j = sum_g E_gj qhat_g for 64 columns: wave w sums the rows g = w (mod 4); wave 0 then adds the other
// three partials in wave order and writes the rows of Z.
template <int R>
__global__ __launch_bounds__(256) void pred_cols_kernel(const float* __restrict__ E, const float* __restrict__ qhat,
                                                        float* __restrict__ Z, int NG, int NB) {
  __shared__ float part[3][R][64];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const size_t bh = (size_t)blockIdx.z * gridDim.y + blockIdx.y;
  const int j = blockIdx.x * 64 + lane;
  const bool ok = j < NB;
  const float* ebh = E + bh * NG * NB;
  const float* qbh = qhat + bh * NG * R;
  float z[R];
#pragma unroll
  for (int r = 0; r < R; ++r) z[r] = 0.f;
  for (int g = wave; g < NG; g += 4) {
    const float e = ok ? ebh[(size_t)g * NB + j] : 0.f;
    const float* q = qbh + (size_t)g * R;
#pragma unroll
    for (int r = 0; r < R; ++r) z[r] = __builtin_fmaf(e, q[r], z[r]);
  }
  if (wave > 0)
#pragma unroll
    for (int r = 0; r < R; ++r) part[wave - 1][r][lane] = z[r];
  __syncthreads();
  if (wave > 0 || !ok) return;
  float* zr = Z + (bh * NB + j) * R;
#pragma unroll
  for (int r = 0; r < R; r += 4) {
    float o[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) o[u] = ((z[r + u] + part[0][r + u][lane]) + part[1][r + u][lane]) + part[2][r + u][lane];
    *reinterpret_cast<float4*>(zr + r) = make_float4(o[0], o[1], o[2], o[3]);
  }
}

constexpr int kWgChunk = 16;  // rows staged in LDS per round
constexpr int kWgParts = kPredWgParts;  // workgroups per (head, matrix); their partials are added in order

// blockIdx.y == 0: partial dW_q of head h = blockIdx.x from (qbar, Y) over part blockIdx.z of the B NG
// group rows; blockIdx.y == 1: partial dW_k from (kbar, Z) over the B NB block rows.  Thread t owns
// entries t + 256 i of the d x r matrix.  Partials: [H][2][kWgParts][d r].
template <int D, int R>
__global__ __launch_bounds__(256) void pred_wgrad_kernel(const float* __restrict__ qbar,
                                                          const float* __restrict__ Y,
                                                          const float* __restrict__ kbar,
                                                          const float* __restrict__ Z, float* __restrict__ part,
                                                          int B, int H, int NG, int NB) {
  constexpr int NE = (D * R + 255) / 256;
  __shared__ float sx[kWgChunk][D];
  __shared__ float sy[kWgChunk][R];
  const int h = blockIdx.x;
  const bool is_q = blockIdx.y == 0;
  const int nrow = is_q ? NG : NB;
  const float* X = is_q ? qbar : kbar;
  const float* G = is_q ? Y : Z;
  // this part's rows of the (b, row) sequence, in order
  const int64_t total = (int64_t)B * nrow;
  const int64_t p0 = total * blockIdx.z / kWgParts, p1 = total * (blockIdx.z + 1) / kWgParts;
  float acc[NE];
#pragma unroll
  for (int i = 0; i < NE; ++i) acc[i] = 0.f;
  for (int64_t r0 = p0; r0 < p1; r0 += kWgChunk) {
    const int nr = (int)min((int64_t)kWgChunk, p1 - r0);
    __syncthreads();
    for (int t = threadIdx.x; t < kWgChunk * D; t += 256) {
      const int rr = t / D, c = t % D;
      float v = 0.f;
      if (rr < nr) {
        const int64_t q = r0 + rr, b = q / nrow, row = q % nrow;
        v = X[(((size_t)b * H + h) * nrow + row) * D + c];
      }
      sx[rr][c] = v;
    }
    for (int t = threadIdx.x; t < kWgChunk * R; t += 256) {
      const int rr = t / R, c = t % R;
      float v = 0.f;
      if (rr < nr) {
        const int64_t q = r0 + rr, b = q / nrow, row = q % nrow;
        v = G[(((size_t)b * H + h) * nrow + row) * R + c];
      }
      sy[rr][c] = v;
    }
    __syncthreads();
    for (int rr = 0; rr < nr; ++rr)
#pragma unroll
      for (int i = 0; i < NE; ++i) {
        const int e = threadIdx.x + 256 * i;
        if (e < D * R) acc[i] = __builtin_fmaf(sx[rr][e / R], sy[rr][e % R], acc[i]);
      }
  }
  float* out = part + (((size_t)h * 2 + blockIdx.y) * kWgParts + blockIdx.z) * D * R;
#pragma unroll
  for (int i = 0; i < NE; ++i) {
    const int e = threadIdx.x + 256 * i;
    if (e < D * R) out[e] = acc[i];
  }
}

// dW = scale * (sum of the parts in order); block (h, 0) also writes loss[h] from the row sums.
template <int D, int R>
__global__ __launch_bounds__(256) void pred_wreduce_kernel(const float* __restrict__ part,
                                                            const float* __restrict__ lrow, float* __restrict__ loss,
                                                            float* __restrict__ dWq, float* __restrict__ dWk, int B,
                                                            int H, int NG, int NB, float tau) {
  __shared__ float sred[256];
  const int h = blockIdx.x;
  const bool is_q = blockIdx.y == 0;
  const float scale = 2.0f * tau / ((float)B * (float)NG * (float)NB);
  const float* pp = part + ((size_t)h * 2 + blockIdx.y) * kWgParts * D * R;
  float* dW = (is_q ? dWq : dWk) + (size_t)h * D * R;
  for (int e = threadIdx.x; e < D * R; e += 256) {
    float s = 0.f;
    for (int q = 0; q < kWgParts; ++q) s += pp[(size_t)q * D * R + e];
    dW[e] = s * scale;
  }
  if (!is_q) return;
  // loss of head h: each thread sums a strided share of the rows, then a fixed-order tree
  float s = 0.f;
  for (int b = 0; b < B; ++b)
    for (int g = threadIdx.x; g < NG; g += 256) s += lrow[((size_t)b * H + h) * NG + g];
  sred[threadIdx.x] = s;
  __syncthreads();
  for (int w = 128; w > 0; w >>= 1) {
    if (threadIdx.x < w) sred[threadIdx.x] += sred[threadIdx.x + w];
    __syncthreads();
  }
  if (threadIdx.x == 0) loss[h] = sred[0] / ((float)B * (float)NG * (float)NB);
}

template <int D, int R>
hipError_t train_dispatch(const Shape& s, const PredWork& w, float* loss, float* dWq, float* dWk, float tau,
                          hipStream_t st) {
  const int ncx = (s.NB + kDiffCols - 1) / kDiffCols;
  dim3 gd((unsigned)(ncx * ((s.NG + kDiffRows - 1) / kDiffRows)), s.H, s.B);
  hipLaunchKernelGGL((pred_diff_kernel<D, R>), gd, dim3(kDiffCols), 0, st, w.qbar, w.kbar, w.qhat, w.khat, w.E,
                     s.NG, s.NB, tau);
  const int64_t waves = (int64_t)s.B * s.H * ((s.NG + kRowsPerWave - 1) / kRowsPerWave);
  hipLaunchKernelGGL((pred_rows_kernel<R>), dim3((unsigned)((waves + 3) / 4)), dim3(256), 0, st, w.E, w.khat, w.Y,
                     w.lrow, s.B * s.H, s.NG, s.NB);
  hipLaunchKernelGGL((pred_cols_kernel<R>), dim3((unsigned)((s.NB + 63) / 64), s.H, s.B), dim3(256), 0, st, w.E,
                     w.qhat, w.Z, s.NG, s.NB);
  hipLaunchKernelGGL((pred_wgrad_kernel<D, R>), dim3(s.H, 2, kWgParts), dim3(256), 0, st, w.qbar, w.Y, w.kbar, w.Z,
                     w.part, s.B, s.H, s.NG, s.NB);
  hipLaunchKernelGGL((pred_wreduce_kernel<D, R>), dim3(s.H, 2), dim3(256), 0, st, w.part, w.lrow, loss, dWq, dWk,
                     s.B, s.H, s.NG, s.NB, tau);
  return hipGetLastError();
}

template <int D>
hipError_t train_dispatch_r(const Shape& s, const PredWork& w, float* loss, float* dWq, float* dWk, float tau,
                            hipStream_t st) {
  switch (s.R) {
    case 8: return train_dispatch<D, 8>(s, w, loss, dWq, dWk, tau, st);
    case 16: return train_dispatch<D, 16>(s, w, loss, dWq, dWk, tau, st);
    case 32: return train_dispatch<D, 32>(s, w, loss, dWq, dWk, tau, st);
    case 64: return train_dispatch<D, 64>(s, w, loss, dWq, dWk, tau, st);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

hipError_t launch_predictor_loss_grad(const Shape& s, const void* Q, const void* K, const float* Wq, const float* Wk,
                                      const PredWork& w, float* loss, float* dWq, float* dWk, hipStream_t st) {
  const float tau = 1.0f / sqrtf((float)s.D);
  hipError_t e = launch_pool_project(s, Q, Wq, w.qhat, s.G, st, w.qbar);
  if (e == hipSuccess) e = launch_pool_project(s, K, Wk, w.khat, kBlock, st, w.kbar);
  if (e != hipSuccess) return e;
  return s.D == 64 ? train_dispatch_r<64>(s, w, loss, dWq, dWk, tau, st)
                   : train_dispatch_r<128>(s, w, loss, dWq, dWk, tau, st);
}

}  // namespace dsa
