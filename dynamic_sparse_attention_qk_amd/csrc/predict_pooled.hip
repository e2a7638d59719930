// Block scores pooled from the token-level low-rank logits, a predictor
// variant: instead of projecting the group and block means (DSV, gist.science
// explainer, hi edition, technical summary §2.A low-rank predictor, §2.B proxy
// query), every token is projected and the logits
//   l[i, m] = tau (q_i W_q) . (k_m W_k)
// of each G x 64 tile are pooled by their maximum or by the log of their mean
// exponential (the predicted attention mass of the tile per key pair).
//
// token_project_kernel: fp16 copies of Q W_q and K W_k, [B, H, N, r] (HBM-bound:
// Q and K read once).  pooled_scores_kernel: one wave per query group, four
// groups per workgroup; per KV block the G x 64 logit tile runs on
// v_mfma_f32_32x32x16_f16 (both operands are row-major slices of the fp16
// projections, read straight from L2) and is reduced in registers.
#include "launch.hpp"

namespace dsa {

namespace {

constexpr int kProjTokens = 64;  // tokens per workgroup of the projection

template <typename T, int D, int R>
__global__ __launch_bounds__(256) void token_project_kernel(const T* __restrict__ X, const float* __restrict__ W,
                                                            _Float16* __restrict__ P, int N, int H) {
  __shared__ float sx[kProjTokens][D + 1];
  __shared__ float sw[D][R];
  const size_t bh = blockIdx.z * (size_t)H + blockIdx.y;
  const int h = blockIdx.y;
  const int64_t t0 = (int64_t)blockIdx.x * kProjTokens;
  const T* xb = X + (bh * N + t0) * D;
  // 16-byte loads: VE elements each
  constexpr int VE = 16 / sizeof(T);
  for (int e = threadIdx.x * VE; e < kProjTokens * D; e += 256 * VE) {
    const int t = e / D, c = e % D;
    uint4 v = make_uint4(0u, 0u, 0u, 0u);
    if (t0 + t < N) v = ldg16(xb + e);
    const uint32_t* w = reinterpret_cast<const uint32_t*>(&v);
    if constexpr (sizeof(T) == 2) {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        sx[t][c + 2 * q] = __uint_as_float(w[q] << 16);
        sx[t][c + 2 * q + 1] = __uint_as_float(w[q] & 0xFFFF0000u);
      }
    } else {
#pragma unroll
      for (int q = 0; q < 4; ++q) sx[t][c + q] = __uint_as_float(w[q]);
    }
  }
  for (int e = threadIdx.x; e < D * R; e += 256) sw[e / R][e % R] = W[(size_t)h * D * R + e];
  __syncthreads();
  // thread -> (token, 4 consecutive outputs)
  for (int o = threadIdx.x; o < kProjTokens * (R / 4); o += 256) {
    const int t = o / (R / 4), r0 = 4 * (o % (R / 4));
    float a0 = 0.f, a1 = 0.f, a2 = 0.f, a3 = 0.f;
#pragma unroll 8
    for (int c = 0; c < D; ++c) {
      const float x = sx[t][c];
      a0 = __builtin_fmaf(x, sw[c][r0], a0);
      a1 = __builtin_fmaf(x, sw[c][r0 + 1], a1);
      a2 = __builtin_fmaf(x, sw[c][r0 + 2], a2);
      a3 = __builtin_fmaf(x, sw[c][r0 + 3], a3);
    }
    if (t0 + t < N) {
      typedef _Float16 h4 __attribute__((ext_vector_type(4)));
      *reinterpret_cast<h4*>(P + (bh * N + t0 + t) * R + r0) = h4{(_Float16)a0, (_Float16)a1, (_Float16)a2,
                                                                  (_Float16)a3};
    }
  }
}

// 8 consecutive fp16 projections of row `row` starting at column c (zero beyond R).
template <int R>
__device__ __forceinline__ f16x8 proj8(const _Float16* __restrict__ base, int64_t row, int c) {
  if (c >= R) return f16x8{};
  return *reinterpret_cast<const f16x8*>(base + row * R + c);
}

// MODE 1: max over the tile; MODE 2: log of the mean of exp over the tile.
template <int G, int R, int MODE>
__global__ __launch_bounds__(256) void pooled_scores_kernel(const _Float16* __restrict__ Pq,
                                                            const _Float16* __restrict__ Pk,
                                                            float* __restrict__ scores, int N, int NG, int NB,
                                                            int chunk, float tau) {
  constexpr int RH = G / 32;                    // 32-row halves of the group
  constexpr int KS = (R + 15) / 16;             // 16-wide steps of the rank (zero-padded)
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const size_t bh = blockIdx.z;
  const int g = blockIdx.y * 4 + wave;
  if (g >= NG) return;                          // wave-uniform; no barriers below
  const int j0 = blockIdx.x * chunk, j1 = min(j0 + chunk, NB);
  const _Float16* pq = Pq + bh * (size_t)N * R;
  const _Float16* pk = Pk + bh * (size_t)N * R;
  const int l32 = lane & 31, hi = lane >> 5;
  // A operands: query row 32*rh + l32 of the group, rank columns 16*ks + 8*hi .. +8
  f16x8 a[RH][KS];
#pragma unroll
  for (int rh = 0; rh < RH; ++rh)
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) a[rh][ks] = proj8<R>(pq, (int64_t)g * G + 32 * rh + l32, 16 * ks + 8 * hi);
  float* srow = scores + (bh * NG + g) * (size_t)NB;
  const float kl2 = tau * 1.4426950408889634f;
  f16x8 b[2][KS], bn[2][KS];
  auto load_b = [&](int j, f16x8 (&dst)[2][KS]) {
#pragma unroll
    for (int kh = 0; kh < 2; ++kh)
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) dst[kh][ks] = proj8<R>(pk, (int64_t)j * 64 + 32 * kh + l32, 16 * ks + 8 * hi);
  };
  if (j0 < j1) load_b(j0, b);
  for (int j = j0; j < j1; ++j) {
    if (j + 1 < j1) load_b(j + 1, bn);
    f32x16 acc[RH][2];
#pragma unroll
    for (int rh = 0; rh < RH; ++rh)
#pragma unroll
      for (int kh = 0; kh < 2; ++kh) {
        acc[rh][kh] = f32x16{};
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) acc[rh][kh] = mfma32h(a[rh][ks], b[kh][ks], acc[rh][kh]);
      }
    float m = -INFINITY;
#pragma unroll
    for (int rh = 0; rh < RH; ++rh)
#pragma unroll
      for (int kh = 0; kh < 2; ++kh)
#pragma unroll
        for (int e = 0; e < 16; ++e) m = fmaxf(m, acc[rh][kh][e]);
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) m = fmaxf(m, __shfl_xor(m, off));
    float out;
    if constexpr (MODE == 1) {
      out = m * tau;
    } else {
      float sum = 0.f;
#pragma unroll
      for (int rh = 0; rh < RH; ++rh)
#pragma unroll
        for (int kh = 0; kh < 2; ++kh)
#pragma unroll
          for (int e = 0; e < 16; ++e) sum += __builtin_amdgcn_exp2f((acc[rh][kh][e] - m) * kl2);
#pragma unroll
      for (int off = 32; off > 0; off >>= 1) sum += __shfl_xor(sum, off);
      out = m * tau + logf(sum * (1.0f / (G * 64)));
    }
    if (lane == 0) srow[j] = out;
#pragma unroll
    for (int kh = 0; kh < 2; ++kh)
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) b[kh][ks] = bn[kh][ks];
  }
}

constexpr int kPooledChunk = 64;  // KV blocks per workgroup

template <typename T, int D, int R>
hipError_t pooled_dispatch(const Shape& s, const void* Q, const void* K, const float* Wq, const float* Wk,
                           int pooling, float* scores, _Float16* pq, _Float16* pk, hipStream_t st) {
  const float tau = 1.0f / sqrtf((float)D);
  dim3 gp((unsigned)((s.N + kProjTokens - 1) / kProjTokens), s.H, s.B);
  hipLaunchKernelGGL((token_project_kernel<T, D, R>), gp, dim3(256), 0, st, static_cast<const T*>(Q), Wq, pq, s.N,
                     s.H);
  hipLaunchKernelGGL((token_project_kernel<T, D, R>), gp, dim3(256), 0, st, static_cast<const T*>(K), Wk, pk, s.N,
                     s.H);
  dim3 gs((unsigned)((s.NB + kPooledChunk - 1) / kPooledChunk), (unsigned)((s.NG + 3) / 4), (unsigned)(s.B * s.H));
  if (s.G == 64) {
    if (pooling == 1)
      hipLaunchKernelGGL((pooled_scores_kernel<64, R, 1>), gs, dim3(256), 0, st, pq, pk, scores, s.N, s.NG, s.NB,
                         kPooledChunk, tau);
    else
      hipLaunchKernelGGL((pooled_scores_kernel<64, R, 2>), gs, dim3(256), 0, st, pq, pk, scores, s.N, s.NG, s.NB,
                         kPooledChunk, tau);
  } else {
    if (pooling == 1)
      hipLaunchKernelGGL((pooled_scores_kernel<128, R, 1>), gs, dim3(256), 0, st, pq, pk, scores, s.N, s.NG, s.NB,
                         kPooledChunk, tau);
    else
      hipLaunchKernelGGL((pooled_scores_kernel<128, R, 2>), gs, dim3(256), 0, st, pq, pk, scores, s.N, s.NG, s.NB,
                         kPooledChunk, tau);
  }
  return hipGetLastError();
}

template <typename T, int D>
hipError_t pooled_dispatch_r(const Shape& s, const void* Q, const void* K, const float* Wq, const float* Wk,
                             int pooling, float* scores, _Float16* pq, _Float16* pk, hipStream_t st) {
  switch (s.R) {
    case 8: return pooled_dispatch<T, D, 8>(s, Q, K, Wq, Wk, pooling, scores, pq, pk, st);
    case 16: return pooled_dispatch<T, D, 16>(s, Q, K, Wq, Wk, pooling, scores, pq, pk, st);
    case 32: return pooled_dispatch<T, D, 32>(s, Q, K, Wq, Wk, pooling, scores, pq, pk, st);
    case 64: return pooled_dispatch<T, D, 64>(s, Q, K, Wq, Wk, pooling, scores, pq, pk, st);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

hipError_t launch_pooled_scores(const Shape& s, const void* Q, const void* K, const float* Wq, const float* Wk,
                                int pooling, float* scores, _Float16* pq, _Float16* pk, hipStream_t st) {
  if (s.bf16)
    return s.D == 64 ? pooled_dispatch_r<bf16_t, 64>(s, Q, K, Wq, Wk, pooling, scores, pq, pk, st)
                     : pooled_dispatch_r<bf16_t, 128>(s, Q, K, Wq, Wk, pooling, scores, pq, pk, st);
  return s.D == 64 ? pooled_dispatch_r<float, 64>(s, Q, K, Wq, Wk, pooling, scores, pq, pk, st)
                   : pooled_dispatch_r<float, 128>(s, Q, K, Wq, Wk, pooling, scores, pq, pk, st);
}

}  // namespace dsa
