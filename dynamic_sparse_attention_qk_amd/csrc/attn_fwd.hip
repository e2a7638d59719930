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

// Split-KV (partial states over parts of each row's kept list, merged by
// log-sum-exp; DiTango explainer, nl edition, Methodologie: attention states
// compose associatively and commutatively; DSV hi §2.C sparse sequence-wise
// CP): tasks are ordered (part, b, h, g), so a launch works through every
// group's first part before any second part and, since lists are ascending,
// streams roughly one n_split-th of each head's K and V at a time; the part
// covers list positions [part k_h / n_split, (part + 1) k_h / n_split).
// n_split = 1 is the plain forward.
//
// Phases (phase >= 0, n_split = the phase count): the same segments of each
// row's list, one launch per segment in order; the launch of phase p > 0
// merges its state into the (O, LSE) the earlier phases stored.  Used for the
// plain forward when one head's K and V fill more than half the MALL, so each launch
// streams about 1/n_split of them.
// How far (log2 units) a block's row max may exceed the running max before the accumulators are rescaled.
// 0: exact running max.  A lazier slack (e.g. 8) skips rescales but puts the dominant weights at arbitrary
// values in [1, 2^slack], each rounded to fp16, which measured 1.6x the error of O (and of D = dO . O in
// the backward) on the 57.6k-token workload.
constexpr float kRescaleSlack = 0.0f;

struct FwdTask {
  int g, h, b, part, kbeg, klen;
};

// cnt (if not null): blocks kept by each (b, h, g) row, clamped to [1, k_h] (k_h: the row's list capacity)
__device__ __forceinline__ FwdTask fwd_task(uint32_t L, int NG, int H, int B, int n_split, int phase,
                                            const HeadTable& ht, const int32_t* __restrict__ cnt) {
  FwdTask t;
  const uint32_t per = (uint32_t)NG * H * B;  // tasks of one part
  const int seg = phase >= 0 ? phase : (int)(L / per);
  t.part = phase >= 0 ? 0 : seg;
  const uint32_t r = phase >= 0 ? L : L % per;
  t.g = r % NG;
  t.h = (r / NG) % H;
  t.b = r / (NG * H);
  const int k = cnt ? min(max(cnt[((size_t)t.b * H + t.h) * NG + t.g], 1), ht.k[t.h]) : ht.k[t.h];
  t.kbeg = seg * k / n_split;
  t.klen = (seg + 1) * k / n_split - t.kbeg;
  return t;
}

// An empty part: O = 0, LSE = -inf for the 32 rows starting at qrow0 (one wave; lane pair l32, l32+32 per row).
template <int D>
__device__ __forceinline__ void write_empty_part(float* O, float* LSE, size_t row, int hh) {
  float* orow = O + row * D;
#pragma unroll
  for (int c = 0; c < D / 32; ++c)
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4)
      *reinterpret_cast<float4*>(orow + 32 * c + 8 * q4 + 4 * hh) = make_float4(0.f, 0.f, 0.f, 0.f);
  if (hh == 0) LSE[row] = -INFINITY;
}

// kLists false: dense attention (no lists; list position t of the part is block kbeg + t).
// kMerge: the phased launches (phase >= 0), which merge into the stored state after the first.
template <int D, int G, bool kLists, bool kMerge>
__global__ __launch_bounds__(G * 4, 2) void attn_fwd_bf16_kernel(const bf16_t* __restrict__ Q,
                                                                 const bf16_t* __restrict__ K,
                                                                 const uint16_t* __restrict__ V16,
                                                                 const int32_t* __restrict__ idx,
                                                                 const int32_t* __restrict__ cnt,
                                                                 float* __restrict__ O, float* __restrict__ LSE,
                                                                 const int32_t* __restrict__ ex,
                                                                 HeadTable ht, XcdSplit sp, int N, int H, int B,
                                                                 int n_split, int phase, float scale_log2) {
  constexpr int NRT = G / 32;                  // 32-row tiles of the group
  constexpr int NW = 2 * NRT;                  // waves: row tile x key half
  constexpr int RB = 2 * D;                    // bytes per tile row
  constexpr int TILE = 64 * RB;                // one 64 x D 16-bit tile
  constexpr int OBUF = D * 128;                // one row tile's O partial: 64 lanes x D/2 floats
  static_assert(OBUF == TILE && NRT <= 4, "merge buffers reuse the four tiles");
  // K ring and V ring of two tiles each, separate objects so the compiler can
  // see that reading one never aliases the DMA filling another.  Block t's K
  // sits in kb[t % 2], its V in vb[t % 2]; K runs one block ahead of V.
  __shared__ __attribute__((aligned(1024))) char kb0[TILE];
  __shared__ __attribute__((aligned(1024))) char kb1[TILE];
  __shared__ __attribute__((aligned(1024))) char vb0[TILE];
  __shared__ __attribute__((aligned(1024))) char vb1[TILE];
  __shared__ float sml[NRT][3][64];            // m, l and the fp32 row sum of the key-half-1 waves

  const int NG = N / G;
  const int64_t task = xcd_task(sp, blockIdx.x);
  if (task < 0) return;
  const FwdTask tk = fwd_task((uint32_t)task, NG, H, B, n_split, phase, ht, kLists ? cnt : nullptr);
  const int g = tk.g, h = tk.h, b = tk.b;
  const int k = tk.klen;  // blocks of this part
  const int NB = N / kBlock;
  const int32_t* irow = kLists ? idx + row_base(ht, b, h, NG) + (int64_t)g * ht.k[h] + tk.kbeg : nullptr;
  const size_t bh = (size_t)b * H + h;
  const bf16_t* Kbh = K + bh * (size_t)N * D;
  const uint16_t* Vbh = V16 + bh * (size_t)N * D;
  O += (size_t)tk.part * B * H * N * D;  // this part's output slice
  LSE += (size_t)tk.part * B * H * N;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int l32 = lane & 31, hh = lane >> 5;
  const int rt = wave % NRT, kh = wave / NRT;  // rows 32*rt.., keys 32*kh.. of every block
  const int qrow = g * G + rt * 32 + l32;
  if (k == 0) {  // uniform over the workgroup, before any barrier; a later phase leaves the stored state
    if (kh == 0 && (!kMerge || phase == 0)) write_empty_part<D>(O, LSE, bh * N + qrow, hh);
    return;
  }
  // block of list position min(t, k-1): past the end the last block is fetched again into a free
  // buffer (keeps the copies branch-free; the data is never used).  Ids are valid by contract;
  // clamping keeps a bad list from reading out of bounds.
  auto block_id = [&](int t) {
    if constexpr (kLists) return min(max(irow[min(t, k - 1)], 0), NB - 1);
    else return tk.kbeg + min(t, k - 1);
  };

  bf16x8 qreg[D / 16];
  {
    const bf16_t* qp = Q + (bh * N + qrow) * (size_t)D + 8 * hh;
#pragma unroll
    for (int t = 0; t < D / 16; ++t) qreg[t] = *reinterpret_cast<const bf16x8*>(qp + 16 * t);
  }
  // LDS byte offsets: K rows for S^T = K Q^T, and the transpose-read windows of V for O^T += V^T P^T
  int kofs[D / 16];
#pragma unroll
  for (int c = 0; c < D / 16; ++c) kofs[c] = tile_off<D>(32 * kh + l32, 2 * c + hh);
  // transpose read r (0/1) of column tile c: lane addresses row 32*kh + 8*r + rl of the 16-key chunk,
  // columns 32*c + 16*(g16 & 1) + 4*(li & 3); the chunk at +16 rows has the same swizzle
  const int li = lane & 15, g16 = lane >> 4;
  const int rl = 4 * hh + (li >> 2);
  int vofs[D / 32][2];
#pragma unroll
  for (int c = 0; c < D / 32; ++c)
#pragma unroll
    for (int r = 0; r < 2; ++r)
      vofs[c][r] = tile_off<D>(32 * kh + 8 * r + rl, 4 * c + 2 * (g16 & 1) + ((li & 3) >> 1)) + 8 * (li & 1);

  // l_run: row sum of the fp16-rounded weights that enter P V (normalises O by exactly the weights it used);
  // l_lse: row sum of the unrounded fp32 weights (the log-sum-exp, free of the fp16 rounding of P)
  float m_used = -INFINITY, l_run = 0.f, l_lse = 0.f;
  f32x16 oacc[D / 32];
#pragma unroll
  for (int c = 0; c < D / 32; ++c) oacc[c] = f32x16{};

  auto fetch_k = [&](int j, char* dst) { dma_tile<D, NW>(Kbh + (size_t)j * kBlock * D, dst, wave, lane); };
  auto fetch_v = [&](int j, char* dst) { dma_tile<D, NW>(Vbh + (size_t)j * kBlock * D, dst, wave, lane); };
  // Block ids of the copies, read ahead: at step t, id_v = block of t+1, id_k = block of t+2 and
  // id_pf = block of t+3 are in registers and the id of t+4 is being read, so no list read stands
  // between a barrier and the copies it releases.
  int id_v, id_k, id_pf;
  // S^T of one block: element e is key 32*kh + 8*(e/4) + 4*hh + e%4 of the block, query row l32
  auto s_tile = [&](const char* kt) {
    f32x16 acc = f32x16{};
#pragma unroll
    for (int c = 0; c < D / 16; ++c) acc = mfma32(*reinterpret_cast<const bf16x8*>(kt + kofs[c]), qreg[c], acc);
    return acc;
  };
  // row maximum of a score tile (log2 domain)
  auto row_max = [&](const f32x16& sc) {
    float bm = sc[0];
#pragma unroll
    for (int e = 1; e < 16; ++e) bm = fmaxf(bm, sc[e]);
    return wave_max_pair(bm) * scale_log2;
  };
  // Block t, in two phases that each pair MFMAs with independent vector work of the same wave:
  //   A: scores of block t+1 (K_{t+1} Q^T)  ||  exponentials of block t
  //   B: O += P_t V_t                        ||  row max of block t+1, row sums of block t
  // At entry K_{t+1} and V_t are in flight into kn and vc and bm holds block t's row max; K_t's and
  // V_{t-1}'s buffers (kfree, vfree) take K_{t+2} and V_{t+1}.
  float bm;
  auto step = [&](int t, const f32x16& sc, f32x16& sn, const char* kn, const char* vc, char* kfree, char* vfree) {
    wait_vmem();
    __syncthreads();  // K_{t+1}, V_t in LDS; every wave is done with K_t and V_{t-1}
    fetch_k(id_k, kfree);
    fetch_v(id_v, vfree);
    id_v = id_k;
    id_k = id_pf;
    id_pf = block_id(t + 4);
    // rescale when block t raises any row's running max: the block that sets a row's max then contributes
    // a weight of exactly 1, so the fp16 rounding of P (2^-12 relative) spares the dominant key
    if (__ballot(bm > m_used + kRescaleSlack)) {
      const float m_new = fmaxf(m_used, bm);
      const float alpha = __builtin_amdgcn_exp2f(m_used - m_new);
      l_run *= alpha;
      l_lse *= alpha;
#pragma unroll
      for (int c = 0; c < D / 32; ++c) oacc[c] *= alpha;
      m_used = m_new;
    }
    sn = s_tile(kn);  // after the last block this reads a stale buffer; the result is unused
    f16x8 p[2];
#pragma unroll
    for (int hf = 0; hf < 2; ++hf)
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float pf = __builtin_amdgcn_exp2f(__builtin_fmaf(sc[8 * hf + e], scale_log2, -m_used));
        p[hf][e] = (_Float16)pf;
        l_lse += pf;
      }
#pragma unroll
    for (int c = 0; c < D / 32; ++c) {
      const char* v0 = vc + vofs[c][0];
      const char* v1 = vc + vofs[c][1];
      oacc[c] = mfma32h(join_f16(lds_read_tr16(v0), lds_read_tr16(v1)), p[0], oacc[c]);
      oacc[c] = mfma32h(join_f16(lds_read_tr16(v0 + 16 * RB), lds_read_tr16(v1 + 16 * RB)), p[1], oacc[c]);
    }
    // row sum of the rounded weights that enter P V
    l_run = sum_f16x8(p[1], sum_f16x8(p[0], l_run));
    bm = row_max(sn);
  };

  {
    const int id0 = block_id(0);
    id_v = block_id(1);
    id_k = block_id(2);
    id_pf = block_id(3);
    fetch_k(id0, kb0);
    fetch_v(id0, vb0);
    fetch_k(id_v, kb1);
  }
  wait_vmem();
  __syncthreads();
  f32x16 sa = s_tile(kb0), sb;
  bm = row_max(sa);
  for (int t = 0; t < k; t += 2) {
    step(t, sa, sb, kb1, vb0, kb0, vb1);
    if (t + 1 < k) step(t + 1, sb, sa, kb0, vb1, kb1, vb0);
  }
  wait_vmem();  // the copies issued by the last blocks land before the buffers are reused

  // merge the two key halves of each row tile (O partials parked in the ring buffers)
  const float l_tot = wave_sum_pair(l_run);
  const float l_tot_lse = wave_sum_pair(l_lse);
  __syncthreads();
  float* mb = reinterpret_cast<float*>(rt == 0 ? kb0 : rt == 1 ? kb1 : rt == 2 ? vb0 : vb1);
  if (kh == 1) {
#pragma unroll
    for (int c = 0; c < D / 32; ++c)
#pragma unroll
      for (int e = 0; e < 16; ++e) mb[(c * 16 + e) * 64 + lane] = oacc[c][e];
    sml[rt][0][lane] = m_used;
    sml[rt][1][lane] = l_tot;
    sml[rt][2][lane] = l_tot_lse;
  }
  __syncthreads();
  if (kh == 0) {
    const float m1 = sml[rt][0][lane], l1 = sml[rt][1][lane], l1_lse = sml[rt][2][lane];
    const float m = fmaxf(m_used, m1);
    const float a0 = __builtin_amdgcn_exp2f(m_used - m), a1 = __builtin_amdgcn_exp2f(m1 - m);
    const float lsum = a0 * l_tot + a1 * l1;
    float lse2 = m + __log2f(a0 * l_tot_lse + a1 * l1_lse);  // this segment's log-sum-exp, log2 domain
    // a later phase: merge with the state of the earlier ones (weights e^{LSE_s - LSE}, normalised)
    float wc = 1.0f, wp = 0.0f;
    if (kMerge && phase > 0) {
      const float lp2 = LSE[bh * N + qrow] * kLog2e;
      const float M = fmaxf(lse2, lp2);
      const float ec = __builtin_amdgcn_exp2f(lse2 - M), ep = __builtin_amdgcn_exp2f(lp2 - M);
      const float W = ec + ep;
      wc = ec / W;
      wp = ep / W;
      lse2 = M + __log2f(W);
    }
    const float inv = __builtin_ldexpf(wc / lsum, -ex[kTV * B * H + bh]);  // V16 carries 2^eV
    const float w0 = a0 * inv, w1 = a1 * inv;
    float* orow = O + (bh * N + qrow) * (size_t)D;
#pragma unroll
    for (int c = 0; c < D / 32; ++c)
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        float* op = orow + 32 * c + 8 * q4 + 4 * hh;
        float4 prev = make_float4(0.f, 0.f, 0.f, 0.f);
        if (kMerge && phase > 0) prev = *reinterpret_cast<const float4*>(op);
        float v[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) v[r] = oacc[c][4 * q4 + r] * w0 + mb[(c * 16 + 4 * q4 + r) * 64 + lane] * w1;
        *reinterpret_cast<float4*>(op) =
            make_float4(v[0] + prev.x * wp, v[1] + prev.y * wp, v[2] + prev.z * wp, v[3] + prev.w * wp);
      }
    if (hh == 0) LSE[bh * N + qrow] = lse2 * kLn2;
  }
}

// fp32 operands: v_mfma_f32_32x32x2_f32, K and V row-major in LDS.  kLists as for the bf16 kernel.
template <int D, int G, bool kLists>
__global__ __launch_bounds__(G * 2) void attn_fwd_f32_kernel(const float* __restrict__ Q, const float* __restrict__ K,
                                                             const float* __restrict__ V,
                                                             const int32_t* __restrict__ idx,
                                                             const int32_t* __restrict__ cnt, float* __restrict__ O,
                                                             float* __restrict__ LSE, HeadTable ht, XcdSplit sp, int N, int H,
                                                             int B, int n_split, float scale_log2) {
  constexpr int NT = G * 2;
  constexpr int LD = D + 1;
  __shared__ float sK[64 * LD];
  __shared__ float sV[64 * LD];

  const int NG = N / G;
  const int64_t task = xcd_task(sp, blockIdx.x);
  if (task < 0) return;
  const FwdTask tk = fwd_task((uint32_t)task, NG, H, B, n_split, -1, ht, kLists ? cnt : nullptr);
  const int g = tk.g, h = tk.h, b = tk.b;
  const int k = tk.klen;  // blocks of this part
  const int32_t* irow = kLists ? idx + row_base(ht, b, h, NG) + (int64_t)g * ht.k[h] + tk.kbeg : nullptr;
  const size_t bh = (size_t)b * H + h;
  const float* Kbh = K + bh * (size_t)N * D;
  const float* Vbh = V + bh * (size_t)N * D;
  O += (size_t)tk.part * B * H * N * D;  // this part's output slice
  LSE += (size_t)tk.part * B * H * N;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int l32 = lane & 31, hh = lane >> 5;
  const int qrow = g * G + wave * 32 + l32;
  if (k == 0) {  // uniform over the workgroup, before any barrier
    write_empty_part<D>(O, LSE, bh * N + qrow, hh);
    return;
  }

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
    const int j = kLists ? min(max(irow[t], 0), NB - 1) : tk.kbeg + t;
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

// O = sum_s exp(LSE_s - LSE) O_s with LSE = ln sum_s exp(LSE_s), per row; a
// part with LSE_s = -inf adds nothing (all parts empty: O = 0, LSE = -inf).
// D/4 lanes per row, four columns each.
template <int D>
__global__ __launch_bounds__(256) void attn_merge_kernel(const float* __restrict__ O_part,
                                                         const float* __restrict__ LSE_part, float* __restrict__ O,
                                                         float* __restrict__ LSE, int n_parts, int64_t rows) {
  constexpr int LPR = D / 4;
  constexpr int RPB = 256 / LPR;
  const int sub = threadIdx.x % LPR;
  for (int64_t row = (int64_t)blockIdx.x * RPB + threadIdx.x / LPR; row < rows; row += (int64_t)gridDim.x * RPB) {
    float m = -INFINITY;
    for (int p = 0; p < n_parts; ++p) m = fmaxf(m, LSE_part[p * rows + row]);
    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
    float l = 0.f;
    if (m > -INFINITY) {
      for (int p = 0; p < n_parts; ++p) {
        const float w = expf(LSE_part[p * rows + row] - m);
        const float4 o = *reinterpret_cast<const float4*>(O_part + (p * rows + row) * D + 4 * sub);
        l += w;
        acc.x += w * o.x;
        acc.y += w * o.y;
        acc.z += w * o.z;
        acc.w += w * o.w;
      }
      const float inv = 1.0f / l;
      acc = make_float4(acc.x * inv, acc.y * inv, acc.z * inv, acc.w * inv);
    }
    *reinterpret_cast<float4*>(O + row * D + 4 * sub) = acc;
    if (sub == 0) LSE[row] = m > -INFINITY ? m + logf(l) : -INFINITY;
  }
}

template <int D, int G>
hipError_t fwd_launch(const Shape& s, const void* Q, const void* K, const void* V, const int32_t* idx,
                      const int32_t* cnt, float* O, float* LSE, const FwdWork& w, const HeadTable& ht, int n_split,
                      hipStream_t st) {
  const float scale_log2 = (1.0f / sqrtf((float)D)) * kLog2e;
  unsigned nwg = 0;
  // a (part, group) task costs k_h / n_split blocks + 1; a head streams its K and V.  The parts are
  // outermost in the task order: to the balancer they are n_split batches of the same heads
  const double head_bytes = 4.0 * s.N * D;  // one head's K (bf16) and V (fp16 copy)
  const XcdSplit sp = make_xcd_split(s.B * n_split, s.H, s.NG, ht, 1.0 / n_split, 1.0, head_bytes, &nwg);
  dim3 grid(nwg);
  if (s.bf16) {
    const hipError_t e = launch_cvt_scaled_v(V, w.V16, w.part, w.ex, (int64_t)s.N * D, s.B * s.H, st);
    if (e != hipSuccess) return e;
    auto kern = idx ? attn_fwd_bf16_kernel<D, G, true, false> : attn_fwd_bf16_kernel<D, G, false, false>;
    // the plain forward over heads whose K and V fill more than half the MALL: kMallPhasesKV launches in sequence
    if (n_split == 1 && head_bytes > 0.5 * kMallBytes) {
      unsigned nwg_p = 0;
      const XcdSplit spp = make_xcd_split(s.B, s.H, s.NG, ht, 1.0 / kMallPhasesKV, 1.0, head_bytes, &nwg_p);
      auto kern_m = idx ? attn_fwd_bf16_kernel<D, G, true, true> : attn_fwd_bf16_kernel<D, G, false, true>;
      for (int ph = 0; ph < kMallPhasesKV; ++ph)
        hipLaunchKernelGGL(kern_m, dim3(nwg_p), dim3(G * 4), 0, st, static_cast<const bf16_t*>(Q),
                           static_cast<const bf16_t*>(K), w.V16, idx, cnt, O, LSE, w.ex, ht, spp, s.N, s.H, s.B,
                           kMallPhasesKV, ph, scale_log2);
      return hipGetLastError();
    }
    hipLaunchKernelGGL(kern, grid, dim3(G * 4), 0, st, static_cast<const bf16_t*>(Q), static_cast<const bf16_t*>(K),
                       w.V16, idx, cnt, O, LSE, w.ex, ht, sp, s.N, s.H, s.B, n_split, -1, scale_log2);
  } else {
    auto kern = idx ? attn_fwd_f32_kernel<D, G, true> : attn_fwd_f32_kernel<D, G, false>;
    hipLaunchKernelGGL(kern, grid, dim3(G * 2), 0, st, static_cast<const float*>(Q), static_cast<const float*>(K),
                       static_cast<const float*>(V), idx, cnt, O, LSE, ht, sp, s.N, s.H, s.B, n_split, scale_log2);
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_attn_fwd(const Shape& s, const void* Q, const void* K, const void* V, const int32_t* idx, float* O,
                           float* LSE, const FwdWork& w, const HeadTable& ht, int n_split, hipStream_t st,
                           const int32_t* cnt) {
  if (s.D == 64)
    return s.G == 64 ? fwd_launch<64, 64>(s, Q, K, V, idx, cnt, O, LSE, w, ht, n_split, st)
                     : fwd_launch<64, 128>(s, Q, K, V, idx, cnt, O, LSE, w, ht, n_split, st);
  if (s.D == 128)
    return s.G == 64 ? fwd_launch<128, 64>(s, Q, K, V, idx, cnt, O, LSE, w, ht, n_split, st)
                     : fwd_launch<128, 128>(s, Q, K, V, idx, cnt, O, LSE, w, ht, n_split, st);
  return hipErrorInvalidValue;
}

hipError_t launch_attn_merge(const Shape& s, int n_parts, const float* O_part, const float* LSE_part, float* O,
                             float* LSE, hipStream_t st) {
  const int64_t rows = (int64_t)s.B * s.H * s.N;
  const int rpb = 256 / (s.D / 4);
  const int64_t nwg = (rows + rpb - 1) / rpb;
  const dim3 grid((unsigned)(nwg < 65536 ? nwg : 65536));
  if (s.D == 64)
    hipLaunchKernelGGL(attn_merge_kernel<64>, grid, dim3(256), 0, st, O_part, LSE_part, O, LSE, n_parts, rows);
  else if (s.D == 128)
    hipLaunchKernelGGL(attn_merge_kernel<128>, grid, dim3(256), 0, st, O_part, LSE_part, O, LSE, n_parts, rows);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace dsa
