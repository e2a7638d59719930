// Host-side launchers of the gfx950 kernels (called by the C ABI in api.hip
// after argument validation).  Each returns a hipError_t of the launch.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "common.hpp"

namespace dsa {

struct Shape {
  int B, H, N, D, R, G, NG, NB;
  bool bf16;
};

// out = pooled means projected by W; mean_out (if not null) also receives the means [B, H, N / pool, d]
hipError_t launch_pool_project(const Shape& s, const void* X, const float* W, float* out, int pool,
                               hipStream_t st, float* mean_out = nullptr);
hipError_t launch_block_scores(const Shape& s, const float* qhat, const float* khat, float* scores,
                               float tau, hipStream_t st);
// Selection and its reverse index.  cnt (if not null): select by attention coverage (kept counts per row to
// cnt [B,H,NG], unused slots -1); diag_group > 0: the blocks holding each group's own diag_group tokens are
// always kept.  Scratch: counts [B*H*NB] int32 and the membership bitmaps [B*H, ceil(NG/32), NB] uint32.
hipError_t launch_select(const Shape& s, const float* scores, const float* qhat, const float* khat, int32_t* idx,
                         float* dump, const HeadTable& ht, float tau, int kmax, int32_t* rev_ptr, int32_t* rev_idx,
                         int32_t* counts, uint32_t* bits, hipStream_t st, int32_t* cnt = nullptr,
                         float coverage = 1.0f, int diag_group = 0);
// The forward's workspace (bf16 inputs): the exponent table [4][B*H] (the forward writes the V entry), the
// partial maxima [4][B*H][kAmaxChunks] and the scaled fp16 copy of V.  Its layout is the start of the
// backward's, so a backward given the same workspace can reuse the copy.
struct FwdWork {
  int32_t* ex;
  uint32_t* part;
  uint16_t* V16;
};

// cnt (if not null): per-row kept counts [B,H,NG] within the k_h-entry rows of idx
hipError_t launch_attn_fwd(const Shape& s, const void* Q, const void* K, const void* V, const int32_t* idx,
                           float* O, float* LSE, const FwdWork& w, const HeadTable& ht, int n_split, hipStream_t st,
                           const int32_t* cnt = nullptr);
hipError_t launch_attn_merge(const Shape& s, int n_parts, const float* O_part, const float* LSE_part, float* O,
                             float* LSE, hipStream_t st);
// Backward workspace: the forward's part (exponent table, partial maxima, V16), then D, -LSE*log2(e), the
// scaled fp16 copy of K (for dQ) and the dK/dV task order.  dK/dV read the bf16 inputs themselves.
struct BwdWork {
  int32_t* ex;
  uint32_t* part;
  float* Dvec;
  float* nl2;
  uint16_t* K16;
  uint16_t* V16;
  int32_t* order;  // dK/dV task order: per XCD range, long reverse lists first
};

// v_from_fwd: V16 and its exponent were left in the workspace by the forward (not converted again)
hipError_t launch_bwd_pre(const Shape& s, const void* Q, const void* K, const void* V, const float* O,
                          const void* dO, const float* LSE, const BwdWork& w, bool v_from_fwd, hipStream_t st);
hipError_t launch_bwd_dkdv(const Shape& s, const BwdWork& w, const void* Q, const void* K, const void* V,
                           const void* dO, const int32_t* rev_ptr, const int32_t* rev_idx, float* dK, float* dV,
                           const HeadTable& ht, hipStream_t st);
hipError_t launch_bwd_dq(const Shape& s, const BwdWork& w, const void* Q, const void* dO, const int32_t* idx,
                         float* dQ, const HeadTable& ht, hipStream_t st, const int32_t* cnt = nullptr);

// Block scores pooled from token-level logits (pooling 1: max, 2: log-mean-exp); pq, pk: fp16 [B,H,N,r]
hipError_t launch_pooled_scores(const Shape& s, const void* Q, const void* K, const float* Wq, const float* Wk,
                                int pooling, float* scores, _Float16* pq, _Float16* pk, hipStream_t st);

// Stage-1 predictor training workspace (fp32): qbar [B,H,NG,d], kbar [B,H,NB,d], qhat [B,H,NG,r],
// khat [B,H,NB,r], E [B,H,NG,NB], Y [B,H,NG,r], Z [B,H,NB,r], lrow [B,H,NG], part [H,2,16,d,r].
constexpr int kPredWgParts = 16;
struct PredWork {
  float* qbar;
  float* kbar;
  float* qhat;
  float* khat;
  float* E;
  float* Y;
  float* Z;
  float* lrow;
  float* part;
};

hipError_t launch_predictor_loss_grad(const Shape& s, const void* Q, const void* K, const float* Wq, const float* Wk,
                                      const PredWork& w, float* loss, float* dWq, float* dWk, hipStream_t st);

// Debug builds: checks of the kept-block lists (idx, optional per-row counts cnt) and of the reverse index
// (rev_ptr, rev_idx); either may be null.  The first failure found goes to err[0..3] (code, row or
// (b, h, block), position, value), which the caller clears beforehand.
enum ListCheck : uint32_t {
  kListBadCount = 1,     // a per-row count outside [1, k_h]
  kListOutOfRange = 2,   // a kept block id outside [0, NB)
  kListNotAscending = 3, // a row's ids not strictly ascending (a repeat included)
  kListBadPadding = 4,   // a slot past a row's count not -1
  kRevBadPointer = 5,    // rev_ptr not starting at 0, decreasing, or past NG * k_h
  kRevOutOfRange = 6,    // a reverse-list group id outside [0, NG)
  kRevNotAscending = 7,  // a reverse list not strictly ascending
};
hipError_t launch_check_lists(const Shape& s, const HeadTable& ht, const int32_t* idx, const int32_t* cnt,
                              const int32_t* rev_ptr, const int32_t* rev_idx, uint32_t* err, hipStream_t st);

}  // namespace dsa
