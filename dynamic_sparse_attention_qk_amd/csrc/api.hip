// C ABI of libdsa.so: argument validation on the host, then asynchronous
// launches on the caller's stream.  Nothing here allocates device memory.
#include <math.h>
#include <stdio.h>
#include <string.h>

#include <mutex>

#include "dsa.h"
#include "launch.hpp"

using dsa::HeadTable;
using dsa::Shape;

namespace {

constexpr int kMaxBlocks = 8192;

bool aligned16(const void* p) { return p != nullptr && ((uintptr_t)p & 15u) == 0; }

int check_problem(const dsa_problem* p, Shape* s) {
  if (!p) return DSA_ERR_INVALID_ARG;
  if (p->dtype != DSA_F32 && p->dtype != DSA_BF16) return DSA_ERR_DTYPE;
  if (p->batch < 1 || p->heads < 1 || p->seq_len < 1) return DSA_ERR_SHAPE;
  if (p->heads > dsa::kMaxHeads) return DSA_ERR_UNSUPPORTED;
  if (p->block != dsa::kBlock) return DSA_ERR_UNSUPPORTED;
  if (p->head_dim != 64 && p->head_dim != 128) return DSA_ERR_UNSUPPORTED;
  if (p->rank != 8 && p->rank != 16 && p->rank != 32 && p->rank != 64) return DSA_ERR_UNSUPPORTED;
  if (p->group != 64 && p->group != 128) return DSA_ERR_UNSUPPORTED;
  if (p->seq_len % p->block != 0 || p->seq_len % p->group != 0) return DSA_ERR_SHAPE;
  if (p->seq_len / p->block > kMaxBlocks) return DSA_ERR_UNSUPPORTED;
  s->B = p->batch;
  s->H = p->heads;
  s->N = p->seq_len;
  s->D = p->head_dim;
  s->R = p->rank;
  s->G = p->group;
  s->NG = p->seq_len / p->group;
  s->NB = p->seq_len / p->block;
  s->bf16 = p->dtype == DSA_BF16;
  return DSA_OK;
}

// Fills the per-head table; returns the largest k_h through kmax.
int check_heads(const Shape& s, const int32_t* kph, HeadTable* ht, int* kmax) {
  if (!kph) return DSA_ERR_INVALID_ARG;
  memset(ht, 0, sizeof(*ht));
  int64_t sum = 0;
  int mx = 0;
  for (int h = 0; h < s.H; ++h) {
    if (kph[h] < 1 || kph[h] > s.NB) return DSA_ERR_SHAPE;
    ht->k[h] = kph[h];
    ht->kofs[h] = (int32_t)sum;
    sum += kph[h];
    if (kph[h] > mx) mx = kph[h];
  }
  ht->kofs[s.H] = (int32_t)sum;
  ht->ksum = (int32_t)sum;
  if ((int64_t)s.B * s.NG * sum >= ((int64_t)1 << 31)) return DSA_ERR_UNSUPPORTED;
  if (kmax) *kmax = mx;
  return DSA_OK;
}

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

// the selection's scratch: per-block counts [B*H*NB] int32, then the membership bitmaps of every 32 groups
// [B*H, ceil(NG/32), NB] uint32 (the reverse index is built from them)
size_t select_counts_bytes(const Shape& s) { return align256((size_t)s.B * s.H * s.NB * sizeof(int32_t)); }
size_t select_ws(const Shape& s, const HeadTable& ht) {
  (void)ht;
  return select_counts_bytes(s) + align256((size_t)s.B * s.H * ((s.NG + 31) / 32) * s.NB * sizeof(uint32_t));
}

// The forward's workspace (bf16 inputs) and the start of the backward's: the exponent table of the scaled
// fp16 copies [4][B*H] int32, the partial maxima [4][B*H][kAmaxChunks] uint32, the copy of V.
size_t ex_bytes(const Shape& s) { return align256((size_t)4 * s.B * s.H * sizeof(int32_t)); }
size_t part_bytes(const Shape& s) { return align256((size_t)4 * s.B * s.H * dsa::kAmaxChunks * sizeof(uint32_t)); }
size_t bwd_tensor_bytes(const Shape& s) { return align256((size_t)s.B * s.H * s.N * s.D * 2); }
size_t fwd_prefix_bytes(const Shape& s) { return ex_bytes(s) + part_bytes(s) + bwd_tensor_bytes(s); }

// forward: the prefix above (bf16 inputs only)
size_t fwd_ws(const Shape& s) { return s.bf16 ? fwd_prefix_bytes(s) : 0; }

dsa::FwdWork fwd_work(const Shape& s, void* ws) {
  char* p = static_cast<char*>(ws);
  dsa::FwdWork w;
  w.ex = reinterpret_cast<int32_t*>(p);
  w.part = reinterpret_cast<uint32_t*>(p + ex_bytes(s));
  w.V16 = reinterpret_cast<uint16_t*>(p + ex_bytes(s) + part_bytes(s));
  return w;
}

size_t bwd_row_bytes(const Shape& s) { return align256((size_t)s.B * s.H * s.N * sizeof(float)); }
size_t bwd_order_bytes(const Shape& s) { return align256((size_t)s.B * s.H * s.NB * sizeof(int32_t)); }
// the forward's part, then D, -LSE*log2(e), the scaled fp16 copy of K and the dK/dV task order
size_t bwd_ws(const Shape& s) { return fwd_prefix_bytes(s) + 2 * bwd_row_bytes(s) + bwd_tensor_bytes(s) + bwd_order_bytes(s); }

dsa::BwdWork bwd_work(const Shape& s, void* ws) {
  const dsa::FwdWork f = fwd_work(s, ws);
  char* p = static_cast<char*>(ws) + fwd_prefix_bytes(s);
  dsa::BwdWork w;
  w.ex = f.ex;
  w.part = f.part;
  w.V16 = f.V16;
  w.Dvec = reinterpret_cast<float*>(p);
  w.nl2 = reinterpret_cast<float*>(p + bwd_row_bytes(s));
  char* t = p + 2 * bwd_row_bytes(s);
  w.K16 = reinterpret_cast<uint16_t*>(t);
  w.order = reinterpret_cast<int32_t*>(t + bwd_tensor_bytes(s));
  return w;
}

// stage-1 predictor training: the means, projections, E and the partial sums of PredWork
size_t pred_ws(const Shape& s) {
  const size_t BH = (size_t)s.B * s.H;
  return align256(BH * s.NG * s.D * 4) + align256(BH * s.NB * s.D * 4) + align256(BH * s.NG * s.R * 4) +
         align256(BH * s.NB * s.R * 4) + align256(BH * s.NG * s.NB * 4) + align256(BH * s.NG * s.R * 4) +
         align256(BH * s.NB * s.R * 4) + align256(BH * s.NG * 4) +
         align256((size_t)s.H * 2 * dsa::kPredWgParts * s.D * s.R * 4);
}

dsa::PredWork pred_work(const Shape& s, void* ws) {
  const size_t BH = (size_t)s.B * s.H;
  char* p = static_cast<char*>(ws);
  auto take = [&](size_t bytes) {
    float* f = reinterpret_cast<float*>(p);
    p += align256(bytes);
    return f;
  };
  dsa::PredWork w;
  w.qbar = take(BH * s.NG * s.D * 4);
  w.kbar = take(BH * s.NB * s.D * 4);
  w.qhat = take(BH * s.NG * s.R * 4);
  w.khat = take(BH * s.NB * s.R * 4);
  w.E = take(BH * s.NG * s.NB * 4);
  w.Y = take(BH * s.NG * s.R * 4);
  w.Z = take(BH * s.NB * s.R * 4);
  w.lrow = take(BH * s.NG * 4);
  w.part = take((size_t)s.H * 2 * dsa::kPredWgParts * s.D * s.R * 4);
  return w;
}

// pooled scores: fp16 token projections of Q and K
size_t pooled_ws(const Shape& s) { return 2 * align256((size_t)s.B * s.H * s.N * s.R * 2); }

int hip_status(hipError_t e) { return e == hipSuccess ? DSA_OK : DSA_ERR_HIP; }

// Dense attention: every head keeps all NB blocks and the kernels take block t at list position t.
HeadTable dense_heads(const Shape& s) {
  HeadTable ht;
  memset(&ht, 0, sizeof(ht));
  for (int h = 0; h <= s.H; ++h) ht.kofs[h] = h * s.NB;
  for (int h = 0; h < s.H; ++h) ht.k[h] = s.NB;
  ht.ksum = s.H * s.NB;
  return ht;
}

// Device bytes the sparse path needs beyond the dense one: qhat, khat, idx, rev_ptr, rev_idx and the
// selection workspace (block scores streamed, not materialised).
size_t sparse_extra_bytes(const Shape& s, const HeadTable& ht) {
  const size_t list = (size_t)s.B * s.NG * ht.ksum * sizeof(int32_t);
  return (size_t)s.B * s.H * ((size_t)s.NG + s.NB) * s.R * sizeof(float) + 2 * list +
         (size_t)s.B * s.H * (s.NB + 1) * sizeof(int32_t) + select_ws(s, ht);
}

}  // namespace

// ---------------------------------------------------------------- the selection without a caller workspace
//
// For callers that cannot allocate: its scratch (the reverse index's counts and membership bitmaps) is this
// static device array, one per GPU the library runs on, held until the process ends.  Host code never
// passes the array's name to a kernel (on the host it is only a stand-in for the device symbol): the
// device address comes from hipGetSymbolAddress, looked up once per device with that device current.
static __device__ __align__(256) char scratch[DSA_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
static void* g_scratch_ptr[kMaxDevices];
static std::mutex g_scratch_mu;

// Device address of `scratch` on the device of `stream` (the current device for the null stream).
static int scratch_for_stream(hipStream_t stream, void** out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return DSA_ERR_HIP;
  const int cur = dev;
  if (stream && hipStreamGetDevice(stream, &dev) != hipSuccess) return DSA_ERR_HIP;
  if (dev < 0 || dev >= kMaxDevices) return DSA_ERR_UNSUPPORTED;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    if (dev != cur && hipSetDevice(dev) != hipSuccess) return DSA_ERR_HIP;
    void* ptr = nullptr;
    const hipError_t e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (dev != cur) (void)hipSetDevice(cur);
    if (e != hipSuccess || !ptr) return DSA_ERR_HIP;
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return DSA_OK;
}

// ---------------------------------------------------------------- list checks of the debug build
#ifdef DSA_DEBUG
static __device__ uint32_t dbg_err[4];  // first failure: code, where, position, value

static const char* list_check_text(uint32_t code) {
  switch (code) {
    case dsa::kListBadCount: return "a per-row count outside [1, k_h]";
    case dsa::kListOutOfRange: return "a kept block id outside [0, NB)";
    case dsa::kListNotAscending: return "kept block ids not strictly ascending";
    case dsa::kListBadPadding: return "a slot past the row's count is not -1";
    case dsa::kRevBadPointer: return "rev_ptr not starting at 0, decreasing, or past NG * k_h";
    case dsa::kRevOutOfRange: return "a reverse-list group id outside [0, NG)";
    case dsa::kRevNotAscending: return "a reverse list not strictly ascending";
    default: return "unknown list error";
  }
}

// Checks the lists a call is about to read (any may be null) on the stream's device and waits for the result.
static int debug_check_lists(const Shape& s, const HeadTable& ht, const int32_t* idx, const int32_t* cnt,
                             const int32_t* rev_ptr, const int32_t* rev_idx, void* stream, const char* call) {
  hipStream_t st = static_cast<hipStream_t>(stream);
  int dev = 0, cur = 0;
  if (hipGetDevice(&cur) != hipSuccess) return DSA_ERR_HIP;
  dev = cur;
  if (st && hipStreamGetDevice(st, &dev) != hipSuccess) return DSA_ERR_HIP;
  if (dev != cur && hipSetDevice(dev) != hipSuccess) return DSA_ERR_HIP;
  uint32_t* err = nullptr;
  uint32_t h[4] = {0, 0, 0, 0};
  hipError_t e = hipGetSymbolAddress(reinterpret_cast<void**>(&err), HIP_SYMBOL(dbg_err));
  if (e == hipSuccess) e = hipMemsetAsync(err, 0, sizeof(h), st);
  if (e == hipSuccess) e = dsa::launch_check_lists(s, ht, idx, cnt, rev_ptr, rev_idx, err, st);
  if (e == hipSuccess) e = hipMemcpyAsync(h, err, sizeof(h), hipMemcpyDeviceToHost, st);
  if (e == hipSuccess) e = hipStreamSynchronize(st);
  if (dev != cur) (void)hipSetDevice(cur);
  if (e != hipSuccess) return DSA_ERR_HIP;
  if (h[0] == 0) return DSA_OK;
  fprintf(stderr, "dsa (debug build) %s: %s -- %s %u, position %d, value %d\n", call, list_check_text(h[0]),
          h[0] >= dsa::kRevBadPointer ? "(b*H + h)*NB + block" : "row (b*H + h)*NG + g", h[1], (int)h[2],
          (int)h[3]);
  return DSA_ERR_BAD_LIST;
}
#define DSA_CHECK_LISTS(...)                          \
  do {                                                \
    const int check_status_ = debug_check_lists(__VA_ARGS__); \
    if (check_status_) return check_status_;          \
  } while (0)
#else
#define DSA_CHECK_LISTS(...) \
  do {                       \
  } while (0)
#endif

extern "C" {

const char* dsa_version(void) { return "dsa-mi355x 0.1.0 (gfx950)"; }

const char* dsa_status_string(int status) {
  switch (status) {
    case DSA_OK: return "ok";
    case DSA_ERR_INVALID_ARG: return "invalid argument (null pointer or bad enum)";
    case DSA_ERR_SHAPE: return "unsupported or inconsistent shape";
    case DSA_ERR_DTYPE: return "unsupported dtype for this call";
    case DSA_ERR_ALIGN: return "device pointer not 16-byte aligned";
    case DSA_ERR_UNSUPPORTED: return "problem outside the supported limits";
    case DSA_ERR_WORKSPACE: return "workspace missing or too small";
    case DSA_ERR_HIP: return "HIP runtime or launch error";
    case DSA_ERR_SCRATCH_LIMIT: return "problem needs more scratch than the library's static buffer holds";
    case DSA_ERR_BAD_LIST: return "malformed kept-block list or reverse index (debug build check)";
    default: return "unknown status";
  }
}

int dsa_index_layout(const dsa_problem* p, const int32_t* k_per_head, int64_t* row_base) {
  Shape s;
  HeadTable ht;
  int st = check_problem(p, &s);
  if (st) return st;
  if ((st = check_heads(s, k_per_head, &ht, nullptr))) return st;
  if (!row_base) return DSA_ERR_INVALID_ARG;
  for (int b = 0; b < s.B; ++b)
    for (int h = 0; h < s.H; ++h) row_base[b * s.H + h] = (int64_t)b * s.NG * ht.ksum + (int64_t)s.NG * ht.kofs[h];
  row_base[s.B * s.H] = (int64_t)s.B * s.NG * ht.ksum;
  return DSA_OK;
}

size_t dsa_workspace_bytes(const dsa_problem* p, const int32_t* k_per_head, int which_call) {
  Shape s;
  HeadTable ht;
  if (check_problem(p, &s)) return 0;
  // the forward and backward workspaces do not depend on the kept counts (dense calls pass none)
  if (!k_per_head && which_call == DSA_WS_FWD) return fwd_ws(s);
  if (!k_per_head && which_call == DSA_WS_BWD) return bwd_ws(s);
  if (which_call == DSA_WS_PRED_GRAD) return pred_ws(s);
  if (which_call == DSA_WS_PRED_POOLED) return pooled_ws(s);
  if (check_heads(s, k_per_head, &ht, nullptr)) return 0;
  if (which_call == DSA_WS_SELECT) return select_ws(s, ht);
  if (which_call == DSA_WS_BWD) return bwd_ws(s);
  if (which_call == DSA_WS_FWD) return fwd_ws(s);
  return 0;
}

int dsa_predict_block_scores(const dsa_problem* p, const void* Q, const void* K, const float* Wq, const float* Wk,
                             float* qhat, float* khat, float* scores, void* stream) {
  Shape s;
  int st = check_problem(p, &s);
  if (st) return st;
  if (!Q || !K || !Wq || !Wk || !qhat || !khat) return DSA_ERR_INVALID_ARG;
  if (!aligned16(Q) || !aligned16(K) || !aligned16(Wq) || !aligned16(Wk) || !aligned16(qhat) || !aligned16(khat) ||
      (scores && !aligned16(scores)))
    return DSA_ERR_ALIGN;
  hipStream_t hs = static_cast<hipStream_t>(stream);
  const float tau = 1.0f / sqrtf((float)s.D);
  hipError_t e = dsa::launch_pool_project(s, Q, Wq, qhat, s.G, hs);
  if (e == hipSuccess) e = dsa::launch_pool_project(s, K, Wk, khat, dsa::kBlock, hs);
  if (e == hipSuccess && scores) e = dsa::launch_block_scores(s, qhat, khat, scores, tau, hs);
  return hip_status(e);
}

// Validates a selection call; fills the shape, head table, largest k and the diagonal group size.
static int select_check(const dsa_problem* p, const float* scores, const float* qhat, const float* khat,
                        const int32_t* k_per_head, int32_t* idx, int flags, int32_t* rev_ptr, int32_t* rev_idx,
                        float* scores_dump, Shape* s, HeadTable* ht, int* kmax, int* diag) {
  int st = check_problem(p, s);
  if (st) return st;
  if ((st = check_heads(*s, k_per_head, ht, kmax))) return st;
  if (flags & ~DSA_SELECT_DIAGONAL) return DSA_ERR_INVALID_ARG;
  *diag = (flags & DSA_SELECT_DIAGONAL) ? s->G : 0;
  for (int h = 0; *diag && h < s->H; ++h)
    if (ht->k[h] < s->G / dsa::kBlock) return DSA_ERR_SHAPE;  // room for the forced blocks
  if (!idx || !rev_ptr || !rev_idx) return DSA_ERR_INVALID_ARG;
  if (!scores && (!qhat || !khat)) return DSA_ERR_INVALID_ARG;
  if ((scores && !aligned16(scores)) || (!scores && (!aligned16(qhat) || !aligned16(khat))) || !aligned16(idx) ||
      !aligned16(rev_ptr) || !aligned16(rev_idx) || (scores_dump && !aligned16(scores_dump)))
    return DSA_ERR_ALIGN;
  return DSA_OK;
}

// The selection's launches, scratch given as a select-layout workspace (counts, then the bitmaps).
static int select_launch(const Shape& s, const HeadTable& ht, int kmax, int diag, const float* scores,
                         const float* qhat, const float* khat, int32_t* idx, int32_t* cnt, float coverage,
                         int32_t* rev_ptr, int32_t* rev_idx, float* scores_dump, void* workspace, hipStream_t hs) {
  const float tau = 1.0f / sqrtf((float)s.D);
  int32_t* counts = static_cast<int32_t*>(workspace);
  uint32_t* bits = reinterpret_cast<uint32_t*>(static_cast<char*>(workspace) + select_counts_bytes(s));
  return hip_status(dsa::launch_select(s, scores, qhat, khat, idx, scores ? nullptr : scores_dump, ht, tau, kmax,
                                       rev_ptr, rev_idx, counts, bits, hs, cnt, coverage, diag));
}

static int select_impl(const dsa_problem* p, const float* scores, const float* qhat, const float* khat,
                       const int32_t* k_per_head, int32_t* idx, int32_t* cnt, float coverage, int flags,
                       int32_t* rev_ptr, int32_t* rev_idx, float* scores_dump, void* workspace,
                       size_t workspace_bytes, void* stream) {
  Shape s;
  HeadTable ht;
  int kmax = 0, diag = 0;
  int st = select_check(p, scores, qhat, khat, k_per_head, idx, flags, rev_ptr, rev_idx, scores_dump, &s, &ht, &kmax,
                        &diag);
  if (st) return st;
  const size_t need = select_ws(s, ht);
  if (!workspace || workspace_bytes < need) return DSA_ERR_WORKSPACE;
  if (!aligned16(workspace)) return DSA_ERR_ALIGN;
  return select_launch(s, ht, kmax, diag, scores, qhat, khat, idx, cnt, coverage, rev_ptr, rev_idx, scores_dump,
                       workspace, static_cast<hipStream_t>(stream));
}

int dsa_predict_block_scores_pooled(const dsa_problem* p, const void* Q, const void* K, const float* Wq,
                                    const float* Wk, int pooling, float* scores, void* workspace,
                                    size_t workspace_bytes, void* stream) {
  Shape s;
  int st = check_problem(p, &s);
  if (st) return st;
  if (pooling != DSA_POOL_MAX && pooling != DSA_POOL_LSE) return DSA_ERR_INVALID_ARG;
  if (!Q || !K || !Wq || !Wk || !scores) return DSA_ERR_INVALID_ARG;
  if (!aligned16(Q) || !aligned16(K) || !aligned16(Wq) || !aligned16(Wk) || !aligned16(scores)) return DSA_ERR_ALIGN;
  if (!workspace || workspace_bytes < pooled_ws(s)) return DSA_ERR_WORKSPACE;
  if (!aligned16(workspace)) return DSA_ERR_ALIGN;
  _Float16* pq = static_cast<_Float16*>(workspace);
  _Float16* pk = reinterpret_cast<_Float16*>(static_cast<char*>(workspace) + pooled_ws(s) / 2);
  return hip_status(dsa::launch_pooled_scores(s, Q, K, Wq, Wk, pooling, scores, pq, pk,
                                              static_cast<hipStream_t>(stream)));
}

int dsa_select_topk_blocks(const dsa_problem* p, const float* scores, const float* qhat, const float* khat,
                           const int32_t* k_per_head, int32_t* idx, int32_t* rev_ptr, int32_t* rev_idx,
                           float* scores_dump, void* workspace, size_t workspace_bytes, void* stream) {
  return select_impl(p, scores, qhat, khat, k_per_head, idx, nullptr, 1.0f, 0, rev_ptr, rev_idx, scores_dump,
                     workspace, workspace_bytes, stream);
}

int dsa_select_topk_blocks_noalloc(const dsa_problem* p, const float* scores, const float* qhat, const float* khat,
                                   const int32_t* k_per_head, int32_t* idx, int32_t* rev_ptr, int32_t* rev_idx,
                                   float* scores_dump, void* stream) {
  Shape s;
  HeadTable ht;
  int kmax = 0, diag = 0;
  int st = select_check(p, scores, qhat, khat, k_per_head, idx, 0, rev_ptr, rev_idx, scores_dump, &s, &ht, &kmax,
                        &diag);
  if (st) return st;
  if (select_ws(s, ht) > (size_t)DSA_NOALLOC_SCRATCH_BYTES) return DSA_ERR_SCRATCH_LIMIT;
  hipStream_t hs = static_cast<hipStream_t>(stream);
  void* ws = nullptr;
  if ((st = scratch_for_stream(hs, &ws))) return st;
  return select_launch(s, ht, kmax, diag, scores, qhat, khat, idx, nullptr, 1.0f, rev_ptr, rev_idx, scores_dump, ws,
                       hs);
}

int dsa_select_blocks(const dsa_problem* p, const float* scores, const float* qhat, const float* khat,
                      const int32_t* k_per_head, double coverage, int flags, int32_t* idx, int32_t* cnt,
                      int32_t* rev_ptr, int32_t* rev_idx, float* scores_dump, void* workspace, size_t workspace_bytes,
                      void* stream) {
  if (!(coverage >= 0.0 && coverage <= 1.0)) return DSA_ERR_INVALID_ARG;
  if (coverage > 0.0) {
    if (!cnt) return DSA_ERR_INVALID_ARG;
    if (!aligned16(cnt)) return DSA_ERR_ALIGN;
  }
  return select_impl(p, scores, qhat, khat, k_per_head, idx, coverage > 0.0 ? cnt : nullptr, (float)coverage, flags,
                     rev_ptr, rev_idx, scores_dump, workspace, workspace_bytes, stream);
}

int dsa_select_coverage_blocks(const dsa_problem* p, const float* scores, const float* qhat, const float* khat,
                               const int32_t* k_per_head, double coverage, int32_t* idx, int32_t* cnt,
                               int32_t* rev_ptr, int32_t* rev_idx, float* scores_dump, void* workspace,
                               size_t workspace_bytes, void* stream) {
  if (!(coverage > 0.0 && coverage <= 1.0)) return DSA_ERR_INVALID_ARG;
  if (!cnt) return DSA_ERR_INVALID_ARG;
  if (!aligned16(cnt)) return DSA_ERR_ALIGN;
  return select_impl(p, scores, qhat, khat, k_per_head, idx, cnt, (float)coverage, 0, rev_ptr, rev_idx, scores_dump,
                     workspace, workspace_bytes, stream);
}

static int fwd_impl(const dsa_problem* p, const void* Q, const void* K, const void* V, const int32_t* idx,
                    const int32_t* cnt, const int32_t* k_per_head, float* O, float* LSE, void* workspace,
                    size_t workspace_bytes, void* stream) {
  Shape s;
  HeadTable ht;
  int st = check_problem(p, &s);
  if (st) return st;
  if ((st = check_heads(s, k_per_head, &ht, nullptr))) return st;
  if (!Q || !K || !V || !idx || !O || !LSE) return DSA_ERR_INVALID_ARG;
  if (!aligned16(Q) || !aligned16(K) || !aligned16(V) || !aligned16(idx) || !aligned16(O) || !aligned16(LSE))
    return DSA_ERR_ALIGN;
  const size_t need = fwd_ws(s);
  if (need && (!workspace || workspace_bytes < need)) return DSA_ERR_WORKSPACE;
  if (need && !aligned16(workspace)) return DSA_ERR_ALIGN;
  DSA_CHECK_LISTS(s, ht, idx, cnt, nullptr, nullptr, stream, cnt ? "sparse_attn_fwd_varlen" : "sparse_attn_fwd");
  return hip_status(dsa::launch_attn_fwd(s, Q, K, V, idx, O, LSE, fwd_work(s, workspace), ht, 1,
                                         static_cast<hipStream_t>(stream), cnt));
}

int dsa_sparse_attn_fwd(const dsa_problem* p, const void* Q, const void* K, const void* V, const int32_t* idx,
                        const int32_t* k_per_head, float* O, float* LSE, void* workspace, size_t workspace_bytes,
                        void* stream) {
  return fwd_impl(p, Q, K, V, idx, nullptr, k_per_head, O, LSE, workspace, workspace_bytes, stream);
}

int dsa_sparse_attn_fwd_varlen(const dsa_problem* p, const void* Q, const void* K, const void* V, const int32_t* idx,
                               const int32_t* cnt, const int32_t* k_per_head, float* O, float* LSE, void* workspace,
                               size_t workspace_bytes, void* stream) {
  if (!cnt) return DSA_ERR_INVALID_ARG;
  if (!aligned16(cnt)) return DSA_ERR_ALIGN;
  return fwd_impl(p, Q, K, V, idx, cnt, k_per_head, O, LSE, workspace, workspace_bytes, stream);
}

int dsa_sparse_attn_fwd_split(const dsa_problem* p, const void* Q, const void* K, const void* V, const int32_t* idx,
                              const int32_t* k_per_head, int n_split, float* O_part, float* LSE_part,
                              void* workspace, size_t workspace_bytes, void* stream) {
  Shape s;
  HeadTable ht;
  int st = check_problem(p, &s);
  if (st) return st;
  if ((st = check_heads(s, k_per_head, &ht, nullptr))) return st;
  if (n_split < 1 || n_split > DSA_MAX_SPLIT) return DSA_ERR_INVALID_ARG;
  if (!Q || !K || !V || !idx || !O_part || !LSE_part) return DSA_ERR_INVALID_ARG;
  if (!aligned16(Q) || !aligned16(K) || !aligned16(V) || !aligned16(idx) || !aligned16(O_part) ||
      !aligned16(LSE_part))
    return DSA_ERR_ALIGN;
  const size_t need = fwd_ws(s);
  if (need && (!workspace || workspace_bytes < need)) return DSA_ERR_WORKSPACE;
  if (need && !aligned16(workspace)) return DSA_ERR_ALIGN;
  DSA_CHECK_LISTS(s, ht, idx, nullptr, nullptr, nullptr, stream, "sparse_attn_fwd_split");
  return hip_status(dsa::launch_attn_fwd(s, Q, K, V, idx, O_part, LSE_part, fwd_work(s, workspace), ht, n_split,
                                         static_cast<hipStream_t>(stream)));
}

int dsa_attn_merge(const dsa_problem* p, int n_parts, const float* O_part, const float* LSE_part, float* O,
                   float* LSE, void* stream) {
  Shape s;
  int st = check_problem(p, &s);
  if (st) return st;
  if (n_parts < 1 || n_parts > DSA_MAX_SPLIT) return DSA_ERR_INVALID_ARG;
  if (!O_part || !LSE_part || !O || !LSE) return DSA_ERR_INVALID_ARG;
  if (!aligned16(O_part) || !aligned16(LSE_part) || !aligned16(O) || !aligned16(LSE)) return DSA_ERR_ALIGN;
  return hip_status(dsa::launch_attn_merge(s, n_parts, O_part, LSE_part, O, LSE, static_cast<hipStream_t>(stream)));
}

static int check_bwd_common(const dsa_problem* p, const int32_t* k_per_head, Shape* s, HeadTable* ht) {
  int st = check_problem(p, s);
  if (st) return st;
  if (!s->bf16) return DSA_ERR_DTYPE;
  return check_heads(*s, k_per_head, ht, nullptr);
}

static int check_ws(const Shape& s, const void* workspace, size_t workspace_bytes) {
  if (!workspace || workspace_bytes < bwd_ws(s)) return DSA_ERR_WORKSPACE;
  return aligned16(workspace) ? DSA_OK : DSA_ERR_ALIGN;
}

int dsa_sparse_attn_bwd_preprocess_ex(const dsa_problem* p, const void* Q, const void* K, const void* V,
                                      const float* O, const void* dO, const float* LSE, int flags, void* workspace,
                                      size_t workspace_bytes, void* stream) {
  Shape s;
  int st = check_problem(p, &s);
  if (st) return st;
  if (!s.bf16) return DSA_ERR_DTYPE;
  if (flags & ~DSA_BWD_V_FROM_FORWARD) return DSA_ERR_INVALID_ARG;
  if (!Q || !K || !V || !O || !dO || !LSE) return DSA_ERR_INVALID_ARG;
  if (!aligned16(Q) || !aligned16(K) || !aligned16(V) || !aligned16(O) || !aligned16(dO) || !aligned16(LSE))
    return DSA_ERR_ALIGN;
  if ((st = check_ws(s, workspace, workspace_bytes))) return st;
  return hip_status(dsa::launch_bwd_pre(s, Q, K, V, O, dO, LSE, bwd_work(s, workspace),
                                        (flags & DSA_BWD_V_FROM_FORWARD) != 0, static_cast<hipStream_t>(stream)));
}

int dsa_sparse_attn_bwd_preprocess(const dsa_problem* p, const void* Q, const void* K, const void* V, const float* O,
                                   const void* dO, const float* LSE, void* workspace, size_t workspace_bytes,
                                   void* stream) {
  return dsa_sparse_attn_bwd_preprocess_ex(p, Q, K, V, O, dO, LSE, 0, workspace, workspace_bytes, stream);
}

int dsa_sparse_attn_bwd_dkdv(const dsa_problem* p, const void* Q, const void* K, const void* V, const void* dO,
                             const int32_t* k_per_head, const int32_t* rev_ptr, const int32_t* rev_idx, float* dK,
                             float* dV, void* workspace, size_t workspace_bytes, void* stream) {
  Shape s;
  HeadTable ht;
  int st = check_bwd_common(p, k_per_head, &s, &ht);
  if (st) return st;
  if (!Q || !K || !V || !dO || !rev_ptr || !rev_idx || !dK || !dV) return DSA_ERR_INVALID_ARG;
  if (!aligned16(Q) || !aligned16(K) || !aligned16(V) || !aligned16(dO) || !aligned16(rev_ptr) ||
      !aligned16(rev_idx) || !aligned16(dK) || !aligned16(dV))
    return DSA_ERR_ALIGN;
  if ((st = check_ws(s, workspace, workspace_bytes))) return st;
  DSA_CHECK_LISTS(s, ht, nullptr, nullptr, rev_ptr, rev_idx, stream, "sparse_attn_bwd_dkdv");
  return hip_status(dsa::launch_bwd_dkdv(s, bwd_work(s, workspace), Q, K, V, dO, rev_ptr, rev_idx, dK, dV, ht,
                                         static_cast<hipStream_t>(stream)));
}

int dsa_sparse_attn_bwd_dq(const dsa_problem* p, const void* Q, const void* dO, const int32_t* idx,
                           const int32_t* k_per_head, float* dQ, void* workspace, size_t workspace_bytes,
                           void* stream) {
  Shape s;
  HeadTable ht;
  int st = check_bwd_common(p, k_per_head, &s, &ht);
  if (st) return st;
  if (!Q || !dO || !idx || !dQ) return DSA_ERR_INVALID_ARG;
  if (!aligned16(Q) || !aligned16(dO) || !aligned16(idx) || !aligned16(dQ)) return DSA_ERR_ALIGN;
  if ((st = check_ws(s, workspace, workspace_bytes))) return st;
  DSA_CHECK_LISTS(s, ht, idx, nullptr, nullptr, nullptr, stream, "sparse_attn_bwd_dq");
  return hip_status(dsa::launch_bwd_dq(s, bwd_work(s, workspace), Q, dO, idx, dQ, ht, static_cast<hipStream_t>(stream)));
}

static int bwd_impl(const dsa_problem* p, const void* Q, const void* K, const void* V, const float* O, const void* dO,
                    const float* LSE, const int32_t* idx, const int32_t* cnt, const int32_t* k_per_head,
                    const int32_t* rev_ptr, const int32_t* rev_idx, float* dQ, float* dK, float* dV, int flags,
                    void* workspace, size_t workspace_bytes, void* stream) {
  Shape s;
  HeadTable ht;
  int st = check_bwd_common(p, k_per_head, &s, &ht);
  if (st) return st;
  if (flags & ~DSA_BWD_V_FROM_FORWARD) return DSA_ERR_INVALID_ARG;
  if (!Q || !K || !V || !O || !dO || !LSE || !idx || !rev_ptr || !rev_idx || !dQ || !dK || !dV)
    return DSA_ERR_INVALID_ARG;
  if (!aligned16(Q) || !aligned16(K) || !aligned16(V) || !aligned16(O) || !aligned16(dO) || !aligned16(LSE) ||
      !aligned16(idx) || !aligned16(rev_ptr) || !aligned16(rev_idx) || !aligned16(dQ) || !aligned16(dK) ||
      !aligned16(dV))
    return DSA_ERR_ALIGN;
  if ((st = check_ws(s, workspace, workspace_bytes))) return st;
  DSA_CHECK_LISTS(s, ht, idx, cnt, rev_ptr, rev_idx, stream, cnt ? "sparse_attn_bwd_varlen" : "sparse_attn_bwd");
  hipStream_t hs = static_cast<hipStream_t>(stream);
  const dsa::BwdWork w = bwd_work(s, workspace);
  hipError_t e = dsa::launch_bwd_pre(s, Q, K, V, O, dO, LSE, w, (flags & DSA_BWD_V_FROM_FORWARD) != 0, hs);
  if (e == hipSuccess) e = dsa::launch_bwd_dkdv(s, w, Q, K, V, dO, rev_ptr, rev_idx, dK, dV, ht, hs);
  if (e == hipSuccess) e = dsa::launch_bwd_dq(s, w, Q, dO, idx, dQ, ht, hs, cnt);
  return hip_status(e);
}

int dsa_sparse_attn_bwd(const dsa_problem* p, const void* Q, const void* K, const void* V, const float* O,
                        const void* dO, const float* LSE, const int32_t* idx, const int32_t* k_per_head,
                        const int32_t* rev_ptr, const int32_t* rev_idx, float* dQ, float* dK, float* dV,
                        void* workspace, size_t workspace_bytes, void* stream) {
  return bwd_impl(p, Q, K, V, O, dO, LSE, idx, nullptr, k_per_head, rev_ptr, rev_idx, dQ, dK, dV, 0, workspace,
                  workspace_bytes, stream);
}

int dsa_sparse_attn_bwd_ex(const dsa_problem* p, const void* Q, const void* K, const void* V, const float* O,
                           const void* dO, const float* LSE, const int32_t* idx, const int32_t* k_per_head,
                           const int32_t* rev_ptr, const int32_t* rev_idx, float* dQ, float* dK, float* dV, int flags,
                           void* workspace, size_t workspace_bytes, void* stream) {
  return bwd_impl(p, Q, K, V, O, dO, LSE, idx, nullptr, k_per_head, rev_ptr, rev_idx, dQ, dK, dV, flags, workspace,
                  workspace_bytes, stream);
}

int dsa_sparse_attn_bwd_varlen(const dsa_problem* p, const void* Q, const void* K, const void* V, const float* O,
                               const void* dO, const float* LSE, const int32_t* idx, const int32_t* cnt,
                               const int32_t* k_per_head, const int32_t* rev_ptr, const int32_t* rev_idx, float* dQ,
                               float* dK, float* dV, void* workspace, size_t workspace_bytes, void* stream) {
  if (!cnt) return DSA_ERR_INVALID_ARG;
  if (!aligned16(cnt)) return DSA_ERR_ALIGN;
  return bwd_impl(p, Q, K, V, O, dO, LSE, idx, cnt, k_per_head, rev_ptr, rev_idx, dQ, dK, dV, 0, workspace,
                  workspace_bytes, stream);
}

int dsa_dense_attn_fwd(const dsa_problem* p, const void* Q, const void* K, const void* V, float* O, float* LSE,
                       void* workspace, size_t workspace_bytes, void* stream) {
  Shape s;
  int st = check_problem(p, &s);
  if (st) return st;
  if (!Q || !K || !V || !O || !LSE) return DSA_ERR_INVALID_ARG;
  if (!aligned16(Q) || !aligned16(K) || !aligned16(V) || !aligned16(O) || !aligned16(LSE)) return DSA_ERR_ALIGN;
  const size_t need = fwd_ws(s);
  if (need && (!workspace || workspace_bytes < need)) return DSA_ERR_WORKSPACE;
  if (need && !aligned16(workspace)) return DSA_ERR_ALIGN;
  return hip_status(dsa::launch_attn_fwd(s, Q, K, V, nullptr, O, LSE, fwd_work(s, workspace), dense_heads(s), 1,
                                         static_cast<hipStream_t>(stream)));
}

int dsa_dense_attn_bwd(const dsa_problem* p, const void* Q, const void* K, const void* V, const float* O,
                       const void* dO, const float* LSE, float* dQ, float* dK, float* dV, void* workspace,
                       size_t workspace_bytes, void* stream) {
  Shape s;
  int st = check_problem(p, &s);
  if (st) return st;
  if (!s.bf16) return DSA_ERR_DTYPE;
  if (!Q || !K || !V || !O || !dO || !LSE || !dQ || !dK || !dV) return DSA_ERR_INVALID_ARG;
  if (!aligned16(Q) || !aligned16(K) || !aligned16(V) || !aligned16(O) || !aligned16(dO) || !aligned16(LSE) ||
      !aligned16(dQ) || !aligned16(dK) || !aligned16(dV))
    return DSA_ERR_ALIGN;
  if ((st = check_ws(s, workspace, workspace_bytes))) return st;
  hipStream_t hs = static_cast<hipStream_t>(stream);
  const dsa::BwdWork w = bwd_work(s, workspace);
  const HeadTable ht = dense_heads(s);
  hipError_t e = dsa::launch_bwd_pre(s, Q, K, V, O, dO, LSE, w, false, hs);
  if (e == hipSuccess) e = dsa::launch_bwd_dkdv(s, w, Q, K, V, dO, nullptr, nullptr, dK, dV, ht, hs);
  if (e == hipSuccess) e = dsa::launch_bwd_dq(s, w, Q, dO, nullptr, dQ, ht, hs);
  return hip_status(e);
}

int dsa_predictor_loss_grad(const dsa_problem* p, const void* Q, const void* K, const float* Wq, const float* Wk,
                            float* loss, float* dWq, float* dWk, void* workspace, size_t workspace_bytes,
                            void* stream) {
  Shape s;
  int st = check_problem(p, &s);
  if (st) return st;
  if (!Q || !K || !Wq || !Wk || !loss || !dWq || !dWk) return DSA_ERR_INVALID_ARG;
  if (!aligned16(Q) || !aligned16(K) || !aligned16(Wq) || !aligned16(Wk) || !aligned16(loss) || !aligned16(dWq) ||
      !aligned16(dWk))
    return DSA_ERR_ALIGN;
  if ((size_t)s.B * s.H * s.NG * s.NB >= ((size_t)1 << 31)) return DSA_ERR_UNSUPPORTED;
  if (!workspace || workspace_bytes < pred_ws(s)) return DSA_ERR_WORKSPACE;
  if (!aligned16(workspace)) return DSA_ERR_ALIGN;
  return hip_status(dsa::launch_predictor_loss_grad(s, Q, K, Wq, Wk, pred_work(s, workspace), loss, dWq, dWk,
                                                    static_cast<hipStream_t>(stream)));
}

int dsa_choose_path(const dsa_problem* p, const int32_t* k_per_head, double min_sparsity, size_t max_sparse_bytes) {
  Shape s;
  HeadTable ht;
  int st = check_problem(p, &s);
  if (st) return st;
  if (!k_per_head) return DSA_ERR_INVALID_ARG;
  memset(&ht, 0, sizeof(ht));
  int64_t kept = 0;
  for (int h = 0; h < s.H; ++h) {
    if (k_per_head[h] < 1 || k_per_head[h] > s.NB) return DSA_ERR_SHAPE;
    kept += k_per_head[h];
  }
  if (!(min_sparsity >= 0.0)) min_sparsity = DSA_DEFAULT_MIN_SPARSITY;  // negative or NaN: the default
  const double sparsity = 1.0 - (double)kept / ((double)s.H * s.NB);
  if (!(sparsity > min_sparsity)) return DSA_PATH_DENSE;
  if (check_heads(s, k_per_head, &ht, nullptr)) return DSA_PATH_DENSE;  // lists beyond the sparse limits
  if (max_sparse_bytes && sparse_extra_bytes(s, ht) > max_sparse_bytes) return DSA_PATH_DENSE;
  return DSA_PATH_SPARSE;
}

}  // extern "C"
