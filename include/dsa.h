/*
 * dsa.h -- C ABI of the MI355X (gfx950) dynamic sparse attention library, libdsa.so.
 *
 * The method is DSV's ("DSV: Exploiting Dynamic Sparsity to Accelerate
 * Large-Scale Video DiT Training"; explainer pages at gist.science, Dutch and
 * Hindi editions, cited below as nl/hi with their technical-summary section):
 * a low-rank predictor estimates query-group x key-block attention scores, the
 * top-k "critical" KV blocks are kept per (head, query group), and exact
 * attention runs forward and backward over the kept blocks only.
 *
 * Conventions shared by every call
 * --------------------------------
 *  - Tensors are dense, row-major, [B, H, N, d] ("BHND", d innermost) unless
 *    stated.  Query groups are G consecutive tokens (G in {64, 128}); KV blocks
 *    are 64 consecutive tokens.  NG = N / G groups, NB = N / 64 blocks.
 *  - Q, K, V, dO are bf16 (DSA_BF16, stored as 16-bit patterns) or fp32
 *    (DSA_F32), as problem->dtype says.  Predictor weights and every output
 *    (scores, qhat, khat, O, LSE, dQ, dK, dV) are fp32.  tau = 1/sqrt(d).
 *  - Kept-block lists ("idx") are ragged by head: head h keeps k_h blocks per
 *    group, 1 <= k_h <= NB.  Row (b, h, g) holds k_h int32 block ids in
 *    ascending order, starting at element row_base[b*H + h] + g * k_h, where
 *    row_base is given by dsa_index_layout.  rev_idx has the same total length.
 *  - All pointers except k_per_head are DEVICE pointers owned by the caller;
 *    the library never allocates, frees or retains memory (beside the one
 *    static per-GPU scratch array of dsa_select_topk_blocks_noalloc, part of
 *    the loaded code object).  k_per_head is a
 *    HOST array of H int32, read during the call only.  Device buffers must be
 *    16-byte aligned.  Scratch memory comes from a caller-provided workspace
 *    whose size dsa_workspace_bytes returns.
 *  - Every compute call is asynchronous on the given HIP stream (a
 *    hipStream_t passed as void*, NULL = the null stream) and does not
 *    synchronise.  Arguments are validated on the host before anything is
 *    launched; on error nothing is launched and a negative status is returned.
 *  - Calls on one stream may be issued from any thread; the library holds no
 *    mutable global state other than that scratch array (see its call).
 *  - Limits: d in {64, 128}; rank r in {8, 16, 32, 64}; H <= 128;
 *    NB <= 8192 (N <= 524288); B*H*NG*max(k_h) < 2^31.
 *  - Lists are taken as written by the selection calls: each idx row strictly
 *    ascending in [0, NB) (with counts: the first cnt entries, the rest -1),
 *    rev_ptr starting at 0 and non-decreasing, each reverse list strictly
 *    ascending in [0, NG).  The release library clamps every id it reads
 *    into range, so a malformed list gives wrong results, never an access out
 *    of bounds.  The debug build (libdsa_debug.so, compiled with DSA_DEBUG)
 *    checks the lists of every attention call on the device first,
 *    synchronises the stream, prints the first bad entry to stderr and returns
 *    DSA_ERR_BAD_LIST without launching the attention kernels.
 */
#ifndef DSA_H_
#define DSA_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  DSA_OK = 0,
  DSA_ERR_INVALID_ARG = -1,   /* null pointer, bad enum, NULL problem */
  DSA_ERR_SHAPE = -2,         /* sizes not supported / not divisible */
  DSA_ERR_DTYPE = -3,         /* dtype not supported for this call */
  DSA_ERR_ALIGN = -4,         /* a device pointer not 16-byte aligned */
  DSA_ERR_UNSUPPORTED = -5,   /* combination outside the limits above */
  DSA_ERR_WORKSPACE = -6,     /* workspace missing or too small */
  DSA_ERR_HIP = -7,           /* a HIP launch or runtime call failed */
  DSA_ERR_SCRATCH_LIMIT = -8, /* a call without a workspace needs more than its static scratch */
  DSA_ERR_BAD_LIST = -9       /* debug builds only: a kept-block list or reverse index is malformed */
} dsa_status;

typedef enum { DSA_F32 = 0, DSA_BF16 = 1 } dsa_dtype;

typedef struct {
  int32_t batch;      /* B */
  int32_t heads;      /* H */
  int32_t seq_len;    /* N tokens per sequence */
  int32_t head_dim;   /* d */
  int32_t rank;       /* predictor rank r (d_lr) */
  int32_t group;      /* query-group size G */
  int32_t block;      /* KV block size, must be 64 */
  int32_t dtype;      /* dsa_dtype of Q, K, V, dO */
} dsa_problem;

/* Which call a workspace is sized for. */
typedef enum {
  DSA_WS_SELECT = 0,
  DSA_WS_BWD = 1,
  DSA_WS_FWD = 2,
  DSA_WS_PRED_GRAD = 3,
  DSA_WS_PRED_POOLED = 4
} dsa_ws_call;

/* Library version string. */
const char* dsa_version(void);

/* Static, human-readable text of a status code. */
const char* dsa_status_string(int status);

/*
 * dsa_index_layout: host-only helper.  Writes row_base[0 .. B*H] (B*H + 1
 * int64 entries, host memory): the element offset of each (b, h) region of the
 * kept-block list; row_base[B*H] is the total number of entries.
 */
int dsa_index_layout(const dsa_problem* p, const int32_t* k_per_head, int64_t* row_base);

/*
 * Bytes of workspace the given call needs (0 if the arguments are invalid).
 * k_per_head may be NULL for DSA_WS_FWD, DSA_WS_BWD, DSA_WS_PRED_GRAD and
 * DSA_WS_PRED_POOLED, whose sizes do not depend on it (the dense calls and
 * the predictor calls take no kept counts).
 */
size_t dsa_workspace_bytes(const dsa_problem* p, const int32_t* k_per_head, int which_call);

/*
 * dsa_predict_block_scores -- the low-rank sparsity predictor (hi §2.A, nl §2.A;
 * query grouping with a proxy query, hi §2.B).
 *   qhat[b,h,g,:]   = mean_{i in group g} Q[b,h,i,:] . Wq[h]      [B,H,NG,r] fp32
 *   khat[b,h,j,:]   = mean_{m in block j} K[b,h,m,:] . Wk[h]      [B,H,NB,r] fp32
 *   scores[b,h,g,j] = tau * qhat[b,h,g,:] . khat[b,h,j,:]         [B,H,NG,NB] fp32
 * Wq, Wk: [H, d, r] fp32.  scores may be NULL (then only qhat, khat are
 * written; dsa_select_topk_blocks can stream the scores itself).
 */
int dsa_predict_block_scores(const dsa_problem* p, const void* Q, const void* K,
                             const float* Wq, const float* Wk, float* qhat, float* khat,
                             float* scores, void* stream);

/* Poolings of dsa_predict_block_scores_pooled. */
#define DSA_POOL_MAX 1
#define DSA_POOL_LSE 2

/*
 * dsa_predict_block_scores_pooled -- a predictor variant (not from the pages,
 * which pool with a proxy query, hi §2.B): every token is projected,
 * l[i,m] = tau (Q_i.Wq[h]) . (K_m.Wk[h]), and each G x 64 tile of these
 * logits is pooled into scores[b,h,g,j]:
 *   DSA_POOL_MAX: max_{i in g, m in j} l[i,m];
 *   DSA_POOL_LSE: ln( mean_{i in g, m in j} exp(l[i,m]) ), the predicted
 *                 attention mass of the tile per key pair, in log form.
 * The projections are rounded to fp16 (workspace) and the products run on
 * fp16 MFMA with fp32 accumulation (|projections| must stay below 65504).
 * scores: [B,H,NG,NB] fp32, then usable by every selection call.
 * Workspace: dsa_workspace_bytes(p, NULL, DSA_WS_PRED_POOLED).  Other
 * pooling values: DSA_ERR_INVALID_ARG.
 */
int dsa_predict_block_scores_pooled(const dsa_problem* p, const void* Q, const void* K, const float* Wq,
                                    const float* Wk, int pooling, float* scores, void* workspace,
                                    size_t workspace_bytes, void* stream);

/*
 * dsa_select_topk_blocks -- critical KV block selection (hi §2.A critical KV
 * estimation; hi §2.B / nl §2.B fused low-rank MatMul + top-k).
 * For each (b, h, g): the k_h block ids j with the largest scores[b,h,g,j],
 * ties broken towards the lowest j (-0.0 equals +0.0), written ascending to
 * idx.  If scores is NULL the scores are recomputed from qhat/khat inside the
 * kernel, bit-identical to dsa_predict_block_scores' and never stored (the
 * O(S*k) memory mode); scores_dump, if not NULL, then receives them
 * [B,H,NG,NB] (debug/checking only).
 * Also builds the reverse index: rev_ptr [B*H, NB+1] int32 holds, per (b, h),
 * offsets into that (b, h)'s region of rev_idx (same row_base as idx); the
 * segment of block j lists, ascending, every group g whose row kept j.
 * Workspace: dsa_workspace_bytes(p, k_per_head, DSA_WS_SELECT).
 */
int dsa_select_topk_blocks(const dsa_problem* p, const float* scores, const float* qhat,
                           const float* khat, const int32_t* k_per_head, int32_t* idx,
                           int32_t* rev_ptr, int32_t* rev_idx, float* scores_dump,
                           void* workspace, size_t workspace_bytes, void* stream);

/*
 * dsa_sparse_attn_fwd -- exact attention over the kept blocks only (hi §2.A
 * stage 2; nl §2.A fase 2).  For query i of group g and the keys m of the
 * blocks in idx row (b,h,g): l_im = tau Q_i.K_m, LSE_i = ln sum_m exp(l_im),
 * O_i = sum_m exp(l_im - LSE_i) V_m.  No causal mask.
 * O: [B,H,N,d] fp32; LSE: [B,H,N] fp32 (natural log).
 * Workspace: dsa_workspace_bytes(p, k_per_head, DSA_WS_FWD) (for bf16 inputs:
 * a scaled fp16 copy of V and its per-(b, h) exponent; 0 bytes, NULL allowed,
 * for fp32 inputs).  A DSA_WS_BWD workspace is accepted as well: the
 * forward's part is its first part, so the backward can reuse the copy
 * (DSA_BWD_V_FROM_FORWARD).
 * Input range: any finite bf16 values.  The forward's P V and the backward's
 * dQ products run on fp16 operands: V and K are copied to fp16 per (b, h)
 * slice, and the dQ kernel converts each wave's 32 rows of Q and dO, each
 * multiplied by the power of two that puts the largest magnitude of its
 * slice (or rows) in [2^a, 2^(a+1)) (a = 3 for V, 2 for dO, 14 for Q and K);
 * the results are scaled back exactly.  Values more than 2^-(a+14) below
 * that largest magnitude (fp16 subnormals after scaling) keep fewer
 * significant bits, and below 2^-(a+24) of it they count as zero.  The
 * backward's dK/dV products run on bf16 operands (fp32's range) straight
 * from the inputs.
 * When one head's K and V copies (4*N*d bytes) fill more than half of the
 * 256 MiB Infinity Cache, the call runs as several launches over segments of
 * every list, the later ones merging into O and LSE in place; O and LSE hold
 * partial states until the call's work on the stream has finished.
 */
int dsa_sparse_attn_fwd(const dsa_problem* p, const void* Q, const void* K, const void* V,
                        const int32_t* idx, const int32_t* k_per_head, float* O, float* LSE,
                        void* workspace, size_t workspace_bytes, void* stream);

/*
 * dsa_sparse_attn_bwd -- gradient of sum(dO * O) for the forward above, the
 * selection held fixed (the pages describe a training system, hi §2 and §3;
 * the gradient itself is the standard softmax-attention one on the kept keys):
 *   D_i = dO_i.O_i, P = exp(l - LSE), dS = P (dO V^T - D),
 *   dQ_g = tau dS K, dK_m = tau sum dS^T Q, dV_m = sum P^T dO,
 * keys of blocks no group kept get dK = dV = 0.  Needs the forward's O and
 * LSE, and rev_ptr/rev_idx from dsa_select_topk_blocks.  dQ, dK, dV:
 * [B,H,N,d] fp32.  bf16 inputs only.  Deterministic (no atomics).  For
 * heads beyond half the Infinity Cache (as for the forward) the dQ and dK/dV
 * stages run as several launches that add into dQ, dK, dV in place.
 * Workspace: dsa_workspace_bytes(p, k_per_head, DSA_WS_BWD).
 */
int dsa_sparse_attn_bwd(const dsa_problem* p, const void* Q, const void* K, const void* V,
                        const float* O, const void* dO, const float* LSE, const int32_t* idx,
                        const int32_t* k_per_head, const int32_t* rev_ptr, const int32_t* rev_idx,
                        float* dQ, float* dK, float* dV, void* workspace, size_t workspace_bytes,
                        void* stream);

/* Flags of dsa_sparse_attn_bwd_ex and dsa_sparse_attn_bwd_preprocess_ex. */
#define DSA_BWD_V_FROM_FORWARD 1

/*
 * dsa_sparse_attn_bwd_ex -- dsa_sparse_attn_bwd with flags (0: the same call).
 * DSA_BWD_V_FROM_FORWARD: the workspace is the one the forward of these inputs
 * (the same problem and V) was given, and nothing has written it since; the
 * backward then reuses the scaled fp16 copy of V the forward left there
 * instead of converting V again (a training step converts V once).  The
 * results are the same bits either way.  Other flags: DSA_ERR_INVALID_ARG.
 */
int dsa_sparse_attn_bwd_ex(const dsa_problem* p, const void* Q, const void* K, const void* V,
                           const float* O, const void* dO, const float* LSE, const int32_t* idx,
                           const int32_t* k_per_head, const int32_t* rev_ptr, const int32_t* rev_idx,
                           float* dQ, float* dK, float* dV, int flags, void* workspace,
                           size_t workspace_bytes, void* stream);

/* Bytes of the static per-GPU scratch of dsa_select_topk_blocks_noalloc. */
#define DSA_NOALLOC_SCRATCH_BYTES (16u << 20)

/*
 * dsa_select_topk_blocks_noalloc -- dsa_select_topk_blocks for callers that
 * cannot allocate device memory or pass a workspace: code under HIP graph
 * capture, tight serving loops, harnesses that forbid allocation.  Same
 * arguments (minus the workspace), same results bit for bit; no allocating
 * call is made.  Its scratch (what DSA_WS_SELECT would hold) is a static
 * device array of DSA_NOALLOC_SCRATCH_BYTES on each GPU the library runs
 * on, kept until the process ends; problems whose DSA_WS_SELECT size exceeds
 * it return DSA_ERR_SCRATCH_LIMIT before anything is launched (16 MiB holds
 * the 57,600-token layer with k = 90 and the 131,072-token layer with
 * k = 102, 24 heads each).  Every call on one GPU shares that array: calls
 * that overlap on one GPU (on different streams, or from several threads
 * without ordering) race and give undefined lists; calls ordered on one
 * stream do not (each call writes all the scratch it reads).
 */
int dsa_select_topk_blocks_noalloc(const dsa_problem* p, const float* scores, const float* qhat,
                                   const float* khat, const int32_t* k_per_head, int32_t* idx,
                                   int32_t* rev_ptr, int32_t* rev_idx, float* scores_dump, void* stream);

/*
 * Selection by attention coverage (hi §2.A: the critical KV pairs are the
 * ones that carry about 90% of the attention score), with per-row counts.
 *
 * dsa_select_coverage_blocks -- as dsa_select_topk_blocks, except that row
 * (b,h,g) keeps the shortest run of blocks, in the order of decreasing score
 * (ties towards the lowest id), whose estimated attention mass reaches
 * `coverage` of the row's total, and at most k_h blocks (k_per_head is the
 * per-head capacity of the rows).  Each block holds 64 keys and its score
 * estimates their mean logit, so the estimated masses are the softmax of the
 * row's scores, computed in fp32 (exp(s_j - max s), summed per wave).
 * Writes the kept count to cnt[b,h,g] (int32 [B,H,NG], 1 <= cnt <= k_h), the
 * cnt ascending ids to the first slots of the row (same layout as idx, rows
 * k_h entries apart) and -1 to the unused slots; rev_ptr/rev_idx index the
 * kept entries only.  0 < coverage <= 1, else DSA_ERR_INVALID_ARG.  Where the
 * cumulative mass comes within fp32 rounding of the target, the run may end
 * earlier or later than an exact computation would (at coverage 1, blocks
 * whose mass is below fp32 resolution of the total are not needed).
 * Workspace DSA_WS_SELECT.
 */
int dsa_select_coverage_blocks(const dsa_problem* p, const float* scores, const float* qhat,
                               const float* khat, const int32_t* k_per_head, double coverage, int32_t* idx,
                               int32_t* cnt, int32_t* rev_ptr, int32_t* rev_idx, float* scores_dump,
                               void* workspace, size_t workspace_bytes, void* stream);

/* Flags of dsa_select_blocks. */
#define DSA_SELECT_DIAGONAL 1

/*
 * dsa_select_blocks -- the general selection call.  coverage == 0: each row
 * keeps its top k_h blocks (dsa_select_topk_blocks; cnt is not written and
 * may be NULL); 0 < coverage <= 1: the coverage rule of
 * dsa_select_coverage_blocks (cnt required).  flags: 0, or
 * DSA_SELECT_DIAGONAL: the blocks holding the row's own G query tokens
 * (blocks g*G/64 .. (g+1)*G/64 - 1) are always kept and come first in the
 * selection order, ahead of every score (a variant, not from the pages: a
 * local window next to the predicted blocks); in coverage mode their
 * estimated masses count towards the target.  With it every k_h must be at
 * least G/64 (else DSA_ERR_SHAPE).  Other flags, or coverage outside
 * [0, 1]: DSA_ERR_INVALID_ARG.  Output layout, workspace and the other
 * arguments as dsa_select_topk_blocks / dsa_select_coverage_blocks.
 */
int dsa_select_blocks(const dsa_problem* p, const float* scores, const float* qhat, const float* khat,
                      const int32_t* k_per_head, double coverage, int flags, int32_t* idx, int32_t* cnt,
                      int32_t* rev_ptr, int32_t* rev_idx, float* scores_dump, void* workspace,
                      size_t workspace_bytes, void* stream);

/*
 * dsa_sparse_attn_fwd_varlen / dsa_sparse_attn_bwd_varlen -- the forward and
 * backward above for rows of different lengths: row (b,h,g) attends to the
 * first cnt[b,h,g] blocks of its idx row (counts outside [1, k_h] are
 * clamped to it).  idx, cnt, rev_ptr and rev_idx as written by
 * dsa_select_coverage_blocks.  Other arguments, workspaces and errors as
 * dsa_sparse_attn_fwd / dsa_sparse_attn_bwd.
 */
int dsa_sparse_attn_fwd_varlen(const dsa_problem* p, const void* Q, const void* K, const void* V,
                               const int32_t* idx, const int32_t* cnt, const int32_t* k_per_head, float* O,
                               float* LSE, void* workspace, size_t workspace_bytes, void* stream);
int dsa_sparse_attn_bwd_varlen(const dsa_problem* p, const void* Q, const void* K, const void* V,
                               const float* O, const void* dO, const float* LSE, const int32_t* idx,
                               const int32_t* cnt, const int32_t* k_per_head, const int32_t* rev_ptr,
                               const int32_t* rev_idx, float* dQ, float* dK, float* dV, void* workspace,
                               size_t workspace_bytes, void* stream);

/* Most parts a split-KV forward or a merge takes. */
#define DSA_MAX_SPLIT 64

/*
 * dsa_sparse_attn_fwd_split -- split-KV forward: attention of every query over
 * one part of its group's kept blocks, as a partial state (DSV hi §2.C sparse
 * sequence-wise CP: a device attends to the critical KV it holds; DiTango
 * explainer, nl edition, Methodologie: attention states, output and
 * log-sum-exp, compose associatively and commutatively).
 * The kept list of row (b,h,g) (k_h ascending ids) is cut into n_split
 * contiguous parts; part s holds list positions [s k_h / n_split,
 * (s+1) k_h / n_split) (integer division).  For every part s and query i of the
 * group, over the keys m of the part's blocks:
 *   LSE_part[s][b,h,i] = ln sum_m exp(tau Q_i.K_m),
 *   O_part[s][b,h,i,:] = sum_m exp(tau Q_i.K_m - LSE_part[s][b,h,i]) V_m;
 * an empty part (n_split > k_h) gives O = 0 and LSE = -inf.  Merging the parts
 * with dsa_attn_merge gives dsa_sparse_attn_fwd's O and LSE.
 * O_part: [n_split, B, H, N, d] fp32; LSE_part: [n_split, B, H, N] fp32;
 * 1 <= n_split <= DSA_MAX_SPLIT (else DSA_ERR_INVALID_ARG).  Workspace, other
 * arguments and errors as dsa_sparse_attn_fwd (DSA_WS_FWD).
 */
int dsa_sparse_attn_fwd_split(const dsa_problem* p, const void* Q, const void* K, const void* V,
                              const int32_t* idx, const int32_t* k_per_head, int n_split, float* O_part,
                              float* LSE_part, void* workspace, size_t workspace_bytes, void* stream);

/*
 * dsa_attn_merge -- combine n_parts partial attention states per query row
 * (DiTango explainer, nl edition, Methodologie: state composition):
 *   LSE = ln sum_s exp(LSE_part[s]),  O = sum_s exp(LSE_part[s] - LSE) O_part[s];
 * a part with LSE = -inf adds nothing; if every part has -inf, O = 0 and
 * LSE = -inf.  O_part [n_parts, B, H, N, d] and LSE_part [n_parts, B, H, N]
 * fp32 as written by dsa_sparse_attn_fwd_split (or by other devices'
 * partial forwards over other blocks); O [B, H, N, d], LSE [B, H, N] fp32.
 * Only batch, heads, seq_len and head_dim of p are read beyond validation.
 * 1 <= n_parts <= DSA_MAX_SPLIT; all pointers 16-byte aligned device memory.
 */
int dsa_attn_merge(const dsa_problem* p, int n_parts, const float* O_part, const float* LSE_part, float* O,
                   float* LSE, void* stream);

/*
 * The three stages dsa_sparse_attn_bwd runs, exposed one launch group each,
 * sharing the DSA_WS_BWD workspace (D_i = dO_i . O_i, -LSE*log2(e) and the
 * scaled fp16 copies of K and V with their exponents, written by the
 * preprocess stage; V's copy may come from the forward, see
 * DSA_BWD_V_FROM_FORWARD):
 *   dsa_sparse_attn_bwd_preprocess  fills the workspace from K, V, O, dO, LSE
 *                                   (Q is not read; _ex: with the flags of
 *                                   dsa_sparse_attn_bwd_ex);
 *   dsa_sparse_attn_bwd_dkdv        dK, dV from the reverse index and the bf16
 *                                   inputs Q, K, V, dO (every key row of every
 *                                   block is written); it also writes its own
 *                                   task order (blocks with long reverse lists
 *                                   first) into the workspace before the launch;
 *   dsa_sparse_attn_bwd_dq          dQ from the kept-block lists, Q, dO and the
 *                                   workspace.
 */
int dsa_sparse_attn_bwd_preprocess(const dsa_problem* p, const void* Q, const void* K, const void* V, const float* O,
                                   const void* dO, const float* LSE, void* workspace, size_t workspace_bytes,
                                   void* stream);
int dsa_sparse_attn_bwd_preprocess_ex(const dsa_problem* p, const void* Q, const void* K, const void* V,
                                      const float* O, const void* dO, const float* LSE, int flags, void* workspace,
                                      size_t workspace_bytes, void* stream);
int dsa_sparse_attn_bwd_dkdv(const dsa_problem* p, const void* Q, const void* K, const void* V, const void* dO,
                             const int32_t* k_per_head, const int32_t* rev_ptr, const int32_t* rev_idx, float* dK,
                             float* dV, void* workspace, size_t workspace_bytes, void* stream);
int dsa_sparse_attn_bwd_dq(const dsa_problem* p, const void* Q, const void* dO, const int32_t* idx,
                           const int32_t* k_per_head, float* dQ, void* workspace, size_t workspace_bytes,
                           void* stream);

/*
 * The OP dispatcher's branches (hi and nl §2.A, stage 2: per transformer
 * block, sparse attention is switched on only when the block's sparsity
 * exceeds a threshold set by offline profiling of speedup against memory
 * overhead; otherwise the block keeps the full attention of stage 1).
 *
 * dsa_dense_attn_fwd -- full attention, every query over every key:
 *   LSE_i = ln sum_m exp(tau Q_i.K_m),  O_i = sum_m exp(tau Q_i.K_m - LSE_i) V_m,
 * i.e. dsa_sparse_attn_fwd with k_h = NB and every block kept, without index
 * lists.  Same dtypes, layouts, workspace (DSA_WS_FWD, k_per_head NULL) and
 * errors as dsa_sparse_attn_fwd.
 */
int dsa_dense_attn_fwd(const dsa_problem* p, const void* Q, const void* K, const void* V, float* O,
                       float* LSE, void* workspace, size_t workspace_bytes, void* stream);

/*
 * dsa_dense_attn_bwd -- gradient of sum(dO * O) for dsa_dense_attn_fwd (the
 * formulas of dsa_sparse_attn_bwd over all keys).  bf16 inputs only;
 * workspace DSA_WS_BWD (k_per_head NULL); deterministic.
 */
int dsa_dense_attn_bwd(const dsa_problem* p, const void* Q, const void* K, const void* V, const float* O,
                       const void* dO, const float* LSE, float* dQ, float* dK, float* dV, void* workspace,
                       size_t workspace_bytes, void* stream);

/*
 * dsa_predictor_loss_grad -- stage-1 training of the low-rank predictor (hi
 * and nl §2.A, stage 1: the per-head predictors are trained beside the full
 * attention of normal training, by a loss that keeps the relative magnitude of
 * the estimated scores).  Per (b, h), with qbar/kbar the group/block means of
 * Q/K (qhat = qbar Wq[h], khat = kbar Wk[h] as in dsa_predict_block_scores):
 *   diff[g,j] = tau (qhat_g.khat_j - qbar_g.kbar_j)  (the block score minus
 *               the mean of tau Q K^T over the G x 64 tile),
 *   E[g,j]    = diff[g,j] - mean_j diff[g,j]          (each row centred),
 *   loss[h]   = mean over b, g, j of E^2,
 *   dWq[h]    = 2 tau / (B NG NB) sum_b qbar^T E khat,
 *   dWk[h]    = 2 tau / (B NG NB) sum_b kbar^T E^T qhat   (the gradients of loss[h]).
 * Q, K: [B,H,N,d] bf16 or fp32; Wq, Wk: [H,d,r] fp32; loss [H], dWq, dWk
 * [H,d,r] fp32 (overwritten).  Workspace: dsa_workspace_bytes(p, NULL,
 * DSA_WS_PRED_GRAD) (means, projections, E and partial sums, all fp32).
 * Deterministic.  B*H*NG*NB >= 2^31: DSA_ERR_UNSUPPORTED.
 */
int dsa_predictor_loss_grad(const dsa_problem* p, const void* Q, const void* K, const float* Wq, const float* Wk,
                            float* loss, float* dWq, float* dWk, void* workspace, size_t workspace_bytes,
                            void* stream);

typedef enum { DSA_PATH_DENSE = 0, DSA_PATH_SPARSE = 1 } dsa_path;

/*
 * Sparsity above which the sparse training step (predict, select, forward,
 * backward) beats the dense one (forward, backward) on these kernels: a
 * sweep of the kept fraction on MI355X put the break-even at a sparsity of
 * 0.06 for a 57,600-token, 24-head, d = 128 layer and at 0 for an
 * 8,192-token, 16-head, d = 64 one (the larger is taken).  Forward-only
 * callers (break-even 0.03 and 0.09 there), or callers with their own
 * profile, pass their own threshold.
 */
#define DSA_DEFAULT_MIN_SPARSITY 0.06

/*
 * dsa_choose_path -- the dispatcher's decision for one attention layer (host
 * only; reads k_per_head, launches nothing).  With the sparsity
 *   s = 1 - sum_h k_h / (H * NB)   (the fraction of (head, group, block)
 *                                   tiles the selection skips),
 * returns DSA_PATH_SPARSE iff s > min_sparsity, the kept lists fit the sparse
 * calls' limits, and (when max_sparse_bytes > 0) the device memory the sparse
 * path needs beyond the dense one -- qhat, khat, idx, rev_ptr, rev_idx and the
 * DSA_WS_SELECT workspace, block scores streamed -- is at most
 * max_sparse_bytes; otherwise DSA_PATH_DENSE.  min_sparsity < 0 (or NaN)
 * selects DSA_DEFAULT_MIN_SPARSITY.  Negative status on invalid arguments
 * (k_h outside [1, NB]: DSA_ERR_SHAPE).
 */
int dsa_choose_path(const dsa_problem* p, const int32_t* k_per_head, double min_sparsity,
                    size_t max_sparse_bytes);

#ifdef __cplusplus
}
#endif

#endif /* DSA_H_ */
