/*
 * sparse_attn.h -- C ABI of the dynamic block-sparse self-attention path on
 * one MI355X (gfx950): block pooling -> block scores -> top-p / top-k block
 * selection -> CSR block lists -> per-head KV demand union and packed gather
 * -> flash-style attention over the selected blocks only.
 *
 * The operation is the one the source pages describe in words:
 *  - "Dynamic Sparsity in Large-Scale Video DiT Training" (DSV explainer),
 *    section "The idea": rank query-key pairs with a cheap surrogate (here the
 *    block means, or a per-head low-rank predictor of inner dimension 16),
 *    keep the critical ones, let neighbouring queries (one query block) share
 *    one selected key/value set, and compute attention only on that set with
 *    kernels that never build the full score matrix.
 *  - The Top-p sparse-attention abstract (mlsift listing, tag "sequence
 *    parallelism"): Top-p routing with a Top-k safety floor over blocks of
 *    video tokens, producing a materialised block mask.
 *  - "SparSP: Exploiting Communication Sparsity for Sequence-Parallel Video
 *    DiTs", Abstract: only the KV blocks some query block demands are moved;
 *    one GPU's part of that is the demand union and its contiguous gather.
 *
 * Conventions shared by every entry point
 *  - Pointers are DEVICE pointers unless marked (host).  The library never
 *    allocates, frees, caches or keeps a pointer: the caller owns every
 *    buffer, including the workspace (size from sa_workspace_size).
 *  - Calls only enqueue work on `stream` (a hipStream_t; NULL = the default
 *    stream) and never synchronise.  Outputs are ready when the stream is.
 *  - Q, K, V are contiguous row-major [H, rows, d] with d innermost, rows a
 *    multiple of the block size B; rows at or beyond the valid count must be
 *    zero.  Every block holds at least one valid row: rows == ceil(valid/B)*B.
 *  - Return value: SA_OK (0) or a negative sa_status.  Argument errors are
 *    detected on the host before any HIP call is made.  A packed-buffer
 *    overflow, which depends on device data, is reported through the
 *    `dev_status` word of kv_demand_pack.
 *  - Identical inputs give bit-identical outputs (no floating-point atomics
 *    on any output path).
 *  - Calls on different streams are independent as long as their output and
 *    workspace buffers do not overlap.
 */
#ifndef SPARSE_ATTN_H
#define SPARSE_ATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum sa_status {
  SA_OK = 0,
  SA_ERR_INVALID_ARG = -1,  /* null pointer, bad size, misaligned buffer      */
  SA_ERR_UNSUPPORTED = -2,  /* valid but not built: head_dim/block/dtype mix  */
  SA_ERR_WORKSPACE = -3,    /* workspace smaller than sa_workspace_size       */
  SA_ERR_HIP = -4,          /* a HIP launch failed                            */
  SA_ERR_CAPACITY = -5,     /* demand union larger than the packed buffers    */
  SA_ERR_SCRATCH = -6       /* problem larger than the static scratch array of
                               sparse_attn_forward_noalloc                    */
} sa_status;

typedef enum sa_dtype { SA_F32 = 0, SA_BF16 = 1 } sa_dtype;
typedef enum sa_select_mode { SA_TOP_P = 0, SA_TOP_K = 1 } sa_select_mode;
typedef enum sa_score_mode {
  SA_SCORE_POOLED = 0,      /* block means, scaled dot product                    */
  SA_SCORE_LOWRANK = 1,     /* mean over the block pair of rank-r predicted scores */
  SA_SCORE_LOWRANK_MAX = 2, /* max over the block pair of rank-16 predicted token
                               scores (rank must be 16)                            */
  SA_SCORE_LOWRANK_MASS = 3 /* ln of the block pair's predicted softmax mass from
                               rank-16 token scores (rank must be 16)              */
} sa_score_mode;
typedef enum sa_stage {
  SA_STAGE_SELECT = 0,   /* sparse_attn_select         */
  SA_STAGE_CSR = 1,      /* sparse_attn_csr_from_mask  */
  SA_STAGE_PACK = 2,     /* kv_demand_pack             */
  SA_STAGE_FORWARD = 3,  /* sparse_attn_forward        */
  SA_STAGE_BACKWARD = 4, /* sparse_attn_backward       */
  SA_STAGE_FUSED = 5     /* sparse_attn_fused          */
} sa_stage;

/* Problem description (host struct, read during the call only).
 * Notation: H = num_heads (batch folded in), d = head_dim, B = block,
 * nQB = q_rows / B, nKB = kv_rows / B, W = ceil(nKB / 32).
 * Size limits (else SA_ERR_UNSUPPORTED): nKB <= 4096, H*nQB*nKB < 2^31,
 * H*nQB < 2^30, H*kv_rows*d < 2^40. */
typedef struct sa_problem {
  int32_t num_heads;    /* H >= 1                                             */
  int32_t head_dim;     /* d: 64 or 128 (bf16 attention: 128)                */
  int32_t block;        /* B: 64 or 128 (bf16 attention: 128); query blocks
                           and key blocks have the same size                  */
  int32_t dtype;        /* sa_dtype of Q, K, V, the output and packed K/V     */
  int64_t q_rows;       /* nQB * B                                            */
  int64_t q_valid;      /* q_rows - B < q_valid <= q_rows                     */
  int64_t kv_rows;      /* nKB * B, nKB <= 4096                               */
  int64_t kv_valid;     /* kv_rows - B < kv_valid <= kv_rows                  */
  float sm_scale;       /* attention logit scale; <= 0 means 1/sqrt(d)        */
  float score_scale;    /* pooled block-score scale and the temperature of
                           SA_SCORE_LOWRANK_MASS; <= 0 means 1/sqrt(d)        */
  int32_t select_mode;  /* sa_select_mode                                     */
  float top_p;          /* SA_TOP_P: mass to reach, > 0; >= 1 keeps all       */
  int32_t top_k;        /* SA_TOP_P: floor (>= 0); SA_TOP_K: k (>= 1); both
                           are clamped to nKB                                 */
  int32_t score_mode;   /* sa_score_mode                                      */
  int32_t rank;         /* low-rank modes: predictor rank r, 1..64 (16 for the
                           token-level MAX and MASS modes)                    */
} sa_problem;

/* Workspace bytes needed by one entry point (`stage`) for this problem.
 * bytes: host pointer.  The workspace passed to that entry point must be at
 * least this large and 256-byte aligned; its contents need not be preserved
 * between calls. */
int sa_workspace_size(const sa_problem* prob, int stage, size_t* bytes);

/* Pool, score and select (DSV explainer "The idea"; Top-p abstract).
 *
 *   qbar[h,i] = mean of the valid rows of query block i   (fp64)
 *   kbar[h,j] = mean of the valid rows of key block j      (fp64)
 *   SA_SCORE_POOLED : S[h,i,j] = score_scale * <qbar[h,i], kbar[h,j]>
 *   SA_SCORE_LOWRANK: S[h,i,j] = <qbar[h,i] Wq[h], kbar[h,j] Wk[h]>, i.e. the
 *                     mean over the block pair of the rank-r predicted
 *                     token-pair scores
 *   SA_SCORE_LOWRANK_MAX: S[h,i,j] = max over valid tokens a of block i and b
 *                     of block j of <q_a Wq[h], k_b Wk[h]> (rank 16; the
 *                     projections are fp64 sums and the token-pair scores
 *                     fp64 dot products on the matrix cores, so S is exact
 *                     to fp64 rounding)
 *   SA_SCORE_LOWRANK_MASS: with the predicted token scores read as logits
 *                     z_ab = tau <q_a Wq[h], k_b Wk[h]> (tau = score_scale,
 *                     0 -> 1/sqrt(d); valid keys only), S[h,i,j] = ln of the
 *                     mean over valid queries a of block i of the softmax
 *                     mass sum_{b in j} exp(z_ab) / sum_b exp(z_ab).  Rows of
 *                     exp(S) sum to one, so SA_TOP_P's softmax gives back the
 *                     masses.  Rank 16; token scores as for
 *                     SA_SCORE_LOWRANK_MAX; each exponential is 2^n exp2(f)
 *                     with f in [-1, 0] formed in fp64 and exp2 in fp32, all
 *                     sums and logarithms fp64 (S within about 2^-22 of the
 *                     exact value); the workspace holds
 *                     ln sum_{b in j} exp(z_ab) for every query token and key
 *                     block in fp64 (8*H*nKB*q_rows bytes).
 *   SA_TOP_P: P = softmax_j S[h,i,:]; blocks ordered by P descending, ties to
 *             the lower j; keep the shortest prefix whose cumulative mass
 *             reaches top_p (all blocks if top_p >= 1 or the prefix never
 *             reaches it), extended to at least min(top_k, nKB) blocks.
 *   SA_TOP_K: keep the min(top_k, nKB) largest S, ties to the lower j.
 * All selection arithmetic is fp64.
 *
 * q [H,q_rows,d], k [H,kv_rows,d]: input dtype.
 * wq, wk: fp32 [H,d,rank] (the low-rank modes only; else ignored, may be NULL).
 * mask_bits: out, uint32 [H*nQB, W]; bit b of word w of row h*nQB+i is block
 *            32w+b; bits at or beyond nKB are 0.
 * row_ptr:   out, int32 [H*nQB+1], CSR row offsets (rows head-major).
 * col_idx:   out, int32, capacity H*nQB*nKB; entries of a row ascending.
 * qbar_opt, kbar_opt: NULL or out fp64 [H,nQB,d] / [H,nKB,d].
 * ws: workspace of sa_workspace_size(SA_STAGE_SELECT) bytes. */
int sparse_attn_select(const sa_problem* prob, const void* q, const void* k,
                       const float* wq, const float* wk, uint32_t* mask_bits,
                       int32_t* row_ptr, int32_t* col_idx, double* qbar_opt,
                       double* kbar_opt, void* ws, size_t ws_bytes, void* stream);

/* CSR of an externally given (for example repaired) block mask, the same
 * layout sparse_attn_select writes (Top-p abstract: the materialised mask).
 * mask_bits: in, uint32 [H*nQB, W] (bits beyond nKB are ignored).
 * row_ptr: out [H*nQB+1]; col_idx: out, capacity H*nQB*nKB. */
int sparse_attn_csr_from_mask(const sa_problem* prob, const uint32_t* mask_bits,
                              int32_t* row_ptr, int32_t* col_idx, void* ws,
                              size_t ws_bytes, void* stream);

/* Per-head KV demand union and packed gather (SparSP Abstract:
 * demand-directed KV routing; this is one GPU's share of it).
 *
 *   demanded[h] = union over the query blocks i of head h of their blocks
 *   demand_ptr [H+1]: out, head h owns slots demand_ptr[h] .. demand_ptr[h+1]-1
 *   demand_idx: out, capacity H*nKB; block id of each slot, ascending in a head
 *   col_slot:   out, capacity H*nQB*nKB; slot of each CSR entry
 *   k_packed, v_packed: out, [packed_cap_blocks, B, d] in the input dtype;
 *               slot s holds a bitwise copy of rows j*B .. j*B+B-1 of head h
 * row_ptr, col_idx: a CSR as written by the calls above.
 * dev_status: out, int32 [1]: 0, or SA_ERR_CAPACITY when the union exceeds
 *             packed_cap_blocks (then only the first packed_cap_blocks slots
 *             are copied; demand_ptr, demand_idx and col_slot are complete).
 * packed_cap_blocks >= 0. */
int kv_demand_pack(const sa_problem* prob, const int32_t* row_ptr,
                   const int32_t* col_idx, const void* k, const void* v,
                   int32_t* demand_ptr, int32_t* demand_idx, int32_t* col_slot,
                   void* k_packed, void* v_packed, int64_t packed_cap_blocks,
                   int32_t* dev_status, void* ws, size_t ws_bytes, void* stream);

/* Attention over the selected blocks only (DSV explainer "The idea": sparse
 * attention kernels that never build the full score matrix).
 *
 * For query a of block i of head h and key b of a selected block j:
 *   z = sm_scale * <q_a, k_b>, with keys b >= kv_valid excluded;
 *   out[h,a] = sum_b softmax(z)_b v_b,  lse[h,a] = ln sum_b exp(z_b).
 * Query rows a >= q_valid, and rows whose block selected nothing, get out = 0
 * and lse = -inf.  bf16 inputs use bf16 MFMA with fp32 accumulation; the
 * output has the input dtype (round to nearest even), lse is fp32.
 *
 * col_slot == NULL: k_src, v_src are the full K, V [H,kv_rows,d].
 * col_slot != NULL: k_src, v_src are packed [slots,B,d] and entry e reads
 *                   slot col_slot[e] (col_idx still gives the block id).
 * Work items (head, query block) are cut into eight contiguous ranges of
 * near-equal work, one per XCD, and taken in (head, query block) order within
 * a range, under the schedule SA_SCHEDULE_AUTO picks for the problem (see
 * sa_schedule).  When whole items would leave the device's last round of
 * work more than 5% idle, each item's block list is processed as two halves
 * whose partial results are combined in a fixed order, so results never
 * depend on timing; the workspace then also holds the halves' partial
 * states (66 KiB per item), and its size depends on the CU count of the
 * device that is current when sa_workspace_size is called.
 * out: [H,q_rows,d] input dtype; lse_opt: NULL or fp32 [H,q_rows]. */
int sparse_attn_forward(const sa_problem* prob, const void* q,
                        const int32_t* row_ptr, const int32_t* col_idx,
                        const int32_t* col_slot, const void* k_src,
                        const void* v_src, void* out, float* lse_opt, void* ws,
                        size_t ws_bytes, void* stream);

/* Work schedules of the attention forward (sparse_attn_forward_ex). */
typedef enum sa_schedule {
  SA_SCHEDULE_PERSISTENT = 0, /* two workgroups per CU take work units from
                                 per-XCD queues until all are done            */
  SA_SCHEDULE_PER_UNIT = 1,   /* one workgroup per work unit, handed out by the
                                 hardware dispatcher (the plain launch)       */
  SA_SCHEDULE_AUTO = 2        /* what sparse_attn_forward runs: PER_UNIT when
                                 prob->select_mode is SA_TOP_K (every row keeps
                                 the same number of blocks, so the dispatcher
                                 balances them and the queue only adds its
                                 pops), PERSISTENT otherwise (rows of unequal
                                 length, where the queue removes the
                                 stragglers of the Top-p abstract)             */
} sa_schedule;

/* Options of sparse_attn_forward_ex (host struct, read synchronously). */
typedef struct sa_forward_opts {
  int32_t schedule;    /* sa_schedule                                          */
  int32_t clock_cap;   /* capacity of wg_clock, in workgroups                  */
  uint64_t* wg_clock;  /* NULL, or device [clock_cap, 2]: for each workgroup of
                          the bf16 attention launch, the device's constant-rate
                          clock (s_memrealtime ticks) when it started and when
                          it found no more work                               */
} sa_forward_opts;

/* Workgroups of the bf16 attention launch under `schedule` for this problem
 * on the current device (an upper bound on the units for SA_SCHEDULE_PER_UNIT,
 * whose surplus workgroups exit at once).  workgroups: host pointer. */
int sa_forward_workgroups(const sa_problem* prob, int32_t schedule, int32_t* workgroups);

/* sparse_attn_forward with a chosen work schedule and optional per-workgroup
 * clock stamps, the measurement behind the load-imbalance figure (max over
 * mean of the workgroups' busy time) that the Top-p sparse-attention
 * abstract reports for its rank-level stragglers.  Results are bit-identical
 * to sparse_attn_forward's under every schedule.  The fp32 path always runs
 * one workgroup per item and writes no clock stamps.  SA_ERR_INVALID_ARG for
 * an unknown schedule, or a wg_clock with clock_cap below
 * sa_forward_workgroups.  opts == NULL is sparse_attn_forward. */
int sparse_attn_forward_ex(const sa_problem* prob, const void* q,
                           const int32_t* row_ptr, const int32_t* col_idx,
                           const int32_t* col_slot, const void* k_src,
                           const void* v_src, void* out, float* lse_opt, void* ws,
                           size_t ws_bytes, const sa_forward_opts* opts, void* stream);

/* Critical-KV estimation and sparse attention in one pass (DSV explainer,
 * "The idea": kernels that fuse the estimation of the critical keys and
 * values with the sparse attention, keep intermediates on chip and never
 * build the full score matrix).  The same result as sparse_attn_select
 * followed by sparse_attn_forward on the full K and V, but after the pooling
 * pass (block means, and their rank-r projections in SA_SCORE_LOWRANK) a
 * single kernel scores each query block against every key block of its head,
 * selects as sparse_attn_select does and attends to the kept blocks; no score
 * matrix, mask or CSR goes to memory.
 *   SA_TOP_K: the min(top_k, nKB) largest scores (ties to the lower block id).
 *   SA_TOP_P (Top-p abstract): the shortest prefix of the blocks ranked by
 *     softmax mass (fp64, ties to the lower id) whose cumulative mass reaches
 *     top_p, raised to min(top_k, nKB) blocks; top_p >= 1 keeps every block.
 *     The cumulative mass is summed exactly in 2^-62 fixed point rather than
 *     as a running fp64 sum.
 *   Supported: bf16, head_dim = block = 128, nKB <= 4096, score_mode
 *   SA_SCORE_POOLED or SA_SCORE_LOWRANK (rank <= 64); else
 *   SA_ERR_UNSUPPORTED.  Scores are fp64 (each a sequential fused
 *   multiply-add over the pooled dimension), so the kept sets equal
 *   sparse_attn_select's except where two ranking values tie to fp64
 *   rounding or, in SA_TOP_P, where top_p lies within rounding of the
 *   cumulative mass at the cut (one block more or fewer).
 * q [H,q_rows,d], k, v [H,kv_rows,d]: bf16; wq, wk: fp32 [H,d,rank] in
 *   SA_SCORE_LOWRANK (else ignored, may be NULL);
 * out [H,q_rows,d] bf16, lse_opt NULL or fp32 [H,q_rows]: as for
 *   sparse_attn_forward;
 * mask_bits_opt: NULL, or out uint32 [H*nQB, W] (the kept sets, laid out as
 *   sparse_attn_select writes them), for checking;
 * ws: workspace of sa_workspace_size(SA_STAGE_FUSED) bytes (the block means
 *   and projections, and in SA_TOP_P the counters of the per-XCD item
 *   queues, which the call zeroes itself). */
int sparse_attn_fused(const sa_problem* prob, const void* q, const void* k, const void* v,
                      const float* wq, const float* wk, void* out, float* lse_opt,
                      uint32_t* mask_bits_opt, void* ws, size_t ws_bytes, void* stream);

/* For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc):
 * sparse_attn_forward without a workspace argument.  Its work queue lives in
 * a file-scope device array of SA_NOALLOC_SCRATCH_BYTES bytes that the
 * library holds on every device it runs on until the process ends; the call
 * itself allocates nothing (no hipMalloc, hipFree or allocating library
 * routine).  It always processes whole items (never halves), so its results
 * are bit-identical to sparse_attn_forward's whenever that call does not
 * halve items, and otherwise equal up to the rounding of the halves'
 * combination.  The queue needs 12 bytes per (head, query block) item plus
 * 68 bytes; a problem needing more than SA_NOALLOC_SCRATCH_BYTES returns
 * SA_ERR_SCRATCH before any HIP call.  Every call on a device shares that
 * device's array (the queue kernel re-initialises what it reads), so calls
 * that overlap in time on one device, from several streams or threads, race
 * and must not be issued.  Other arguments as for sparse_attn_forward. */
#define SA_NOALLOC_SCRATCH_BYTES (1u << 20)
int sparse_attn_forward_noalloc(const sa_problem* prob, const void* q, const int32_t* row_ptr,
                                const int32_t* col_idx, const int32_t* col_slot,
                                const void* k_src, const void* v_src, void* out, float* lse_opt,
                                void* stream);

/* Gradients of sparse_attn_forward for an upstream gradient dout (the
 * training workload: the DSV explainer's speedups, "What it costs", are
 * training numbers).  With P = softmax(z) of the forward (same selected
 * blocks, same padding rules, P recomputed from lse):
 *   dV = P^T dO,  dP = dO V^T,  D = rowsum(dO * O),  dS = P * (dP - D),
 *   dQ = sm_scale dS K,  dK = sm_scale dS^T Q.
 * bf16 only, head_dim = block = 128 (else SA_ERR_UNSUPPORTED).
 * q, k, v: the forward's inputs, [H,q_rows,d] and full [H,kv_rows,d];
 * out, lse: the forward's outputs for these inputs and blocks;
 * dout: [H,q_rows,d], zero in padded rows;
 * row_ptr, col_idx: the CSR of the forward; column ids ascending and unique
 *   within each row (as sparse_attn_select / sparse_attn_csr_from_mask write);
 * dq [H,q_rows,d], dk, dv [H,kv_rows,d]: out, bf16 (fp32 accumulation, P and
 *   dS rounded to bf16 as MFMA operands); padded rows and key blocks that no
 *   query block selected get zero;
 * ws: workspace of sa_workspace_size(SA_STAGE_BACKWARD) bytes (D, the
 *   transposed block lists: per key block the query blocks that selected it,
 *   and the launch order of the dK/dV work: per head, longest lists first). */
int sparse_attn_backward(const sa_problem* prob, const void* q, const void* k, const void* v,
                         const void* out, const void* dout, const float* lse,
                         const int32_t* row_ptr, const int32_t* col_idx, void* dq, void* dk,
                         void* dv, void* ws, size_t ws_bytes, void* stream);

/* ---- video-aware block organisation --------------------------------------
 * The Top-p sparse-attention abstract (mlsift listing, tag "sequence
 * parallelism") organises video tokens into blocks in a video-aware way; the
 * page gives no layout.  Reading implemented here: the tokens of a
 * (frames, height, width) latent, raster order, are reordered so consecutive
 * positions fill 3-D tiles of (tile_t, tile_h, tile_w) tokens: tiles in
 * raster order over the tile grid, tokens in raster order inside a tile,
 * tiles at the far edges clipped to the latent.  The path then runs on the
 * reordered rows unchanged (blocks are runs of B consecutive positions); with
 * tile_t*tile_h*tile_w == B and dimensions divisible by the tile, every block
 * is one tile. */
typedef struct sa_video_tiling {   /* host struct, read synchronously */
  int32_t frames, height, width;   /* latent (T, Hl, Wl), each >= 1 */
  int32_t tile_t, tile_h, tile_w;  /* tile shape, each >= 1 */
} sa_video_tiling;

/* The orders of one latent and one query share (raster tokens q_start ..
 * q_start + q_valid - 1, 0 <= q_start, 1 <= q_valid, q_start + q_valid <= N,
 * N = frames * height * width < 2^31):
 *   kv_order[p]   = raster index of the token at position p        int32 [N]
 *   kv_inverse[r] = position of raster token r                     int32 [N]
 *   q_order[p]    = query-local raster row (0 .. q_valid-1) of the p-th
 *                   query token in kv_order                        int32 [q_valid]
 *   q_inverse[r]  = position in q_order of query-local row r       int32 [q_valid]
 * The query share keeps its tokens and takes them in the order they appear
 * in kv_order.  Computed on the device once per shape; no workspace. */
int sa_video_block_order(const sa_video_tiling* tiling, int64_t q_start, int64_t q_valid,
                         int32_t* kv_order, int32_t* kv_inverse, int32_t* q_order,
                         int32_t* q_inverse, void* stream);

/* Row gather for every head: dst[h, r] = src[h, idx[r]] for r < rows, and
 * dst[h, r] = 0 for rows <= r < dst_rows (the zero padding the path needs).
 * Rows are row_bytes bytes (a multiple of 4, at most 65536); src is
 * [heads, src_rows, row_bytes], dst [heads, dst_rows, row_bytes].  An index
 * outside [0, src_rows) yields a zero row.  With kv_order / q_order this puts
 * Q, K, V into the tiled layout; with q_inverse it brings O (row_bytes =
 * d * element size) and the LSE (row_bytes = 4) back to raster order.  src
 * and dst must not overlap; 16-byte aligned pointers and rows take the wide
 * path. */
int sa_permute_rows(int32_t heads, int64_t rows, int32_t row_bytes, const int32_t* idx,
                    const void* src, int64_t src_rows, void* dst, int64_t dst_rows,
                    void* stream);

/* Static description of a status code (never NULL). */
const char* sa_status_string(int status);

/* ABI version of this header: 8 (1, plus the video block order entry points
 * in 2, plus sparse_attn_backward in 3, plus sparse_attn_forward_ex and
 * sa_forward_workgroups in 4, plus sparse_attn_forward_noalloc and
 * SA_ERR_SCRATCH in 5, plus sparse_attn_fused and SA_STAGE_FUSED in 6, plus
 * SA_SCHEDULE_AUTO, the per-problem schedule sparse_attn_forward runs, in 7,
 * plus SA_TOP_P in sparse_attn_fused in 8). */
int sa_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* SPARSE_ATTN_H */
