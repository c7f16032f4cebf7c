/*
 * sol_attn.h - C ABI of the Sol-Attn sparse attention forward on AMD Instinct
 * MI355X (gfx950).
 *
 * What is computed. Page "Sol-Attn: Accelerating Video Generation Inference
 * via On-the-Fly Attention Sparsification" (paperlayer.ai summary of arXiv
 * 2607.24027):
 *   - §2 "Block-Sparse Attention": q and k are cut into blocks of Bq and Bk
 *     consecutive tokens; each (query block i, key block j) pair gets a proxy
 *     score from the block means,  s_ij = mean(q_i) . mean(k_j) / sqrt(d).
 *   - §3 "Dynamic threshold routing" / "On-the-fly sparsification": a
 *     query-dependent threshold selects blocks on chip, without a proxy map or
 *     routing indices in device memory. Here the threshold is the row maximum
 *     minus tau: block j is kept for query block i iff s_ij >= max_j' s_ij' - tau
 *     (ties kept, so the best block is always kept; tau = +inf is dense).
 *   - §3 "Approximate correction": kept blocks get exact attention; every
 *     skipped block j adds exp(s_ij - m) * n_j * mean(v_j) to the softmax
 *     numerator and exp(s_ij - m) * n_j to the denominator of every row of
 *     query block i, n_j being the number of tokens in block j.
 *   - §3 "Unified execution": exact and corrected terms share one
 *     online-softmax state, so for row r of query block i
 *       out_r = (sum_kept_t e^{x_rt} v_t + sum_skip_j n_j e^{s_ij} vbar_j)
 *             / (sum_kept_t e^{x_rt}     + sum_skip_j n_j e^{s_ij}),
 *     x_rt = q_r . k_t / sqrt(d) (stabilised by a common maximum).
 *   - §2 "Attention and Online Softmax", App. B: forward only, bidirectional,
 *     no masks; a ragged last block pools only its valid tokens.
 *
 * Layouts. q, k, v: bf16, contiguous [B][H][N][d], d fastest. out: fp32, same
 * shape. kpool, vmean: fp32 [B][H][Nk][d] with Nk = ceil(N/Bk). Pointers are
 * device pointers and must be 16-byte aligned.
 *
 * Ownership. The caller allocates and frees every buffer. The library never
 * allocates device memory, never copies between host and device and never
 * synchronises: each call validates its arguments on the host and enqueues
 * kernels on `stream` (a hipStream_t; NULL = the default stream), then
 * returns. Device-side faults surface at the caller's next synchronisation.
 *
 * Errors. Every entry point returns SOL_OK or a negative code, and validates
 * all arguments before any launch; on an error nothing has been enqueued.
 *
 * Re-entrancy. Calls are stateless apart from the caller's workspace: two
 * forwards that overlap in time (different streams) need separate workspaces.
 */
#ifndef SOL_ATTN_H
#define SOL_ATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Return codes. */
enum {
  SOL_OK = 0,
  SOL_EINVAL = -1,       /* null or misaligned pointer, size <= 0, tau NaN or < 0, bad flag */
  SOL_EUNSUPPORTED = -2, /* d not in {64, 128}, Bq != 64, Bk != 64, or N too large */
  SOL_EWORKSPACE = -3,   /* workspace smaller than sol_attn_workspace_bytes() */
  SOL_EHIP = -4,         /* the HIP runtime refused a launch or a query */
  SOL_ESCRATCH = -5      /* sol_attn_forward_noalloc: the problem needs more than SOL_ATTN_SCRATCH_BYTES */
};

/* Flags of sol_attn_forward. */
enum {
  /* kpool/vmean already hold sol_attn_pool() of these k and v: skip that pass. */
  SOL_F_POOLED = 1u << 0,
  /* Ablation: drop skipped blocks instead of correcting them (keep-or-drop).
   * With SOL_ROUTE_GAUSS or SOL_ROUTE_GAUSS_DIAG it needs a sink range
   * (SOL_EINVAL otherwise): a Gaussian threshold above a query block's best
   * proxy keeps nothing, which leaves that block's rows without any term. */
  SOL_F_EXACT_ONLY = 1u << 1,
  /* The workspace holds the result of sol_attn_plan() (for these shapes;
   * ideally for these q, kpool and tau), possibly followed by other forwards
   * on it: launch only the fused kernel, taking the items in the planned
   * order. The order only schedules work, so a plan made for other inputs
   * of the same shapes gives the same result, only scheduled worse; a plan
   * made for another number of work items (the automatic group size depends
   * on tau) is ignored and the items go in sequence. A workspace that was
   * never planned must not be used with this flag. Requires SOL_F_POOLED. */
  SOL_F_PLANNED = 1u << 2,
  /* Token-to-block correction (§3 "Unified execution": one score tile per
   * query row and key block; App. B analyses one query row): a skipped block
   * j adds, for every row r of the query block, the logit q_r . kbar_j /
   * sqrt(d) (instead of the block's s_ij) with weight n_j and value vbar_j.
   * Routing stays block-level. Computed in bf16 MFMA tiles over the pooled
   * keys and values (bf16-rounded copies made in the workspace), in the same
   * online softmax as the kept blocks. Not with SOL_F_EXACT_ONLY. */
  SOL_F_ROW_CORRECTION = 1u << 3,
  /* `out` is bf16 [B][H][N][d] instead of fp32: the same fp32 result, rounded
   * to nearest even as it is stored (half the output bytes). */
  SOL_F_OUT_BF16 = 1u << 4,
  /* Bits 5-6, 8 and 9: query blocks per work item of the fused kernel; the
   * group's routing pass reads the head's pooled keys and values once for
   * all of them. None set (the default): chosen by the library. For
   * row-max routing with tau <= 4 the largest of 16, 8 (both only up to
   * 2048 key blocks) and 6 that gives the call at least 4 such items per
   * CU; otherwise 8 when there are at least 6 items per CU and at most 2048
   * key blocks, else 4 under the item rule, else 2. SOL_F_GROUP2 / 4 / 6 /
   * 8 / 16 ask for a size; 8 and 16 need ceil(N/64) <= 2048
   * (SOL_EUNSUPPORTED otherwise); two sizes at once, or any size with
   * SOL_F_PLANNED, is SOL_EINVAL. The size only schedules work: results
   * agree within floating-point rounding (sums are taken in another order),
   * and are bitwise reproducible for a given size. */
  SOL_F_GROUP2 = 1u << 5,
  SOL_F_GROUP4 = 2u << 5,
  SOL_F_GROUP8 = 3u << 5,
  SOL_F_GROUP16 = 1u << 8,
  SOL_F_GROUP6 = 1u << 9,
  /* The workspace holds sol_attn_prepare() of these q, kpool and vmean (with
   * the same SOL_F_ROW_CORRECTION bit): skip the pre-pass. Requires
   * SOL_F_POOLED. With SOL_F_PLANNED only the fused kernel is launched. */
  SOL_F_PREPARED = 1u << 7
};
#define SOL_F_GROUP_SHIFT 5
#define SOL_F_GROUP_MASK (3u << SOL_F_GROUP_SHIFT)

/* Routing rules of sol_attn_forward_ex (§3 "Dynamic threshold routing":
 * a query-dependent threshold on the block proxy scores s_ij). */
enum {
  /* keep key block j of query block i iff s_ij >= max_j s_ij - tau */
  SOL_ROUTE_ROWMAX = 0,
  /* keep iff s_ij >= mean_j s_ij + beta * std_j s_ij: the Gaussian-calibrated
   * threshold with a shared standardized cutoff beta (population statistics
   * over the key blocks of the row), computed before any score from the
   * head's pooled-key first and second moments (App. B "Threshold variance
   * derivation"): mean = qbar_i . m_K / sqrt(d), var = qbar_i^T C_K qbar_i / d,
   * m_K and C_K the mean and population covariance of the pooled keys
   * (O(d^2) per head, in the workspace); the scores are then routed chunk by
   * chunk as they are produced (§3 "On-the-fly sparsification") */
  SOL_ROUTE_GAUSS = 1,
  /* the same threshold with the diagonal estimator of App. B "Diagonal
   * threshold estimator": mean_j s_ij = qbar_i . m_K / sqrt(d) and
   * var_j s_ij ~= sum_c qbar_ic^2 v_Kc / d, from the mean m_K and the
   * per-dimension (population) variance v_K of the head's pooled keys, so the
   * threshold is known before the proxy row is formed. Forward only. */
  SOL_ROUTE_GAUSS_DIAG = 2
};

/* Routing of sol_attn_forward_ex, read from HOST memory during the call. */
typedef struct sol_attn_route {
  int rule;        /* SOL_ROUTE_ROWMAX or SOL_ROUTE_GAUSS */
  float tau;       /* ROWMAX: 0 <= tau <= +inf (ignored by GAUSS) */
  float beta;      /* GAUSS: any finite value (ignored by ROWMAX) */
  int sink_first;  /* key blocks sink_first .. sink_first + sink_count - 1 are */
  int sink_count;  /* always kept, computed exactly (App. A: text key-value    */
                   /* tokens retained as sinks); sink_count = 0: none          */
} sol_attn_route;

/* Largest supported sequence length: the kept bits and the kept list of a
 * query block are held on chip (4096 key blocks). */
#define SOL_ATTN_MAX_N (4096 * 64)

/* Per-call counters, written by sol_attn_forward into DEVICE memory: every
 * field is overwritten when the forward's last workgroup finishes. */
typedef struct sol_attn_stats {
  unsigned long long kept_blocks;  /* number of kept (i, j) block pairs */
  unsigned long long total_blocks; /* B * H * Nq * Nk */
  unsigned long long kept_pairs;   /* sum over kept (i, j) of n_i * n_j: exact query-key pairs */
  unsigned int min_kept;           /* fewest kept blocks of any query block */
  unsigned int max_kept;           /* most kept blocks of any query block */
} sol_attn_stats;

/* Bytes of device workspace sol_attn_forward and sol_attn_plan need: the
 * work-queue and stats words, one cost and one order slot per pair of query
 * blocks, the pooled queries [B][H][Nq][d] (fp32), the routing pass's bf16
 * operand planes of the pooled keys (three parts) and values, each
 * [B][H][Nk rounded up to 64][d], bf16 pooled values [B][H][Nk][d] for
 * SOL_F_ROW_CORRECTION, the pooled-key statistics [B][H][2][d] of
 * SOL_ROUTE_GAUSS_DIAG and the pooled-key mean and covariance
 * [B][H][d + 1][d] of SOL_ROUTE_GAUSS. Returns 0 for unsupported sizes. */
size_t sol_attn_workspace_bytes(int B, int H, int N, int d, int Bq, int Bk);

/*
 * Pooling pre-pass (§2 "Block-Sparse Attention" mean pooling; §3 "Approximate
 * correction": pooled keys and summed values = n_j * mean).
 *   kpool[b][h][j][:] = mean of k[b][h][t][:] over the valid tokens t of block j
 *   vmean[b][h][j][:] = mean of v[b][h][t][:] over the same tokens
 * k, v: bf16 [B][H][N][d]; kpool, vmean: fp32 [B][H][ceil(N/Bk)][d], written.
 * Means are accumulated in fp32.
 */
int sol_attn_pool(const void* k, const void* v, float* kpool, float* vmean,
                  int B, int H, int N, int d, int Bk, void* stream);

/*
 * The planning stage of the forward, callable on its own for forwards with
 * SOL_F_PLANNED (e.g. one plan reused over several diffusion steps of a
 * layer): for finite tau, estimates every work item's kept budget (bf16
 * products of query means sampled from every 4th row and the pooled keys)
 * and orders each work queue: its first two thirds in sequence (neighbouring
 * query blocks keep overlapping key blocks and share them in L2), its last
 * third heaviest first; an item estimated at a quarter of the head's key
 * blocks or more (its routing pass then a small part of it) is handed out
 * one pair of query blocks at a time, each routing the item again. A
 * scheduling aid only: the forward still routes every block itself, in
 * fp32, and nothing routing-related is written to device memory beyond one
 * count per item and the order. For tau = +inf (and very large B*H*N)
 * the order is the identity. The items are those of the forward's automatic
 * group size at this tau (their count is recorded with the order). Resets
 * the workspace's queue and stats words.
 *   q         bf16 [B][H][N][d]
 *   kpool     fp32 [B][H][Nk][d], sol_attn_pool() of k
 *   workspace as for sol_attn_forward
 */
int sol_attn_plan(const void* q, const float* kpool, int B, int H, int N, int d, int Bq, int Bk, float tau,
                  void* workspace, size_t workspace_bytes, void* stream);

/*
 * The forward's pre-pass on its own, for forwards with SOL_F_PREPARED (so that
 * a caller or a benchmark can launch and time the fused kernel alone): pools
 * q (fp32 [B][H][Nq][d] in the workspace) and writes the routing pass's bf16
 * operand planes of kpool and vmean into the workspace (section "pooling
 * pre-pass" of the forward below), one launch.
 *   q          bf16 [B][H][N][d]
 *   kpool, vmean  fp32 [B][H][Nk][d], sol_attn_pool() of k and v
 *   flags      0 or SOL_F_ROW_CORRECTION (also writes the row-major bf16
 *              pooled values that mode reads)
 *   workspace  as for sol_attn_forward; only its prepared regions are
 *              written (the queue words and any plan are left as they are)
 * Errors: SOL_EINVAL for null or misaligned pointers or other flags, those
 * of the sizes as for sol_attn_forward, SOL_EWORKSPACE, SOL_EHIP.
 */
int sol_attn_prepare(const void* q, const float* kpool, const float* vmean, int B, int H, int N, int d, int Bq,
                     int Bk, unsigned flags, void* workspace, size_t workspace_bytes, void* stream);

/*
 * Sparse attention forward with proxy correction (all sections cited above).
 *   q, k, v   bf16 [B][H][N][d] (read)
 *   out       fp32 [B][H][N][d] (written), or bf16 with SOL_F_OUT_BF16
 *   tau       threshold offset in natural-log units, 0 <= tau <= +inf
 *   flags     SOL_F_* bits
 *   stats     device sol_attn_stats or NULL
 *   kpool, vmean  fp32 [B][H][Nk][d]; written by the pre-pass unless
 *                 SOL_F_POOLED, in which case they are read as given
 *   workspace device memory of at least sol_attn_workspace_bytes() bytes,
 *             256-byte aligned; its content on entry does not matter unless
 *             SOL_F_PLANNED is set. Every forward leaves its queue and stats
 *             words clean.
 * Launches the pooling pre-pass (means of q, and of k and v unless
 * SOL_F_POOLED; the routing pass's bf16 operand planes of the pooled keys and
 * values; a reset of the workspace words unless SOL_F_PLANNED), the planning
 * kernels of sol_attn_plan where the order repays them (row-max rule with
 * 8 <= tau < +inf, where the per-block budgets spread widest, at most 4096
 * items and at least 2^21 query-block x key-block pairs in the call) and one
 * fused kernel; with SOL_F_PLANNED no planning kernel, with SOL_F_PREPARED
 * no pre-pass (then a one-workgroup reset unless SOL_F_PLANNED). The fused
 * kernel's persistent grid takes groups of query blocks from eight atomic
 * queues (one per XCD, each over a contiguous range of items, stealing from
 * the others once drained); for each it routes the group in one pass over
 * the pooled keys and values on the matrix cores (scores consumed as they
 * are produced), then, pair by pair, runs bf16 MFMA attention over the kept
 * key blocks with an online softmax and folds the skipped blocks' correction
 * into the same accumulator. Two calls that share a workspace must not
 * overlap in time.
 */
int sol_attn_forward(const void* q, const void* k, const void* v, void* out,
                     int B, int H, int N, int d, int Bq, int Bk, float tau,
                     unsigned flags, sol_attn_stats* stats,
                     float* kpool, float* vmean,
                     void* workspace, size_t workspace_bytes, void* stream);

/*
 * sol_attn_forward with a routing rule and forced-keep sink blocks.
 *   route       host pointer to the routing parameters (not NULL)
 *   kept_bitmap NULL, or as for sol_attn_forward_debug
 * All other arguments, the launches and the errors are those of
 * sol_attn_forward; in addition SOL_EINVAL for an unknown rule, a NaN or
 * negative tau (ROWMAX), a non-finite beta (GAUSS), or a sink range outside
 * 0 .. ceil(N/Bk) - 1, and for SOL_F_EXACT_ONLY under a Gaussian rule with
 * sink_count = 0. sol_attn_forward(..., tau, ...) is this call with
 * {SOL_ROUTE_ROWMAX, tau, 0, 0, 0}.
 */
int sol_attn_forward_ex(const void* q, const void* k, const void* v, void* out,
                        int B, int H, int N, int d, int Bq, int Bk,
                        const sol_attn_route* route, unsigned flags, sol_attn_stats* stats,
                        float* kpool, float* vmean,
                        void* workspace, size_t workspace_bytes, void* stream,
                        uint32_t* kept_bitmap);

/*
 * Routing alone: the kept-block bitmap, without attention. Three routers with
 * one output layout (that of sol_attn_forward_debug), for comparing routing
 * costs (§2 "Block-Sparse Attention": top-k sets a fixed budget, top-p a
 * dynamic one, both traversing the proxy scores; §4 "Efficient On-the-Fly
 * Sparsification" compares their cost with on-chip threshold routing).
 *   q          bf16 [B][H][N][d]; kpool fp32 [B][H][Nk][d] (sol_attn_pool)
 *   kept_bitmap device uint32 [B][H][Nq][ceil(Nk/32)], written in full
 * Errors as for sol_attn_forward; SOL_EUNSUPPORTED also when B * H > 65535,
 * and from sol_attn_mask_threshold for the Gaussian rules (their pooled-key
 * statistics live in the forward's workspace).
 *
 * sol_attn_mask_threshold: the forward's own fused kernel, stopped after its
 * routing pass (pooled queries from the query rows, scores consumed chunk by
 * chunk on chip, the row-max rule and sinks of `route`), one workgroup per
 * work item; the workspace receives the pooled keys as the three bf16 parts
 * the kernel's score products take (as in the forward's workspace), and
 * nothing but the bitmap is written beyond it: the same bits a forward of
 * these inputs exports.
 *
 * sol_attn_mask_topk / sol_attn_mask_topp: pool q into the workspace, write
 * the full fp32 proxy map [B][H][Nq][Nk] to the workspace, then sort each
 * row: top-k keeps the k highest scores (k clipped to 0..Nk; equal scores by
 * lower block index); top-p keeps the fewest highest scores whose share of
 * the row's softmax mass over the proxy scores reaches p (p <= 0: the top
 * block; p >= 1: all; SOL_EINVAL for NaN). The workspace must hold
 * sol_attn_mask_workspace_bytes() bytes, 256-byte aligned.
 */
size_t sol_attn_mask_workspace_bytes(int B, int H, int N, int d, int Bq, int Bk);
int sol_attn_mask_threshold(const void* q, const float* kpool, int B, int H, int N, int d, int Bq, int Bk,
                            const sol_attn_route* route, uint32_t* kept_bitmap, void* workspace,
                            size_t workspace_bytes, void* stream);
int sol_attn_mask_topk(const void* q, const float* kpool, int B, int H, int N, int d, int Bq, int Bk, int k,
                       uint32_t* kept_bitmap, void* workspace, size_t workspace_bytes, void* stream);
int sol_attn_mask_topp(const void* q, const float* kpool, int B, int H, int N, int d, int Bq, int Bk, float p,
                       uint32_t* kept_bitmap, void* workspace, size_t workspace_bytes, void* stream);

/*
 * sol_attn_forward plus an export of the routing decisions it used: the same
 * kernel, with the kept-block bitmap written as it routes.
 *   kept_bitmap  device uint32 [B][H][Nq][ceil(Nk/32)]; bit (j % 32) of word
 *                j / 32 of row (b, h, i) is 1 iff key block j was kept for
 *                query block i. Must not be NULL.
 */
int sol_attn_forward_debug(const void* q, const void* k, const void* v, void* out,
                           int B, int H, int N, int d, int Bq, int Bk, float tau,
                           unsigned flags, sol_attn_stats* stats,
                           float* kpool, float* vmean,
                           void* workspace, size_t workspace_bytes, void* stream,
                           uint32_t* kept_bitmap);

/*
 * For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid allocation):
 * sol_attn_forward_ex with the pooled keys and values and the workspace taken
 * from a static device array of the library instead of the caller. The
 * caller passes only inputs and outputs; the call makes no allocation, free
 * or allocating library call.
 *   arguments    as for sol_attn_forward_ex, without kpool, vmean and the
 *                workspace
 *   scratch      SOL_ATTN_SCRATCH_BYTES of device memory per GPU, reserved
 *                when the library is loaded and held until the process ends,
 *                laid out as [workspace | kpool | vmean]: a problem needs
 *                sol_attn_workspace_bytes() + 2 * round_up(B*H*ceil(N/Bk)*d*4,
 *                256) bytes of it (about 126 MiB for B*H = 24 heads of
 *                118800 tokens at d = 128)
 * Errors: those of sol_attn_forward_ex; SOL_EINVAL also for SOL_F_POOLED or
 * SOL_F_PLANNED (the array holds whatever the previous call on this GPU left,
 * so every call pools afresh); SOL_ESCRATCH, before any launch, when the
 * problem needs more than SOL_ATTN_SCRATCH_BYTES; SOL_EHIP if the runtime
 * cannot resolve the array's address on the current GPU (looked up once per
 * device, on the first call made with that device current).
 * Every call on one GPU uses that GPU's one array (one per process): two
 * calls of one process that overlap in time on the same GPU (different
 * streams or threads) race and may both return wrong results. Calls on one
 * stream are ordered and safe.
 */
#define SOL_ATTN_SCRATCH_BYTES (128u << 20)
int sol_attn_forward_noalloc(const void* q, const void* k, const void* v, void* out,
                             int B, int H, int N, int d, int Bq, int Bk,
                             const sol_attn_route* route, unsigned flags, sol_attn_stats* stats,
                             void* stream, uint32_t* kept_bitmap);

/* Static description of a return code. */
const char* sol_attn_strerror(int code);

#ifdef __cplusplus
}
#endif

#endif /* SOL_ATTN_H */
