/*
 * sparse_mla.h -- C ABI of the MI355X (gfx950) sparse MLA attention library.
 *
 * Operation (sparse multi-head latent attention in its MQA / absorbed form):
 * for every query row t, gather the cache rows named by its top-k index list,
 * score them against the row's h query heads -- all heads share the same
 * latent rows -- apply a softmax over the listed rows, and accumulate the
 * first 512 dims of those rows.  Per row and head the call writes
 *     out[t, h, 0:512]  (bf16)   and   lse[t, h]  (fp32, natural log).
 *
 * Sources on the pages this library is built from:
 *   - vLLM PR #60220 ("FlashMLA sparse: stage fp8 mixed-batch q/out in the
 *     workspace"), section "Claims": query rows are 576 wide (T x 64 x 576
 *     bf16), outputs 512 wide (T x 64 x 512 bf16), passed in by the caller;
 *     section "Details": one call covers all T tokens of a step, lse is fp32
 *     T x heads, and the output feeds the v_up projection (so it stays in
 *     the 512-dim latent space); sections "Overview" and "Limitations": the
 *     fp32 split-KV partial buffer must not be allocated per call.
 *   - prhub report on vLLM PR #55738, section "Motivation": each prefill
 *     token goes through a per-token top-k MQA kernel whose cost is the KV
 *     gather; section "Key source snippets": the K row is the 512-dim
 *     latent ("nope") part followed by the 64-dim rope part.
 *   - vLLM PR #54951, section "Summary": top-k lists are int32, 2048 per
 *     row, stored in buffers wider than top-k (2051 columns).
 *   - vLLM PR #64510, section "Details": the real head count (8/16/32) is
 *     run natively instead of padding heads to 64.
 *   - prhub report on vLLM PR #55738, "Implementation breakdown" items 1
 *     and 3: a NoPE MLA layout has a zero-width rope part (qk_rope 0), and K
 *     is then the latent part alone (SMLA_GEOM_NOPE below); item 5: with a
 *     quantised cache such layers stay on the per-token top-k MQA path.
 *
 * Conventions fixed by this ABI (the pages leave them open):
 *   - A cache row is 576 values: dims 0..511 latent, 512..575 rope.  The
 *     value vector of a row is its first 512 dims.  With geometry
 *     SMLA_GEOM_NOPE rows and query heads are the 512 latent dims alone
 *     (bf16 cache: row `slot` at byte slot * 1024; fp8 cache: rows of the
 *     512 codes alone, see below).
 *   - The cache is paged; page_size rows per page (a power of two; 64 in
 *     the configurations this library is tuned for).
 *       bf16 cache: row `slot` lives at byte slot * 1152.
 *       fp8 cache (SMLA_KV_FP8_E4M3): page p starts at byte
 *         p * page_size * 656 and holds page_size rows of 640 bytes
 *         [512 OCP E4M3FN codes | 64 bf16 rope values], followed by
 *         page_size x 4 fp32 scales (one per 128 latent dims).  The latent
 *         value of dim d is e4m3(code[d]) * scale[d / 128]; rope is bf16.
 *         SMLA_GEOM_NOPE: page p starts at byte p * page_size * 528 and
 *         holds page_size rows of the 512 codes, then the page_size x 4
 *         scales.
 *   - Index entries equal to -1 are skipped.  Any entry that is negative,
 *     or whose physical row falls outside [0, num_pages * page_size) (or,
 *     in LOGICAL mode, whose block lies outside the block table, or whose
 *     block-table entry is negative), is skipped the same way.  Repeated
 *     entries are repeated softmax terms.
 *   - Index modes: SMLA_IDX_SLOT -- entries are physical rows.
 *     SMLA_IDX_LOGICAL -- entries are positions j in the query row's
 *     sequence s = token_seq[t]; the physical row is
 *     block_table[s * block_table_stride + j / page_size] * page_size
 *     + j % page_size.
 *   - A row with no valid entry gets out = 0 and lse = -inf.
 *
 * Ownership and side effects: every buffer is owned by the caller.  The
 * library keeps no per-call state, performs no device allocation, no
 * host<->device copy and no synchronisation inside sparse_mla_fwd; all work
 * is enqueued on `stream` (a hipStream_t; NULL = the default stream) and the
 * buffers must stay valid until that work completes.  Device properties are
 * queried once per device and cached (thread-safe).
 *
 * Errors: arguments are validated on the host before anything is enqueued;
 * on any error nothing is launched and out / lse / workspace are untouched.
 */
#ifndef SPARSE_MLA_H
#define SPARSE_MLA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Status codes. */
#define SMLA_OK 0
#define SMLA_ERR_INVALID_ARG 1          /* null/misaligned pointer, bad size or stride      */
#define SMLA_ERR_UNSUPPORTED 2          /* valid request outside what the kernels implement */
#define SMLA_ERR_WORKSPACE_TOO_SMALL 3  /* workspace NULL or smaller than required          */
#define SMLA_ERR_HIP 4                  /* HIP runtime error (no device, launch failure)    */

/* kv_format */
#define SMLA_KV_BF16 0
#define SMLA_KV_FP8_E4M3 1

/* index_mode */
#define SMLA_IDX_SLOT 0
#define SMLA_IDX_LOGICAL 1

/* tiling: which head tile the kernel runs.  NATIVE runs groups of 16 heads
 * (1, 2 or 4 groups for h <= 16, <= 32, <= 64); PAD64 always runs 4 groups
 * (64 head slots, the unused ones on zero queries), the padded mode that
 * vLLM PR #64510 compares against.  AUTO picks NATIVE. */
#define SMLA_TILING_AUTO 0
#define SMLA_TILING_NATIVE 1
#define SMLA_TILING_PAD64 2

/* geometry (smla_params.geometry): the width of query heads and cache rows.
 * MLA: 576 = 512 latent + 64 rope dims.  NOPE: 512 latent dims, no rope
 * part (bf16 caches: kernel_variant 0, or 2 at h <= 32; fp8 caches:
 * kernel_variant 0, or 2 at h <= 16; anything else -> SMLA_ERR_UNSUPPORTED).
 * The output is 512 wide either way.  0 is MLA, so zero-initialised params
 * keep the rope part. */
#define SMLA_GEOM_MLA 0
#define SMLA_GEOM_NOPE 1

/* Gather order (smla_params.gather_order).  LIST follows the index list;
 * SLOT groups each row's entries (stably) into 16 ranges of physical cache
 * row, so that the rows computed at the same time on one XCD read nearby
 * cache rows and share its L2.  AUTO picks SLOT for unsplit bf16 batches of
 * at least 1024 query rows (prefill-sized; rows of one sequence overlap in
 * their history) and LIST otherwise. */
#define SMLA_GATHER_AUTO 0
#define SMLA_GATHER_LIST 1
#define SMLA_GATHER_SLOT 2

#define SMLA_D_QK 576
#define SMLA_D_V 512
#define SMLA_MAX_HEADS 64
/* Bound on split work units (query row x KV split) of an automatic plan. */
#define SMLA_MAX_SPLIT_UNITS 1024

typedef struct smla_params {
  int32_t num_tokens;          /* T >= 0 query rows                                   */
  int32_t num_heads;           /* h, 1..64 query heads sharing the latent             */
  int32_t topk;                /* >= 1 meaningful columns per index row               */
  int32_t page_size;           /* rows per cache page, power of two in [1, 4096]      */
  int64_t idx_stride;          /* int32 elements between index rows, >= topk          */
  int64_t q_stride_t;          /* bf16 elements between query rows (multiple of 8)    */
  int64_t q_stride_h;          /* bf16 elements between heads (>= 576, or >= 512 for  */
                               /* SMLA_GEOM_NOPE; multiple of 8)                      */
  int64_t out_stride_t;        /* bf16 elements between output rows (multiple of 8)   */
  int64_t out_stride_h;        /* bf16 elements between output heads (>= 512, mult 8) */
  int64_t lse_stride_t;        /* fp32 elements between lse rows (>= h)               */
  int64_t num_pages;           /* pages in the cache pool (>= 1 when T > 0)           */
  int32_t kv_format;           /* SMLA_KV_*                                           */
  int32_t index_mode;          /* SMLA_IDX_*                                          */
  int32_t num_seqs;            /* LOGICAL: rows of block_table                        */
  int32_t max_blocks_per_seq;  /* LOGICAL: valid columns of block_table               */
  int64_t block_table_stride;  /* LOGICAL: int32 elements between block-table rows    */
  float softmax_scale;         /* multiplies q.k (e.g. 1/sqrt(576)); finite           */
  int32_t tiling;              /* SMLA_TILING_*                                       */
  int32_t num_splits;          /* 0 = automatic; n >= 1 forces n KV splits per row    */
  int32_t kernel_variant;      /* 0 = default (the plan picks the shape); 1 = the     */
                               /* alternative shape (bf16 MLA any h; fp8 h <= 16);    */
                               /* 2 = two work-groups per CU at h <= 32 (bf16, MLA or */
                               /* NoPE) or h <= 16 (fp8), and at 33..64 heads (or     */
                               /* PAD64, bf16 MLA) the row-half score split; anything */
                               /* else -> SMLA_ERR_UNSUPPORTED.  A tuning knob, see   */
                               /* smla_plan; same results to tolerance.               */
  int32_t gather_order;        /* SMLA_GATHER_*: order in which a row's listed cache  */
                               /* rows are gathered (the result is the same set sum;  */
                               /* fp32 summation order, hence rounding, follows it)   */
  int32_t geometry;            /* SMLA_GEOM_*: row width (576 with rope, 512 NoPE)    */
} smla_params;

/* Read-only description of how a call with these parameters is executed. */
typedef struct smla_plan {
  int32_t head_groups;         /* 16-head groups the kernel runs (1, 2 or 4)          */
  int32_t row_groups;          /* independent row streams (tile sequences) per        */
                               /* work-group                                          */
  int32_t tile_rows;           /* cache rows per pipeline stage                       */
  int32_t stages;              /* pipeline depth (tiles in LDS per row group)         */
  int32_t num_splits;          /* KV splits per query row (1 = unsplit)               */
  int32_t threads;             /* threads per work-group                              */
  int64_t units;               /* work-groups doing attention = T * num_splits        */
  int64_t grid;                /* launched work-groups (units rounded up to 8)        */
  int64_t workspace_bytes;     /* workspace sparse_mla_fwd writes (0 if unsplit)      */
  int64_t partials_bytes;      /* workspace sparse_mla_fwd_partials writes            */
  int32_t lds_bytes;           /* LDS per work-group                                  */
  int32_t num_cus;             /* compute units assumed by the plan                   */
  int32_t gather_order;        /* resolved SMLA_GATHER_LIST or SMLA_GATHER_SLOT        */
  int32_t kernel_variant;      /* resolved kernel shape: the requested variant, or   */
                               /* for variant 0 the shape the plan picks (2 for      */
                               /* unsplit batches of >= 2 rows per CU at h <= 32     */
                               /* bf16 or h <= 16 fp8, else 0)                       */
} smla_plan;

/* Bytes of workspace sparse_mla_fwd needs for calls described by *p: the
 * fp32 split-KV partials that vLLM PR #60220 ("Limitations"; "Details",
 * root cause) reports a kernel allocating on every call, outside the startup
 * memory profile (2 x T x 64 x 512 x 4 B = 8 GiB at T = 32K), held here in a
 * caller buffer sized once.
 * Host-only, pure and independent of the device.  For num_splits == 0 the
 * result does not depend on num_tokens (it covers every automatic plan:
 * SMLA_MAX_SPLIT_UNITS * h * 513 * 4 bytes), so a caller can size the
 * workspace once.  For num_splits == n > 1 it is T * n * h * 513 * 4 bytes;
 * for n == 1 it is 0.  The workspace holds fp32 split partials (out and lse
 * per unit and head); its contents are scratch between calls.  Returns 0
 * for a NULL or invalid *p. */
size_t sparse_mla_workspace_size(const smla_params* p);

/* Execution plan for *p on the current device (queries the device's compute
 * unit count once).  Returns SMLA_OK or an error code; *plan is written on
 * success only.  Pure host function besides that one cached query. */
int sparse_mla_plan(const smla_params* p, smla_plan* plan);

/* Same, for an explicit compute-unit count (no device query at all). */
int sparse_mla_plan_for(const smla_params* p, int32_t num_cus, smla_plan* plan);

/* The forward pass.  Device pointers:
 *   q           bf16  [T, h, 576] ([T, h, 512] for SMLA_GEOM_NOPE) with strides
 *               q_stride_t / q_stride_h (16-B aligned)
 *   kv_cache    bf16 [num_pages, page_size, 576] ([.., 512] for SMLA_GEOM_NOPE) or the
 *               fp8 page layout above (16-B aligned)
 *   block_table int32 [num_seqs, block_table_stride]  (LOGICAL mode; NULL in SLOT mode)
 *   token_seq   int32 [T]                             (LOGICAL mode; NULL in SLOT mode)
 *   topk_idx    int32 [T, idx_stride]                 (4-B aligned)
 *   out         bf16  [T, h, 512] with strides out_stride_t / out_stride_h (16-B aligned)
 *   lse         fp32  [T, h] with stride lse_stride_t (4-B aligned)
 *   workspace   >= sparse_mla_workspace_size(p) bytes (16-B aligned), or
 *               NULL / any size when the plan is unsplit
 *   stream      hipStream_t the work is enqueued on
 * T == 0 returns SMLA_OK without touching the device.  Returns SMLA_OK or an
 * error code (nothing enqueued on error). */
int sparse_mla_fwd(const smla_params* p, const void* q, const void* kv_cache,
                   const int32_t* block_table, const int32_t* token_seq,
                   const int32_t* topk_idx, void* out, float* lse,
                   void* workspace, size_t workspace_bytes, void* stream);

/* sparse_mla_fwd without a workspace argument, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc).  The split partials go to a static
 * device array of SMLA_NOALLOC_SCRATCH_BYTES that the library holds on every
 * GPU it runs on until the process ends (looked up on the first call per
 * device; nothing is allocated per call).  Same arguments, plan, kernels,
 * results and validation as sparse_mla_fwd; a plan whose partials exceed
 * the static array (a forced num_splits with T * num_splits * h * 513 * 4 >
 * SMLA_NOALLOC_SCRATCH_BYTES; every automatic plan on up to 256 compute
 * units fits) returns SMLA_ERR_WORKSPACE_TOO_SMALL with nothing enqueued.
 * Every call on one GPU shares that GPU's array: calls that overlap on one
 * GPU (on different streams) race and must not be issued; stream-ordered
 * calls are safe, since every partial is written before it is read. */
#define SMLA_NOALLOC_SCRATCH_BYTES ((size_t)256 * 64 * 513 * 4)
int sparse_mla_fwd_noalloc(const smla_params* p, const void* q, const void* kv_cache,
                           const int32_t* block_table, const int32_t* token_seq,
                           const int32_t* topk_idx, void* out, float* lse, void* stream);

/* The attention kernel alone, leaving the split results unmerged: for every
 * query row t and KV split s < S (S = the plan's num_splits; 1 when unsplit)
 * it writes the split's normalised fp32 output and its lse to the workspace,
 *     part_out = (float*)workspace                 fp32 [T * S, h, 512]
 *     part_lse = part_out + T * S * h * 512        fp32 [T * S, h]
 * with unit u = t * S + s; split s covers index columns
 * [topk * s / S, topk * (s + 1) / S).  An empty split has lse = -inf and a
 * zero output.  Needs plan.partials_bytes (= T * S * h * 513 * 4) bytes of
 * workspace.  This is the fp32 split-KV partial of vLLM PR #60220
 * ("Overview", "Limitations") held in caller memory; the partials can be
 * merged with sparse_mla_lse_combine, also after stacking the partials of
 * several producers.  Same validation and error behaviour as sparse_mla_fwd. */
int sparse_mla_fwd_partials(const smla_params* p, const void* q, const void* kv_cache,
                            const int32_t* block_table, const int32_t* token_seq,
                            const int32_t* topk_idx, void* workspace, size_t workspace_bytes,
                            void* stream);

/* Merge S partial results per query row by their lse, in split order:
 *     lse = log sum_s exp(lse_s),  out = sum_s exp(lse_s - lse) * out_s
 * (splits with lse_s = -inf weigh nothing; a row whose splits are all -inf
 * gets out = 0, lse = -inf).  part_out fp32 [T * S, h, 512] and part_lse fp32
 * [T * S, h] (unit u = t * S + s, 16-B / 4-B aligned device memory); out bf16
 * with the given strides (elements), lse fp32 with lse_stride_t.  Enqueued on
 * `stream`; no allocation, no synchronisation. */
int sparse_mla_lse_combine(const float* part_out, const float* part_lse, int32_t num_tokens,
                           int32_t num_splits, int32_t num_heads, void* out, int64_t out_stride_t,
                           int64_t out_stride_h, float* lse, int64_t lse_stride_t, void* stream);

/* Dense causal fallback: every query row t attends to all positions
 * 0 .. positions[t] of its sequence -- the same result as sparse_mla_fwd with
 * the index list 0, 1, .., positions[t] (prhub report on vLLM PR #55738,
 * "Motivation": a prefix no longer than top-k is better served densely,
 * about 1.6 ms per layer through the top-k kernel against 0.2 ms dense for
 * 8 x 2048 tokens).  A work-group takes up to 64 / h consecutive query rows
 * of one sequence and gathers each cache row once for all of them.
 *   query_start int32 [num_seqs + 1] (device): rows of sequence s are
 *               [query_start[s], query_start[s + 1]) -- nondecreasing, first
 *               0, last num_tokens (a varlen "cu_seqlens" layout)
 *   positions   int32 [num_tokens] (device): the causal position of each row
 *   block_table as for SMLA_IDX_LOGICAL (positions past the table, or blocks
 *               whose page is outside the pool, are skipped like -1 entries)
 * Requirements (else SMLA_ERR_UNSUPPORTED): kv_format bf16, index_mode
 * SMLA_IDX_LOGICAL, page_size >= 16, max_blocks_per_seq and num_seqs at most
 * 2048, num_splits 0 or 1, tiling AUTO / NATIVE, kernel_variant 0.
 * topk / idx_stride must be valid but are not used; geometry may be MLA or
 * NOPE.  Other validation, ownership and error behaviour as sparse_mla_fwd;
 * no workspace. */
int sparse_mla_dense_fwd(const smla_params* p, const void* q, const void* kv_cache,
                         const int32_t* block_table, const int32_t* query_start,
                         const int32_t* positions, void* out, float* lse, void* stream);

/* Per-row top-k selection: the last step of the sparse indexer, producing
 * the int32 index lists the attention consumes (vLLM PR #54951, "Summary":
 * each query row keeps the indices of its top-k scored keys; "Additional
 * checks": selected sets are compared, the order inside a row is not
 * defined).  The score function itself is not on the pages and is not part
 * of this library: the caller passes the scores.
 *   scores  fp32 [num_rows, ld] (device, ld >= n_keys elements, 4-B aligned)
 *   lens    int32 [num_rows] (device) or NULL: row t's valid keys are
 *           0 .. lens[t]-1, clamped to [0, n_keys] (NULL: all n_keys)
 *   idx     int32 [num_rows, idx_stride] (device, idx_stride >= k): receives
 *           min(k, lens[t]) selected key indices in an unspecified order,
 *           then -1 in the remaining columns of the first k
 * Selection order: higher score first, NaN below every number (-inf
 * included), equal scores by lower key index.  Errors: SMLA_ERR_INVALID_ARG
 * for negative sizes, k < 1, ld < n_keys, idx_stride < k, null or
 * misaligned pointers (nothing is launched); SMLA_ERR_HIP on launch failure.
 * Enqueued on `stream`; no allocation, no synchronisation. */
int sparse_mla_topk(const float* scores, int64_t ld, const int32_t* lens, int32_t num_rows,
                    int32_t n_keys, int32_t k, int32_t* idx, int64_t idx_stride, void* stream);

/* Indexer scoring, the step before sparse_mla_topk: MQA logits of every
 * query row against its key history (vLLM PR #54951, "TL;DR" and
 * "Summary": each row is scored against the full available key history,
 * then top-k; "Additional checks": valid logits of a row are the same
 * whatever other rows share the batch).  The pages do not give the head
 * count, head width or head reduction; this library computes
 *     logits[t, s] = sum_j w[t, j] * max(0, q[t, j, :] . k[s, :]),  s < lens[t]
 * (per-head ReLU, then a sum weighted by per-row head weights: the form of
 * the MQA-logits kernel those checks run), with every indexer head of a row
 * sharing one key per history position (MQA).
 *   q       bf16 [num_rows, num_heads, head_dim] (device), element strides
 *           q_stride_t / q_stride_h (multiples of 8; 16-B aligned)
 *   k       bf16 [n_keys, head_dim] (device), row stride k_stride elements
 *           (multiple of 8; 16-B aligned): token keys, or pooled keys when
 *           the caller pools its history
 *   w       fp32 [num_rows, num_heads] (device), row stride w_stride_t
 *           (multiple of 4; 16-B aligned)
 *   lens    int32 [num_rows] (device) or NULL: row t scores keys
 *           0 .. lens[t] - 1 (clamped to [0, n_keys]); NULL: all n_keys
 *   logits  fp32 [num_rows, ld] (device, ld >= n_keys): columns s < lens[t]
 *           are written, the others are left untouched
 * head_dim must be SMLA_INDEXER_HEAD_DIM and num_heads a multiple of 16 up
 * to 64 (else SMLA_ERR_UNSUPPORTED).  Sizes / strides / pointers as stated
 * or SMLA_ERR_INVALID_ARG (nothing launched).  Enqueued on `stream`; no
 * allocation, no synchronisation.  The logits feed sparse_mla_topk (scores =
 * logits, ld, lens) to produce the index lists. */
#define SMLA_INDEXER_HEAD_DIM 128
int sparse_mla_indexer_logits(const void* q, int64_t q_stride_t, int64_t q_stride_h, const void* k,
                              int64_t k_stride, const float* w, int64_t w_stride_t, const int32_t* lens,
                              int32_t num_rows, int32_t n_keys, int32_t num_heads, int32_t head_dim,
                              float* logits, int64_t ld, void* stream);

/* Static, human-readable text for a status code. */
const char* sparse_mla_status_string(int status);

#ifdef __cplusplus
}
#endif

#endif /* SPARSE_MLA_H */
