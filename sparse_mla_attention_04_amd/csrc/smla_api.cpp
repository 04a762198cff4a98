// C ABI of the sparse MLA library: validation, planning, workspace sizing and
// launch.  Validation runs entirely on the host before any HIP call, so every
// argument error returns without touching the device.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <mutex>

#include "../../include/sparse_mla.h"
#include "smla_internal.h"

namespace {

constexpr int64_t kPartialFloatsPerHead = SMLA_D_V + 1;   // normalised out + lse

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

bool is_pow2(int64_t v) { return v > 0 && (v & (v - 1)) == 0; }

int log2i(int64_t v) {
  int s = 0;
  while ((int64_t(1) << s) < v) ++s;
  return s;
}

int head_groups_for(const smla_params* p) {
  if (p->tiling == SMLA_TILING_PAD64) return 4;
  if (p->num_heads <= 16) return 1;
  if (p->num_heads <= 32) return 2;
  return 4;
}

int d_qk_of(const smla_params* p) { return p->geometry == SMLA_GEOM_NOPE ? SMLA_D_V : SMLA_D_QK; }

// Parameter checks that need no pointers (and no device).
int check_params(const smla_params* p) {
  if (!p) return SMLA_ERR_INVALID_ARG;
  if (p->kernel_variant < 0) return SMLA_ERR_INVALID_ARG;
  if (p->geometry != SMLA_GEOM_MLA && p->geometry != SMLA_GEOM_NOPE) return SMLA_ERR_INVALID_ARG;
  if (p->gather_order < SMLA_GATHER_AUTO || p->gather_order > SMLA_GATHER_SLOT) return SMLA_ERR_INVALID_ARG;
  if (p->num_tokens < 0) return SMLA_ERR_INVALID_ARG;
  if (p->num_heads < 1) return SMLA_ERR_INVALID_ARG;
  if (p->num_heads > SMLA_MAX_HEADS) return SMLA_ERR_UNSUPPORTED;
  if (p->topk < 1 || p->idx_stride < p->topk) return SMLA_ERR_INVALID_ARG;
  if (!is_pow2(p->page_size) || p->page_size > 4096) return SMLA_ERR_INVALID_ARG;
  if (p->kv_format != SMLA_KV_BF16 && p->kv_format != SMLA_KV_FP8_E4M3) return SMLA_ERR_INVALID_ARG;
  if (p->index_mode != SMLA_IDX_SLOT && p->index_mode != SMLA_IDX_LOGICAL) return SMLA_ERR_INVALID_ARG;
  if (p->tiling < SMLA_TILING_AUTO || p->tiling > SMLA_TILING_PAD64) return SMLA_ERR_INVALID_ARG;
  if (p->num_splits < 0) return SMLA_ERR_INVALID_ARG;
  if (p->num_heads >= 1 && p->num_heads <= SMLA_MAX_HEADS &&
      (p->kv_format == SMLA_KV_BF16 || p->kv_format == SMLA_KV_FP8_E4M3) &&
      p->tiling >= SMLA_TILING_AUTO && p->tiling <= SMLA_TILING_PAD64) {
    smla::FwdShape sh{};
    if (!smla::fwd_shape(p->kv_format, head_groups_for(p), p->kernel_variant, p->geometry == SMLA_GEOM_NOPE, &sh))
      return SMLA_ERR_UNSUPPORTED;
  }
  if (!std::isfinite(p->softmax_scale)) return SMLA_ERR_INVALID_ARG;
  if (p->q_stride_h < d_qk_of(p) || p->q_stride_h % 8 || p->q_stride_t < 0 || p->q_stride_t % 8)
    return SMLA_ERR_INVALID_ARG;
  if (p->out_stride_h < SMLA_D_V || p->out_stride_h % 8 || p->out_stride_t < 0 || p->out_stride_t % 8)
    return SMLA_ERR_INVALID_ARG;
  if (p->lse_stride_t < 0) return SMLA_ERR_INVALID_ARG;
  if (p->num_tokens > 1 && (p->q_stride_t < (int64_t)p->num_heads * p->q_stride_h - (p->q_stride_h - d_qk_of(p)) ||
                            p->out_stride_t < (int64_t)p->num_heads * p->out_stride_h - (p->out_stride_h - SMLA_D_V) ||
                            p->lse_stride_t < p->num_heads))
    return SMLA_ERR_INVALID_ARG;   // rows of q / out / lse would overlap
  if (p->num_tokens > 0) {
    if (p->num_pages < 1) return SMLA_ERR_INVALID_ARG;
    if (p->num_pages > (int64_t)INT32_MAX / p->page_size) return SMLA_ERR_UNSUPPORTED;
    if (p->index_mode == SMLA_IDX_LOGICAL) {
      if (p->num_seqs < 1 || p->max_blocks_per_seq < 1 || p->block_table_stride < p->max_blocks_per_seq)
        return SMLA_ERR_INVALID_ARG;
    }
  }
  return SMLA_OK;
}


int splits_for(const smla_params* p, int32_t num_cus, const smla::FwdShape& sh) {
  if (p->num_splits > 0) return p->num_splits;
  const int64_t T = p->num_tokens;
  if (T <= 0 || T >= num_cus) return 1;
  int64_t s = num_cus / T;
  // one head group: a row streams its gathers at ~50 GB/s per work-group, so
  // from #CU / 4 rows on the unsplit batch already draws most of the gather
  // bandwidth and the merge launch costs more than splitting gains (MI355X,
  // rows of 2048 entries over a 604 MB pool: T = 128 at h = 8 ran 51.8 us
  // unsplit, 54.7 us in two splits; T = 64 ran 34.9 us in four splits, 42.2
  // unsplit; at h = 32, T = 128 still gains from two splits, 59.7 vs 75.8 us)
  if (sh.head_groups == 1 && s < 4) return 1;
  // keep at least one tile per row group in every split; with one head
  // group, at least 256 list entries (a split's fixed start-up and merge cost
  // outweighs a shorter share: T = 64 rows of 128 entries at h = 8 ran
  // 13.4 us per call in two splits, 11.2 us unsplit, on MI355X)
  int64_t rows_per_wg = (int64_t)sh.tile_rows * sh.row_groups;
  if (sh.head_groups == 1 && rows_per_wg < 256) rows_per_wg = 256;
  int64_t smax = p->topk / rows_per_wg;
  if (smax < 1) smax = 1;
  if (s > smax) s = smax;
  if (T * s > SMLA_MAX_SPLIT_UNITS) s = SMLA_MAX_SPLIT_UNITS / T;
  return s < 1 ? 1 : (int)s;
}

// Unsplit bf16 batches of at least this many query rows gather in slot order
// (measured on MI355X: c3 h=8 -9%, c4 -2%; the fp8 c5 batch ran 3% slower).
constexpr int64_t kSlotOrderMinTokens = 1024;

int bucket_shift_for(int64_t num_slots) {
  int bits = 0;
  while (bits < 62 && ((int64_t)1 << bits) < num_slots) ++bits;
  return bits > 4 ? bits - 4 : 0;
}

int make_plan(const smla_params* p, int32_t num_cus, smla_plan* plan) {
  int rc = check_params(p);
  if (rc != SMLA_OK) return rc;
  if (num_cus < 1) return SMLA_ERR_INVALID_ARG;
  smla::FwdShape sh{};
  const int hg = head_groups_for(p);
  if (!smla::fwd_shape(p->kv_format, hg, p->kernel_variant, p->geometry == SMLA_GEOM_NOPE, &sh))
    return SMLA_ERR_UNSUPPORTED;
  const int S = splits_for(p, num_cus, sh);
  // Unsplit batches with at least two rows per CU run, at h <= 32 (bf16) or
  // h <= 16 (fp8), the shapes that fit two work-groups on a CU (kernel
  // variant 2): one row's start-up and epilogue overlap another's tiles.
  // Measured on MI355X, rows of 2048 entries: 4096 rows at h = 8 714 -> 656
  // us, h = 16 758 -> 672 us, h = 32 1057 -> 853 us; 32768 fp8 rows at h = 8
  // 7050 -> 6532 us; 64 rows (one per CU) ran 13.4 -> 15.6 us, hence the row
  // threshold.
  int variant = p->kernel_variant;
  if (variant == 0 && S == 1 && p->num_tokens >= 2 * (int64_t)num_cus &&
      (p->kv_format == SMLA_KV_BF16 ? hg <= 2 : hg == 1)) {
    variant = 2;
    if (!smla::fwd_shape(p->kv_format, hg, variant, p->geometry == SMLA_GEOM_NOPE, &sh)) return SMLA_ERR_UNSUPPORTED;
  }
  smla_plan pl{};
  pl.kernel_variant = variant;
  pl.head_groups = sh.head_groups;
  pl.row_groups = sh.row_groups;
  pl.tile_rows = sh.tile_rows;
  pl.stages = sh.stages;
  pl.threads = sh.threads;
  pl.lds_bytes = sh.lds_bytes;
  pl.num_splits = S;
  pl.units = (int64_t)p->num_tokens * S;
  pl.grid = (pl.units + 7) / 8 * 8;
  pl.workspace_bytes = S > 1 ? pl.units * p->num_heads * kPartialFloatsPerHead * 4 : 0;
  pl.partials_bytes = pl.units * p->num_heads * kPartialFloatsPerHead * 4;
  pl.num_cus = num_cus;
  pl.gather_order = p->gather_order != SMLA_GATHER_AUTO                    ? p->gather_order
                    : (S == 1 && p->num_tokens >= kSlotOrderMinTokens && p->kv_format == SMLA_KV_BF16)
                        ? SMLA_GATHER_SLOT
                        : SMLA_GATHER_LIST;
  *plan = pl;
  return SMLA_OK;
}

std::mutex g_mu;
int g_cus[256];

// Keys per indexer work unit: each unit loads its 16 rows' queries (256 KB at
// 64 heads) once, so longer chunks load them less often; they are doubled
// from 4096 up to 16384 keys while at least four units per CU remain
// (4096 rows x 65536 keys on 256 CUs: 3.29 ms at 4096, 3.24 at 8192, 3.22 at
// 16384 keys per chunk).
int indexer_chunk_keys(int32_t row_blocks, int32_t n_keys, int32_t cus) {
  int chunk = 4096;
  while (chunk < 16384 && (int64_t)row_blocks * ((n_keys + 2 * chunk - 1) / (2 * chunk)) >= 4 * (int64_t)cus)
    chunk *= 2;
  return chunk;
}

int device_cus(int32_t* cus) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 256) return SMLA_ERR_HIP;
  std::lock_guard<std::mutex> lk(g_mu);
  if (g_cus[dev] == 0) {
    int v = 0;
    if (hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || v < 1)
      return SMLA_ERR_HIP;
    g_cus[dev] = v;
  }
  *cus = g_cus[dev];
  return SMLA_OK;
}

}  // namespace

extern "C" {

size_t sparse_mla_workspace_size(const smla_params* p) {
  if (check_params(p) != SMLA_OK) return 0;
  const int64_t per_unit = (int64_t)p->num_heads * kPartialFloatsPerHead * 4;
  if (p->num_splits == 0) return (size_t)(SMLA_MAX_SPLIT_UNITS * per_unit);
  if (p->num_splits == 1) return 0;
  return (size_t)((int64_t)p->num_tokens * p->num_splits * per_unit);
}

int sparse_mla_plan_for(const smla_params* p, int32_t num_cus, smla_plan* plan) {
  if (!plan) return SMLA_ERR_INVALID_ARG;
  return make_plan(p, num_cus, plan);
}

int sparse_mla_plan(const smla_params* p, smla_plan* plan) {
  if (!plan) return SMLA_ERR_INVALID_ARG;
  int rc = check_params(p);
  if (rc != SMLA_OK) return rc;
  int32_t cus = 0;
  rc = device_cus(&cus);
  if (rc != SMLA_OK) return rc;
  return make_plan(p, cus, plan);
}

}  // extern "C"

namespace {

enum class Mode { kFull, kPartials };

int run(Mode mode, const smla_params* p, const void* q, const void* kv_cache, const int32_t* block_table,
        const int32_t* token_seq, const int32_t* topk_idx, void* out, float* lse, void* workspace,
        size_t workspace_bytes, void* stream) {
  int rc = check_params(p);
  if (rc != SMLA_OK) return rc;
  if (p->num_tokens == 0) return SMLA_OK;
  if (!q || !kv_cache || !topk_idx) return SMLA_ERR_INVALID_ARG;
  if (!aligned(q, 16) || !aligned(kv_cache, 16) || !aligned(topk_idx, 4)) return SMLA_ERR_INVALID_ARG;
  if (mode == Mode::kFull && (!out || !lse || !aligned(out, 16) || !aligned(lse, 4))) return SMLA_ERR_INVALID_ARG;
  if (p->index_mode == SMLA_IDX_LOGICAL) {
    if (!block_table || !token_seq || !aligned(block_table, 4) || !aligned(token_seq, 4))
      return SMLA_ERR_INVALID_ARG;
  }
  const int64_t per_unit = (int64_t)p->num_heads * kPartialFloatsPerHead * 4;
  if (p->num_splits > 0 && (mode == Mode::kPartials || p->num_splits > 1)) {
    // forced split count: the workspace need is known without the device
    const size_t need = (size_t)((int64_t)p->num_tokens * p->num_splits * per_unit);
    if (!workspace || !aligned(workspace, 16) || workspace_bytes < need) return SMLA_ERR_WORKSPACE_TOO_SMALL;
  }
  int32_t cus = 0;
  rc = device_cus(&cus);
  if (rc != SMLA_OK) return rc;
  smla_plan pl{};
  rc = make_plan(p, cus, &pl);
  if (rc != SMLA_OK) return rc;
  const bool partials = (mode == Mode::kPartials) || pl.num_splits > 1;
  if (partials) {
    const size_t need = (size_t)(pl.units * per_unit);
    if (!workspace || !aligned(workspace, 16) || workspace_bytes < need) return SMLA_ERR_WORKSPACE_TOO_SMALL;
  }

  smla::FwdArgs a{};
  a.q = static_cast<const uint16_t*>(q);
  a.kv = static_cast<const uint8_t*>(kv_cache);
  a.block_table = block_table;
  a.token_seq = token_seq;
  a.topk_idx = topk_idx;
  a.out = static_cast<uint16_t*>(out);
  a.lse = lse;
  a.ws_out = partials ? static_cast<float*>(workspace) : nullptr;
  a.ws_lse = partials ? a.ws_out + pl.units * p->num_heads * SMLA_D_V : nullptr;
  a.q_st = p->q_stride_t;
  a.q_sh = p->q_stride_h;
  a.out_st = p->out_stride_t;
  a.out_sh = p->out_stride_h;
  a.lse_st = p->lse_stride_t;
  a.idx_stride = p->idx_stride;
  a.bt_stride = p->block_table_stride;
  a.num_slots = p->num_pages * p->page_size;
  a.num_pages = p->num_pages;
  a.units = pl.units;
  a.T = p->num_tokens;
  a.h = p->num_heads;
  a.topk = p->topk;
  a.num_splits = pl.num_splits;
  a.page_shift = log2i(p->page_size);
  a.index_mode = p->index_mode;
  a.num_seqs = p->num_seqs;
  a.max_blocks = p->max_blocks_per_seq;
  a.grid_per_xcd = (int32_t)(pl.grid / 8);
  a.write_partials = partials ? 1 : 0;
  a.scale_log2 = std::fabs(p->softmax_scale) * 1.44269504088896340736f;
  a.q_neg = p->softmax_scale < 0.f;
  // slot order: 16 ranges of physical row (the top 4 bits of the row number)
  a.bucket_shift = pl.gather_order == SMLA_GATHER_SLOT ? bucket_shift_for(a.num_slots) : -1;

  hipStream_t st = static_cast<hipStream_t>(stream);
  if (smla::launch_fwd(a, p->kv_format, pl.head_groups, pl.kernel_variant, p->geometry == SMLA_GEOM_NOPE, pl.grid,
                       st) != hipSuccess)
    return SMLA_ERR_HIP;
  if (mode == Mode::kFull && pl.num_splits > 1) {
    smla::CombineArgs c{};
    c.ws_out = a.ws_out;
    c.ws_lse = a.ws_lse;
    c.out = a.out;
    c.lse = lse;
    c.out_st = p->out_stride_t;
    c.out_sh = p->out_stride_h;
    c.lse_st = p->lse_stride_t;
    c.T = p->num_tokens;
    c.h = p->num_heads;
    c.num_splits = pl.num_splits;
    if (smla::launch_combine(c, st) != hipSuccess) return SMLA_ERR_HIP;
  }
  return SMLA_OK;
}

}  // namespace

extern "C" {

int sparse_mla_fwd(const smla_params* p, const void* q, const void* kv_cache, const int32_t* block_table,
                   const int32_t* token_seq, const int32_t* topk_idx, void* out, float* lse, void* workspace,
                   size_t workspace_bytes, void* stream) {
  return run(Mode::kFull, p, q, kv_cache, block_table, token_seq, topk_idx, out, lse, workspace,
             workspace_bytes, stream);
}

int sparse_mla_fwd_noalloc(const smla_params* p, const void* q, const void* kv_cache, const int32_t* block_table,
                           const int32_t* token_seq, const int32_t* topk_idx, void* out, float* lse, void* stream) {
  int rc = check_params(p);
  if (rc != SMLA_OK) return rc;
  if (p->num_tokens == 0) return SMLA_OK;
  void* ws = nullptr;
  if (smla::noalloc_scratch(&ws) != hipSuccess) return SMLA_ERR_HIP;
  return run(Mode::kFull, p, q, kv_cache, block_table, token_seq, topk_idx, out, lse, ws,
             smla::kNoallocScratchBytes, stream);
}

int sparse_mla_fwd_partials(const smla_params* p, const void* q, const void* kv_cache,
                            const int32_t* block_table, const int32_t* token_seq, const int32_t* topk_idx,
                            void* workspace, size_t workspace_bytes, void* stream) {
  return run(Mode::kPartials, p, q, kv_cache, block_table, token_seq, topk_idx, nullptr, nullptr, workspace,
             workspace_bytes, stream);
}

int sparse_mla_lse_combine(const float* part_out, const float* part_lse, int32_t num_tokens, int32_t num_splits,
                           int32_t num_heads, void* out, int64_t out_stride_t, int64_t out_stride_h, float* lse,
                           int64_t lse_stride_t, void* stream) {
  if (num_tokens < 0 || num_splits < 1 || num_heads < 1 || num_heads > SMLA_MAX_HEADS) return SMLA_ERR_INVALID_ARG;
  if (out_stride_h < SMLA_D_V || out_stride_h % 8 || out_stride_t < 0 || out_stride_t % 8 || lse_stride_t < 0)
    return SMLA_ERR_INVALID_ARG;
  if (num_tokens > 1 && (out_stride_t < (int64_t)(num_heads - 1) * out_stride_h + SMLA_D_V || lse_stride_t < num_heads))
    return SMLA_ERR_INVALID_ARG;
  if (num_tokens == 0) return SMLA_OK;
  if (!part_out || !part_lse || !out || !lse) return SMLA_ERR_INVALID_ARG;
  if (!aligned(part_out, 16) || !aligned(part_lse, 4) || !aligned(out, 16) || !aligned(lse, 4))
    return SMLA_ERR_INVALID_ARG;
  smla::CombineArgs c{};
  c.ws_out = part_out;
  c.ws_lse = part_lse;
  c.out = static_cast<uint16_t*>(out);
  c.lse = lse;
  c.out_st = out_stride_t;
  c.out_sh = out_stride_h;
  c.lse_st = lse_stride_t;
  c.T = num_tokens;
  c.h = num_heads;
  c.num_splits = num_splits;
  if (smla::launch_combine(c, static_cast<hipStream_t>(stream)) != hipSuccess) return SMLA_ERR_HIP;
  return SMLA_OK;
}

int sparse_mla_dense_fwd(const smla_params* p, const void* q, const void* kv_cache, const int32_t* block_table,
                         const int32_t* query_start, const int32_t* positions, void* out, float* lse,
                         void* stream) {
  int rc = check_params(p);
  if (rc != SMLA_OK) return rc;
  if (p->kv_format != SMLA_KV_BF16 || p->index_mode != SMLA_IDX_LOGICAL || p->page_size < 16 ||
      p->max_blocks_per_seq > smla::kListCap || p->num_seqs > smla::kListCap || p->num_splits > 1 ||
      p->tiling == SMLA_TILING_PAD64 || p->kernel_variant != 0)
    return SMLA_ERR_UNSUPPORTED;
  if (p->num_tokens == 0) return SMLA_OK;
  if (!q || !kv_cache || !block_table || !query_start || !positions || !out || !lse) return SMLA_ERR_INVALID_ARG;
  if (!aligned(q, 16) || !aligned(kv_cache, 16) || !aligned(block_table, 4) || !aligned(query_start, 4) ||
      !aligned(positions, 4) || !aligned(out, 16) || !aligned(lse, 4))
    return SMLA_ERR_INVALID_ARG;
  int32_t cus = 0;
  rc = device_cus(&cus);
  if (rc != SMLA_OK) return rc;
  (void)cus;
  const int qb = SMLA_MAX_HEADS / p->num_heads;
  // blocks: sum over sequences of ceil(n_s / qb) <= ceil(T / qb) + num_seqs
  const int64_t units = ((int64_t)p->num_tokens + qb - 1) / qb + p->num_seqs;
  smla::FwdArgs a{};
  a.q = static_cast<const uint16_t*>(q);
  a.kv = static_cast<const uint8_t*>(kv_cache);
  a.block_table = block_table;
  a.out = static_cast<uint16_t*>(out);
  a.lse = lse;
  a.q_st = p->q_stride_t;
  a.q_sh = p->q_stride_h;
  a.out_st = p->out_stride_t;
  a.out_sh = p->out_stride_h;
  a.lse_st = p->lse_stride_t;
  a.bt_stride = p->block_table_stride;
  a.num_slots = p->num_pages * p->page_size;
  a.num_pages = p->num_pages;
  a.units = units;
  a.T = p->num_tokens;
  a.h = p->num_heads;
  a.topk = 1;
  a.num_splits = 1;
  a.page_shift = log2i(p->page_size);
  a.index_mode = SMLA_IDX_LOGICAL;
  a.num_seqs = p->num_seqs;
  a.max_blocks = p->max_blocks_per_seq;
  a.grid_per_xcd = (int32_t)((units + 7) / 8);
  a.write_partials = 0;
  a.scale_log2 = std::fabs(p->softmax_scale) * 1.44269504088896340736f;
  a.q_neg = p->softmax_scale < 0.f;
  a.bucket_shift = -1;
  a.query_start = query_start;
  a.positions = positions;
  a.dense_qb = qb;
  if (smla::launch_dense(a, p->geometry == SMLA_GEOM_NOPE, (units + 7) / 8 * 8, static_cast<hipStream_t>(stream)) !=
      hipSuccess)
    return SMLA_ERR_HIP;
  return SMLA_OK;
}

int sparse_mla_topk(const float* scores, int64_t ld, const int32_t* lens, int32_t num_rows, int32_t n_keys,
                    int32_t k, int32_t* idx, int64_t idx_stride, void* stream) {
  if (num_rows < 0 || n_keys < 0 || k < 1 || ld < n_keys || idx_stride < k) return SMLA_ERR_INVALID_ARG;
  if (num_rows == 0) return SMLA_OK;
  if (!scores || !idx || !aligned(scores, 4) || !aligned(idx, 4) || (lens && !aligned(lens, 4)))
    return SMLA_ERR_INVALID_ARG;
  smla::TopkArgs a{};
  a.scores = scores;
  a.lens = lens;
  a.idx = idx;
  a.ld = ld;
  a.idx_stride = idx_stride;
  a.T = num_rows;
  a.n_keys = n_keys;
  a.k = k;
  if (smla::launch_topk(a, static_cast<hipStream_t>(stream)) != hipSuccess) return SMLA_ERR_HIP;
  return SMLA_OK;
}

int sparse_mla_indexer_logits(const void* q, int64_t q_stride_t, int64_t q_stride_h, const void* k, int64_t k_stride,
                              const float* w, int64_t w_stride_t, const int32_t* lens, int32_t num_rows,
                              int32_t n_keys, int32_t num_heads, int32_t head_dim, float* logits, int64_t ld,
                              void* stream) {
  if (num_rows < 0 || n_keys < 0 || num_heads < 1 || head_dim < 1) return SMLA_ERR_INVALID_ARG;
  if (head_dim != SMLA_INDEXER_HEAD_DIM || num_heads % 16 != 0 || num_heads > SMLA_MAX_HEADS)
    return SMLA_ERR_UNSUPPORTED;
  if (q_stride_h < head_dim || q_stride_h % 8 || q_stride_t < 0 || q_stride_t % 8 || k_stride < head_dim ||
      k_stride % 8 || w_stride_t < 0 || w_stride_t % 4 || ld < n_keys)
    return SMLA_ERR_INVALID_ARG;
  if (num_rows > 1 && (q_stride_t < (int64_t)(num_heads - 1) * q_stride_h + head_dim || w_stride_t < num_heads))
    return SMLA_ERR_INVALID_ARG;
  if (num_rows == 0 || n_keys == 0) return SMLA_OK;
  if (!q || !k || !w || !logits) return SMLA_ERR_INVALID_ARG;
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(w, 16) || !aligned(logits, 4) || (lens && !aligned(lens, 4)))
    return SMLA_ERR_INVALID_ARG;
  int32_t cus = 0;
  const int dev_rc = device_cus(&cus);
  if (dev_rc != SMLA_OK) return dev_rc;
  const int rpb = smla::indexer_rows_per_block();
  const int32_t row_blocks = (num_rows + rpb - 1) / rpb;
  const int chunk_keys = indexer_chunk_keys(row_blocks, n_keys, cus);
  smla::IndexerArgs a{};
  a.q = static_cast<const uint16_t*>(q);
  a.k = static_cast<const uint16_t*>(k);
  a.w = w;
  a.lens = lens;
  a.logits = logits;
  a.q_st = q_stride_t;
  a.q_sh = q_stride_h;
  a.k_st = k_stride;
  a.w_st = w_stride_t;
  a.ld = ld;
  a.T = num_rows;
  a.n_keys = n_keys;
  a.H = num_heads;
  a.chunk_keys = chunk_keys;
  a.row_blocks = row_blocks;
  a.units = (int64_t)a.row_blocks * ((n_keys + chunk_keys - 1) / chunk_keys);
  const int64_t grid = (a.units + 7) / 8 * 8;
  a.grid_per_xcd = (int32_t)(grid / 8);
  if (smla::launch_indexer(a, grid, static_cast<hipStream_t>(stream)) != hipSuccess) return SMLA_ERR_HIP;
  return SMLA_OK;
}

const char* sparse_mla_status_string(int status) {
  switch (status) {
    case SMLA_OK: return "ok";
    case SMLA_ERR_INVALID_ARG: return "invalid argument (null or misaligned pointer, bad size or stride)";
    case SMLA_ERR_UNSUPPORTED: return "unsupported configuration";
    case SMLA_ERR_WORKSPACE_TOO_SMALL: return "workspace missing or smaller than sparse_mla_workspace_size()";
    case SMLA_ERR_HIP: return "HIP runtime error";
    default: return "unknown status";
  }
}

}  // extern "C"
