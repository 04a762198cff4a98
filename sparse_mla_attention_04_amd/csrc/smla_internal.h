// Internal interface between the C-ABI host code and the HIP kernels.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace smla {

// Index entries (or, in the dense mode, block-table pages) a work-group holds
// in LDS per pass.
constexpr int kListCap = 2048;

// Bytes of the static device scratch of the allocation-free entry point:
// 256 split units x 64 heads x 513 fp32, the largest partials buffer of any
// automatic plan on a GPU of up to 256 compute units (an automatic plan
// splits only when T < #CU, and then into at most #CU units).
constexpr size_t kNoallocScratchBytes = (size_t)256 * 64 * 513 * 4;
constexpr int kMaxDevices = 256;

// This GPU's copy of the static scratch (the current device), looked up on
// the first call per device; never freed.
hipError_t noalloc_scratch(void** ptr);

// Everything a forward launch needs, passed by value as the kernel argument.
struct FwdArgs {
  const uint16_t* q;          // bf16 [T, h, 576] (strided)
  const uint8_t* kv;          // cache pool base
  const int32_t* block_table; // LOGICAL mode
  const int32_t* token_seq;   // LOGICAL mode
  const int32_t* topk_idx;    // int32 [T, idx_stride]
  uint16_t* out;              // bf16 [T, h, 512] (strided)
  float* lse;                 // fp32 [T, h] (strided)
  float* ws_out;              // fp32 [units, h, 512] split partials
  float* ws_lse;              // fp32 [units, h]
  int64_t q_st, q_sh, out_st, out_sh, lse_st, idx_stride, bt_stride;
  int64_t num_slots;          // num_pages * page_size (<= INT32_MAX)
  int64_t num_pages;
  int64_t units;              // T * num_splits
  int32_t T, h, topk, num_splits;
  int32_t page_shift, index_mode, num_seqs, max_blocks;
  int32_t grid_per_xcd;       // launched work-groups / 8
  int32_t write_partials;     // 1: write fp32 partials to ws_out / ws_lse instead of out / lse
  float scale_log2;           // |softmax_scale| * log2(e) (never negative)
  int32_t q_neg;              // softmax_scale < 0: queries enter with their sign flipped, so
                              // every score is |scale| * (-q) . k = scale * q . k exactly
  int32_t bucket_shift;       // >= 0: gather each row's entries grouped by (slot >> shift), 16 groups; -1: list order
  // dense causal mode only
  const int32_t* query_start; // int32 [num_seqs + 1]: rows of sequence s are [query_start[s], query_start[s+1])
  const int32_t* positions;   // int32 [T]: row t attends to positions 0 .. positions[t] of its sequence
  int32_t dense_qb;           // query rows per work-group (64 / h)
};

struct CombineArgs {
  const float* ws_out;
  const float* ws_lse;
  uint16_t* out;
  float* lse;
  int64_t out_st, out_sh, lse_st;
  int32_t T, h, num_splits;
};

// Per-row top-k selection.
struct TopkArgs {
  const float* scores;        // fp32 [T, ld]
  const int32_t* lens;        // int32 [T] valid keys per row, or null (n_keys)
  int32_t* idx;               // int32 [T, idx_stride]
  int64_t ld, idx_stride;
  int32_t T, n_keys, k;
};
hipError_t launch_topk(const TopkArgs& a, hipStream_t stream);

// Indexer scoring (MQA logits): one work-group per (8 query rows, key chunk).
struct IndexerArgs {
  const uint16_t* q;          // bf16 [T, H, 128] (strided)
  const uint16_t* k;          // bf16 [n_keys, 128] (row stride k_st)
  const float* w;             // fp32 [T, H] (row stride w_st)
  const int32_t* lens;        // int32 [T] or null (every row sees n_keys keys)
  float* logits;              // fp32 [T, ld]
  int64_t q_st, q_sh, k_st, w_st, ld;
  int64_t units;              // row_blocks * key chunks
  int32_t row_blocks, chunk_keys, grid_per_xcd;
  int32_t T, n_keys, H;
};
hipError_t launch_indexer(const IndexerArgs& a, int64_t grid, hipStream_t stream);
int indexer_rows_per_block();

// Pipeline shape of one forward kernel instantiation.
struct FwdShape {
  int head_groups, row_groups, tile_rows, stages, threads, lds_bytes;
};

// Shape of kernel `variant` for `head_groups`; returns false when no such kernel exists.
bool fwd_shape(int kv_format, int head_groups, int variant, int nope, FwdShape* shape);

// Launches; return a hipError_t.
hipError_t launch_fwd(const FwdArgs& a, int kv_format, int head_groups, int variant, int nope, int64_t grid,
                      hipStream_t stream);
hipError_t launch_combine(const CombineArgs& a, hipStream_t stream);
// Dense causal mode (bf16, rows of 576 or 512 dims): grid work-groups of 256 threads.
hipError_t launch_dense(const FwdArgs& a, int nope, int64_t grid, hipStream_t stream);
int dense_lds_bytes(int nope);

}  // namespace smla
