// Sparse indexer scoring (MQA logits), CDNA4 (gfx950) kernel.
//
// What is computed (vLLM PR #54951, "TL;DR" and "Summary": every query row is
// scored against its full available key history by "MQA logits", and the
// top-k of those logits become its int32 index list; "Additional checks":
// the logits of a row do not depend on which other rows share the batch):
//     logits[t, s] = sum_j w[t, j] * max(0, q[t, j, :] . k[s, :])   for s < lens[t]
// with H indexer heads of D = 128 dims per row sharing one key vector per
// history position (MQA), fp32 head weights, bf16 queries and keys.
//
// Design (one work-group = 16 query rows x one chunk of keys):
//   * the 16 rows' queries sit in registers as MFMA A operands (wave w holds
//     rows 2w and 2w + 1: H/16 head groups x 4 k-steps of 32 dims each), so
//     every K operand read from LDS feeds both rows' MFMAs (measured on
//     4096 x 65536, H = 64: 3.55 ms with one row per wave, 3.33 ms with two);
//     eight waves, two per SIMD, so one wave's ReLU / weight / reduction work
//     overlaps the other's MFMAs;
//   * 64-key tiles of K (16 KB) stream through a double-buffered LDS ring,
//     loaded into registers two tiles ahead and written with a 16-byte chunk
//     swizzle (chunk c of key s at c ^ (s & 15)) so the operand reads of 16
//     keys x one chunk hit 16 distinct bank groups;
//   * per 16-key block, D[head][key] = Q . K^T on v_mfma_f32_16x16x32_bf16
//     (lane: key n, heads 4*g4 + j), then ReLU, the head weight and the sum
//     over the lane's heads and head groups, and a two-step butterfly over
//     the four lane groups; lane group g keeps the block g result, so a wave
//     stores 64 consecutive logits of a row with one coalesced write;
//   * work units are chunk-major and mapped so the units of one XCD share its
//     key chunks in their L2.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "smla_internal.h"

namespace smla {
namespace {

#define LDS_AS __attribute__((address_space(3)))

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4;
typedef __attribute__((__vector_size__(4 * sizeof(uint32_t)))) uint32_t u32x4;

constexpr int IX_D = 128;          // dims per indexer head
constexpr int IX_KT = 64;          // keys per tile
constexpr int IX_RPW = 2;          // query rows per wave
constexpr int IX_NW = 8;           // waves per work-group (two per SIMD)
constexpr int IX_RB = IX_RPW * IX_NW;   // query rows per work-group
constexpr int IX_TILE_BYTES = IX_KT * IX_D * 2;
constexpr int IX_LPT = IX_TILE_BYTES / (IX_NW * 64 * 16);   // 16-byte loads per thread per tile

// Word 3 of a raw buffer descriptor on gfx950 (32-bit data format, no
// swizzle): offsets at or past num_records are out of range, and a store
// there is dropped.
constexpr int kBufferFlags = 0x00020000;

// max(x, 0) as one integer max on the bit pattern: non-negative floats are
// non-negative integers in the same order, negative floats negative integers
__device__ __forceinline__ float relu(float x) { return __int_as_float(max(__float_as_int(x), 0)); }

// LDS position (bytes) of 16-byte chunk c of tile key s
__device__ __forceinline__ uint32_t ix_pos(int s, int c) { return (uint32_t)(s * 256 + ((c ^ (s & 15)) << 4)); }

template <int HB>   // 16-head groups (H = 16 * HB)
__global__ void __launch_bounds__(IX_NW * 64, 1) smla_indexer_logits(IndexerArgs a) {
  __shared__ __attribute__((aligned(1024))) uint8_t smem[2 * IX_TILE_BYTES];
  const int b = blockIdx.x;
  const int64_t unit = (int64_t)(b & 7) * a.grid_per_xcd + (b >> 3);
  if (unit >= a.units) return;
  const int chunk = (int)(unit / a.row_blocks);
  const int rb = (int)(unit - (int64_t)chunk * a.row_blocks);
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
  const int g4 = lane >> 4, n = lane & 15;

  // rows of this work-group and the longest history among them
  const int t0 = rb * IX_RB;
  int myrow_len = 0;
  if (lane < IX_RB && t0 + lane < a.T) {
    int L = a.lens ? a.lens[t0 + lane] : a.n_keys;
    myrow_len = L < 0 ? 0 : (L > a.n_keys ? a.n_keys : L);
  }
  int maxlen = myrow_len;
#pragma unroll
  for (int d = 1; d < IX_RB; d <<= 1) maxlen = max(maxlen, __shfl_xor(maxlen, d, 64));
  maxlen = __shfl(maxlen, 0, 64);   // lanes 0..IX_RB-1 hold the rows' lengths; make it wave-uniform
  const int c0 = chunk * a.chunk_keys;
  const int cend = min(min(c0 + a.chunk_keys, a.n_keys), maxlen);
  if (cend <= c0) return;   // every row's history ends before this chunk (uniform over the work-group)
  const int ntiles = (cend - c0 + IX_KT - 1) / IX_KT;

  // this wave's rows: queries (A operands) and weights
  // (a row past the batch reads the last row's queries and has length 0:
  // nothing of it is stored)
  __amdgpu_buffer_rsrc_t orow[IX_RPW];   // logits row t: records = its length, so keys >= lens[t] are dropped
  bf16x8 qa[IX_RPW][HB][4];
  f32x4 wv[IX_RPW][HB];
#pragma unroll
  for (int r = 0; r < IX_RPW; ++r) {
    const int t = t0 + IX_RPW * wave + r;
    const int tq = t < a.T ? t : a.T - 1;
    const int len = __builtin_amdgcn_readfirstlane(__shfl(myrow_len, IX_RPW * wave + r, 64));
    orow[r] = __builtin_amdgcn_make_buffer_rsrc(a.logits + (int64_t)tq * a.ld, (short)0, len * 4, kBufferFlags);
#pragma unroll
    for (int mb = 0; mb < HB; ++mb) {
      const uint16_t* qp = a.q + (int64_t)tq * a.q_st + (int64_t)(16 * mb + n) * a.q_sh + 8 * g4;
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) qa[r][mb][kk] = *reinterpret_cast<const bf16x8*>(qp + 32 * kk);
      wv[r][mb] = *reinterpret_cast<const f32x4*>(a.w + (int64_t)tq * a.w_st + 16 * mb + 4 * g4);
    }
  }

  // K tile loads: thread tid moves 16-byte chunks L = i * 256 + tid (key L / 16, chunk L % 16)
  auto load_tile = [&](int kt, u32x4 (&st)[IX_LPT]) {
#pragma unroll
    for (int i = 0; i < IX_LPT; ++i) {
      const int L = i * (IX_NW * 64) + tid;
      int key = c0 + kt * IX_KT + (L >> 4);
      key = key < a.n_keys ? key : a.n_keys - 1;   // tail keys repeat the last key (never stored)
      st[i] = *reinterpret_cast<const u32x4*>(a.k + (int64_t)key * a.k_st + 8 * (L & 15));
    }
  };
  auto store_tile = [&](int buf, const u32x4 (&st)[IX_LPT]) {
    LDS_AS uint8_t* base = (LDS_AS uint8_t*)smem + buf * IX_TILE_BYTES;
#pragma unroll
    for (int i = 0; i < IX_LPT; ++i) {
      const int L = i * (IX_NW * 64) + tid;
      *reinterpret_cast<LDS_AS u32x4*>(base + ix_pos(L >> 4, L & 15)) = st[i];
    }
  };

  // one tile: 4 blocks of 16 keys; lane (g4, n) ends with the logit of key
  // 16 * g4 + n of the tile for each of the wave's rows
  auto compute = [&](int buf, float (&res)[IX_RPW]) {
    const LDS_AS uint8_t* base = (const LDS_AS uint8_t*)smem + buf * IX_TILE_BYTES;
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
      bf16x8 kbop[4];
#pragma unroll
      for (int kk = 0; kk < 4; ++kk)
        kbop[kk] = *reinterpret_cast<const LDS_AS bf16x8*>(base + ix_pos(16 * kb + n, 4 * kk + g4));
#pragma unroll
      for (int r = 0; r < IX_RPW; ++r) {
        // one accumulation chain per head group, interleaved so consecutive
        // MFMAs are independent
        f32x4 acc[HB];
#pragma unroll
        for (int mb = 0; mb < HB; ++mb) acc[mb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kk = 0; kk < 4; ++kk)
#pragma unroll
          for (int mb = 0; mb < HB; ++mb)
            acc[mb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qa[r][mb][kk], kbop[kk], acc[mb], 0, 0, 0);
        float v = 0.f;
#pragma unroll
        for (int mb = 0; mb < HB; ++mb)
#pragma unroll
          for (int j = 0; j < 4; ++j) v += wv[r][mb][j] * relu(acc[mb][j]);
        v += __shfl_xor(v, 16, 64);
        v += __shfl_xor(v, 32, 64);
        res[r] = (g4 == kb) ? v : res[r];
      }
    }
  };
  // every lane stores; the row's buffer descriptor drops keys at or past its length
  auto store_logits = [&](int kt, const float (&res)[IX_RPW]) {
    const int key = c0 + kt * IX_KT + 16 * g4 + n;
#pragma unroll
    for (int r = 0; r < IX_RPW; ++r)
      __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(res[r]), orow[r], key * 4, 0, 0);
  };

  // ---- pipeline: LDS double buffer; register sets A (even tiles) and B (odd
  // tiles) each loaded two tiles before their LDS write.  Every step issues the
  // same loads and stores (past the last tile the loads repeat the last key), so
  // the compiler's memory-counter waits stay exact and each wait covers only the
  // tile being written.
  // the queries and weights have landed before any tile load is in flight
  // (their first use would otherwise put memory waits inside the loop)
#pragma unroll
  for (int r = 0; r < IX_RPW; ++r)
#pragma unroll
    for (int mb = 0; mb < HB; ++mb) {
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) asm volatile("" : : "v"(qa[r][mb][kk]));
      asm volatile("" : : "v"(wv[r][mb]));
    }
  u32x4 stA[IX_LPT], stB[IX_LPT];
  load_tile(0, stA);
  load_tile(1, stB);
  store_tile(0, stA);
  load_tile(2, stA);
  __syncthreads();
  for (int kt = 0;; kt += 2) {
    // even step: tile kt in buffer 0; tile kt + 1 (set B) to buffer 1
    float res[IX_RPW];
    store_tile(1, stB);
    load_tile(kt + 3, stB);
    compute(0, res);
    store_logits(kt, res);
    __syncthreads();
    if (kt + 1 >= ntiles) break;
    // odd step: tile kt + 1 in buffer 1; tile kt + 2 (set A) to buffer 0
    store_tile(0, stA);
    load_tile(kt + 4, stA);
    compute(1, res);
    store_logits(kt + 1, res);
    __syncthreads();
    if (kt + 2 >= ntiles) break;
  }
}

}  // namespace

hipError_t launch_indexer(const IndexerArgs& a, int64_t grid, hipStream_t stream) {
  switch (a.H / 16) {
    case 1: hipLaunchKernelGGL(smla_indexer_logits<1>, dim3((unsigned)grid), dim3(IX_NW * 64), 0, stream, a); break;
    case 2: hipLaunchKernelGGL(smla_indexer_logits<2>, dim3((unsigned)grid), dim3(IX_NW * 64), 0, stream, a); break;
    case 3: hipLaunchKernelGGL(smla_indexer_logits<3>, dim3((unsigned)grid), dim3(IX_NW * 64), 0, stream, a); break;
    case 4: hipLaunchKernelGGL(smla_indexer_logits<4>, dim3((unsigned)grid), dim3(IX_NW * 64), 0, stream, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

int indexer_rows_per_block() { return IX_RB; }

}  // namespace smla
