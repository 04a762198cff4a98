// Sparse MLA forward over top-k selected cache rows, CDNA4 (gfx950) kernels.
//
// What is computed: for each query row t, attention of its h heads over the
// cache rows its index list names, all heads sharing the same 576-wide rows
// (MQA / absorbed form; prhub report on vLLM PR #55738, "Motivation"), with
// the output in the 512-dim latent space and an fp32 log-sum-exp per head
// (vLLM PR #60220, "Claims" and "Details").
//
// Design (one work-group = one query row, or one KV split of it):
//   * index compaction: the row's entries are translated to physical rows
//     (block table in LOGICAL mode), -1 / out-of-range entries dropped, and
//     the surviving rows stored in order in LDS;
//   * gather: rows are copied HBM -> LDS with direct-to-LDS 16-byte loads
//     (global_load_lds_dwordx4), a ring of `NST` tiles per row group, issued
//     and waited on by hand so several tiles stay in flight; eight lanes
//     fetch one 128-byte line of a row, the 16-byte chunks of a line being
//     XOR-swizzled so MFMA operand reads are free of LDS bank conflicts;
//   * scores: S^T = K . Q^T on v_mfma_f32_16x16x32_bf16 (K from LDS, the
//     row's queries for 16 heads held in registers), so each lane ends up
//     owning one head's scores;
//   * online softmax in base 2 with wave-level reductions (max over the four
//     lanes that share a head);
//   * P.V: O^T += V^T . P^T on MFMA, V^T read straight from the same LDS
//     tile with ds_read_b64_tr_b16 (the transposing LDS read of gfx950); the
//     pipelined h = 64 kernels use v_mfma_f32_32x32x16_bf16 there (half the
//     MFMA instructions of 16x16x32 for the same work);
//   * waves that split the rows of one query are merged through LDS at the
//     end; a split work-group writes its fp32 partial (normalised output
//     and lse) to the caller's workspace instead, and a second kernel merges
//     the splits by their lse (the fp32 split-KV path of PR #60220,
//     "Overview"/"Limitations", with the buffer owned by the caller);
//   * at up to 32 heads, shapes of two waves and at most 80 KB of LDS let two
//     work-groups share a CU, so one row's start-up loads and epilogue
//     overlap another row's tiles.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <mutex>
#include <type_traits>

#include "smla_internal.h"

// Device scratch of the allocation-free entry point: the fp32 split partials
// of one call (units x h x 513 fp32).  Each GPU the library runs on holds its
// own copy until the process ends; host code never uses this name as an
// address, only the per-device pointer hipGetSymbolAddress returns for it.
static __device__ __align__(256) uint8_t scratch[smla::kNoallocScratchBytes];

namespace smla {
namespace {

#define LDS_AS __attribute__((address_space(3)))

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(4 * sizeof(__bf16)))) __bf16 bf16x4;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16;
typedef __attribute__((__vector_size__(4 * sizeof(uint32_t)))) uint32_t u32x4;
typedef __attribute__((__vector_size__(2 * sizeof(uint32_t)))) uint32_t u32x2;

constexpr int D_QK = 576;
constexpr int D_V = 512;
constexpr int ROW_BYTES = D_QK * 2;     // bf16 cache row
constexpr int NOPE_ROW_BYTES = D_V * 2; // bf16 cache row of the NoPE geometry (no rope part)
constexpr int FP8_ROW_BYTES = 640;      // fp8 cache row: 512 code bytes + 64 bf16 rope
constexpr int FP8_NOPE_ROW_BYTES = 512; // fp8 cache row of the NoPE geometry: the 512 code bytes
constexpr int FP8_SCALE_BYTES = 16;     // four fp32 block scales per fp8 row, after the page's rows
constexpr int LIST_CAP = kListCap;      // index entries compacted per pass
constexpr float NEG_INF = -__builtin_inff();
constexpr float LN2 = 0.69314718055994530942f;
constexpr float REF_HEADROOM = 64.0f;   // p = 2^(x - ref) may reach 2^64 before a second pass is forced

template <int HG_, int NRG_, int RT_, int NST_, int FMT_, bool DSPLIT_ = false, bool PIPE_ = false,
          bool PAIR_ = false, bool RSPLIT_ = false, bool NOPE_ = false, bool DENSE_ = false, bool TWO_ = false>
struct Shape {
  static constexpr int HG = HG_;            // 16-head groups (waves per row group)
  static constexpr int NRG = NRG_;          // row groups (independent KV row streams)
  static constexpr int RT = RT_;            // rows per tile
  static constexpr int NST = NST_;          // tiles in flight per row group
  static constexpr bool FP8 = FMT_ == 1;    // fp8 latent + bf16 rope rows, per-128-dim scales
  static constexpr int NW = HG * NRG;       // waves
  static constexpr int NTHR = NW * 64;
  static constexpr int NF = RT / 16;        // 16-row score fragments per tile
  static constexpr int NRH = RT / 8;        // 8-row DMA groups per tile
  static constexpr int RH_PER_WAVE = NRH / HG;
  // NOPE: the NoPE geometry, rows and queries of the 512 latent dims only
  static constexpr bool NOPE = NOPE_;
  static constexpr int ROWB = FP8 ? (NOPE ? FP8_NOPE_ROW_BYTES : FP8_ROW_BYTES)
                                 : NOPE ? NOPE_ROW_BYTES : ROW_BYTES;  // bytes per cache row
  static constexpr int KS = NOPE ? 16 : 18;           // 32-dim k-steps of a score
  static constexpr int NLINES = ROWB / 128;           // 128-B lines per row
  static constexpr int BODY_BYTES = RT * NLINES * 128;
  static constexpr int TILE_BYTES = BODY_BYTES + (FP8 ? RT * 16 : 0);       // + fp32 block scales
  static constexpr int PER = NLINES * RH_PER_WAVE + (FP8 ? 1 : 0);  // DMA instructions per wave per tile
  static constexpr int RING_BYTES = NRG * NST * TILE_BYTES;
  static constexpr int LIST_OFF = RING_BYTES;
  // TWO: at most 80 KB of LDS, so two work-groups share a CU and one's
  // start-up and epilogue overlap the other's tiles.  The compaction counts
  // and the epilogue statistics then live in the tile ring, which is idle
  // whenever they are used (before the first gather of a pass, after the
  // last tile has been consumed).
  static constexpr bool TWO = TWO_;
  static constexpr int TWO_STAT_OFF = HG * NRG * 32 * 64 * 16;   // above the epilogue staging
  static constexpr int CNT_OFF = TWO ? TWO_STAT_OFF + HG * NRG * 16 * 2 * 4 : LIST_OFF + LIST_CAP * 4;
  // DSPLIT: every wave computes P for its 16 heads, the waves exchange P
  // through LDS, and wave w accumulates output dims [128w, 128w + 128) for all
  // 4 head groups, so each V element is read from LDS once per tile.
  static constexpr bool DSPLIT = DSPLIT_;
  // PIPE (with DSPLIT): software pipeline over tiles; the scores of tile i+1
  // are computed while tile i's softmax runs and tile i+NST's gathers are
  // issued, and tile i+1's V^T operands are read while tile i's P.V runs.
  static constexpr bool PIPE = PIPE_;
  // PAIR (fp8, h <= 16): the two waves of a row stream share its tiles; wave
  // hp forms the scores and softmax of the tile's rows 16hp .. 16hp + 15 and
  // accumulates output dims [256hp, 256hp + 256) over all 32 rows, the scaled
  // P of the 4 dim blocks being exchanged through LDS.  The pair shares one
  // exponent reference.
  static constexpr bool PAIR = PAIR_;
  // RSPLIT (with PIPE): wave w forms the scores and softmax of tile rows
  // 16(w & 1) .. +15 for the 32 heads 32(w >> 1) .. +31, so every K operand read
  // from LDS feeds two MFMAs; the two waves holding one head's row halves share
  // its exponent reference and add their row sums at the end.
  static constexpr bool RSPLIT = RSPLIT_;
  // PV32 (pipelined, without RSPLIT): P.V on v_mfma_f32_32x32x16_bf16, each
  // wave's 128 output dims x 64 heads as 4 x 2 accumulators of 32 x 32
  static constexpr bool PV32 = PIPE_ && !RSPLIT_;
  static constexpr int NE = RSPLIT ? 2 : 1;            // 16-head groups in a wave's scores
  static constexpr int HEAD_GROUPS = PAIR ? 1 : HG;   // 16-head groups the shape covers
  // per-wave counts (NW x 8 words) at CNT_OFF.  The pipelined shapes keep the
  // counts (compaction only), the P exchange (tile loop only) and the
  // statistics (epilogue only) in one region; P is double-buffered there.
  static constexpr int STAT_BYTES = NW * 16 * 2 * 4 * NE;
  static constexpr int PEX_OFF = PIPE ? CNT_OFF : CNT_OFF + 512;
  static constexpr int PEX_BYTES = DSPLIT ? 2 * 4 * 64 * 16 : PAIR ? NRG * 4 * 64 * 16 : 0;
  static constexpr int MEX_OFF = PEX_OFF + PEX_BYTES;
  static constexpr int STAT_OFF = TWO ? TWO_STAT_OFF : PIPE ? CNT_OFF : MEX_OFF + (PAIR ? NW * 64 * 4 : 0);
  static constexpr int LDS_BYTES =
      TWO    ? LIST_OFF + LIST_CAP * 4
      : PIPE ? CNT_OFF + (PEX_BYTES > STAT_BYTES ? (PEX_BYTES > 512 ? PEX_BYTES : 512) : (STAT_BYTES > 512 ? STAT_BYTES : 512))
             : STAT_OFF + STAT_BYTES;
  static constexpr int EPT = LIST_CAP / NTHR;   // index entries per thread per pass
  static constexpr bool SYNC = HG > 1;          // waves share tiles -> barrier per tile
  static_assert(RT == 16 || RT == 32, "tile rows");
  static_assert(!FP8 || RT == 32, "the fp8 P.V step pairs two 16-row fragments");
  static_assert(NRH % HG == 0, "DMA groups must split evenly over the waves of a row group");
  static_assert((NST - 1) * PER <= 63, "vmcnt holds at most 63 outstanding loads");
  // epilogue staging: every wave's 32 accumulator fragments (a wave pair
  // stages its row stream's 32 fragments once)
  static_assert((PAIR_ ? NRG : NW) * 32 * 64 * 16 <= STAT_OFF, "epilogue staging must fit below the statistics");
  static_assert(NW * 8 * 4 <= 512, "compaction counts");
  static_assert(LDS_BYTES <= 160 * 1024, "LDS");
  static_assert(LIST_CAP % NTHR == 0, "compaction split");
  static_assert(!DSPLIT || (HG == 4 && NRG == 1 && RT == 32 && !FP8), "output-dim split layout");
  static_assert(!PIPE || (DSPLIT && NST >= 3 && PER == NLINES), "pipelined variant layout");
  // DENSE (with PIPE): dense causal mode.  A work-group takes a block of up to
  // 64 / h consecutive query rows of one sequence; its 64 query slots are
  // (row, head) pairs m = row * h + head, and every cache row of positions
  // 0 .. max position is gathered once for all of them (tile i = positions
  // 32i .. 32i + 31 through the block table), each slot masking positions
  // past its own row's.
  static constexpr bool DENSE = DENSE_;
  static_assert(!DENSE || (PIPE && !RSPLIT && !FP8), "dense mode runs the pipelined bf16 schedule");
  static_assert(!DSPLIT || PIPE, "the output-dim split runs in the pipelined schedule");
  static_assert(!PAIR || (FP8 && HG == 2 && RT == 32 && !DSPLIT), "row/dim-split pair layout");
  static_assert(!RSPLIT || PIPE, "the row-half score split runs in the pipelined schedule");
  static_assert(!TWO || (!PIPE && !PAIR && !FP8 && NE == 1), "two-per-CU layout: plain bf16 row streams");
  static_assert(!TWO || (CNT_OFF + NW * 8 * 4 <= RING_BYTES && LDS_BYTES <= 80 * 1024), "two-per-CU layout");
};

__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(const LDS_AS void*)p;
}

// One 64 x 16-byte direct-to-LDS gather: lane l reads 16 bytes at
// gaddr + OFF and writes them to LDS at m0 + OFF + 16 * l.
template <int OFF>
__device__ __forceinline__ void dma16(const void* gaddr, uint32_t m0) {
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off offset:%2"
               :
               : "v"(gaddr), "s"(__builtin_amdgcn_readfirstlane(m0)), "n"(OFF)
               : "memory", "m0");
}

// The KS 16-byte pieces of a lane's query (k-step kk at qp + 32 kk bf16
// elements) to LDS bytes qd + 1024 kk + 16 lane: one direct-to-LDS load per
// k-step, each covering 1 KB of contiguous LDS for the wave.
template <int KS>
__device__ __forceinline__ void dma_queries(const uint16_t* qp, uint32_t qd) {
#pragma unroll
  for (int kk = 0; kk < KS; ++kk) {
    switch (kk) {   // dma16 writes LDS at m0 + offset + 16 lane
      case 0: dma16<0>(qp, qd); break;
      case 1: dma16<64>(qp, qd + 1 * 960); break;
      case 2: dma16<128>(qp, qd + 2 * 960); break;
      case 3: dma16<192>(qp, qd + 3 * 960); break;
      case 4: dma16<256>(qp, qd + 4 * 960); break;
      case 5: dma16<320>(qp, qd + 5 * 960); break;
      case 6: dma16<384>(qp, qd + 6 * 960); break;
      case 7: dma16<448>(qp, qd + 7 * 960); break;
      case 8: dma16<512>(qp, qd + 8 * 960); break;
      case 9: dma16<576>(qp, qd + 9 * 960); break;
      case 10: dma16<640>(qp, qd + 10 * 960); break;
      case 11: dma16<704>(qp, qd + 11 * 960); break;
      case 12: dma16<768>(qp, qd + 12 * 960); break;
      case 13: dma16<832>(qp, qd + 13 * 960); break;
      case 14: dma16<896>(qp, qd + 14 * 960); break;
      case 15: dma16<960>(qp, qd + 15 * 960); break;
      case 16: dma16<1024>(qp, qd + 16 * 960); break;
      default: dma16<1088>(qp, qd + 17 * 960); break;
    }
  }
}

template <int N>
__device__ __forceinline__ void wait_vm() {
  asm volatile("s_waitcnt vmcnt(%0)" : : "n"(N) : "memory");
}

// Wait until at most pend * PER of this wave's gathers are outstanding.
template <int PER, int NST>
__device__ __forceinline__ void wait_tiles(int pend) {
  if (pend <= 0) { wait_vm<0>(); return; }
  if constexpr (NST > 2) {
    if (pend == 1) { wait_vm<PER>(); return; }
    if constexpr (NST > 3) {
      if (pend == 2) { wait_vm<2 * PER>(); return; }
      if constexpr (NST > 4) {
        if (pend == 3) { wait_vm<3 * PER>(); return; }
      }
    }
  }
  // pend >= NST - 1: nothing newer than (NST - 1) tiles can be pending
  wait_vm<(NST - 1) * PER>();
}

__device__ __forceinline__ void lds_barrier() { asm volatile("s_barrier" : : : "memory"); }

__device__ __forceinline__ float wave_xor(float v, int m) { return __shfl_xor(v, m, 64); }


__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Exponent reference of a head: a base-2 score maximum rounded up to an
// integer.  With integer references P = 2^(x - m) is, for any m, the same
// bf16 value up to an exact power of two, so a row split into KV chunks
// (each with its own reference) rounds every P exactly as the unsplit row
// does, and the lse-weighted merge of the chunks reproduces the unsplit
// result up to fp32 summation order.  -inf (no score yet) stays -inf.
__device__ __forceinline__ float int_ref(float m) { return __builtin_ceilf(m); }

// max over lanes l, l^16, l^32, l^48 with the gfx950 lane-swap instructions
// (rows of 16 lanes swapped, then halves of 32), no LDS traffic
__device__ __forceinline__ float max_xor16_32(float v) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}

// two floats to a packed bf16 pair (round to nearest even), one instruction
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  typedef float f32x2v __attribute__((ext_vector_type(2)));
  typedef __bf16 bf16x2v __attribute__((ext_vector_type(2)));
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2v{lo, hi}, bf16x2v));
}

__device__ __forceinline__ uint16_t f32_to_bf16_bits(float x) {
  __bf16 b = (__bf16)x;
  return __builtin_bit_cast(uint16_t, b);
}

// Byte offset of a cache row: bf16 rows are contiguous; fp8 pages hold the
// page's rows first ([512 codes | 64 bf16 rope] each, or the 512 codes alone
// in the NoPE geometry) and then their scales.
template <bool FP8, int ROWB>
__device__ __forceinline__ int64_t row_offset(const FwdArgs& a, int slot) {
  if constexpr (FP8) {
    const int64_t page = slot >> a.page_shift;
    const int64_t rin = slot & ((1 << a.page_shift) - 1);
    return page * ((int64_t)(ROWB + FP8_SCALE_BYTES) << a.page_shift) + rin * ROWB;
  } else {
    return (int64_t)slot * ROWB;
  }
}

// 8 fp8 E4M3 codes (two 32-bit words) -> 8 bf16 values, exact.
__device__ __forceinline__ bf16x8 fp8x8_to_bf16(uint32_t w0, uint32_t w1) {
  typedef __attribute__((__vector_size__(2 * sizeof(__bf16)))) __bf16 bf16x2;
  const bf16x2 a0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)w0, 1.0f, false);
  const bf16x2 a1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)w0, 1.0f, true);
  const bf16x2 a2 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)w1, 1.0f, false);
  const bf16x2 a3 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)w1, 1.0f, true);
  return bf16x8{a0[0], a0[1], a1[0], a1[1], a2[0], a2[1], a3[0], a3[1]};
}

// XOR swizzle of the 16-byte chunks of tile row r (3 bits).  gfx950's LDS
// has 64 banks (256 B); measured with single-pattern probes, an 8-byte read
// (plain or transposing) serves lanes 0-31 and then 32-63, and a 16-byte read
// serves the lane sets {0-7, 24-31}, {8-23}, {32-39, 56-63}, {40-55} one per
// cycle.  A tile row is 128 B, so the bank group of chunk c of row r is
// 8 (r & 1) + (c ^ swz(r)), and each cycle's lanes need distinct groups:
//   bf16 tiles (16-row K operand reads of one chunk per lane group; 4-row x
//     2-chunk transposing V reads; the 32x32 P.V reads, which take rows r0
//     and r0 + 16 with the swizzle of r0): r & 7 is conflict-free for all;
//   fp8 tiles (the same K reads; transposing reads of rows 4g + j and
//     16 + 4g + j): the K reads put rows r and r + 8 in one cycle with chunks
//     c and c ^ 1, the transposing reads rows r and r + 16 with one chunk.
// Bit 2 of the swizzle also decides, for each row of a gather instruction,
// which 64-byte half of the row's line its first four lanes fetch.  On the
// 640-byte fp8 rows, gathers ran 4% faster when that bit follows row bit 1
// (or 0) than when it follows row bit 2 or is constant; bf16 and the 512-byte
// NoPE rows showed no difference.  Among the conflict-free fp8 swizzles this
// one takes bit 2 from row bit 1.
template <bool FP8>
__device__ __forceinline__ int swz(int r) {
  if constexpr (FP8) return ((r & 2) << 1) | ((r & 4) >> 1) | ((r >> 4) & 1);
  else return r & 7;
}

// Translate a thread's EPT index entries to physical cache rows (-1 when
// skipped).  LOGICAL mode requests every entry's block-table word before
// using any of them, so the thread waits for one round trip, not EPT: a
// skipped entry reads the row's first word instead (block tables hold at
// least one sequence of at least one block), and its result is discarded.
template <int EPT>
__device__ __forceinline__ void translate_all(const FwdArgs& a, const int (&raw)[EPT], int seq_ok, int64_t bt_row,
                                              int (&sl)[EPT]) {
  if (a.index_mode == 0) {
#pragma unroll
    for (int i = 0; i < EPT; ++i) sl[i] = (raw[i] >= 0 && raw[i] < a.num_slots) ? raw[i] : -1;
    return;
  }
  bool ok[EPT];
  int pg[EPT];
#pragma unroll
  for (int i = 0; i < EPT; ++i) {
    const int blk = raw[i] >> a.page_shift;
    ok[i] = seq_ok && raw[i] >= 0 && blk < a.max_blocks;
    pg[i] = a.block_table[bt_row + (ok[i] ? blk : 0)];
  }
  // every looked-up word is waited for here, unconditionally: waits the
  // compiler would otherwise place on the later, lane-dependent uses leave
  // it counting these loads as pending into the tile loop, where its waits
  // would also drain the gathers
#pragma unroll
  for (int i = 0; i < EPT; ++i) asm volatile("" : : "v"(pg[i]));
#pragma unroll
  for (int i = 0; i < EPT; ++i)
    sl[i] = (ok[i] && pg[i] >= 0 && pg[i] < a.num_pages)
                ? (pg[i] << a.page_shift) | (raw[i] & ((1 << a.page_shift) - 1))
                : -1;
}

// LDS word of compacted list entry k: each 64-word block rotated by its block
// index, so the compaction's writes (a thread stores its survivors at
// consecutive positions, neighbouring lanes 8 or 16 words apart) spread over
// the banks; reads of consecutive entries stay consecutive words modulo 64.
__device__ __forceinline__ int lpos(int k) { return (k & ~63) | ((k + (k >> 6)) & 63); }

// Position of a staged accumulator fragment f of lane (g4, n) in the epilogue
// staging area: each 16-lane row rotated by f + 8 * (g4 >> 1), so the
// merge's reads (16 lanes, one head n, fragments c / 2 and lane rows
// 2 * (c & 1)) hit 16 different bank groups.  A bijection within each row.
__device__ __forceinline__ int spos(int f, int g4, int n) { return f * 64 + g4 * 16 + ((n + f + 8 * (g4 >> 1)) & 15); }

// 16-bit field g of a packed array (two fields per word), g a runtime value
__device__ __forceinline__ uint32_t field16(const uint32_t (&w)[8], int g) {
  uint32_t v = 0;
#pragma unroll
  for (int k = 0; k < 8; ++k) v = ((g >> 1) == k) ? w[k] : v;
  return (v >> ((g & 1) * 16)) & 0xffffu;
}

// Translate a thread's EPT raw index entries and compact the surviving rows
// into list[]; returns the chunk's count.  Two work-group barriers.
//   list order (a.bucket_shift < 0): survivors keep the index list's order
//     (a wave prefix sum, then the waves' offsets);
//   slot order: a stable counting sort of the survivors into 16 groups of
//     physical row (slot >> bucket_shift), list order inside a group, so the
//     rows that run together on one XCD read nearby cache rows.  Counts are
//     packed two groups per 32-bit word (each at most 2048 per pass).
//   after_lookups() runs once every entry's lookup has landed and before the
//   first barrier: loads issued there are not waited for by the compaction.
template <int NW, int EPT, class AfterLookups>
__device__ __forceinline__ int compact_chunk(const FwdArgs& a, const int (&raw)[EPT], int seq_ok, int64_t bt_row,
                                             int* list, int* wcnt, int wave, int lane, AfterLookups&& after_lookups) {
  int sl[EPT];
  translate_all<EPT>(a, raw, seq_ok, bt_row, sl);
  after_lookups();
  int cnt = 0;
#pragma unroll
  for (int i = 0; i < EPT; ++i) cnt += (sl[i] >= 0);
  if (a.bucket_shift < 0) {
    int incl = cnt;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
      const int v = __shfl_up(incl, d, 64);
      if (lane >= d) incl += v;
    }
    if (lane == 63) wcnt[wave] = incl;
    __syncthreads();
    int base = 0, n_valid = 0;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      const int c = wcnt[w];
      base += (w < wave) ? c : 0;
      n_valid += c;
    }
    int pos = base + incl - cnt;
#pragma unroll
    for (int i = 0; i < EPT; ++i) {
      if (sl[i] >= 0) { list[lpos(pos)] = sl[i]; ++pos; }
    }
    __syncthreads();
    return n_valid;
  }
  int grp[EPT];
  uint32_t own[8];
#pragma unroll
  for (int k = 0; k < 8; ++k) own[k] = 0;
#pragma unroll
  for (int i = 0; i < EPT; ++i) {
    const int g = (sl[i] >= 0) ? (sl[i] >> a.bucket_shift) : -1;
    grp[i] = g;
    const uint32_t one = (g >= 0) ? (1u << ((g & 1) * 16)) : 0u;
#pragma unroll
    for (int k = 0; k < 8; ++k) own[k] += ((g >> 1) == k) ? one : 0u;
  }
  uint32_t inc[8];
#pragma unroll
  for (int k = 0; k < 8; ++k) inc[k] = own[k];
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const uint32_t v = __shfl_up(inc[k], d, 64);
      if (lane >= d) inc[k] += v;
    }
  }
  uint32_t* wc = reinterpret_cast<uint32_t*>(wcnt);
  if (lane == 63) {
#pragma unroll
    for (int k = 0; k < 8; ++k) wc[wave * 8 + k] = inc[k];
  }
  __syncthreads();
  uint32_t before[8], total[8];
#pragma unroll
  for (int k = 0; k < 8; ++k) before[k] = total[k] = 0;
#pragma unroll
  for (int w = 0; w < NW; ++w)
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const uint32_t v = wc[w * 8 + k];
      total[k] += v;
      before[k] += (w < wave) ? v : 0u;
    }
  // base of each group for this thread: group start + earlier waves + earlier lanes
  uint32_t base[8];
  uint32_t running = 0;
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    const uint32_t t0 = total[k] & 0xffffu, t1 = total[k] >> 16;
    const uint32_t start = running | ((running + t0) << 16);
    running += t0 + t1;
    base[k] = start + before[k] + (inc[k] - own[k]);
  }
#pragma unroll
  for (int i = 0; i < EPT; ++i) {
    const int g = grp[i];
    if (g >= 0) {
      list[lpos((int)field16(base, g))] = sl[i];
      const uint32_t one = 1u << ((g & 1) * 16);
#pragma unroll
      for (int k = 0; k < 8; ++k) base[k] += ((g >> 1) == k) ? one : 0u;
    }
  }
  __syncthreads();
  return (int)running;
}

template <class S>
__global__ void __launch_bounds__(S::NTHR, 1) smla_fwd(FwdArgs a) {
  __shared__ __attribute__((aligned(1024))) uint8_t smem[S::LDS_BYTES];
  int* list = reinterpret_cast<int*>(smem + S::LIST_OFF);
  int* wcnt = reinterpret_cast<int*>(smem + S::CNT_OFF);
  float* stat = reinterpret_cast<float*>(smem + S::STAT_OFF);
  const LDS_AS uint8_t* lds = (const LDS_AS uint8_t*)smem;
  const uint32_t ring0 = lds_addr(smem);

  // XCD-aware unit mapping: consecutive units share an XCD (and its L2).
  const int b = blockIdx.x;
  const int64_t unit = (int64_t)(b & 7) * a.grid_per_xcd + (b >> 3);
  if (unit >= a.units) return;
  const int S_ = a.num_splits;
  const int t = (int)(unit / S_);
  const int sp = (int)(unit - (int64_t)t * S_);

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
  const int hg = wave % S::HG, rg = wave / S::HG;
  const int g4 = lane >> 4, n = lane & 15;

  // ---- dense mode: block `unit` -> (sequence, first row, rows).  Sequence s
  // has ceil(n_s / qb) blocks; wave 0 scans the block counts 64 sequences at
  // a time and the lane owning `unit` publishes it through LDS.
  int d_seq = 0, d_r0 = 0, d_nr = 0;
  if constexpr (S::DENSE) {
    const int qb = a.dense_qb;
    int* found = reinterpret_cast<int*>(smem + S::CNT_OFF);
    if (tid == 0) found[0] = -1;
    __syncthreads();
    if (wave == 0) {
      int64_t base = 0;
      for (int c = 0; c < a.num_seqs; c += 64) {
        const int s_ = c + lane;
        int q0 = 0, q1 = 0;
        if (s_ < a.num_seqs) {
          q0 = a.query_start[s_];
          q1 = a.query_start[s_ + 1];
        }
        const int nb = (q1 > q0) ? (q1 - q0 + qb - 1) / qb : 0;
        int incl = nb;
#pragma unroll
        for (int d = 1; d < 64; d <<= 1) {
          const int v = __shfl_up(incl, d, 64);
          if (lane >= d) incl += v;
        }
        const int64_t lo = base + incl - nb, hi = base + incl;
        if (unit >= lo && unit < hi) {
          const int r0 = q0 + (int)(unit - lo) * qb;
          found[0] = s_;
          found[1] = r0;
          found[2] = (q1 - r0 < qb) ? q1 - r0 : qb;
        }
        base += __shfl(incl, 63, 64);
        if (base > unit) break;
      }
    }
    __syncthreads();
    d_seq = found[0];
    d_r0 = found[1];
    d_nr = found[2];
    __syncthreads();
    if (d_seq < 0) return;   // past the last block (the grid is an upper bound)
  }
  // dense mode: this lane's query slot m = 16 * hg + n as (row, head); slots
  // past the block's rows repeat its last row (computed, never written)
  const int d_m = 16 * hg + n;
  const int d_row = S::DENSE ? (d_m / a.h < d_nr ? d_m / a.h : d_nr - 1) : 0;
  const int d_head = S::DENSE ? d_m - (d_m / a.h) * a.h : 0;

  // ---- per-lane LDS offsets inside a tile
  // tile layout: position(r, c) = (c / 8) * RT * 8 + r * 8 + ((c % 8) ^ swz(r)), 16 B each
  uint32_t kofs[S::NF][2];     // K operand: row 16f+n, chunk 4*kk+g4
  uint32_t vofs[S::NF][4];     // V^T operand (transposing read): row 16f+4*g4+(n>>2), dims 4*(n&3)
#pragma unroll
  for (int f = 0; f < S::NF; ++f) {
    const int r = 16 * f + n;
    const int sw = swz<S::FP8>(r);
#pragma unroll
    for (int p = 0; p < 2; ++p) kofs[f][p] = (uint32_t)(r * 8 + ((4 * p + g4) ^ sw)) * 16u;
    const int rv = 16 * f + 4 * g4 + (n >> 2);
    const int swv = swz<S::FP8>(rv);
    const int cq = n & 3;
#pragma unroll
    for (int p = 0; p < 4; ++p)
      vofs[f][p] = (uint32_t)(rv * 8 + ((2 * p + (cq >> 1)) ^ swv)) * 16u + (uint32_t)(cq & 1) * 8u;
  }

  // RSPLIT: K operand of this wave's 16 tile rows 16*(wave & 1) + n, chunk 4p + g4
  uint32_t krs[2];
  {
    const int r = 16 * (wave & 1) + n;
#pragma unroll
    for (int p = 0; p < 2; ++p) krs[p] = (uint32_t)(r * 8 + ((4 * p + g4) ^ swz<S::FP8>(r))) * 16u;
  }

  // fp8 rows: 40 chunks of 16 B ([512 codes | 64 bf16 rope]) laid out like the bf16 tile
  uint32_t tr8ofs[S::FP8 ? 8 : 1];         // transposing fp8 read: row kmap(g4, n>>1), 8 B at dims 16f + 8*(n&1)
  if constexpr (S::FP8) {
    const int kq = n >> 1;
    const int rr = (kq < 4) ? 4 * g4 + kq : 16 + 4 * g4 + (kq - 4);
    const int swr = swz<S::FP8>(rr);
#pragma unroll
    for (int p = 0; p < 8; ++p) tr8ofs[p] = (uint32_t)(rr * 8 + (p ^ swr)) * 16u + (uint32_t)(n & 1) * 8u;
  }

  f32x4 o[S::PV32 ? 1 : 32];
#pragma unroll
  for (int f = 0; f < (S::PV32 ? 1 : 32); ++f) o[f] = f32x4{0.f, 0.f, 0.f, 0.f};
  // PV32: accumulator (db, hb) = o16[2 * db + hb]: lane l holds head (or dense
  // slot) 32 hb + (l & 31) and, for i = 4q + j, dim 128 hg + 64 (db >> 1) +
  // 16 ((db & 1) + 2 (q >> 1)) + 8 (q & 1) + 4 (l >> 5) + j
  f32x16 o16[S::PV32 ? 8 : 1];
#pragma unroll
  for (int k = 0; k < (S::PV32 ? 8 : 1); ++k)
#pragma unroll
    for (int i = 0; i < 16; ++i) o16[k][i] = 0.f;
  // per 16-head group of the wave's scores (lane n: head n of the group)
  float m_run[S::NE], l_run[S::NE];       // exponent reference and row sum
  float m_seen[S::NE];                    // true running maximum
#pragma unroll
  for (int e = 0; e < S::NE; ++e) {
    m_run[e] = NEG_INF;
    l_run[e] = 0.f;
    m_seen[e] = NEG_INF;
  }
  bool overflow = false;

  // ---- index range of this split
  const int64_t c0 = (int64_t)a.topk * sp / S_;
  const int64_t c1 = (int64_t)a.topk * (sp + 1) / S_;
  const int32_t* idx_row = a.topk_idx + (int64_t)t * a.idx_stride;

  // raw index entries of the first pass are requested before the queries so
  // that their latencies overlap; thread tid owns entries cs + tid*EPT + i
  int raw[S::EPT];
  auto load_raw = [&](int64_t cs, int64_t ce) {
#pragma unroll
    for (int i = 0; i < S::EPT; ++i) {
      const int64_t e = cs + (int64_t)tid * S::EPT + i;
      raw[i] = (e < ce) ? idx_row[e] : -1;
    }
  };
  if constexpr (!S::DENSE) load_raw(c0, (c0 + LIST_CAP < c1) ? c0 + LIST_CAP : c1);

  // ---- queries of this wave's 16 heads, in the MFMA B-operand layout:
  //      lane (g4, n) holds head hg*16+n, dims 32*kk + 8*g4 .. +7
  bf16x8 qb[18 * S::NE];   // RSPLIT: group e's k-step kk at qb[18e + kk]
  // QDMA (the pipelined shapes: h = 64 and dense): the queries (64 heads or
  // slots x 576 dims = two tiles' bytes) are not loaded here.  Loads retire in
  // issue order on one counter, so the wait for the block-table words would
  // also wait for 73.7 KB of queries requested before them.  They are instead
  // requested once those words have landed, straight into ring slots 2..3
  // (idle until the first tiles are gathered), and read into registers after
  // tiles 0..1 are issued and before slots 2..3 are.
  constexpr bool QDMA = S::PV32;
  if constexpr (QDMA) {
#pragma unroll
    for (int kk = 0; kk < 18; ++kk) qb[kk] = bf16x8{};
  }
#pragma unroll
  for (int e = 0; e < (QDMA ? 0 : S::NE); ++e) {
    const int head = (S::RSPLIT ? 32 * (wave >> 1) + 16 * e : (S::PAIR ? 0 : hg) * 16) + n;
    if (S::DENSE || head < a.h) {
      const uint16_t* qp = S::DENSE ? a.q + (int64_t)(d_r0 + d_row) * a.q_st + (int64_t)d_head * a.q_sh + 8 * g4
                                    : a.q + (int64_t)t * a.q_st + (int64_t)head * a.q_sh + 8 * g4;
#pragma unroll
      for (int kk = 0; kk < S::KS; ++kk) {
        // fp8 latent k-steps take their dims in the order the 16-byte code reads
        // deliver them: step (block b, s) of a lane covers dims
        // 128b + 64(s >> 1) + 16*g4 + 8(s & 1) .. +7 (a permutation of the block's
        // dims, applied to q and k alike); the rope steps keep 32kk + 8*g4
        const int off = (S::FP8 && kk < 16)
                            ? 128 * (kk >> 2) + 64 * ((kk & 3) >> 1) + 8 * g4 + 8 * (kk & 1)
                            : 32 * kk;
        qb[18 * e + kk] = *reinterpret_cast<const bf16x8*>(qp + off);
      }
    } else {
#pragma unroll
      for (int kk = 0; kk < S::KS; ++kk) qb[18 * e + kk] = bf16x8{};
    }
    // a negative softmax scale: the kernels scale by |scale| and take -q
    // (negating a bf16 value is exact), so the scaled scores are unchanged and
    // the softmax code may assume a non-negative scale
    if (a.q_neg) {
#pragma unroll
      for (int kk = 0; kk < S::KS; ++kk)
        qb[18 * e + kk] = __builtin_bit_cast(bf16x8, __builtin_bit_cast(u32x4, qb[18 * e + kk]) ^ 0x80008000u);
    }
  }

  // the row's sequence (LOGICAL mode) is requested after the index entries and
  // queries so its latency overlaps theirs
  int seq_ok = 1;
  int64_t bt_row = 0;
  if constexpr (S::DENSE) {
    bt_row = (int64_t)d_seq * a.bt_stride;
  } else if (a.index_mode == 1) {
    const int seq = a.token_seq[t];
    seq_ok = (seq >= 0 && seq < a.num_seqs);
    bt_row = seq_ok ? (int64_t)seq * a.bt_stride : 0;
  }
  // dense mode: this slot's causal limit, and the sequence's block-table row
  // (max_blocks <= LIST_CAP words, requested with the limits so that one round
  // trip brings both); then the queries, once both have landed
  int d_plim = 0;
  int d_btw[S::DENSE ? LIST_CAP / S::NTHR : 1];
  if constexpr (S::DENSE) {
    const int lastpos = a.max_blocks * (1 << a.page_shift) - 1;   // beyond the block table: skipped
    int pl = a.positions[d_r0 + d_row];
#pragma unroll
    for (int j = 0; j < LIST_CAP / S::NTHR; ++j) {
      const int i = tid + j * S::NTHR;
      d_btw[j] = (i < a.max_blocks) ? a.block_table[bt_row + i] : -1;
    }
    pl = pl < lastpos ? pl : lastpos;
    d_plim = pl;
    asm volatile("" : : "v"(pl));
#pragma unroll
    for (int j = 0; j < LIST_CAP / S::NTHR; ++j) asm volatile("" : : "v"(d_btw[j]));
    // slot m = 16 hg + n is (row d_row, head d_head) of the block
    const uint16_t* qp = a.q + (int64_t)(d_r0 + d_row) * a.q_st + (int64_t)d_head * a.q_sh + 8 * g4;
    dma_queries<S::KS>(qp, ring0 + 2u * S::TILE_BYTES + (uint32_t)(hg * S::KS) * 1024u);
  }

  for (int pass = 0; pass < 2; ++pass) {
  for (int64_t cs = c0; cs < c1; cs += LIST_CAP) {
    const int64_t ce = (cs + LIST_CAP < c1) ? cs + LIST_CAP : c1;
    int n_valid;
    if constexpr (S::DENSE) {
      // positions 0 .. the block's largest limit; list[i] = the block-table
      // page of block i (-1 when invalid: those positions are skipped)
      float pm = (float)d_plim;
      pm = max_xor16_32(pm);
      pm = fmaxf(pm, wave_xor(pm, 1));
      pm = fmaxf(pm, wave_xor(pm, 2));
      pm = fmaxf(pm, wave_xor(pm, 4));
      pm = fmaxf(pm, wave_xor(pm, 8));
      float* wmax = reinterpret_cast<float*>(smem + S::CNT_OFF);
      if (lane == 0) wmax[wave] = pm;
      __syncthreads();
      float bm = wmax[0];
#pragma unroll
      for (int w = 1; w < S::NW; ++w) bm = fmaxf(bm, wmax[w]);
      const int pmax = (int)bm;
      const int npg = (pmax >> a.page_shift) + 1;
#pragma unroll
      for (int j = 0; j < LIST_CAP / S::NTHR; ++j) {
        const int i = tid + j * S::NTHR;
        if (i < npg) list[i] = (d_btw[j] >= 0 && d_btw[j] < a.num_pages) ? d_btw[j] : -1;
      }
      __syncthreads();
      n_valid = pmax + 1;
    } else {
      if (cs != c0 || pass != 0) load_raw(cs, ce);
      n_valid = compact_chunk<S::NW, S::EPT>(a, raw, seq_ok, bt_row, list, wcnt, wave, lane, [&]() {
        if constexpr (QDMA) {
          if (cs == c0 && pass == 0) {
            // lane (g4, n): head 16 hg + n, dims 32 kk + 8 g4 .. +7 -> slot
            // bytes 2 TILE_BYTES + 1024 (KS hg + kk) + 16 lane (heads past h
            // read head 0 and are zeroed when read out)
            const int head = hg * 16 + n;
            const uint16_t* qp = a.q + (int64_t)t * a.q_st + (int64_t)(head < a.h ? head : 0) * a.q_sh + 8 * g4;
            dma_queries<S::KS>(qp, ring0 + 2u * S::TILE_BYTES + (uint32_t)(hg * S::KS) * 1024u);
          }
        }
      });
    }

    // ---- tiles: tile i belongs to row group i % NRG
    const int ntile = (n_valid + S::RT - 1) / S::RT;
    const int nt_rg = (ntile > rg) ? (ntile - rg + S::NRG - 1) / S::NRG : 0;
    const int nit = S::SYNC ? (ntile + S::NRG - 1) / S::NRG : nt_rg;

    auto tile_lds = [&](int it) -> uint32_t {
      return ring0 + (uint32_t)((rg * S::NST + (it % S::NST)) * S::TILE_BYTES);
    };
    auto issue = [&](int it) {
      const int tstart = (rg + S::NRG * it) * S::RT;
      const uint32_t tl = tile_lds(it);
#pragma unroll
      for (int k = 0; k < S::RH_PER_WAVE; ++k) {
        const int rh = hg + k * S::HG;
        const int r = 8 * rh + (lane >> 3);
        int li = tstart + r;
        li = (li < n_valid) ? li : n_valid - 1;           // tail rows repeat the last valid row
        const int slot = list[lpos(li)];
        const int q = (lane & 7) ^ swz<S::FP8>(r);
        const uint8_t* g = a.kv + row_offset<S::FP8, S::ROWB>(a, slot) + q * 16;
        const uint32_t mb = tl + (uint32_t)rh * 1024u;
        // line L of the row lands at tile position L*RT*8 + rh*64 + lane
        dma16<0 * 128>(g, mb + 0 * (S::RT * 128 - 128));
        dma16<1 * 128>(g, mb + 1 * (S::RT * 128 - 128));
        dma16<2 * 128>(g, mb + 2 * (S::RT * 128 - 128));
        dma16<3 * 128>(g, mb + 3 * (S::RT * 128 - 128));
        if constexpr (S::NLINES > 4) dma16<4 * 128>(g, mb + 4 * (S::RT * 128 - 128));
        if constexpr (S::NLINES > 5) {
          dma16<5 * 128>(g, mb + 5 * (S::RT * 128 - 128));
          dma16<6 * 128>(g, mb + 6 * (S::RT * 128 - 128));
          dma16<7 * 128>(g, mb + 7 * (S::RT * 128 - 128));
        }
        if constexpr (S::NLINES > 8) dma16<8 * 128>(g, mb + 8 * (S::RT * 128 - 128));
      }
      if constexpr (S::FP8) {
        // the block scales of this wave's share of the tile rows, 16 B per row
        constexpr int SR = S::RT / S::HG;
        if (lane < SR) {
          const int r = hg * SR + lane;
          int li = tstart + r;
          li = (li < n_valid) ? li : n_valid - 1;
          const int slot = list[lpos(li)];
          const int64_t page = slot >> a.page_shift;
          const int64_t rin = slot & ((1 << a.page_shift) - 1);
          const uint8_t* g = a.kv + page * ((int64_t)(S::ROWB + FP8_SCALE_BYTES) << a.page_shift) +
                             ((int64_t)S::ROWB << a.page_shift) + rin * FP8_SCALE_BYTES;
          dma16<0>(g, tl + S::BODY_BYTES + (uint32_t)(hg * SR * 16));
        }
      }
    };
    auto compute = [&](int it) {
      const int tstart = (rg + S::NRG * it) * S::RT;
      const uint32_t toff = tile_lds(it) - ring0;
      const LDS_AS uint8_t* tp = lds + toff;
      // scores S^T[row][head] for this wave's 16 heads
      f32x4 sc[S::NF];
      f32x4 sv[S::FP8 ? S::NF : 1][4];   // fp8: block scales of the lane's accumulator rows 16f+4*g4+j
      if constexpr (S::FP8) {
#pragma unroll
        for (int f = 0; f < S::NF; ++f)
#pragma unroll
          for (int j = 0; j < 4; ++j)
            sv[f][j] = *reinterpret_cast<const LDS_AS f32x4*>(tp + S::BODY_BYTES + (16 * f + 4 * g4 + j) * 16);
#pragma unroll
        for (int f = 0; f < S::NF; ++f) {
          // latent: 16 k-steps of 8 fp8 codes per lane, dequantised exactly to
          // bf16; each 128-dim block accumulates separately and is scaled in fp32
          // 16 codes per lane per read: k-steps (b, 2m) and (b, 2m + 1) of block b
          u32x4 kq[8];
#pragma unroll
          for (int i = 0; i < 8; ++i)
            kq[i] = *reinterpret_cast<const LDS_AS u32x4*>(tp + kofs[f][i & 1] + (i >> 1) * S::RT * 128);
          u32x2 kw[16];
#pragma unroll
          for (int kk = 0; kk < 16; ++kk) {
            const u32x4 v = kq[2 * (kk >> 2) + ((kk & 3) >> 1)];
            kw[kk] = (kk & 1) ? u32x2{v[2], v[3]} : u32x2{v[0], v[1]};
          }
          bf16x8 kr[2];   // rope k-steps (line group 4; none in the NoPE geometry)
          if constexpr (!S::NOPE) {
#pragma unroll
            for (int kk = 0; kk < 2; ++kk)
              kr[kk] = *reinterpret_cast<const LDS_AS bf16x8*>(tp + kofs[f][kk] + 4 * S::RT * 128);
          }
          __builtin_amdgcn_sched_barrier(0);
          // one accumulation chain per 128-dim block (interleaved, so consecutive
          // MFMAs are independent) and one per rope k-step
          f32x4 ab[4], ar[2];
#pragma unroll
          for (int blk = 0; blk < 4; ++blk) ab[blk] = f32x4{0.f, 0.f, 0.f, 0.f};
          ar[0] = ar[1] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int ks = 0; ks < 4; ++ks) {
#pragma unroll
            for (int blk = 0; blk < 4; ++blk) {
              const int kk = 4 * blk + ks;
              ab[blk] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fp8x8_to_bf16(kw[kk][0], kw[kk][1]), qb[kk], ab[blk], 0, 0, 0);
            }
            if constexpr (!S::NOPE)
              if (ks < 2) ar[ks] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kr[ks], qb[16 + ks], ar[ks], 0, 0, 0);
          }
          f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int blk = 0; blk < 4; ++blk)
#pragma unroll
            for (int j = 0; j < 4; ++j) acc[j] += ab[blk][j] * sv[f][j][blk];
          sc[f] = acc + (ar[0] + ar[1]);
        }
      } else
#pragma unroll
      for (int f = 0; f < S::NF; ++f) {
        // all 18 K operands of the fragment are requested before its first
        // MFMA, so the LDS latency is paid once per fragment
        bf16x8 kb[S::KS];
#pragma unroll
        for (int kk = 0; kk < S::KS; ++kk)
          kb[kk] = *reinterpret_cast<const LDS_AS bf16x8*>(tp + kofs[f][kk & 1] + (kk >> 1) * S::RT * 128);
        __builtin_amdgcn_sched_barrier(0);
        // one accumulation chain: back-to-back dependent MFMAs measured
        // 10-13% faster on the c3 head sweep than six chains summed afterwards
        // (those cost accumulator moves and adds per tile)
        f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kk = 0; kk < S::KS; ++kk) acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kb[kk], qb[kk], acc, 0, 0, 0);
        sc[f] = acc;
      }
      // online softmax (base 2); lane owns head n, rows 16f + 4*g4 + j
      const int left = n_valid - tstart;
      float x[S::NF][4];
      float mx = NEG_INF;
#pragma unroll
      for (int f = 0; f < S::NF; ++f)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int r = 16 * f + 4 * g4 + j;
          const float v = sc[f][j] * a.scale_log2;
          x[f][j] = (r < left) ? v : NEG_INF;
          mx = fmaxf(mx, x[f][j]);
        }
      mx = fmaxf(mx, wave_xor(mx, 16));
      mx = fmaxf(mx, wave_xor(mx, 32));
      // Fixed exponent reference: the first tile's max, rounded up to an
      // integer, becomes the row's reference and later tiles use it unchanged
      // (p <= 2^REF_HEADROOM), so the accumulators never need rescaling.  A
      // tile that exceeds the reference by more than the headroom flags the
      // work-group, which then recomputes the row once with its true maximum
      // (rounded up) as the reference.
      m_seen[0] = fmaxf(m_seen[0], mx);
      if (m_run[0] == NEG_INF) m_run[0] = int_ref(mx);
      overflow |= (mx > m_run[0] + REF_HEADROOM);
      float psum = 0.f;
      float pv[S::NF][4];
#pragma unroll
      for (int f = 0; f < S::NF; ++f)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          pv[f][j] = fast_exp2(x[f][j] - m_run[0]);
          psum += pv[f][j];
        }
      l_run[0] += psum;
      // P.V
      // V^T operands are read in groups of 8 output fragments, the next
      // group's transposing reads in flight while the current group's MFMAs run
      if constexpr (S::FP8) {
        // P' = P * scale(row, block): one bf16 operand per 128-dim block, the
        // 8 k-slots of a lane being rows 4*g4+j (fragment 0) and 16+4*g4+j (fragment 1)
        bf16x8 pb[4];
#pragma unroll
        for (int blk = 0; blk < 4; ++blk)
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            pb[blk][j] = (__bf16)(pv[0][j] * sv[0][j][blk]);
            pb[blk][4 + j] = (__bf16)(pv[1][j] * sv[1][j][blk]);
          }
        typedef __attribute__((__vector_size__(2 * sizeof(int)))) int i32x2;
        i32x2 vw[2][8];
        auto load_grp = [&](int g, int buf) {
#pragma unroll
          for (int i = 0; i < 8; ++i) {
            const int f = 8 * g + i;
            vw[buf][i] = __builtin_amdgcn_ds_read_tr8_b64_v2i32((LDS_AS i32x2*)(tp + tr8ofs[f & 7] + (f >> 3) * S::RT * 128));
          }
        };
        load_grp(0, 0);
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          if (g + 1 < 4) load_grp(g + 1, (g + 1) & 1);
          __builtin_amdgcn_sched_barrier(0);
#pragma unroll
          for (int i = 0; i < 8; ++i)
            o[8 * g + i] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                fp8x8_to_bf16((uint32_t)vw[g & 1][i][0], (uint32_t)vw[g & 1][i][1]), pb[g], o[8 * g + i], 0, 0, 0);
        }
      } else if constexpr (S::RT == 16) {
        bf16x4 pb;
#pragma unroll
        for (int j = 0; j < 4; ++j) pb[j] = (__bf16)pv[0][j];
        bf16x4 va[2][8];
        auto load_grp = [&](int g, int buf) {
#pragma unroll
          for (int i = 0; i < 8; ++i) {
            const int f = 8 * g + i;
            va[buf][i] = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
                (LDS_AS bf16x4*)(tp + vofs[0][f & 3] + (f >> 2) * S::RT * 128));
          }
        };
        load_grp(0, 0);
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          if (g + 1 < 4) load_grp(g + 1, (g + 1) & 1);
          __builtin_amdgcn_sched_barrier(0);
#pragma unroll
          for (int i = 0; i < 8; ++i)
            o[8 * g + i] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(va[g & 1][i], pb, o[8 * g + i], 0, 0, 0);
        }
      } else {
        bf16x8 pb;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          pb[j] = (__bf16)pv[0][j];
          pb[4 + j] = (__bf16)pv[1][j];
        }
        bf16x8 va[2][8];
        auto load_grp = [&](int g, int buf) {
#pragma unroll
          for (int i = 0; i < 8; ++i) {
            const int f = 8 * g + i;
            const bf16x4 v0 = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
                (LDS_AS bf16x4*)(tp + vofs[0][f & 3] + (f >> 2) * S::RT * 128));
            const bf16x4 v1 = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
                (LDS_AS bf16x4*)(tp + vofs[1][f & 3] + (f >> 2) * S::RT * 128));
            va[buf][i] = __builtin_shufflevector(v0, v1, 0, 1, 2, 3, 4, 5, 6, 7);
          }
        };
        load_grp(0, 0);
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          if (g + 1 < 4) load_grp(g + 1, (g + 1) & 1);
          __builtin_amdgcn_sched_barrier(0);
#pragma unroll
          for (int i = 0; i < 8; ++i)
            o[8 * g + i] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(va[g & 1][i], pb, o[8 * g + i], 0, 0, 0);
        }
      }
    };

    // fp8 row/dim-split pair: every wave runs this each step (barriers inside);
    // `active` is false once the row stream has no tile at this step
    auto compute_pair = [&](int it, bool active) {
      if constexpr (S::PAIR) {
        const int tstart = (rg + S::NRG * it) * S::RT;
        const LDS_AS uint8_t* tp = lds + (tile_lds(it) - ring0);
        const int f = hg;   // this wave's 16-row fragment
        f32x4 sv[4];        // block scales of the lane's rows 16f + 4*g4 + j
        float x[4];
        float mx = NEG_INF;
        if (active) {
#pragma unroll
          for (int j = 0; j < 4; ++j)
            sv[j] = *reinterpret_cast<const LDS_AS f32x4*>(tp + S::BODY_BYTES + (16 * f + 4 * g4 + j) * 16);
          u32x4 kq[8];
#pragma unroll
          for (int i = 0; i < 8; ++i)
            kq[i] = *reinterpret_cast<const LDS_AS u32x4*>(tp + kofs[f][i & 1] + (i >> 1) * S::RT * 128);
          bf16x8 kr[2];   // rope k-steps (none in the NoPE geometry)
          if constexpr (!S::NOPE) {
#pragma unroll
            for (int kk = 0; kk < 2; ++kk)
              kr[kk] = *reinterpret_cast<const LDS_AS bf16x8*>(tp + kofs[f][kk] + 4 * S::RT * 128);
          }
          f32x4 ab[4], ar[2];
#pragma unroll
          for (int blk = 0; blk < 4; ++blk) ab[blk] = f32x4{0.f, 0.f, 0.f, 0.f};
          ar[0] = ar[1] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int ks = 0; ks < 4; ++ks) {
#pragma unroll
            for (int blk = 0; blk < 4; ++blk) {
              const int kk = 4 * blk + ks;
              const u32x4 v = kq[2 * blk + (ks >> 1)];
              const bf16x8 kb = (ks & 1) ? fp8x8_to_bf16(v[2], v[3]) : fp8x8_to_bf16(v[0], v[1]);
              ab[blk] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kb, qb[kk], ab[blk], 0, 0, 0);
            }
            if constexpr (!S::NOPE)
              if (ks < 2) ar[ks] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kr[ks], qb[16 + ks], ar[ks], 0, 0, 0);
          }
          f32x4 sc = ar[0] + ar[1];
#pragma unroll
          for (int blk = 0; blk < 4; ++blk)
#pragma unroll
            for (int j = 0; j < 4; ++j) sc[j] += ab[blk][j] * sv[j][blk];
          const int left = n_valid - tstart;
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const float v = sc[j] * a.scale_log2;
            x[j] = (16 * f + 4 * g4 + j < left) ? v : NEG_INF;
            mx = fmaxf(mx, x[j]);
          }
          mx = max_xor16_32(mx);
        }
        LDS_AS float* mex = (LDS_AS float*)(lds + S::MEX_OFF);
        if (it == 0) {
          // the pair's exponent reference (set once per row): the first tile's
          // maximum over its 32 rows; both waves of a pair hold the same state
          mex[wave * 64 + lane] = (m_run[0] == NEG_INF) ? mx : m_run[0];
          asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
          const float other = mex[(wave ^ 1) * 64 + lane];
          if (m_run[0] == NEG_INF) m_run[0] = int_ref(fmaxf(mx, other));
        }
        bf16x4 pb[4];   // P scaled by each 128-dim block's scale of the row
        if (active) {
          m_seen[0] = fmaxf(m_seen[0], mx);
          overflow |= (mx > m_run[0] + REF_HEADROOM);
          float psum = 0.f;
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const float pj = fast_exp2(x[j] - m_run[0]);
            psum += pj;
#pragma unroll
            for (int blk = 0; blk < 4; ++blk) pb[blk][j] = (__bf16)(pj * sv[j][blk]);
          }
          l_run[0] += psum;
          // P of block blk from wave f: 8 bytes per lane, contiguous over the
          // lanes ([stream][block][wave][lane]), so the writes are free of bank
          // conflicts
#pragma unroll
          for (int blk = 0; blk < 4; ++blk)
            *(LDS_AS bf16x4*)(lds + S::PEX_OFF + (((rg * 4 + blk) * 2 + f) * 64 + lane) * 8) = pb[blk];
        }
        asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
        if (active) {
          // B operands of this wave's two blocks: rows 4*g4 + j (fragment 0), 16 + 4*g4 + j (fragment 1)
          bf16x8 pall[2];
#pragma unroll
          for (int b2 = 0; b2 < 2; ++b2) {
            const LDS_AS uint8_t* pp = lds + S::PEX_OFF + ((rg * 4 + 2 * f + b2) * 2 * 64 + lane) * 8;
            const bf16x4 lo = *(const LDS_AS bf16x4*)pp;              // rows 4*g4 + j (wave 0's fragment)
            const bf16x4 hi = *(const LDS_AS bf16x4*)(pp + 64 * 8);   // rows 16 + 4*g4 + j (wave 1's)
            pall[b2] = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
          }
          typedef __attribute__((__vector_size__(2 * sizeof(int)))) int i32x2;
          i32x2 vw[16];
#pragma unroll
          for (int i = 0; i < 16; ++i)
            vw[i] = __builtin_amdgcn_ds_read_tr8_b64_v2i32(
                (LDS_AS i32x2*)(tp + tr8ofs[i & 7] + (2 * f + (i >> 3)) * S::RT * 128));
#pragma unroll
          for (int i = 0; i < 16; ++i)
            o[i] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fp8x8_to_bf16((uint32_t)vw[i][0], (uint32_t)vw[i][1]),
                                                           pall[i >> 3], o[i], 0, 0, 0);
        }
      }
    };

    // the compiler's wait for the query loads lands here, before any gather is in flight
#pragma unroll
    for (int e = 0; e < S::NE; ++e)
#pragma unroll
      for (int kk = 0; kk < S::KS; ++kk) asm volatile("" : : "v"(qb[18 * e + kk]));

    if constexpr (S::PIPE) {
      // ---- software-pipelined schedule (one tile stream, four waves):
      //   prologue: gather tiles 0..NST-2; scores of tile 0 (gather NST-1 under it); V^T of tile 0
      //   step i:   [tile i+1 landed, barrier]
      //             scores of tile i+1  ||  softmax of tile i  ||  gathers of tile i+NST
      //             P of tile i exchanged (barrier)
      //             P.V of tile i       ||  V^T operands of tile i+1
      // Tile i's slot is free after step i-1 (its K and V^T were read then), so
      // the gathers of step i refill it.  Gathers stop at the last tile and the
      // waits count the tiles actually in flight (the row-half split variant
      // instead keeps issuing past the list, with a constant count).
      constexpr int KRING = 8;
      const uint8_t* dg = a.kv;
      uint32_t dmb = 0;
      auto dma_prep = [&](int itd) {
        const int r = 8 * hg + (lane >> 3);
        int li = itd * S::RT + r;
        li = (li < n_valid) ? li : n_valid - 1;
        int slot;
        if constexpr (S::DENSE) {
          // position li of the sequence (an invalid page reads page 0; masked)
          const int pg = list[li >> a.page_shift];
          slot = ((pg < 0 ? 0 : pg) << a.page_shift) | (li & ((1 << a.page_shift) - 1));
        } else {
          slot = list[lpos(li)];
        }
        dg = a.kv + (int64_t)slot * S::ROWB + ((lane & 7) ^ swz<S::FP8>(r)) * 16;
        dmb = tile_lds(itd) + (uint32_t)hg * 1024u;
      };
      auto dma_line = [&](int L) {
        constexpr uint32_t LS = S::RT * 128 - 128;
        switch (L) {
          case 0: dma16<0 * 128>(dg, dmb + 0 * LS); break;
          case 1: dma16<1 * 128>(dg, dmb + 1 * LS); break;
          case 2: dma16<2 * 128>(dg, dmb + 2 * LS); break;
          case 3: dma16<3 * 128>(dg, dmb + 3 * LS); break;
          case 4: dma16<4 * 128>(dg, dmb + 4 * LS); break;
          case 5: dma16<5 * 128>(dg, dmb + 5 * LS); break;
          case 6: dma16<6 * 128>(dg, dmb + 6 * LS); break;
          case 7: dma16<7 * 128>(dg, dmb + 7 * LS); break;
          default: dma16<8 * 128>(dg, dmb + 8 * LS); break;
        }
      };
      auto tptr = [&](int it) { return lds + (tile_lds(it) - ring0); };
      // online softmax of one tile (base 2, fixed exponent reference).  The
      // lane owns head n of a 16-head group and rows 4*g4 + j of a 16-row
      // fragment: scv[q] is fragment q (rows 16q + ..) of the wave's group, or
      // with RSPLIT head group q of the wave's rows 16*(wave & 1) + ..; P comes
      // back as pb[4q + j].  With RSPLIT, `first` (work-group uniform) sets the
      // exponent reference of each head from the tile's maximum over both
      // row halves, exchanged with the partner wave through LDS.
      // The softmax runs in stages so that, in a pipeline step, each stage
      // can sit between two groups of P.V MFMAs (which do not depend on it):
      //   sm_scale(q): scale and mask fragment q, partial maximum;
      //   sm_reduce:   maximum over the lanes sharing a head, reference, overflow;
      //   sm_exp(q):   P of fragment q and its row sum;
      //   sm_finish:   row sums into l_run.
      struct SmState {
        float x[2][4];
        float mx[2];
        float psum[2];
        bf16x8 pb;
      };
      auto sm_init = [&](SmState& st) {
        st.mx[0] = st.mx[1] = NEG_INF;
        st.psum[0] = st.psum[1] = 0.f;
      };
      // MASK false (a whole tile: every row is listed): the raw scores are
      // kept, their maximum is scaled once (the scale is non-negative), and the
      // exponent is one fma; MASK true: rows past the list are -inf.
      auto sm_scale = [&](int it, const f32x4* scv, int q, SmState& st, auto mask_tag) {
        constexpr bool MASK = decltype(mask_tag)::value;
        if constexpr (!MASK) {
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            st.x[q][j] = scv[q][j];
            st.mx[S::RSPLIT ? q : 0] = fmaxf(st.mx[S::RSPLIT ? q : 0], scv[q][j]);
          }
          return;
        }
        const int left = n_valid - it * S::RT;
        // dense mode: positions past the slot's own row, or on an invalid
        // page (pages hold >= 16 rows, so a 16-row fragment has one page)
        bool pgok = true;
        if constexpr (S::DENSE) {
          const int p0 = it * S::RT + 16 * q;
          pgok = p0 < n_valid && list[p0 >> a.page_shift] >= 0;
        }
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int row = (S::RSPLIT ? 16 * (wave & 1) : 16 * q) + 4 * g4 + j;
          const float v = scv[q][j] * a.scale_log2;
          const bool keep = S::DENSE ? (pgok && it * S::RT + row <= d_plim) : (row < left);
          st.x[q][j] = keep ? v : NEG_INF;
          st.mx[S::RSPLIT ? q : 0] = fmaxf(st.mx[S::RSPLIT ? q : 0], st.x[q][j]);
        }
      };
      auto sm_reduce = [&](SmState& st, bool first, auto mask_tag) {
        constexpr bool MASK = decltype(mask_tag)::value;
#pragma unroll
        for (int e = 0; e < S::NE; ++e) {
          st.mx[e] = max_xor16_32(st.mx[e]);
          if constexpr (!MASK) st.mx[e] *= a.scale_log2;
        }
        if constexpr (S::RSPLIT) {
          if (first) {
            // in exchange buffer 1: buffer 0 receives P of this tile right after
            LDS_AS float* mex = (LDS_AS float*)(lds + S::PEX_OFF + 4096);
#pragma unroll
            for (int e = 0; e < 2; ++e) mex[(wave * 2 + e) * 64 + lane] = (m_run[e] == NEG_INF) ? st.mx[e] : m_run[e];
            asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
#pragma unroll
            for (int e = 0; e < 2; ++e) {
              const float other = mex[((wave ^ 1) * 2 + e) * 64 + lane];
              if (m_run[e] == NEG_INF) m_run[e] = int_ref(fmaxf(st.mx[e], other));
            }
          }
        } else {
          if (m_run[0] == NEG_INF) m_run[0] = int_ref(st.mx[0]);
        }
#pragma unroll
        for (int e = 0; e < S::NE; ++e) {
          m_seen[e] = fmaxf(m_seen[e], st.mx[e]);
          overflow |= (st.mx[e] > m_run[e] + REF_HEADROOM);
        }
      };
      auto sm_exp = [&](int q, SmState& st, auto mask_tag) {
        constexpr bool MASK = decltype(mask_tag)::value;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          float pj = MASK ? fast_exp2(st.x[q][j] - m_run[S::RSPLIT ? q : 0])
                          : fast_exp2(__builtin_fmaf(st.x[q][j], a.scale_log2, -m_run[S::RSPLIT ? q : 0]));
          // dense mode: a slot may see no valid position yet (reference unset)
          if constexpr (S::DENSE) pj = (m_run[0] == NEG_INF) ? 0.f : pj;
          st.psum[S::RSPLIT ? q : 0] += pj;
          st.pb[4 * q + j] = (__bf16)pj;
        }
      };
      auto sm_finish = [&](SmState& st) {
#pragma unroll
        for (int e = 0; e < S::NE; ++e) l_run[e] += st.psum[e];
      };
      // online softmax of one tile (base 2, fixed exponent reference).  The
      // lane owns head n of a 16-head group and rows 4*g4 + j of a 16-row
      // fragment: scv[q] is fragment q (rows 16q + ..) of the wave's group, or
      // with RSPLIT head group q of the wave's rows 16*(wave & 1) + ..; P comes
      // back as pb[4q + j].  With RSPLIT, `first` (work-group uniform) sets the
      // exponent reference of each head from the tile's maximum over both
      // row halves, exchanged with the partner wave through LDS.
      auto softmax = [&](int it, const f32x4* scv, bool first) -> bf16x8 {
        SmState st;
        sm_init(st);
        sm_scale(it, scv, 0, st, std::true_type{});
        sm_scale(it, scv, 1, st, std::true_type{});
        sm_reduce(st, first, std::true_type{});
        sm_exp(0, st, std::true_type{});
        sm_exp(1, st, std::true_type{});
        sm_finish(st);
        return st.pb;
      };
      // scores of tile itq (K operands through a ring of KRING reads) with the
      // gathers of tile itd interleaved, one 128-B line per four MFMAs
      auto scores = [&](int itq, f32x4* out) {
        const LDS_AS uint8_t* tp = tptr(itq);
        if constexpr (S::RSPLIT) {
          // k-step kk's K operand (this wave's 16 rows) feeds the MFMAs of both
          // head groups, one accumulation chain per group
          constexpr int KR = 4;
          bf16x8 kr[S::KS];
#pragma unroll
          for (int i = 0; i < KR; ++i)
            kr[i] = *reinterpret_cast<const LDS_AS bf16x8*>(tp + krs[i & 1] + (i >> 1) * S::RT * 128);
          __builtin_amdgcn_sched_group_barrier(0x100, KR, 0);
          f32x4 acc[2];
          acc[0] = acc[1] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int kk = 0; kk < S::KS; ++kk) {
#pragma unroll
            for (int e = 0; e < 2; ++e)
              acc[e] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kr[kk], qb[18 * e + kk], acc[e], 0, 0, 0);
            const int j = kk + KR;
            if (j < S::KS) kr[j] = *reinterpret_cast<const LDS_AS bf16x8*>(tp + krs[j & 1] + (j >> 1) * S::RT * 128);
            __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
            if (j < S::KS) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
          }
          out[0] = acc[0];
          out[1] = acc[1];
          return;
        }
        // MFMA i is (fragment i & 1, k-step i >> 1), accumulating into its
        // fragment's chain: consecutive MFMAs belong to different fragments.
        // (Four chains per fragment, summed afterwards, measured 2% slower on
        // the long-prefill batch: the extra accumulator moves and adds cost
        // more than the dependent-MFMA spacing.)
        constexpr int NM = 2 * S::KS;   // score MFMAs of a tile
        bf16x8 kr[NM];
#pragma unroll
        for (int i = 0; i < KRING; ++i)
          kr[i] = *reinterpret_cast<const LDS_AS bf16x8*>(tp + kofs[i & 1][(i >> 1) & 1] + (i >> 2) * S::RT * 128);
        __builtin_amdgcn_sched_group_barrier(0x100, KRING, 0);   // the ring's first reads
        f32x4 acc[2];
        acc[0] = acc[1] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int i = 0; i < NM; ++i) {
          const int f = i & 1, kk = i >> 1;
          acc[f] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kr[i], qb[kk], acc[f], 0, 0, 0);
          const int j = i + KRING;
          if (j < NM)
            kr[j] = *reinterpret_cast<const LDS_AS bf16x8*>(tp + kofs[j & 1][(j >> 1) & 1] + (j >> 2) * S::RT * 128);
          // one MFMA, then its ring read
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
          if (j < NM) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        }
        out[0] = acc[0];
        out[1] = acc[1];
      };
      // V^T operands of tile itv for this wave's output dims 128*hg ..
      auto read_vt = [&](int itv, int f) -> bf16x8 {
        const LDS_AS uint8_t* tpd = tptr(itv) + hg * 2 * S::RT * 128;
        const bf16x4 v0 = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
            (LDS_AS bf16x4*)(tpd + vofs[0][f & 3] + (f >> 2) * S::RT * 128));
        const bf16x4 v1 = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
            (LDS_AS bf16x4*)(tpd + vofs[1][f & 3] + (f >> 2) * S::RT * 128));
        return __builtin_shufflevector(v0, v1, 0, 1, 2, 3, 4, 5, 6, 7);
      };
      // PV32: V^T operand k = 4 ks + db of tile itv: lane (b, n) = (lane >> 4,
      // lane & 15) holds dim 64 (db >> 1) + 16 ((db & 1) + 2 (b & 1)) + n of the
      // wave's 128 and the eight rows of P's writer lane group g = 2 ks + (b >> 1):
      // 4g + j, 16 + 4g + j
      auto read_vt32 = [&](int itv, int k) -> bf16x8 {
        const int ks = k >> 2, db = k & 3;
        const int b = lane >> 4, cq = n & 3;
        const int g = 2 * ks + (b >> 1);
        const int r0 = 4 * g + (n >> 2);
        // 16-dim group p of line db >> 1: the block's two halves sit in the
        // line's chunks 0..3 and 4..7, so that lanes 0..31 (four rows, both
        // halves) hit sixteen distinct bank groups under the r & 7 swizzle
        const int p = (db & 1) + 2 * (b & 1);
        const uint32_t col = (uint32_t)(db >> 1) * S::RT * 128u +
                             (uint32_t)(((2 * p + (cq >> 1)) ^ swz<S::FP8>(r0)) * 16 + (cq & 1) * 8);
        const LDS_AS uint8_t* tpd = tptr(itv) + hg * 2 * S::RT * 128 + col;
        const bf16x4 v0 = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((LDS_AS bf16x4*)(tpd + r0 * 128));
        const bf16x4 v1 = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((LDS_AS bf16x4*)(tpd + (r0 + 16) * 128));
        return __builtin_shufflevector(v0, v1, 0, 1, 2, 3, 4, 5, 6, 7);
      };

      // QDMA: the queries out of slots 2..3 into registers (this wave's own
      // loads have landed), then a barrier before any wave gathers into them
      const bool qread = QDMA && cs == c0 && pass == 0;
      auto read_q = [&]() {
        if constexpr (QDMA) {
          const LDS_AS uint8_t* qs = lds + 2 * S::TILE_BYTES + hg * S::KS * 1024 + 16 * lane;
#pragma unroll
          for (int kk = 0; kk < S::KS; ++kk) qb[kk] = *reinterpret_cast<const LDS_AS bf16x8*>(qs + 1024 * kk);
          if (!S::DENSE && hg * 16 + n >= a.h) {
#pragma unroll
            for (int kk = 0; kk < S::KS; ++kk) qb[kk] = bf16x8{};
          }
          if (a.q_neg) {
#pragma unroll
            for (int kk = 0; kk < S::KS; ++kk)
              qb[kk] = __builtin_bit_cast(bf16x8, __builtin_bit_cast(u32x4, qb[kk]) ^ 0x80008000u);
          }
          asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
        }
      };
      if (qread && nit == 0) {
        wait_vm<0>();
        read_q();
      }
      if (nit > 0) {
        // (the row-half split variant issues a full ring even past the list:
        // its steps wait on a constant count)
        constexpr int NPRE = QDMA ? 2 : S::NST;   // tiles gathered before the queries are read out
#pragma unroll
        for (int st = 0; st < NPRE; ++st) {
          if (S::RSPLIT || st < nit) {
            dma_prep(st);
#pragma unroll
            for (int L = 0; L < S::NLINES; ++L) dma_line(L);
          }
        }
        if (qread) {
          wait_tiles<S::PER, S::NST>(nit < 2 ? nit : 2);
          read_q();
        }
#pragma unroll
        for (int st = NPRE; st < S::NST; ++st) {
          if (S::RSPLIT || st < nit) {
            dma_prep(st);
#pragma unroll
            for (int L = 0; L < S::NLINES; ++L) dma_line(L);
          }
        }
        if constexpr (S::RSPLIT) wait_vm<(S::NST - 1) * S::PER>();       // tile 0 has landed
        else wait_tiles<S::PER, S::NST>((nit < S::NST ? nit : S::NST) - 1);
        lds_barrier();
        // P of tile i is published into exchange buffer i & 1 at the end of
        // step i - 1 (the prologue for tile 0); the barrier that opens step i
        // makes it visible, and the buffer's previous readers (step i - 2's
        // P.V operands) finished before that barrier
        LDS_AS bf16x8* pex = (LDS_AS bf16x8*)(lds + S::PEX_OFF);
        auto publish = [&](const bf16x8& pbv, int buf) {
          if constexpr (S::RSPLIT) {
            // rows 16*(wave & 1) + 4*g4 + j of head groups 2*(wave >> 1) + e:
            // the half of each group's B operand that this wave owns
            LDS_AS uint8_t* pw = (LDS_AS uint8_t*)lds + S::PEX_OFF + buf * 4096 +
                                 (2 * (wave >> 1) * 64 + lane) * 16 + (wave & 1) * 8;
            *(LDS_AS bf16x4*)pw = __builtin_shufflevector(pbv, pbv, 0, 1, 2, 3);
            *(LDS_AS bf16x4*)(pw + 64 * 16) = __builtin_shufflevector(pbv, pbv, 4, 5, 6, 7);
          } else {
            pex[buf * 256 + hg * 64 + lane] = pbv;
          }
        };
        f32x4 sc[2];
        scores(0, sc);
        publish(softmax(0, sc, true), 0);   // P of tile 0
        bf16x8 vpre[8];
#pragma unroll
        for (int f = 0; f < 8; ++f) vpre[f] = S::PV32 ? read_vt32(0, f) : read_vt(0, f);
        // step it; REFILL: the gathers of tile it + NST (all but the last NST
        // steps), so those steps keep a full ring and wait on a constant count
        auto step = [&](int it, auto refill_tag) {
          constexpr bool REFILL = decltype(refill_tag)::value;
          // tile it+1 has landed (this wave's share); tiles up to
          // min(it + NST - 1, nit - 1) have been issued
          if constexpr (REFILL) {
            wait_vm<(S::NST - 2) * S::PER>();
          } else {
            if (it + 1 < nit) wait_tiles<S::PER, S::NST>(nit - it - 2 < S::NST - 2 ? nit - it - 2 : S::NST - 2);
          }
          // every wave's reads of tile it (its V^T operands) have completed
          // before any gather refills that slot, and P of tile it is published
          asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
          f32x4 scn[2];
          if (it + 1 < nit) {
            scores(it + 1, scn);
          } else {
            scn[0] = scn[1] = f32x4{0.f, 0.f, 0.f, 0.f};
          }
          // P of tile it, read after the score phase: read before it, these four
          // reads took slots of the K operand ring's first group of reads
          bf16x8 pall[4];
#pragma unroll
          for (int hf = 0; hf < 4; ++hf) {
            if constexpr (S::PV32) {
              // B operand (hb, ks) = pall[2 * hb + ks]: head 32 hb + (lane & 31),
              // the rows of writer lane group 2 ks + (lane >> 5)
              const int hb = hf >> 1, ks = hf & 1;
              pall[hf] = pex[(it & 1) * 256 + (2 * hb + ((lane & 31) >> 4)) * 64 + (2 * ks + (lane >> 5)) * 16 + (lane & 15)];
            } else {
              pall[hf] = pex[(it & 1) * 256 + hf * 64 + lane];
            }
          }
          // P.V of tile it over this wave's 8 output fragments x 4 head groups;
          // each fragment's V^T registers are refilled from tile it+1 once used;
          // the gathers of tile it + NST (into tile it's slot, free since the
          // last step) and the softmax stages of tile it+1 sit between these
          // MFMA groups, so their VALU work overlaps the MFMAs instead of
          // running before them (past the list the softmax sees only masked
          // rows: no effect)
          if constexpr (REFILL) dma_prep(it + S::NST);
          SmState st;
          sm_init(st);
#pragma unroll
          for (int f = 0; f < 8; ++f) {
            if constexpr (S::PV32) {
              const int ks = f >> 2, db = f & 3;
#pragma unroll
              for (int hb = 0; hb < 2; ++hb)
                o16[2 * db + hb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vpre[f], pall[2 * hb + ks], o16[2 * db + hb], 0, 0, 0);
              vpre[f] = read_vt32(it + 1, f);
            } else {
#pragma unroll
              for (int hf = 0; hf < 4; ++hf)
                o[4 * f + hf] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vpre[f], pall[hf], o[4 * f + hf], 0, 0, 0);
              vpre[f] = read_vt(it + 1, f);
            }
            // tiles before the last NST are whole (only the last listed tile
            // can be partial): no masking in the refill steps
            using MT = std::integral_constant<bool, !REFILL || S::RSPLIT || S::DENSE>;
            if (f == 0) sm_scale(it + 1, scn, 0, st, MT{});
            if (f == 1) sm_scale(it + 1, scn, 1, st, MT{});
            if (f == 2) sm_reduce(st, false, MT{});
            if (f == 3) sm_exp(0, st, MT{});
            if (f == 4) sm_exp(1, st, MT{});
            if (f == 5) sm_finish(st);
            if constexpr (REFILL) dma_line(f);
            __builtin_amdgcn_sched_barrier(0);
          }
          if constexpr (REFILL && S::NLINES > 8) dma_line(8);
          publish(st.pb, (it + 1) & 1);
        };
        int it = 0;
        if constexpr (S::RSPLIT) {
          // the row-half split keeps one loop body: past the list its gathers
          // re-read the last listed row into a free slot (two bodies measured
          // 17% slower for it on the 4096-row sweep at h = 64)
          for (; it < nit; ++it) step(it, std::true_type{});
        } else {
          for (; it < nit - S::NST; ++it) step(it, std::true_type{});
          for (; it < nit; ++it) step(it, std::false_type{});
        }
      }
    } else {
      // ---- the pipeline
      int iss = 0;
  #pragma unroll
      for (int st = 0; st < S::NST - 1; ++st) {
        if (iss < nit) {
          if (iss < nt_rg) issue(iss);
          ++iss;
        }
      }
      for (int it = 0; it < nit; ++it) {
        if constexpr (!S::SYNC) {
          if (iss < nit) {
            if (iss < nt_rg) issue(iss);
            ++iss;
          }
        }
        const int real = (iss < nt_rg) ? iss : nt_rg;
        wait_tiles<S::PER, S::NST>(real - (it + 1));
        if constexpr (S::SYNC) {
          lds_barrier();
          if (iss < nit) {
            if (iss < nt_rg) issue(iss);
            ++iss;
          }
        }
        if constexpr (S::PAIR) compute_pair(it, it < nt_rg);
        else if (it < nt_rg) compute(it);
      }
    }
    wait_vm<0>();
    __syncthreads();   // the list is rewritten by the next pass
  }
  // rare: some tile exceeded the reference headroom -> recompute the row
  // (every wave of the work-group takes the same decision)
  // (a work-group OR through one LDS word of the compaction counts, free
  // here; __syncthreads_or would take LDS of its own beyond the tile ring)
  {
    volatile int* flag = reinterpret_cast<volatile int*>(smem + S::CNT_OFF);
    if (tid == 0) *flag = 0;
    __syncthreads();
    if (overflow) *flag = 1;
    __syncthreads();
    const bool any = *flag != 0;
    __syncthreads();
    if (!any) break;
  }
  if constexpr (S::PAIR) {
    LDS_AS float* mex = (LDS_AS float*)(lds + S::MEX_OFF);
    mex[wave * 64 + lane] = m_seen[0];
    __syncthreads();
    m_run[0] = int_ref(fmaxf(m_seen[0], mex[(wave ^ 1) * 64 + lane]));
    __syncthreads();
  } else if constexpr (S::RSPLIT) {
    // the two waves holding a head's row halves take their common maximum
    LDS_AS float* mex = (LDS_AS float*)(lds + S::PEX_OFF);
#pragma unroll
    for (int e = 0; e < 2; ++e) mex[(wave * 2 + e) * 64 + lane] = m_seen[e];
    __syncthreads();
#pragma unroll
    for (int e = 0; e < 2; ++e) m_run[e] = int_ref(fmaxf(m_seen[e], mex[((wave ^ 1) * 2 + e) * 64 + lane]));
    __syncthreads();
  } else {
    m_run[0] = int_ref(m_seen[0]);
  }
#pragma unroll
  for (int e = 0; e < S::NE; ++e) l_run[e] = 0.f;
  overflow = false;
#pragma unroll
  for (int f = 0; f < (S::PV32 ? 1 : 32); ++f) o[f] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int k = 0; k < (S::PV32 ? 8 : 1); ++k)
#pragma unroll
    for (int i = 0; i < 16; ++i) o16[k][i] = 0.f;
  }

  // ---- epilogue: merge the row groups of each head group, normalise, write
  // statistics slot of (head group, row half): RSPLIT 2 * group + (wave & 1), else the wave
  float l_tot[S::NE];
#pragma unroll
  for (int e = 0; e < S::NE; ++e) {
    l_tot[e] = l_run[e] + wave_xor(l_run[e], 16);
    l_tot[e] += wave_xor(l_tot[e], 32);
  }
  __syncthreads();
  if (lane < 16) {
#pragma unroll
    for (int e = 0; e < S::NE; ++e) {
      const int slot = S::RSPLIT ? 2 * (2 * (wave >> 1) + e) + (wave & 1) : wave;
      stat[(slot * 16 + lane) * 2 + 0] = m_run[e];
      stat[(slot * 16 + lane) * 2 + 1] = l_tot[e];
    }
  }
  if constexpr (S::DSPLIT) {
    // one row stream: every wave writes its own output dims straight from
    // its accumulators.  Lane (g4, n) holds, in fragment (f, head group hf),
    // dims 128 * wave + 16f + 4 * g4 .. +3 of head (or dense slot) 16hf + n.
    __syncthreads();   // the statistics are visible
    const bool split = a.write_partials != 0;
    if constexpr (S::PV32) {
      // lane l holds slot (head, or dense slot) m = 32 hb + (l & 31) and, in
      // accumulator (db, hb) at i = 4q + j, dim dl + j of the wave's 128 with
      // dl = 64 (db >> 1) + 16 ((db & 1) + 2 (q >> 1)) + 8 (q & 1) + 4 (l >> 5)
      float inv[2];
      int64_t obase[2];
      bool okv[2];
#pragma unroll
      for (int hb = 0; hb < 2; ++hb) {
        const int m = 32 * hb + (lane & 31);
        const int sa = m >> 4, nn = m & 15;
        const float M = stat[(sa * 16 + nn) * 2];
        const float L = (M != NEG_INF) ? stat[(sa * 16 + nn) * 2 + 1] : 0.f;
        const bool empty = !(L > 0.f);
        inv[hb] = empty ? 0.f : 1.f / L;
        const float lse_v = empty ? NEG_INF : (M + __log2f(L)) * LN2;
        int orow = t, ohead = m;
        bool ok = m < a.h;
        if constexpr (S::DENSE) {
          const int r = m / a.h;
          ok = r < d_nr;
          orow = d_r0 + r;
          ohead = m - r * a.h;
        }
        okv[hb] = ok;
        obase[hb] = split ? (unit * a.h + ohead) * D_V : (int64_t)orow * a.out_st + (int64_t)ohead * a.out_sh;
        if (ok && hg == 0 && lane < 32) {
          if (!split) a.lse[(int64_t)orow * a.lse_st + ohead] = lse_v;
          else a.ws_lse[unit * a.h + ohead] = lse_v;
        }
      }
      if (!split) {
        // bf16 output in 16-byte pieces: for q = 2r, 2r + 1 a lane holds dims
        // dl .. dl + 3 of both; one lane-half swap gives lane l < 32 the two
        // pieces of q = 2r (dims dl .. dl + 7) and lane l + 32 those of q = 2r + 1,
        // so each store instruction writes 32 contiguous bytes per slot.  With
        // 8-byte stores straight from the accumulators the epilogue was 2%
        // of c4's kernel time slower.
#pragma unroll
        for (int hb = 0; hb < 2; ++hb) {
          if (!okv[hb]) continue;
          uint16_t* ob = a.out + obase[hb] + 128 * hg + 8 * (lane >> 5);
#pragma unroll
          for (int db = 0; db < 4; ++db)
#pragma unroll
            for (int qp = 0; qp < 4; qp += 2) {
              const f32x16& v = o16[2 * db + hb];
              uint32_t r0[2], r1[2];
              r0[0] = pack_bf16x2(v[4 * qp] * inv[hb], v[4 * qp + 1] * inv[hb]);
              r0[1] = pack_bf16x2(v[4 * qp + 2] * inv[hb], v[4 * qp + 3] * inv[hb]);
              r1[0] = pack_bf16x2(v[4 * qp + 4] * inv[hb], v[4 * qp + 5] * inv[hb]);
              r1[1] = pack_bf16x2(v[4 * qp + 6] * inv[hb], v[4 * qp + 7] * inv[hb]);
#pragma unroll
              for (int w = 0; w < 2; ++w) {
                const auto sw = __builtin_amdgcn_permlane32_swap(r0[w], r1[w], false, false);
                r0[w] = sw[0];
                r1[w] = sw[1];
              }
              *reinterpret_cast<u32x4*>(ob + 64 * (db >> 1) + 16 * ((db & 1) + 2 * (qp >> 1))) = u32x4{r0[0], r0[1], r1[0], r1[1]};
            }
        }
      } else {
#pragma unroll
        for (int hb = 0; hb < 2; ++hb) {
          if (!okv[hb]) continue;
          float* wb = a.ws_out + obase[hb] + 128 * hg + 4 * (lane >> 5);
#pragma unroll
          for (int db = 0; db < 4; ++db)
#pragma unroll
            for (int q = 0; q < 4; ++q) {
              const f32x16& v = o16[2 * db + hb];
              f32x4 w;
#pragma unroll
              for (int j = 0; j < 4; ++j) w[j] = v[4 * q + j] * inv[hb];
              *reinterpret_cast<f32x4*>(wb + 64 * (db >> 1) + 16 * ((db & 1) + 2 * (q >> 1)) + 8 * (q & 1)) = w;
            }
        }
      }
      return;
    }
#pragma unroll
    for (int hf = 0; hf < 4; ++hf) {
      const int sa = S::RSPLIT ? 2 * hf : hf;   // statistics slot(s) of head group hf
      const int m = 16 * hf + n;
      const float M = stat[(sa * 16 + n) * 2];
      const float L = (M != NEG_INF) ? stat[(sa * 16 + n) * 2 + 1] + (S::RSPLIT ? stat[((sa + 1) * 16 + n) * 2 + 1] : 0.f)
                                     : 0.f;
      const bool empty = !(L > 0.f);
      const float inv = empty ? 0.f : 1.f / L;
      const float lse_v = empty ? NEG_INF : (M + __log2f(L)) * LN2;
      int orow = t, ohead = m;
      bool ok = m < a.h;
      if constexpr (S::DENSE) {
        const int r = m / a.h;
        ok = r < d_nr;
        orow = d_r0 + r;
        ohead = m - r * a.h;
      }
      if (!ok) continue;
#pragma unroll
      for (int f = 0; f < 8; ++f) {
        const int d0 = 128 * hg + 16 * f + 4 * g4;
        const f32x4 v = o[4 * f + hf];
        if (!split) {
          u32x2 pk;
          pk[0] = (uint32_t)f32_to_bf16_bits(v[0] * inv) | ((uint32_t)f32_to_bf16_bits(v[1] * inv) << 16);
          pk[1] = (uint32_t)f32_to_bf16_bits(v[2] * inv) | ((uint32_t)f32_to_bf16_bits(v[3] * inv) << 16);
          *reinterpret_cast<u32x2*>(a.out + (int64_t)orow * a.out_st + (int64_t)ohead * a.out_sh + d0) = pk;
        } else {
          f32x4 w;
#pragma unroll
          for (int j = 0; j < 4; ++j) w[j] = v[j] * inv;
          *reinterpret_cast<f32x4*>(a.ws_out + (unit * a.h + ohead) * D_V + d0) = w;
        }
      }
      if (hg == 0 && g4 == 0) {
        if (!split) a.lse[(int64_t)orow * a.lse_st + ohead] = lse_v;
        else a.ws_lse[unit * a.h + ohead] = lse_v;
      }
    }
    return;
  } else if constexpr (S::PAIR) {
    // the row stream's 32 fragments, staged where its first wave's would be
    f32x4* ost = reinterpret_cast<f32x4*>(smem) + (size_t)(rg * S::HG) * 32 * 64;
#pragma unroll
    for (int i = 0; i < 16; ++i) ost[spos(16 * hg + i, g4, n)] = o[i];
  } else {
    f32x4* ost = reinterpret_cast<f32x4*>(smem) + (size_t)wave * 32 * 64;
#pragma unroll
    for (int f = 0; f < 32; ++f) ost[spos(f, g4, n)] = o[f];
  }
  // (only shapes without the output-dim split reach here: one query row per
  // work-group, row streams merged through LDS)
  __syncthreads();
  const bool split = a.write_partials != 0;
  const int n_items = a.h * 64;
  // unrolled so the LDS reads of several items are in flight together
#pragma unroll 4
  for (int item = tid; item < n_items; item += S::NTHR) {
    const int head = item >> 6, c = item & 63;
    const int hgi = head >> 4, nn = head & 15;
    float M = NEG_INF;
#pragma unroll
    for (int r = 0; r < S::NRG; ++r)
      M = fmaxf(M, stat[((r * S::HG + hgi) * 16 + nn) * 2]);
    float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    float L = 0.f;
    if (M != NEG_INF) {
#pragma unroll
      for (int r = 0; r < S::NRG; ++r) {
        const int w = r * S::HG + hgi;
        // PAIR: waves w, w + 1 hold one head's row halves
        const float fct = fast_exp2(stat[(w * 16 + nn) * 2] - M);
        L += fct * (stat[(w * 16 + nn) * 2 + 1] + (S::PAIR ? stat[((w + 1) * 16 + nn) * 2 + 1] : 0.f));
        // dims 8c..8c+7 = fragment c/2, lanes (2*(c&1) + {0,1})*16 + nn, j = 0..3
        const f32x4* ost = reinterpret_cast<const f32x4*>(smem) + (size_t)w * 32 * 64;
        const f32x4 v0 = ost[spos(c >> 1, 2 * (c & 1) + 0, nn)];
        const f32x4 v1 = ost[spos(c >> 1, 2 * (c & 1) + 1, nn)];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          acc[j] += fct * v0[j];
          acc[4 + j] += fct * v1[j];
        }
      }
    }
    const bool empty = !(L > 0.f);
    const float inv = empty ? 0.f : 1.f / L;
    const float lse_v = empty ? NEG_INF : (M + __log2f(L)) * LN2;
    if (!split) {
      u32x4 pk;
#pragma unroll
      for (int j = 0; j < 4; ++j)
        pk[j] = (uint32_t)f32_to_bf16_bits(acc[2 * j] * inv) |
                ((uint32_t)f32_to_bf16_bits(acc[2 * j + 1] * inv) << 16);
      *reinterpret_cast<u32x4*>(a.out + (int64_t)t * a.out_st + (int64_t)head * a.out_sh + 8 * c) = pk;
      if (c == 0) a.lse[(int64_t)t * a.lse_st + head] = lse_v;
    } else {
      float* wo = a.ws_out + ((unit * a.h + head) * D_V) + 8 * c;
      f32x4 w0, w1;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        w0[j] = acc[j] * inv;
        w1[j] = acc[4 + j] * inv;
      }
      reinterpret_cast<f32x4*>(wo)[0] = w0;
      reinterpret_cast<f32x4*>(wo)[1] = w1;
      if (c == 0) a.ws_lse[unit * a.h + head] = lse_v;
    }
  }
}


// Merge the KV splits of each query row by their lse, in split order.
// Thread = (row, head, 8 output dims); SMAX > 0 unrolls the split loop so the
// loads of all splits are in flight together (SMAX = 0: any split count).
template <int SMAX>
__global__ void __launch_bounds__(256) smla_lse_combine(CombineArgs a) {
  const int t = blockIdx.x;
  const int item = blockIdx.y * blockDim.x + threadIdx.x;
  if (item >= a.h * 64) return;
  const int head = item >> 6, c = item & 63;
  const int S_ = a.num_splits;
  const int64_t u0 = (int64_t)t * S_;
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  float M = NEG_INF, L = 0.f;
  if constexpr (SMAX > 0) {
    float ls[SMAX];
#pragma unroll
    for (int s = 0; s < SMAX; ++s) ls[s] = (s < S_) ? a.ws_lse[(u0 + s) * a.h + head] : NEG_INF;
    f32x4 v0[SMAX], v1[SMAX];
#pragma unroll
    for (int s = 0; s < SMAX; ++s) {
      if (s < S_) {
        const f32x4* src = reinterpret_cast<const f32x4*>(a.ws_out + ((u0 + s) * a.h + head) * D_V + 8 * c);
        v0[s] = src[0];
        v1[s] = src[1];
      }
    }
#pragma unroll
    for (int s = 0; s < SMAX; ++s) M = fmaxf(M, ls[s]);
    if (M != NEG_INF) {
#pragma unroll
      for (int s = 0; s < SMAX; ++s) {
        if (s < S_) {
          const float w = fast_exp2((ls[s] - M) * 1.44269504088896340736f);
          L += w;
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            acc[j] += w * v0[s][j];
            acc[4 + j] += w * v1[s][j];
          }
        }
      }
    }
  } else {
    for (int s = 0; s < S_; ++s) M = fmaxf(M, a.ws_lse[(u0 + s) * a.h + head]);
    if (M != NEG_INF) {
      for (int s = 0; s < S_; ++s) {
        const int64_t u = u0 + s;
        const float w = fast_exp2((a.ws_lse[u * a.h + head] - M) * 1.44269504088896340736f);
        L += w;
        const f32x4* src = reinterpret_cast<const f32x4*>(a.ws_out + (u * a.h + head) * D_V + 8 * c);
        const f32x4 x0 = src[0], x1 = src[1];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          acc[j] += w * x0[j];
          acc[4 + j] += w * x1[j];
        }
      }
    }
  }
  const bool empty = !(L > 0.f);
  const float inv = empty ? 0.f : 1.f / L;
  u32x4 pk;
#pragma unroll
  for (int j = 0; j < 4; ++j)
    pk[j] = (uint32_t)f32_to_bf16_bits(acc[2 * j] * inv) | ((uint32_t)f32_to_bf16_bits(acc[2 * j + 1] * inv) << 16);
  *reinterpret_cast<u32x4*>(a.out + (int64_t)t * a.out_st + (int64_t)head * a.out_sh + 8 * c) = pk;
  if (c == 0) a.lse[(int64_t)t * a.lse_st + head] = empty ? NEG_INF : M + __logf(L);
}

// Kernel variants: (head groups, row groups, tile rows, stages, format).
using V_H1_A = Shape<1, 4, 16, 2, 0>;
using V_H1_B = Shape<1, 2, 16, 4, 0>;
using V_H1_T = Shape<1, 2, 16, 2, 0, false, false, false, false, false, false, true>;   // two per CU
using V_H2_A = Shape<2, 2, 32, 2, 0>;
using V_H2_B = Shape<2, 1, 32, 4, 0>;
using V_H2_T = Shape<2, 1, 32, 2, 0, false, false, false, false, false, false, true>;   // two per CU
using V_H4_A = Shape<4, 1, 32, 4, 0, true, true>;
using V_H4_B = Shape<4, 1, 32, 4, 0>;
using V_H4_C = Shape<4, 1, 32, 4, 0, true, true, false, true>;
// NoPE geometry (bf16, 512-wide rows): the default shapes
using N_H1_A = Shape<1, 4, 16, 2, 0, false, false, false, false, true>;
using N_H2_A = Shape<2, 2, 32, 2, 0, false, false, false, false, true>;
using N_H4_A = Shape<4, 1, 32, 4, 0, true, true, false, false, true>;
// NoPE, two work-groups per CU (the 1 KB rows leave room for the usual layout)
using N_H1_T = Shape<1, 2, 16, 2, 0, false, false, false, false, true>;
using N_H2_T = Shape<2, 1, 32, 2, 0, false, false, false, false, true>;
// dense causal mode (576- and 512-wide rows)
using D_H4 = Shape<4, 1, 32, 4, 0, true, true, false, false, false, true>;
using D_H4_N = Shape<4, 1, 32, 4, 0, true, true, false, false, true, true>;
using F_H1_A = Shape<2, 2, 32, 3, 1, false, false, true>;
using F_H1_B = Shape<1, 2, 32, 3, 1>;
using F_H1_T = Shape<2, 1, 32, 3, 1, false, false, true>;   // one wave-pair stream: two per CU
using F_H2_A = Shape<2, 1, 32, 4, 1>;
using F_H4_A = Shape<4, 1, 32, 7, 1>;
// fp8 NoPE geometry (rows of the 512 codes, no rope part): the fp8 shapes
// (the 528-byte slots leave room for one more stage than the 656-byte ones)
using NF_H1_A = Shape<2, 2, 32, 4, 1, false, false, true, false, true>;
using NF_H1_T = Shape<2, 1, 32, 4, 1, false, false, true, false, true>;   // two per CU
using NF_H2_A = Shape<2, 1, 32, 4, 1, false, false, false, false, true>;
using NF_H4_A = Shape<4, 1, 32, 8, 1, false, false, false, false, true>;

template <class S>
FwdShape shape_of() {
  return FwdShape{S::HEAD_GROUPS, S::NRG, S::RT, S::NST, S::NTHR, S::LDS_BYTES};
}

template <class S>
hipError_t launch_one(const FwdArgs& a, int64_t grid, hipStream_t stream) {
  hipLaunchKernelGGL(smla_fwd<S>, dim3((unsigned)grid), dim3(S::NTHR), 0, stream, a);
  return hipGetLastError();
}

}  // namespace

bool fwd_shape(int kv_format, int head_groups, int variant, int nope, FwdShape* shape) {
  if (nope && kv_format == 1) {
    if (!(variant == 0 || (variant == 2 && head_groups == 1))) return false;
    switch (head_groups) {
      case 1: *shape = variant == 2 ? shape_of<NF_H1_T>() : shape_of<NF_H1_A>(); return true;
      case 2: *shape = shape_of<NF_H2_A>(); return true;
      case 4: *shape = shape_of<NF_H4_A>(); return true;
      default: return false;
    }
  }
  if (nope) {
    if (kv_format != 0 || !(variant == 0 || (variant == 2 && head_groups <= 2))) return false;
    switch (head_groups) {
      case 1: *shape = variant == 2 ? shape_of<N_H1_T>() : shape_of<N_H1_A>(); return true;
      case 2: *shape = variant == 2 ? shape_of<N_H2_T>() : shape_of<N_H2_A>(); return true;
      case 4: *shape = shape_of<N_H4_A>(); return true;
      default: return false;
    }
  }
  if (kv_format == 1) {
    if (variant != 0 && !((variant == 1 || variant == 2) && head_groups == 1)) return false;
    switch (head_groups) {
      case 1:
        *shape = variant == 2 ? shape_of<F_H1_T>() : variant == 1 ? shape_of<F_H1_B>() : shape_of<F_H1_A>();
        return true;
      case 2: *shape = shape_of<F_H2_A>(); return true;
      case 4: *shape = shape_of<F_H4_A>(); return true;
      default: return false;
    }
  }
  switch (head_groups) {
    case 1:
      *shape = variant == 2 ? shape_of<V_H1_T>() : variant == 1 ? shape_of<V_H1_B>() : shape_of<V_H1_A>();
      return variant <= 2;
    case 2:
      *shape = variant == 2 ? shape_of<V_H2_T>() : variant == 1 ? shape_of<V_H2_B>() : shape_of<V_H2_A>();
      return variant <= 2;
    case 4:
      *shape = variant == 2 ? shape_of<V_H4_C>() : variant == 1 ? shape_of<V_H4_B>() : shape_of<V_H4_A>();
      return variant <= 2;
    default: return false;
  }
}

hipError_t launch_fwd(const FwdArgs& a, int kv_format, int head_groups, int variant, int nope, int64_t grid,
                      hipStream_t stream) {
  if (nope && kv_format == 1) {
    switch (head_groups) {
      case 1: return variant == 2 ? launch_one<NF_H1_T>(a, grid, stream) : launch_one<NF_H1_A>(a, grid, stream);
      case 2: return launch_one<NF_H2_A>(a, grid, stream);
      case 4: return launch_one<NF_H4_A>(a, grid, stream);
      default: return hipErrorInvalidValue;
    }
  }
  if (nope) {
    switch (head_groups) {
      case 1: return variant == 2 ? launch_one<N_H1_T>(a, grid, stream) : launch_one<N_H1_A>(a, grid, stream);
      case 2: return variant == 2 ? launch_one<N_H2_T>(a, grid, stream) : launch_one<N_H2_A>(a, grid, stream);
      case 4: return launch_one<N_H4_A>(a, grid, stream);
      default: return hipErrorInvalidValue;
    }
  }
  if (kv_format == 1) {
    switch (head_groups) {
      case 1:
        return variant == 2   ? launch_one<F_H1_T>(a, grid, stream)
               : variant == 1 ? launch_one<F_H1_B>(a, grid, stream)
                              : launch_one<F_H1_A>(a, grid, stream);
      case 2: return launch_one<F_H2_A>(a, grid, stream);
      case 4: return launch_one<F_H4_A>(a, grid, stream);
      default: return hipErrorInvalidValue;
    }
  }
  switch (head_groups) {
    case 1:
      return variant == 2   ? launch_one<V_H1_T>(a, grid, stream)
             : variant == 1 ? launch_one<V_H1_B>(a, grid, stream)
                            : launch_one<V_H1_A>(a, grid, stream);
    case 2:
      return variant == 2   ? launch_one<V_H2_T>(a, grid, stream)
             : variant == 1 ? launch_one<V_H2_B>(a, grid, stream)
                            : launch_one<V_H2_A>(a, grid, stream);
    case 4:
      return variant == 2   ? launch_one<V_H4_C>(a, grid, stream)
             : variant == 1 ? launch_one<V_H4_B>(a, grid, stream)
                            : launch_one<V_H4_A>(a, grid, stream);
    default: return hipErrorInvalidValue;
  }
}
hipError_t launch_dense(const FwdArgs& a, int nope, int64_t grid, hipStream_t stream) {
  return nope ? launch_one<D_H4_N>(a, grid, stream) : launch_one<D_H4>(a, grid, stream);
}
int dense_lds_bytes(int nope) { return nope ? D_H4_N::LDS_BYTES : D_H4::LDS_BYTES; }

// Device address of this GPU's `scratch` array (the current device's), looked
// up once per device with that device current and kept.
hipError_t noalloc_scratch(void** ptr) {
  static std::mutex mu;
  static void* addr[kMaxDevices] = {};
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lk(mu);
  if (!addr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    addr[dev] = p;
  }
  *ptr = addr[dev];
  return hipSuccess;
}

hipError_t launch_combine(const CombineArgs& a, hipStream_t stream) {
  // one 64-thread work-group per (row, head): a decode batch's few rows still
  // spread over every CU (c2: 256 work-groups of 16 KB of partials each
  // instead of 64 of 64 KB; the step 23.8 -> 23.4 us)
  const dim3 grid((unsigned)a.T, (unsigned)a.h);
  if (a.num_splits <= 4) hipLaunchKernelGGL(smla_lse_combine<4>, grid, dim3(64), 0, stream, a);
  else if (a.num_splits <= 8) hipLaunchKernelGGL(smla_lse_combine<8>, grid, dim3(64), 0, stream, a);
  else if (a.num_splits <= 16) hipLaunchKernelGGL(smla_lse_combine<16>, grid, dim3(64), 0, stream, a);
  else hipLaunchKernelGGL(smla_lse_combine<0>, grid, dim3(64), 0, stream, a);
  return hipGetLastError();
}

}  // namespace smla
