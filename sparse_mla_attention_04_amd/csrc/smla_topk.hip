// Per-row top-k selection over caller-provided key scores: the last step of
// the sparse indexer that produces the int32 index lists the attention
// consumes (vLLM PR #54951, "Summary": per query row, the indices of its
// top-k scored keys; "Additional checks": the selected sets are compared, the
// order inside a row is not defined).
//
// One work-group (four waves) per query row.  The k-th largest score is found
// by a radix select over an order-preserving 32-bit key.
//   One read (long rows): every 32nd 128-byte line of the row is read as a
//   sample, and a threshold tau is found in LDS: the lowest key of the 22-bit
//   bucket holding the sample's r-th largest key, r chosen so that about
//   (k + CAP) / 2 keys of the row are expected at or above it.
//   One pass over the row then copies every key >= tau (and its index) to
//   LDS.  When k <= that count <= CAP, the candidates hold the whole top-k and
//   every key equal to the k-th, and the selection finishes in LDS.  Any
//   other count (an unrepresentative sample) takes the two-read route below.
//   Measured on MI355X (4096 rows x 65536 N(0,1) scores, k = 2048): 0.476 ms
//   with two reads, 0.474 ms with one read while each wave kept one load in
//   flight, 0.339 ms with one read in batches of eight loads per thread,
//   0.296 ms with the candidates appended one LDS atomic per wave and batch.
//   Two reads: an LDS histogram of the key's top 11 bits over the whole row
//   names the bucket holding the k-th key.  When that bucket fits in LDS, a
//   second read of the row writes every key above the bucket and copies the
//   bucket's keys to LDS, where the remaining 11 + 10 bits are resolved and
//   ties are cut by index.  A larger bucket (heavily tied rows) takes two
//   more histogram rounds over the row and a final pass that writes the keys
//   above the k-th key and the lowest-index keys equal to it.
#include "smla_internal.h"

namespace smla {
namespace {

typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4;

// Order-preserving key of a score: larger score -> larger key, equal scores
// (-0 and +0 included) -> equal keys; NaN maps below every number (-inf
// included).
__device__ __forceinline__ uint32_t order_key(float x) {
  uint32_t b = __float_as_uint(x);
  if (b == 0x80000000u) b = 0u;
  if ((b & 0x7fffffffu) > 0x7f800000u) return 0u;
  return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}

// Digits of the radix select, most significant first: 11 + 11 + 10 bits, so
// the first histogram already spreads typical scores (sign, exponent and two
// mantissa bits) over many bins.
constexpr int NB = 2048;                 // bins of the widest digit
constexpr int SHIFTS[3] = {21, 10, 0};
constexpr int WIDTHS[3] = {11, 11, 10};
// Candidate keys (and indices) held in LDS: the one-read route's keys >= tau
// (about 3072 for k = 2048), or the two-read route's top-digit bucket (about
// 1200 for N(0,1) scores, 65536 keys, k = 2048).
// 4084 rather than 4096: with it the work-group's LDS (histogram,
// candidates, counters) is 40,912 bytes, so four work-groups share a CU.
constexpr int CAP = 4084;
// The one-read route runs for k <= KMAX_ONE: its threshold aims at
// (k + CAP) / 2 keys, which leaves (CAP - k) / 2 keys of room below CAP and
// above k.
constexpr int KMAX_ONE = 2048;
static_assert((CAP - KMAX_ONE) / 2 >= 1000, "one-read route margin");
// One-read route: sampled lines are every LSTRIDE-th 128-byte line, at most
// CAP sample keys, and the sample rank r behind tau at least MIN_RANK (the
// count of row keys >= tau then has a relative spread of at most about
// 1 / sqrt(MIN_RANK)).
constexpr int LSTRIDE = 32;
constexpr int MIN_RANK = 48;

// Radix step on a filled histogram of nb bins: the bin in which the count of
// keys, taken from the top bin down, reaches kr.  Thread j owns bins
// [j * per, (j + 1) * per); suffix sums over the threads locate the owner of
// the crossing bin, which writes ctl[0] = bin, ctl[1] = keys still to take
// inside it, ctl[4] = the bin's count.  Ends with a barrier.
// Inclusive prefix sum over a wave's 64 lanes without LDS: shifts by 1, 2,
// 4 and 8 lanes inside each 16-lane row (lanes with no source add 0), then
// row 0's total into row 1 and row 2's into row 3 (broadcast of lanes 15 and
// 47), then the first two rows' total into rows 2 and 3 (lane 31).
__device__ __forceinline__ int wave_incl_scan(int x) {
  x += __builtin_amdgcn_update_dpp(0, x, 0x111, 0xf, 0xf, false);   // row_shr:1
  x += __builtin_amdgcn_update_dpp(0, x, 0x112, 0xf, 0xf, false);   // row_shr:2
  x += __builtin_amdgcn_update_dpp(0, x, 0x114, 0xf, 0xf, false);   // row_shr:4
  x += __builtin_amdgcn_update_dpp(0, x, 0x118, 0xf, 0xf, false);   // row_shr:8
  x += __builtin_amdgcn_update_dpp(0, x, 0x142, 0xa, 0xf, false);   // row_bcast:15
  x += __builtin_amdgcn_update_dpp(0, x, 0x143, 0xc, 0xf, false);   // row_bcast:31
  return x;
}

__device__ __forceinline__ void find_bin(const uint32_t* hist, int nb, int kr, int* ctl, int* wsum, int tid,
                                         int lane, int wave) {
  const int per = nb / 256;
  int own = 0;
  for (int q = 0; q < per; ++q) own += (int)hist[tid * per + q];
  // inclusive suffix sum over thread index, high to low: the wave's total
  // minus the inclusive prefix sum, plus the lane's own count
  const int pre = wave_incl_scan(own);
  const int wtot = __builtin_amdgcn_readlane(pre, 63);
  const int incl = wtot - pre + own;
  if (lane == 0) wsum[wave] = incl;   // the wave's total
  __syncthreads();
  int above_waves = 0;
  for (int w = wave + 1; w < 4; ++w) above_waves += wsum[w];
  const int suffix = incl + above_waves;          // keys in bins owned by threads >= tid
  const int above_me = suffix - own;              // keys in bins owned by threads > tid
  if (above_me < kr && suffix >= kr) {
    int acc = above_me, d = (tid + 1) * per - 1;
    for (; d > tid * per; --d) {
      if (acc + (int)hist[d] >= kr) break;
      acc += (int)hist[d];
    }
    ctl[0] = d;
    ctl[1] = kr - acc;
    ctl[4] = (int)hist[d];
  }
  __syncthreads();
}

__global__ void __launch_bounds__(256) smla_topk_kernel(TopkArgs a) {
  __shared__ uint32_t hist[NB];
  __shared__ int ctl[8];     // chosen digit, keys still to take in its bucket, above-count, tie-count, bin count
  __shared__ int wsum[4];
  __shared__ uint32_t cand_key[CAP];   // the top-digit bucket's keys and indices
  __shared__ int32_t cand_idx[CAP];
  const int t = blockIdx.x;
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const float* row = a.scores + (int64_t)t * a.ld;
  int32_t* out = a.idx + (int64_t)t * a.idx_stride;
  int len = a.lens ? a.lens[t] : a.n_keys;
  len = len < 0 ? 0 : (len > a.n_keys ? a.n_keys : len);
  const int k = a.k;
  if (len <= k) {
    for (int i = tid; i < k; i += 256) out[i] = i < len ? i : -1;
    return;
  }
  const bool vec = ((reinterpret_cast<uintptr_t>(row) & 15u) == 0) && ((a.ld & 3) == 0);
  // invariant: at least kr of the keys matching (prefix, mask) remain, and
  // the keys above that bucket (k - kr of them) are all selected
  uint32_t prefix = 0, mask = 0;
  int kr = k;
  auto hist_pass = [&](int shift, int nb) {
    for (int i = tid; i < nb; i += 256) hist[i] = 0u;
    __syncthreads();
    auto count = [&](float x) {
      const uint32_t u = order_key(x);
      if ((u & mask) == prefix) atomicAdd(&hist[(u >> shift) & (uint32_t)(nb - 1)], 1u);
    };
    // 16-byte loads (four scores per lane, four loads in flight) when the
    // row allows them; the last len % 4 scores one by one
    int done = 0;
    if (vec) {
      const f32x4* row4 = reinterpret_cast<const f32x4*>(row);
      const int n4 = len >> 2;
#pragma unroll 4
      for (int j = tid; j < n4; j += 256) {
        const f32x4 v = row4[j];
        count(v[0]);
        count(v[1]);
        count(v[2]);
        count(v[3]);
      }
      done = n4 << 2;
    }
    for (int i = done + tid; i < len; i += 256) count(row[i]);
    __syncthreads();
    find_bin(hist, nb, kr, ctl, wsum, tid, lane, wave);
    prefix |= (uint32_t)ctl[0] << shift;
    mask |= (uint32_t)(nb - 1) << shift;
    kr = ctl[1];
  };
  // radix select over the nc LDS candidates: with (prefix, mask, kr) on entry
  // describing the keys still open, leaves prefix = the kr-th largest key,
  // kr = how many keys equal to it are taken, ctl[4] = how many there are
  auto lds_select = [&](int nc, int first_pass, int end_pass = 3) {
    for (int pass = first_pass; pass < end_pass; ++pass) {
      const int shift = SHIFTS[pass];
      const int nb = 1 << WIDTHS[pass];
      for (int i = tid; i < nb; i += 256) hist[i] = 0u;
      __syncthreads();
      for (int c = tid; c < nc; c += 256) {
        const uint32_t u = cand_key[c];
        if ((u & mask) == prefix) atomicAdd(&hist[(u >> shift) & (uint32_t)(nb - 1)], 1u);
      }
      __syncthreads();
      find_bin(hist, nb, kr, ctl, wsum, tid, lane, wave);
      prefix |= (uint32_t)ctl[0] << shift;
      mask |= (uint32_t)(nb - 1) << shift;
      kr = ctl[1];
    }
  };
  // writes the selection from the nc LDS candidates, which hold every key
  // >= prefix (the k-th largest key); keys above it were already written to
  // out[0 .. n_out) when n_out > 0.  kr of the ctl[4] keys equal to prefix
  // are taken, the lowest-index ones.
  auto write_selection = [&](int nc, int n_out) {
    const int n_eq = ctl[4];
    uint32_t vsel = 0u;   // ties are taken while ~index >= vsel
    if (n_eq > kr) {
      // radix select of the kr-th largest ~index among the ties (indices are
      // distinct, so exactly kr ties reach it)
      uint32_t vpre = 0u, vmask = 0u;
      int kv = kr;
#pragma unroll
      for (int pass = 0; pass < 3; ++pass) {
        const int shift = SHIFTS[pass];
        const int nb = 1 << WIDTHS[pass];
        __syncthreads();
        for (int i = tid; i < nb; i += 256) hist[i] = 0u;
        __syncthreads();
        for (int c = tid; c < nc; c += 256) {
          const uint32_t v = ~(uint32_t)cand_idx[c];
          if (cand_key[c] == prefix && (v & vmask) == vpre) atomicAdd(&hist[(v >> shift) & (uint32_t)(nb - 1)], 1u);
        }
        __syncthreads();
        find_bin(hist, nb, kv, ctl, wsum, tid, lane, wave);
        vpre |= (uint32_t)ctl[0] << shift;
        vmask |= (uint32_t)(nb - 1) << shift;
        kv = ctl[1];
      }
      vsel = vpre;
    }
    __syncthreads();
    if (tid == 0) {
      ctl[2] = n_out;
      ctl[3] = 0;
    }
    __syncthreads();
    // wave-aggregated output slots: one atomic per wave and kind of key
    for (int c0 = 0; c0 < nc; c0 += 256) {
      const int c = c0 + tid;
      uint32_t u = 0u;
      int ix = 0;
      if (c < nc) {
        u = cand_key[c];
        ix = cand_idx[c];
      }
      const int above = (c < nc && u > prefix) ? 1 : 0;
      const int tie = (c < nc && u == prefix && ~(uint32_t)ix >= vsel) ? 1 : 0;
      const int ia = wave_incl_scan(above), it = wave_incl_scan(tie);
      const int ta = __builtin_amdgcn_readlane(ia, 63), tt = __builtin_amdgcn_readlane(it, 63);
      int ba = 0, bt = 0;
      if (lane == 0) {
        if (ta > 0) ba = atomicAdd(&ctl[2], ta);
        if (tt > 0) bt = atomicAdd(&ctl[3], tt);
      }
      ba = __builtin_amdgcn_readfirstlane(ba);
      bt = __builtin_amdgcn_readfirstlane(bt);
      if (above) out[ba + ia - 1] = ix;
      else if (tie) out[(k - kr) + bt + it - 1] = ix;
    }
  };

  // ---- one read: a sampled threshold, then one pass collecting keys >= tau
  if (vec && k <= KMAX_ONE) {
    const int lines = len >> 5;                       // whole 128-byte lines of the row
    const int nsl_all = lines / LSTRIDE;              // sampled lines
    const int nsl = nsl_all < CAP / 32 ? nsl_all : CAP / 32;
    const int ns = nsl * 32;                          // sample keys
    const int64_t rank = ((int64_t)(k + CAP) / 2 * ns + len / 2) / len;
    if (nsl > 0 && rank >= MIN_RANK && rank <= ns) {
      // sample line m is line m * (lines / nsl): thread j of the 8 per line
      // reads 16 bytes of it
      const f32x4* row4 = reinterpret_cast<const f32x4*>(row);
      const int lstep = lines / nsl;
      for (int j = tid; j < nsl * 8; j += 256) {
        const int m = j >> 3;
        const f32x4 v = row4[(int64_t)m * lstep * 8 + (j & 7)];
#pragma unroll
        for (int q = 0; q < 4; ++q) cand_key[4 * j + q] = order_key(v[q]);
      }
      // batches of U 16-byte loads per thread, all issued before any key of
      // the batch is examined (the appends branch, which would otherwise
      // leave one load in flight per wave), the next batch requested before
      // the current one is examined; the first batch is requested here, so
      // that it is in flight while the sample's digits are selected (the
      // barriers of that selection wait for LDS operations only)
      const int n4 = len >> 2;
      constexpr int U = 8;
      f32x4 cur[U], nxt[U];
      auto load_batch = [&](int j0, f32x4 (&v)[U]) {
#pragma unroll
        for (int u = 0; u < U; ++u) {
          const int j = j0 + u * 256 + tid;
          v[u] = row4[j < n4 ? j : n4 - 1];
        }
      };
      if (n4 > 0) load_batch(0, cur);
      __syncthreads();
      kr = (int)rank;
      // two of the three digits: tau is the lowest key of the 22-bit bucket
      // holding the sample's rank-th largest key (a threshold only needs to
      // be about right; the bucket spans 2^-13 of a score's magnitude)
      lds_select(ns, 0, 2);
      const uint32_t tau = prefix;
      // one pass: every key >= tau to LDS.  Per batch of 4U keys per lane, the
      // lanes count their keys >= tau, a wave prefix sum gives each lane its
      // place, and one LDS atomic per wave reserves the wave's range (about
      // 5% of keys pass, so a per-key atomic ran in nearly every key slot of
      // every wave, each waiting for its return)
      __syncthreads();
      if (tid == 0) ctl[3] = 0;
      __syncthreads();
      auto append = [&](uint32_t u, int i, bool ok) {
        if (ok && u >= tau) {
          const int c = atomicAdd(&ctl[3], 1);
          if (c < CAP) {
            cand_key[c] = u;
            cand_idx[c] = i;
          }
        }
      };
      for (int j0 = 0; j0 < n4; j0 += 256 * U) {
        if (j0 + 256 * U < n4) load_batch(j0 + 256 * U, nxt);
        uint32_t key[U][4];
        int cnt = 0;
#pragma unroll
        for (int u = 0; u < U; ++u) {
          const bool ok = j0 + u * 256 + tid < n4;
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            key[u][q] = order_key(cur[u][q]);
            cnt += (ok && key[u][q] >= tau) ? 1 : 0;
          }
        }
        const int incl = wave_incl_scan(cnt);
        const int total = __builtin_amdgcn_readlane(incl, 63);
        int base = 0;
        if (total > 0) {
          if (lane == 0) base = atomicAdd(&ctl[3], total);
          base = __builtin_amdgcn_readfirstlane(base);
        }
        int pos = base + incl - cnt;
#pragma unroll
        for (int u = 0; u < U; ++u) {
          const int j = j0 + u * 256 + tid;
          const bool ok = j < n4;
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            if (ok && key[u][q] >= tau) {
              if (pos < CAP) {
                cand_key[pos] = key[u][q];
                cand_idx[pos] = 4 * j + q;
              }
              ++pos;
            }
          }
        }
        if (j0 + 256 * U < n4) {
#pragma unroll
          for (int u = 0; u < U; ++u) cur[u] = nxt[u];
        }
      }
      for (int i0 = n4 << 2; i0 < len; i0 += 256) {
        const int i = i0 + tid;
        append(i < len ? order_key(row[i]) : 0u, i, i < len);
      }
      __syncthreads();
      const int nc = ctl[3];
      if (nc >= k && nc <= CAP) {
        prefix = 0u;
        mask = 0u;
        kr = k;
        lds_select(nc, 0);
        write_selection(nc, 0);
        return;
      }
      // an unrepresentative sample: start over on the two-read route
      prefix = 0u;
      mask = 0u;
      kr = k;
      __syncthreads();
    }
  }

  // invariant: at least kr of the keys matching (prefix, mask) remain, and
  // the keys above that bucket (k - kr of them) are all selected
  hist_pass(SHIFTS[0], 1 << WIDTHS[0]);
  const int nbucket = ctl[4];
  if (nbucket <= CAP) {
    // ---- second read: keys above the bucket out, the bucket's keys to LDS
    const uint32_t d0 = prefix >> SHIFTS[0];
    __syncthreads();
    if (tid == 0) {
      ctl[2] = 0;
      ctl[3] = 0;
    }
    __syncthreads();
    auto route = [&](float x, int i) {
      const uint32_t u = order_key(x);
      const uint32_t d = u >> SHIFTS[0];
      if (d > d0) {
        out[atomicAdd(&ctl[2], 1)] = i;
      } else if (d == d0) {
        const int c = atomicAdd(&ctl[3], 1);
        cand_key[c] = u;
        cand_idx[c] = i;
      }
    };
    int done = 0;
    if (vec) {
      const f32x4* row4 = reinterpret_cast<const f32x4*>(row);
      const int n4 = len >> 2;
#pragma unroll 4
      for (int j = tid; j < n4; j += 256) {
        const f32x4 v = row4[j];
        route(v[0], 4 * j);
        route(v[1], 4 * j + 1);
        route(v[2], 4 * j + 2);
        route(v[3], 4 * j + 3);
      }
      done = n4 << 2;
    }
    for (int i = done + tid; i < len; i += 256) route(row[i], i);
    __syncthreads();
    const int nc = ctl[3];   // == nbucket
    const int n_out = ctl[2];
    // ---- the remaining digits over the LDS copy of the bucket
    lds_select(nc, 1);
    // prefix is the k-th largest key; kr of the keys equal to it are taken
    write_selection(nc, n_out);
    return;
  }
  hist_pass(SHIFTS[1], 1 << WIDTHS[1]);
  hist_pass(SHIFTS[2], 1 << WIDTHS[2]);
  // prefix is the k-th largest key: the k - kr keys above it go to
  // out[0 .. k - kr), the kr lowest-index keys equal to it to out[k - kr .. k)
  if (tid == 0) {
    ctl[2] = 0;
    ctl[3] = 0;
  }
  __syncthreads();
  int tail0 = 0;
  if (vec) {
    // chunks of 1024 scores, four consecutive ones per thread (thread order
    // is index order); ties ranked by a wave scan of the per-thread counts
    const f32x4* row4 = reinterpret_cast<const f32x4*>(row);
    const int n4 = len >> 2;
    for (int b4 = 0; b4 < n4; b4 += 256) {
      const int j = b4 + tid;
      const bool ok = j < n4;
      f32x4 v = ok ? row4[j] : f32x4{0.f, 0.f, 0.f, 0.f};
      bool tq[4];
      int ties = 0;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const uint32_t u = order_key(v[q]);
        if (ok && u > prefix) out[atomicAdd(&ctl[2], 1)] = 4 * j + q;
        tq[q] = ok && u == prefix;
        ties += tq[q] ? 1 : 0;
      }
      int incl = ties;
#pragma unroll
      for (int d = 1; d < 64; d <<= 1) {
        const int t2 = __shfl_up(incl, d, 64);
        if (lane >= d) incl += t2;
      }
      if (lane == 63) wsum[wave] = incl;
      __syncthreads();
      int r = ctl[3] + incl - ties;
      for (int w = 0; w < wave; ++w) r += wsum[w];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        if (tq[q]) {
          if (r < kr) out[(k - kr) + r] = 4 * j + q;
          ++r;
        }
      }
      __syncthreads();
      if (tid == 0) ctl[3] += wsum[0] + wsum[1] + wsum[2] + wsum[3];
      __syncthreads();
    }
    tail0 = n4 << 2;
  }
  for (int base = tail0; base < len; base += 256) {
    const int i = base + tid;
    const uint32_t u = i < len ? order_key(row[i]) : 0u;
    const bool above = i < len && u > prefix;
    const bool tie = i < len && u == prefix;
    if (above) out[atomicAdd(&ctl[2], 1)] = i;
    const uint64_t bal = __ballot(tie);
    const int wrank = __popcll(bal & ((1ull << lane) - 1ull));
    if (lane == 0) wsum[wave] = __popcll(bal);
    __syncthreads();
    int before = ctl[3];
    for (int w = 0; w < wave; ++w) before += wsum[w];
    if (tie && before + wrank < kr) out[(k - kr) + before + wrank] = i;
    __syncthreads();
    if (tid == 0) ctl[3] += wsum[0] + wsum[1] + wsum[2] + wsum[3];
    __syncthreads();
  }
}

}  // namespace

hipError_t launch_topk(const TopkArgs& a, hipStream_t stream) {
  hipLaunchKernelGGL(smla_topk_kernel, dim3((unsigned)a.T), dim3(256), 0, stream, a);
  return hipGetLastError();
}

}  // namespace smla
