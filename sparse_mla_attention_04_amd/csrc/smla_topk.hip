// Per-row top-k selection over caller-provided key scores: the last step of
// the sparse indexer that produces the int32 index lists the attention
// consumes (vLLM PR #54951, "Summary": per query row, the indices of its
// top-k scored keys; "Additional checks": the selected sets are compared, the
// order inside a row is not defined).
//
// One work-group (four waves) per query row.  The k-th largest score is found
// by a radix select over an order-preserving 32-bit key (three rounds of an
// LDS histogram); a final pass writes every key above it (in any order) and
// the lowest-index keys equal to it (in index order).
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

__global__ void __launch_bounds__(256) smla_topk_kernel(TopkArgs a) {
  __shared__ uint32_t hist[NB];
  __shared__ int part[256];  // per-thread bin sums (suffix-scanned)
  __shared__ int ctl[4];     // chosen digit, keys still to take in its bucket, above-count, tie-count
  __shared__ int wsum[4];
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
#pragma unroll
  for (int pass = 0; pass < 3; ++pass) {
    const int shift = SHIFTS[pass];
    const int nb = 1 << WIDTHS[pass];
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
    // thread j owns bins [j * per, (j + 1) * per); suffix sums over threads
    // (from the top bin down) locate the bin where the count reaches kr
    const int per = nb / 256;
    int own = 0;
    for (int q = 0; q < per; ++q) own += (int)hist[tid * per + q];
    // inclusive suffix sum over thread index, high to low: scan the reversed order
    int incl = own;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
      const int v = __shfl_down(incl, d, 64);
      if (lane + d < 64) incl += v;
    }
    if (lane == 0) wsum[wave] = incl;   // the wave's total
    __syncthreads();
    int above_waves = 0;
    for (int w = wave + 1; w < 4; ++w) above_waves += wsum[w];
    const int suffix = incl + above_waves;          // keys in bins owned by threads >= tid
    const int above_me = suffix - own;              // keys in bins owned by threads > tid
    if (above_me < kr && suffix >= kr) {
      // the crossing bin is one of this thread's
      int acc = above_me, d = (tid + 1) * per - 1;
      for (; d > tid * per; --d) {
        if (acc + (int)hist[d] >= kr) break;
        acc += (int)hist[d];
      }
      ctl[0] = d;
      ctl[1] = kr - acc;
    }
    __syncthreads();
    prefix |= (uint32_t)ctl[0] << shift;
    mask |= (uint32_t)(nb - 1) << shift;
    kr = ctl[1];
    __syncthreads();
  }
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
