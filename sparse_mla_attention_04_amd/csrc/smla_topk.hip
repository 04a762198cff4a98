// Per-row top-k selection over caller-provided key scores: the last step of
// the sparse indexer that produces the int32 index lists the attention
// consumes (vLLM PR #54951, "Summary": per query row, the indices of its
// top-k scored keys; "Additional checks": the selected sets are compared, the
// order inside a row is not defined).
//
// One work-group (four waves) per query row.  The k-th largest score is found
// by a radix select over an order-preserving 32-bit key, eight bits per round
// with a 256-bin LDS histogram; a final pass writes every key above it (in any
// order) and the lowest-index keys equal to it (in index order).
#include "smla_internal.h"

namespace smla {
namespace {

// Order-preserving key of a score: larger score -> larger key, equal scores
// (-0 and +0 included) -> equal keys; NaN maps below every number (-inf
// included).
__device__ __forceinline__ uint32_t order_key(float x) {
  uint32_t b = __float_as_uint(x);
  if (b == 0x80000000u) b = 0u;
  if ((b & 0x7fffffffu) > 0x7f800000u) return 0u;
  return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}

__global__ void __launch_bounds__(256) smla_topk_kernel(TopkArgs a) {
  __shared__ uint32_t hist[256];
  __shared__ int ctl[4];    // chosen digit, keys still to take in its bucket, above-count, tie-count
  __shared__ int wsum[4];
  const int t = blockIdx.x;
  const int tid = threadIdx.x;
  const float* row = a.scores + (int64_t)t * a.ld;
  int32_t* out = a.idx + (int64_t)t * a.idx_stride;
  int len = a.lens ? a.lens[t] : a.n_keys;
  len = len < 0 ? 0 : (len > a.n_keys ? a.n_keys : len);
  const int k = a.k;
  if (len <= k) {
    for (int i = tid; i < k; i += 256) out[i] = i < len ? i : -1;
    return;
  }
  // invariant: at least kr of the keys matching (prefix, mask) remain, and
  // the keys above that bucket (k - kr of them) are all selected
  uint32_t prefix = 0, mask = 0;
  int kr = k;
  for (int shift = 24; shift >= 0; shift -= 8) {
    hist[tid] = 0u;
    __syncthreads();
    for (int i = tid; i < len; i += 256) {
      const uint32_t u = order_key(row[i]);
      if ((u & mask) == prefix) atomicAdd(&hist[(u >> shift) & 255u], 1u);
    }
    __syncthreads();
    if (tid == 0) {
      int acc = 0, d = 255;
      for (; d > 0; --d) {
        if (acc + (int)hist[d] >= kr) break;
        acc += (int)hist[d];
      }
      ctl[0] = d;
      ctl[1] = kr - acc;
    }
    __syncthreads();
    prefix |= (uint32_t)ctl[0] << shift;
    mask |= 255u << shift;
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
  const int lane = tid & 63, wave = tid >> 6;
  for (int base = 0; base < len; base += 256) {
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
