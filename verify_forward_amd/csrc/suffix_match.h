// Suffix-match search shared by the proposal kernels (CopyLoop §2 "Block
// Construction"; Copy-as-Decode §5 "Composition with speculative decoding"
// drafts inside gen bodies the same way).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace cad {

// one work-group of SUFFIX_THREADS scans every start p for each suffix
// length n (max_n down to min_n) and keeps the largest matching p
constexpr int SUFFIX_THREADS = 1024;

// The search over x[0 .. T-1] (T may come from device memory): the largest
// start p of each suffix length n (max_n down to min_n) with x[p .. p+n-1]
// == x[T-n .. T-1] and p + n <= T - 1; the first n that matches gives the
// proposal x[p+n .. min(p+n+K, T) - 1].  Every thread of the work-group must
// call it; out_len / out_pos are written by thread 0 (visible to the
// work-group after its next barrier).
static __device__ void suffix_match_body(const int32_t* __restrict__ x, int64_t T, int max_n, int min_n, int K,
                                         int32_t* __restrict__ out_tokens, int32_t* __restrict__ out_len,
                                         int64_t* __restrict__ out_pos) {
  __shared__ int32_t suf[64];
  __shared__ long long red[SUFFIX_THREADS / 64];
  __shared__ long long found;
  const int top = (int)((T - 1 < (int64_t)max_n) ? (T - 1) : max_n);
  if (threadIdx.x == 0) found = -1;
  __syncthreads();
  for (int n = top; n >= min_n && n >= 1; --n) {
    if (threadIdx.x < n) suf[threadIdx.x] = x[T - n + threadIdx.x];
    __syncthreads();
    long long best = -1;
    const int64_t last = T - 1 - n;  // p + n <= T - 1
    for (int64_t p = threadIdx.x; p <= last; p += blockDim.x) {
      bool m = true;
      for (int j = 0; j < n && m; ++j) m = x[p + j] == suf[j];
      if (m && p > best) best = p;
    }
    for (int o = 32; o > 0; o >>= 1) {
      const long long ob = __shfl_xor(best, o);
      best = ob > best ? ob : best;
    }
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = best;
    __syncthreads();
    if (threadIdx.x == 0) {
      long long b = -1;
      for (int i = 0; i < SUFFIX_THREADS / 64; ++i) b = red[i] > b ? red[i] : b;
      if (b >= 0) found = b + n;
    }
    __syncthreads();
    if (found >= 0) break;
  }
  const long long start = found;
  if (start < 0) {
    if (threadIdx.x == 0) { *out_len = 0; *out_pos = -1; }
    return;
  }
  const long long end = (start + K < T) ? start + K : T;
  const int len = (int)(end - start);
  for (int j = threadIdx.x; j < len; j += blockDim.x) out_tokens[j] = x[start + j];
  if (threadIdx.x == 0) { *out_len = len; *out_pos = start; }
}

}  // namespace cad
