// Row gather / scatter through a segment-wise permutation.
//
// PBS-Attn page §1: permuting key/value pairs together leaves attention
// unchanged, permuted queries give a permuted output and the inverse
// permutation restores the order; §2: permutations stay inside segments.
// Pure data movement, HBM-bound: each thread moves 16 bytes (fast path) so a
// 256-byte bf16 row of d = 128 is one coalesced 16-lane access.
#include "spa_internal.h"

namespace spa {

namespace {

template <typename U>
__global__ void permute_kernel(const U* __restrict__ src, U* __restrict__ dst, int T,
                               int units_per_row, const int32_t* __restrict__ perm, int inverse) {
  const int64_t o = blockIdx.y;
  const int64_t per_outer = (int64_t)T * units_per_row;
  const U* s = src + o * per_outer;
  U* d = dst + o * per_outer;
  for (int64_t u = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; u < per_outer;
       u += (int64_t)gridDim.x * blockDim.x) {
    const int t = (int)(u / units_per_row);
    const int c = (int)(u - (int64_t)t * units_per_row);
    const int pt = perm[t];
    if (!inverse)
      d[u] = s[(int64_t)pt * units_per_row + c];
    else
      d[(int64_t)pt * units_per_row + c] = s[u];
  }
}

}  // namespace

hipError_t launch_permute(const void* src, void* dst, int64_t outer, int T, size_t row_bytes,
                          const int32_t* perm, int inverse, hipStream_t s) {
  const int threads = 256;
  auto grid_for = [&](int64_t units) {
    int64_t blocks = (units + threads - 1) / threads;
    if (blocks > 65535) blocks = 65535;
    return dim3((unsigned)blocks, (unsigned)outer);
  };
  const bool a16 = row_bytes % 16 == 0 && ((uintptr_t)src % 16 == 0) && ((uintptr_t)dst % 16 == 0);
  const bool a4 = row_bytes % 4 == 0 && ((uintptr_t)src % 4 == 0) && ((uintptr_t)dst % 4 == 0);
  if (a16) {
    const int upr = (int)(row_bytes / 16);
    permute_kernel<uint4><<<grid_for((int64_t)T * upr), threads, 0, s>>>(
        (const uint4*)src, (uint4*)dst, T, upr, perm, inverse);
  } else if (a4) {
    const int upr = (int)(row_bytes / 4);
    permute_kernel<uint32_t><<<grid_for((int64_t)T * upr), threads, 0, s>>>(
        (const uint32_t*)src, (uint32_t*)dst, T, upr, perm, inverse);
  } else {
    const int upr = (int)row_bytes;
    permute_kernel<uint8_t><<<grid_for((int64_t)T * upr), threads, 0, s>>>(
        (const uint8_t*)src, (uint8_t*)dst, T, upr, perm, inverse);
  }
  return hipGetLastError();
}

}  // namespace spa
