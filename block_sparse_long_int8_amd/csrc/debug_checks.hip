// Optional device-side checks of the values the entry points otherwise trust:
// sequence lengths, block lists, positions used as row numbers, head modes and
// segment permutations.  They run only when the checks are switched on: the
// C-ABI layer then resets the violation word, launches the checks of the call
// on the caller's stream, reads the word back and, on a violation, returns an
// error before it launches the call's own kernels.
//
// The violation word is a file-scope device variable (no allocation).  It
// holds (code << 40) | element index of the smallest violation code found, and
// all ones when there is none.
#include "../../include/spa.h"
#include "spa_internal.h"

namespace spa {

namespace {

constexpr unsigned long long kNone = ~0ull;
constexpr int kPermBitmapWords = 8192;  // 32 KiB of LDS: duplicate test for segments up to 262144 rows

__device__ unsigned long long g_violation;

__device__ __forceinline__ void report(int code, long long at) {
  atomicMin(&g_violation, ((unsigned long long)code << 40) | ((unsigned long long)at & ((1ull << 40) - 1)));
}

__global__ void reset_kernel() { g_violation = kNone; }

template <typename T>
__global__ void range_kernel(const T* __restrict__ v, long long n, long long lo, long long hi, int code) {
  for (long long i = blockIdx.x * (long long)blockDim.x + threadIdx.x; i < n; i += (long long)gridDim.x * blockDim.x) {
    const long long x = v[i];
    if (x < lo || x > hi) report(code, i);
  }
}

// One thread per list row: 0 <= count <= cap, entries strictly ascending in
// [0, limit), limit = ceil(seq_len[row / rows_per_seq] / blk) when seq_len is
// given, else nb.
__global__ void lists_kernel(const int32_t* __restrict__ idx, const int32_t* __restrict__ count, long long rows,
                             int cap, int rows_per_seq, const int32_t* __restrict__ seq_len, int blk, int nb) {
  const long long row = blockIdx.x * (long long)blockDim.x + threadIdx.x;
  if (row >= rows) return;
  const int c = count[row];
  if (c < 0 || c > cap) {
    report(SPA_DBG_COUNT, row);
    return;
  }
  long long limit = nb;
  if (seq_len) limit = ((long long)seq_len[row / rows_per_seq] + blk - 1) / blk;
  const int32_t* r = idx + row * cap;
  long long prev = -1;
  for (int j = 0; j < c; ++j) {
    const long long x = r[j];
    if (x < 0 || x >= limit) report(SPA_DBG_IDX_RANGE, row * cap + j);
    else if (x <= prev) report(SPA_DBG_IDX_ORDER, row * cap + j);
    prev = x;
  }
}

// One workgroup per segment: every perm[t] lies in t's segment and, for
// segments that fit the LDS bitmap, no value repeats.
__global__ void __launch_bounds__(256) perm_kernel(const int32_t* __restrict__ perm, int T, int seg) {
  __shared__ unsigned bits[kPermBitmapWords];
  const long long s0 = (long long)blockIdx.x * seg;
  const long long s1 = s0 + seg < T ? s0 + seg : T;
  const bool dup_test = seg <= kPermBitmapWords * 32;
  if (dup_test)
    for (int i = threadIdx.x; i < kPermBitmapWords; i += blockDim.x) bits[i] = 0;
  __syncthreads();
  for (long long t = s0 + threadIdx.x; t < s1; t += blockDim.x) {
    const long long p = perm[t];
    if (p < s0 || p >= s1) {
      report(SPA_DBG_PERM_RANGE, t);
    } else if (dup_test) {
      const unsigned o = (unsigned)(p - s0);
      const unsigned m = 1u << (o & 31);
      if (atomicOr(&bits[o >> 5], m) & m) report(SPA_DBG_PERM_DUP, t);
    }
  }
}

int grid_for(long long n) {
  const long long g = (n + 255) / 256;
  return (int)(g < 1 ? 1 : (g > 4096 ? 4096 : g));
}

}  // namespace

hipError_t dbg_reset(hipStream_t s) {
  reset_kernel<<<1, 1, 0, s>>>();
  return hipGetLastError();
}

hipError_t dbg_range_i32(const int32_t* v, long long n, long long lo, long long hi, int code, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  range_kernel<int32_t><<<grid_for(n), 256, 0, s>>>(v, n, lo, hi, code);
  return hipGetLastError();
}

hipError_t dbg_range_u8(const uint8_t* v, long long n, long long lo, long long hi, int code, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  range_kernel<uint8_t><<<grid_for(n), 256, 0, s>>>(v, n, lo, hi, code);
  return hipGetLastError();
}

hipError_t dbg_lists(const int32_t* idx, const int32_t* count, long long rows, int cap, int rows_per_seq,
                     const int32_t* seq_len, int blk, int nb, hipStream_t s) {
  if (rows <= 0) return hipSuccess;
  lists_kernel<<<(unsigned)((rows + 255) / 256), 256, 0, s>>>(idx, count, rows, cap, rows_per_seq, seq_len, blk, nb);
  return hipGetLastError();
}

hipError_t dbg_perm(const int32_t* perm, int T, int seg, hipStream_t s) {
  if (T <= 0) return hipSuccess;
  perm_kernel<<<(unsigned)((T + (long long)seg - 1) / seg), 256, 0, s>>>(perm, T, seg);
  return hipGetLastError();
}

hipError_t dbg_fetch(unsigned long long* word, hipStream_t s) {
  hipError_t e = hipMemcpyFromSymbolAsync(word, HIP_SYMBOL(g_violation), sizeof(*word), 0, hipMemcpyDeviceToHost, s);
  if (e != hipSuccess) return e;
  return hipStreamSynchronize(s);
}

}  // namespace spa
