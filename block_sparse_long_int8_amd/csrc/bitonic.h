// Register bitonic sorting networks shared by the selection and the
// importance-permutation kernels (gfx950, 64-wide waves).
//
// A workgroup sorts blockDim.x * EPT keys held in registers, thread t owning
// elements t*EPT .. t*EPT+EPT-1.  A compare-exchange stage with partner
// distance J runs inside the thread when J < EPT, across lanes of one wave
// when J < EPT * 64 (DPP row moves for lane distances up to 8, a swizzle for
// 16, a permute beyond), and through LDS with two workgroup barriers only when
// the partner lives in another wave.  Both sorts put the largest key first.
#pragma once

#include "spa_internal.h"

namespace spa {

__device__ inline unsigned long long shfl_xor_u64(unsigned long long v, int m) {
  const unsigned lo = __shfl_xor((unsigned)v, m, kWave);
  const unsigned hi = __shfl_xor((unsigned)(v >> 32), m, kWave);
  return ((unsigned long long)hi << 32) | lo;
}

// One compare-exchange stage (k, j) of a descending bitonic sort on 32-bit
// keys, EPT keys per thread (thread t owns elements t*EPT .. t*EPT+EPT-1).
template <int EPT, int K, int J>
__device__ __forceinline__ void stage32(unsigned (&x)[EPT], unsigned* lds, int tid) {
  if constexpr (J < EPT) {
#pragma unroll
    for (int i = 0; i < EPT; ++i) {
      if ((i ^ J) > i) {
        const int e = tid * EPT + i;
        const bool desc = (e & K) == 0;
        const unsigned lo = x[i], hi = x[i ^ J];
        const unsigned mx = lo > hi ? lo : hi, mn = lo > hi ? hi : lo;
        x[i] = desc ? mx : mn;
        x[i ^ J] = desc ? mn : mx;
      }
    }
  } else if constexpr (J < EPT * kWave) {
#pragma unroll
    for (int i = 0; i < EPT; ++i) {
      const int e = tid * EPT + i;
      const unsigned p = lane_xor<J / EPT>(x[i]);
      const bool take_max = ((e & J) == 0) == ((e & K) == 0);
      x[i] = take_max ? (x[i] > p ? x[i] : p) : (x[i] > p ? p : x[i]);
    }
  } else {
#pragma unroll
    for (int i = 0; i < EPT; ++i) lds[tid * EPT + i] = x[i];
    __syncthreads();
#pragma unroll
    for (int i = 0; i < EPT; ++i) {
      const int e = tid * EPT + i;
      const unsigned p = lds[e ^ J];
      const bool take_max = ((e & J) == 0) == ((e & K) == 0);
      x[i] = take_max ? (x[i] > p ? x[i] : p) : (x[i] > p ? p : x[i]);
    }
    __syncthreads();
  }
}

template <int EPT, int K, int J>
__device__ __forceinline__ void merge_steps32(unsigned (&x)[EPT], unsigned* lds, int tid) {
  stage32<EPT, K, J>(x, lds, tid);
  if constexpr (J > 1) merge_steps32<EPT, K, J / 2>(x, lds, tid);
}

template <int EPT, int N, int K>
__device__ __forceinline__ void bitonic32(unsigned (&x)[EPT], unsigned* lds, int tid) {
  merge_steps32<EPT, K, K / 2>(x, lds, tid);
  if constexpr (K < N) bitonic32<EPT, N, K * 2>(x, lds, tid);
}

// Descending bitonic sort of 64-bit keys (fallback when a row's score range
// does not fit a 32-bit key); same layout, runtime stage loop.
template <int EPT>
__device__ void bitonic64(unsigned long long (&x)[EPT], int n_sort, unsigned long long* lds) {
  const int tid = threadIdx.x;
  for (int k = 2; k <= n_sort; k <<= 1) {
    for (int j = k >> 1; j > 0; j >>= 1) {
      if (j < EPT) {
#pragma unroll
        for (int i = 0; i < EPT; ++i) {
          const int pi = i ^ j;
          if (pi > i) {
            const int e = tid * EPT + i;
            const bool desc = (e & k) == 0;
            const unsigned long long lo = x[i], hi = x[pi];
            if (desc ? (lo < hi) : (lo > hi)) {
              x[i] = hi;
              x[pi] = lo;
            }
          }
        }
      } else if (j < EPT * kWave) {
        const int lm = j / EPT;
#pragma unroll
        for (int i = 0; i < EPT; ++i) {
          const int e = tid * EPT + i;
          const unsigned long long p = shfl_xor_u64(x[i], lm);
          const bool take_max = ((e & j) == 0) == ((e & k) == 0);
          x[i] = take_max ? (x[i] > p ? x[i] : p) : (x[i] < p ? x[i] : p);
        }
      } else {
#pragma unroll
        for (int i = 0; i < EPT; ++i) lds[tid * EPT + i] = x[i];
        __syncthreads();
#pragma unroll
        for (int i = 0; i < EPT; ++i) {
          const int e = tid * EPT + i;
          const unsigned long long p = lds[e ^ j];
          const bool take_max = ((e & j) == 0) == ((e & k) == 0);
          x[i] = take_max ? (x[i] > p ? x[i] : p) : (x[i] < p ? x[i] : p);
        }
        __syncthreads();
      }
    }
  }
}

// Static-stage descending bitonic sort of N 64-bit keys (N = blockDim.x * EPT):
// every stage's distances are compile-time constants, so the keys stay in
// registers (a runtime stage loop would index the key array dynamically).
template <int M>
__device__ __forceinline__ unsigned long long lane_xor64(unsigned long long v) {
  const unsigned lo = lane_xor<M>((unsigned)v);
  const unsigned hi = lane_xor<M>((unsigned)(v >> 32));
  return ((unsigned long long)hi << 32) | lo;
}

template <int EPT, int K, int J>
__device__ __forceinline__ void stage64(unsigned long long (&x)[EPT], unsigned long long* lds, int tid) {
  if constexpr (J < EPT) {
#pragma unroll
    for (int i = 0; i < EPT; ++i) {
      if ((i ^ J) > i) {
        const int e = tid * EPT + i;
        const bool desc = (e & K) == 0;
        const unsigned long long lo = x[i], hi = x[i ^ J];
        const unsigned long long mx = lo > hi ? lo : hi, mn = lo > hi ? hi : lo;
        x[i] = desc ? mx : mn;
        x[i ^ J] = desc ? mn : mx;
      }
    }
  } else if constexpr (J < EPT * kWave) {
#pragma unroll
    for (int i = 0; i < EPT; ++i) {
      const int e = tid * EPT + i;
      const unsigned long long p = lane_xor64<J / EPT>(x[i]);
      const bool take_max = ((e & J) == 0) == ((e & K) == 0);
      x[i] = take_max ? (x[i] > p ? x[i] : p) : (x[i] > p ? p : x[i]);
    }
  } else {
#pragma unroll
    for (int i = 0; i < EPT; ++i) lds[tid * EPT + i] = x[i];
    __syncthreads();
#pragma unroll
    for (int i = 0; i < EPT; ++i) {
      const int e = tid * EPT + i;
      const unsigned long long p = lds[e ^ J];
      const bool take_max = ((e & J) == 0) == ((e & K) == 0);
      x[i] = take_max ? (x[i] > p ? x[i] : p) : (x[i] > p ? p : x[i]);
    }
    __syncthreads();
  }
}

template <int EPT, int K, int J>
__device__ __forceinline__ void merge_steps64(unsigned long long (&x)[EPT], unsigned long long* lds, int tid) {
  stage64<EPT, K, J>(x, lds, tid);
  if constexpr (J > 1) merge_steps64<EPT, K, J / 2>(x, lds, tid);
}

template <int EPT, int N, int K = 2>
__device__ __forceinline__ void bitonic64s(unsigned long long (&x)[EPT], unsigned long long* lds, int tid) {
  merge_steps64<EPT, K, K / 2>(x, lds, tid);
  if constexpr (K < N) bitonic64s<EPT, N, K * 2>(x, lds, tid);
}

}  // namespace spa
