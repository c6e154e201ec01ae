// Block selection: static top-k and dual top-p, one workgroup per query row.
//
// RTPurbo page §3 (top-k budget vs. top-p: accumulate mass until it reaches
// p), SpotAttention page §3 (sink prefix and recency suffix always kept; the
// nucleus runs over the residual distribution of the other blocks; floor
// K_min), HGA page "Mecanismo Central" (current, sink and local chunks always
// visible).
//
// A row's candidates are packed into unique 64-bit keys
//     ((score ^ 0x80000000) << 32) | ~index
// so that sorting keys in descending order ranks by score descending and, on
// equal scores, by lowest block index.  The keys are bitonic-sorted in LDS;
// top-k keeps the first k, top-p turns the sorted scores into fp32 masses
// exp(beta * (s - s_max)), scans them in rank order and keeps the shortest
// prefix whose normalised mass reaches p (clamped to [k_min, k_max]).  A
// bitmask over block indices then emits the reserved and kept blocks in
// ascending order with a block-wide prefix count.
#include "spa_internal.h"

namespace spa {

namespace {

constexpr int kSelThreads = 512;
constexpr int kSelWaves = kSelThreads / kWave;
constexpr int kMaxBlocks = 4096;

__device__ __forceinline__ unsigned long long make_key(int score, int j) {
  return ((unsigned long long)((unsigned)score ^ 0x80000000u) << 32) | (unsigned)(~(unsigned)j);
}
__device__ __forceinline__ int key_score(unsigned long long k) {
  return (int)((unsigned)(k >> 32) ^ 0x80000000u);
}
__device__ __forceinline__ int key_index(unsigned long long k) { return (int)(~(unsigned)k); }

// Exclusive prefix sum of one int per thread across the workgroup; returns
// the exclusive value and writes the total to *total.
__device__ int block_excl_scan_int(int v, int* scratch, int* total) {
  const int lane = threadIdx.x & (kWave - 1);
  const int wid = threadIdx.x / kWave;
  int x = v;
#pragma unroll
  for (int o = 1; o < kWave; o <<= 1) {
    int y = __shfl_up(x, o, kWave);
    if (lane >= o) x += y;
  }
  if (lane == kWave - 1) scratch[wid] = x;
  __syncthreads();
  int off = 0, tot = 0;
#pragma unroll
  for (int w = 0; w < kSelWaves; ++w) {
    const int s = scratch[w];
    off += (w < wid) ? s : 0;
    tot += s;
  }
  __syncthreads();
  *total = tot;
  return off + x - v;
}

__device__ float block_excl_scan_float(float v, float* scratch, float* total) {
  const int lane = threadIdx.x & (kWave - 1);
  const int wid = threadIdx.x / kWave;
  float x = v;
#pragma unroll
  for (int o = 1; o < kWave; o <<= 1) {
    float y = __shfl_up(x, o, kWave);
    if (lane >= o) x += y;
  }
  if (lane == kWave - 1) scratch[wid] = x;
  __syncthreads();
  float off = 0.f, tot = 0.f;
#pragma unroll
  for (int w = 0; w < kSelWaves; ++w) {
    const float s = scratch[w];
    off += (w < wid) ? s : 0.f;
    tot += s;
  }
  __syncthreads();
  *total = tot;
  return off + (x - v);
}

// grid: B*M rows; block kSelThreads; dynamic LDS: n_pad * 8 bytes of keys.
__global__ void __launch_bounds__(kSelThreads) select_kernel(SelectArgs a) {
  extern __shared__ unsigned long long keys[];
  __shared__ unsigned mask[kMaxBlocks / 32];
  __shared__ int iscratch[kSelWaves];
  __shared__ float fscratch[kSelWaves];

  const int row = blockIdx.x;
  const int b = row / a.M;
  const int i = row - b * a.M;
  const int tid = threadIdx.x;
  const int nKb = a.nKb;

  // valid blocks, reserved ranges and the candidate range [c0, c1)
  const int nbv = a.seq_len ? min(nKb, (a.seq_len[b] + a.blk - 1) / a.blk) : nKb;
  int e, sink_end, loc0, loc1, diag, c0, c1;
  if (!a.prefill) {
    e = nbv;
    sink_end = min(a.n_sink, e);
    loc0 = max(0, e - a.n_local);
    loc1 = e;
    diag = -1;
    c0 = a.n_sink;
    c1 = e - a.n_local;
  } else {
    const int qa = a.q_blk0 + i;
    e = min(qa, nbv);
    sink_end = min(min(a.n_sink, qa + 1), nKb);
    loc0 = max(0, qa - a.n_local);
    loc1 = min(qa, nKb);
    diag = qa < nKb ? qa : -1;
    c0 = a.n_sink;
    c1 = min(e, qa - a.n_local);
  }
  const int n_cand = max(0, c1 - c0);
  int n_pad = 1;
  while (n_pad < n_cand) n_pad <<= 1;

  const int32_t* srow = a.scores + (size_t)row * nKb;
  for (int t = tid; t < n_pad; t += kSelThreads)
    keys[t] = t < n_cand ? make_key(srow[c0 + t], c0 + t) : 0ull;
  for (int t = tid; t < kMaxBlocks / 32; t += kSelThreads) mask[t] = 0u;
  __syncthreads();

  // bitonic sort, descending
  for (int kk = 2; kk <= n_pad; kk <<= 1) {
    for (int jj = kk >> 1; jj > 0; jj >>= 1) {
      for (int t = tid; t < (n_pad >> 1); t += kSelThreads) {
        const int lo = 2 * jj * (t / jj) + (t % jj);
        const int hi = lo + jj;
        const unsigned long long x = keys[lo], y = keys[hi];
        const bool desc = (lo & kk) == 0;
        if (desc ? (x < y) : (x > y)) {
          keys[lo] = y;
          keys[hi] = x;
        }
      }
      __syncthreads();
    }
  }

  // how many ranked candidates to keep
  int k_sel;
  if (a.mode == 0) {
    k_sel = min(a.k, n_cand);
  } else if (n_cand == 0) {
    k_sel = 0;
  } else {
    // each thread owns a contiguous run of ranks
    const int per = (n_cand + kSelThreads - 1) / kSelThreads;
    const int r0 = tid * per;
    const int r1 = min(n_cand, r0 + per);
    const int smax = key_score(keys[0]);
    float local = 0.f;
    for (int t = r0; t < r1; ++t) local += expf(a.beta * (float)(key_score(keys[t]) - smax));
    float Z;
    const float off = block_excl_scan_float(local, fscratch, &Z);
    // count ranks whose normalised cumulative mass is still below p
    float run = off;
    int below = 0;
    for (int t = r0; t < r1; ++t) {
      run += expf(a.beta * (float)(key_score(keys[t]) - smax));
      below += (run / Z < a.p) ? 1 : 0;
    }
    int n_below;
    block_excl_scan_int(below, iscratch, &n_below);
    const int kp = min(n_below + 1, n_cand);
    k_sel = min(n_cand, max(a.k_min, min(kp, a.k_max)));
  }

  // mark reserved and kept blocks
  for (int t = tid; t < k_sel; t += kSelThreads) {
    const int j = key_index(keys[t]);
    atomicOr(&mask[j >> 5], 1u << (j & 31));
  }
  for (int j = tid; j < sink_end; j += kSelThreads) atomicOr(&mask[j >> 5], 1u << (j & 31));
  for (int j = loc0 + tid; j < loc1; j += kSelThreads) atomicOr(&mask[j >> 5], 1u << (j & 31));
  if (tid == 0 && diag >= 0) atomicOr(&mask[diag >> 5], 1u << (diag & 31));
  __syncthreads();

  // ascending output: one 32-block word per thread
  const int nwords = (nKb + 31) >> 5;
  int32_t* out = a.idx + (size_t)row * a.cap;
  int written = 0;
  for (int w0 = 0; w0 < nwords; w0 += kSelThreads) {
    const int wdx = w0 + tid;
    const unsigned m = wdx < nwords ? mask[wdx] : 0u;
    int tot;
    int pos = written + block_excl_scan_int(__popc(m), iscratch, &tot);
    unsigned mm = m;
    while (mm) {
      const int bit = __ffs(mm) - 1;
      mm &= mm - 1;
      if (pos < a.cap) out[pos] = (wdx << 5) + bit;
      ++pos;
    }
    written += tot;
  }
  for (int t = written + tid; t < a.cap; t += kSelThreads) out[t] = -1;
  if (tid == 0) a.count[row] = min(written, a.cap);
}

}  // namespace

int select_max_blocks() { return kMaxBlocks; }

hipError_t launch_select(const SelectArgs& a, hipStream_t s) {
  // LDS for keys sized by the widest candidate range any row can have
  int n_pad = 1;
  while (n_pad < a.nKb) n_pad <<= 1;
  const size_t lds = (size_t)n_pad * sizeof(unsigned long long);
  select_kernel<<<a.B * a.M, kSelThreads, lds, s>>>(a);
  return hipGetLastError();
}

}  // namespace spa
