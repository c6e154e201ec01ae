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
// equal scores, by lowest block index; when a row's score range leaves room,
// the key is 32-bit, (score - min) << index_bits | inverted index, which halves
// the compare and exchange work.  Keys are bitonic-sorted in registers (two to
// four per thread): in-thread stages need no exchange, lane strides up to 8 use
// DPP row moves, 16 a swizzle, 32 a permute, and only stages that pair
// different waves go through LDS;
// top-k keeps the first k, top-p turns the sorted scores into fp32 masses
// exp(beta * (s - s_max)) (one hardware exp2 each), scans them in rank order
// and keeps the shortest prefix whose mass reaches p times the total (clamped
// to [k_min, k_max]).  A
// bitmask over block indices then emits the reserved and kept blocks in
// ascending order with a block-wide prefix count.
#include "bitonic.h"
#include "spa_internal.h"

namespace spa {

namespace {

constexpr int kMaxThreads = 1024;
constexpr int kSortThreads = 512;  // keys per thread: max(2, N / 512)
constexpr int kMaxWaves = kMaxThreads / kWave;
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
  const int x = wave_incl_scan_int(v);
  if (lane == kWave - 1) scratch[wid] = x;
  __syncthreads();
  int off = 0, tot = 0;
  const int nw = blockDim.x / kWave;
  for (int w = 0; w < nw; ++w) {
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
  const float x = wave_incl_scan_float(v);
  if (lane == kWave - 1) scratch[wid] = x;
  __syncthreads();
  float off = 0.f, tot = 0.f;
  const int nw = blockDim.x / kWave;
  for (int w = 0; w < nw; ++w) {
    const float s = scratch[w];
    off += (w < wid) ? s : 0.f;
    tot += s;
  }
  __syncthreads();
  *total = tot;
  return off + (x - v);
}

// Block-wide maximum of a and of b (one exchange through LDS).
template <int M>
__device__ __forceinline__ void max2_step(int& a, int& b) {
  a = max(a, (int)lane_xor<M>((unsigned)a));
  b = max(b, (int)lane_xor<M>((unsigned)b));
}
__device__ __forceinline__ void block_max2_int(int& a, int& b, int* scratch) {
  max2_step<1>(a, b);
  max2_step<2>(a, b);
  max2_step<4>(a, b);
  max2_step<8>(a, b);
  max2_step<16>(a, b);
  max2_step<32>(a, b);
  const int wid = threadIdx.x / kWave;
  if ((threadIdx.x & (kWave - 1)) == 0) {
    scratch[2 * wid] = a;
    scratch[2 * wid + 1] = b;
  }
  __syncthreads();
  a = scratch[0];
  b = scratch[1];
  for (int w = 1; w < (int)(blockDim.x / kWave); ++w) {
    a = max(a, scratch[2 * w]);
    b = max(b, scratch[2 * w + 1]);
  }
  __syncthreads();
}

// grid: B*M rows; block N / EPT threads; dynamic LDS: N * 8 bytes.
// Sorts the row's candidates (N = 2^LOG2N >= candidates) in rank order.
template <int LOG2N, bool SCORED>
__global__ void __launch_bounds__(kSortThreads) select_kernel(SelectArgs a) {
  constexpr int N = 1 << LOG2N;
  constexpr int EPT = N > 2 * kSortThreads ? N / kSortThreads : 2;
  extern __shared__ unsigned long long lds64[];
  unsigned* lds32 = reinterpret_cast<unsigned*>(lds64);
  __shared__ unsigned mask[kMaxBlocks / 32];
  __shared__ int iscratch[2 * kMaxWaves];
  __shared__ int kp_s;
  __shared__ float fscratch[kMaxWaves];
  __shared__ int smax_s;

  const int row = blockIdx.x;
  const int b = row / a.M;
  const int i = row - b * a.M;
  const int tid = threadIdx.x;
  const int nKb = a.nKb;

  // valid blocks, reserved ranges and the candidate range [c0, c1)
  const RowRange rr = row_range(a, b, i);
  const int nbv = rr.nbv, sink_end = rr.sink_end, loc0 = rr.loc0, loc1 = rr.loc1, diag = rr.diag, c0 = rr.c0;
  const int n_cand = rr.n_cand;

  int sc[EPT];
  int lmax = INT32_MIN, lmin = INT32_MAX;
  if constexpr (SCORED) {
    // one lane per (block, head): coalesced 16-byte loads, four v_dot4, a
    // shuffle sum over the block's H lanes; scores land in LDS
    __shared__ int4 q4[64];
    __shared__ int w_s[64];
    __shared__ int s_lds[kMaxBlocks];
    for (int t = tid; t < a.H; t += blockDim.x) {
      q4[t] = reinterpret_cast<const int4*>(a.qI)[(size_t)b * a.H + t];
      w_s[t] = a.w[(size_t)b * a.H + t];
    }
    __syncthreads();
    int log2H = 0;
    while ((1 << log2H) < a.H) ++log2H;
    const int H = a.H;
    const int4* krow = reinterpret_cast<const int4*>(a.kI + (size_t)b * nKb * H * 16);
    const int npairs = nbv << log2H;
    constexpr int U = 16;  // loads in flight per thread
    for (int p0 = 0; p0 < npairs; p0 += U * (int)blockDim.x) {
      int4 kv[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int p = p0 + u * blockDim.x + tid;
        kv[u] = p < npairs ? krow[p] : int4{0, 0, 0, 0};
      }
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int p = p0 + u * blockDim.x + tid;
        const int h = p & (H - 1);
        const int4 qv = q4[h];
        int dot = __builtin_amdgcn_sdot4(qv.x, kv[u].x, 0, false);
        dot = __builtin_amdgcn_sdot4(qv.y, kv[u].y, dot, false);
        dot = __builtin_amdgcn_sdot4(qv.z, kv[u].z, dot, false);
        dot = __builtin_amdgcn_sdot4(qv.w, kv[u].w, dot, false);
        int v = p < npairs ? w_s[h] * max(dot, 0) : 0;
        // sum over the block's H neighbouring lanes (lane moves, no LDS round trip)
        if (H >= 2) v += (int)lane_xor<1>((unsigned)v);
        if (H >= 4) v += (int)lane_xor<2>((unsigned)v);
        if (H >= 8) v += (int)lane_xor<4>((unsigned)v);
        if (H >= 16) v += (int)lane_xor<8>((unsigned)v);
        if (H >= 32) v += (int)lane_xor<16>((unsigned)v);
        if (H >= 64) v += (int)lane_xor<32>((unsigned)v);
        if (p < npairs && h == 0) s_lds[p >> log2H] = v;
      }
    }
    __syncthreads();
#pragma unroll
    for (int e = 0; e < EPT; ++e) {
      const int r = tid * EPT + e;
      sc[e] = r < n_cand ? s_lds[c0 + r] : 0;
    }
    if (a.scores_out)
      for (int j = tid; j < nKb; j += blockDim.x) a.scores_out[(size_t)b * nKb + j] = j < nbv ? s_lds[j] : INT32_MIN;
  } else {
    // loaded over the whole row, independent of seq_len, so that both global
    // loads are in flight together; ranks past n_cand are ignored below
    const int32_t* srow = a.scores + (size_t)row * nKb;
#pragma unroll
    for (int e = 0; e < EPT; ++e) {
      const int r = tid * EPT + e;
      sc[e] = c0 + r < nKb ? srow[c0 + r] : 0;
    }
  }
#pragma unroll
  for (int e = 0; e < EPT; ++e) {
    const int r = tid * EPT + e;
    if (r < n_cand) {
      lmax = max(lmax, sc[e]);
      lmin = min(lmin, sc[e]);
    }
  }
  for (int t = tid; t < kMaxBlocks / 32; t += blockDim.x) mask[t] = 0u;
  int smax = lmax, nsmin = lmin == INT32_MIN ? INT32_MAX : -lmin;
  if (tid == 0) kp_s = n_cand;  // ordered before its readers by the barriers below
  block_max2_int(smax, nsmin, iscratch);
  const int smin = -nsmin;
  // 32-bit keys when (score - smin) and the inverted index fit side by side
  int ib = 1;
  while ((1 << ib) <= nKb) ++ib;
  const bool key32 = n_cand > 0 && ib < 32 &&
                     (unsigned long long)((long long)smax - (long long)smin) < (1ull << (32 - ib));

  int rscore[EPT];  // scores in rank order
  int rindex[EPT];  // block indices in rank order
  if (key32) {
    const unsigned imask = (1u << ib) - 1u;
    unsigned x[EPT];
#pragma unroll
    for (int e = 0; e < EPT; ++e) {
      const int r = tid * EPT + e;
      x[e] = r < n_cand ? (((unsigned)(sc[e] - smin) << ib) | (imask - (unsigned)(c0 + r))) : 0u;
    }
    bitonic32<EPT, N, 2>(x, lds32, tid);
#pragma unroll
    for (int e = 0; e < EPT; ++e) {
      rscore[e] = (int)(x[e] >> ib) + smin;
      rindex[e] = (int)(imask - (x[e] & imask));
    }
  } else {
    unsigned long long x[EPT];
#pragma unroll
    for (int e = 0; e < EPT; ++e) {
      const int r = tid * EPT + e;
      x[e] = r < n_cand ? make_key(sc[e], c0 + r) : 0ull;
    }
    int n_sort = 2;
    while (n_sort < n_cand) n_sort <<= 1;
    bitonic64<EPT>(x, n_sort, lds64);
#pragma unroll
    for (int e = 0; e < EPT; ++e) {
      rscore[e] = key_score(x[e]);
      rindex[e] = key_index(x[e]);
    }
  }

  // how many ranked candidates to keep
  int k_sel;
  if (a.mode == 0) {
    k_sel = min(a.k, n_cand);
  } else if (n_cand == 0) {
    k_sel = 0;
  } else {
    // masses exp(beta (s - s_max)) as exp2 of a prescaled argument (one
    // v_exp_f32 each); the cumulative mass is compared with p * Z
    float mass[EPT];
    float local = 0.f;
    const float bl2 = a.beta * 1.4426950408889634f;
#pragma unroll
    for (int e = 0; e < EPT; ++e) {
      const int r = tid * EPT + e;
      mass[e] = r < n_cand ? __builtin_amdgcn_exp2f(bl2 * (float)((long long)rscore[e] - smax)) : 0.f;
      local += mass[e];
    }
    float Z;
    float run = block_excl_scan_float(local, fscratch, &Z);
    const float pz = a.p * Z;
    // k_p = 1 + the first rank at which the cumulative mass reaches p * Z
    // (cumulative mass does not decrease with rank, so this is one rank up to
    // rounding at thread boundaries; the minimum keeps it deterministic; no
    // crossing only if rounding keeps the total below p * Z)
#pragma unroll
    for (int e = 0; e < EPT; ++e) {
      const int r = tid * EPT + e;
      const bool before = run < pz;
      run += mass[e];
      if (r < n_cand && before && !(run < pz)) atomicMin(&kp_s, r + 1);
    }
    __syncthreads();
    const int kp = min(kp_s, n_cand);
    k_sel = min(n_cand, max(a.k_min, min(kp, a.k_max)));
  }

  // mark kept and reserved blocks
#pragma unroll
  for (int e = 0; e < EPT; ++e) {
    const int r = tid * EPT + e;
    if (r < k_sel) atomicOr(&mask[rindex[e] >> 5], 1u << (rindex[e] & 31));
  }
  for (int j = tid; j < sink_end; j += blockDim.x) atomicOr(&mask[j >> 5], 1u << (j & 31));
  for (int j = loc0 + tid; j < loc1; j += blockDim.x) atomicOr(&mask[j >> 5], 1u << (j & 31));
  if (tid == 0 && diag >= 0) atomicOr(&mask[diag >> 5], 1u << (diag & 31));
  __syncthreads();

  // ascending output: one 32-block word per lane of wave 0 (rows of up to
  // 2048 blocks), else one word per thread
  const int nwords = (nKb + 31) >> 5;
  int32_t* out = a.idx + (size_t)row * a.cap;
  if (nwords <= kWave) {
    if (tid >= kWave) return;
    const unsigned m = tid < nwords ? mask[tid] : 0u;
    const int c = __popc(m);
    const int incl = wave_incl_scan_int(c);
    const int written = __builtin_amdgcn_readlane(incl, kWave - 1);
    int pos = incl - c;
    unsigned mm = m;
    while (mm) {
      const int bit = __ffs(mm) - 1;
      mm &= mm - 1;
      if (pos < a.cap) out[pos] = (tid << 5) + bit;
      ++pos;
    }
    for (int t = written + tid; t < a.cap; t += kWave) out[t] = -1;
    if (tid == 0) a.count[row] = min(written, a.cap);
    return;
  }
  int written = 0;
  for (int w0 = 0; w0 < nwords; w0 += blockDim.x) {
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
  for (int t = written + tid; t < a.cap; t += blockDim.x) out[t] = -1;
  if (tid == 0) a.count[row] = min(written, a.cap);
}

}  // namespace

int select_max_blocks() { return kMaxBlocks; }

hipError_t launch_select(const SelectArgs& a, hipStream_t s) {
  // N: the smallest power of two >= every row's candidate count (>= 128)
  int log2n = 7;
  while ((1 << log2n) < a.nKb) ++log2n;
  const int n = 1 << log2n;
  const int ept = n > 2 * kSortThreads ? n / kSortThreads : 2;
  const int threads = n / ept;
  const size_t lds = (size_t)n * sizeof(unsigned long long);
  const int grid = a.B * a.M;
  const bool scored = a.scores == nullptr;
#define SPA_SEL_CASE(L)                                                   \
  case L:                                                                 \
    if (scored)                                                           \
      select_kernel<L, true><<<grid, threads, lds, s>>>(a);               \
    else                                                                  \
      select_kernel<L, false><<<grid, threads, lds, s>>>(a);              \
    break;
  switch (log2n) {
    SPA_SEL_CASE(7)
    SPA_SEL_CASE(8)
    SPA_SEL_CASE(9)
    SPA_SEL_CASE(10)
    SPA_SEL_CASE(11)
    default:
      if (scored)
        select_kernel<12, true><<<grid, threads, lds, s>>>(a);
      else
        select_kernel<12, false><<<grid, threads, lds, s>>>(a);
      break;
  }
#undef SPA_SEL_CASE
  return hipGetLastError();
}

}  // namespace spa
