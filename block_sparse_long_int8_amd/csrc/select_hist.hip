// Sort-free block selection: static top-k and dual top-p by histograms over
// the integer scores, one workgroup per query row.
//
// Same selection rule as the sorting kernel (RTPurbo page §3: keep blocks in
// rank order until the mass reaches p; SpotAttention page §3: reserved sink
// and recency blocks, nucleus over the residual distribution, floor K_min),
// reached the way RTPurbo page §5 suggests for speed: without a sort.
//
// Rank order is (score descending, block index ascending), so the kept set
// of size k is {candidates with score > v} plus the lowest-index candidates
// with score == v, for the threshold score v of rank k.  With integer scores
// the threshold is found exactly by a radix search on d = s_max - s, eight
// bits per level: each level builds a 256-bin LDS histogram of the elements
// whose higher bits match the prefix chosen so far, and one wave scans it.
//
// A histogram word packs (count << 51) | mass, the mass in fixed point with
// 38 fraction bits (each candidate's softmax numerator exp(beta (s - s_max))
// <= 1 is computed in fp32 and converted exactly or to the nearest 2^-38).
// A row has at most 4096 candidates, so both fields add without overflow
// and one 64-bit LDS atomic per element updates both; the sums are exact,
// hence independent of the order of the atomics.  Top-p finds the rank k_p
// at which the cumulative mass first reaches p * Z (Z = total mass, compared
// in fp64), clamps it to [k_min, k_max], and if clamping moved it, searches
// again by count.  Ties at the threshold score take the lowest indices: a
// block-wide prefix count in index order.
#include "spa_internal.h"

namespace spa {

namespace {

constexpr int kThreads = 512;
constexpr int kWaves = kThreads / kWave;
constexpr int kBins = 256;
constexpr int kMaxBlocksH = 4096;
constexpr int kMassBits = 38;
constexpr unsigned long long kOne = 1ull << 51;  // count unit of a histogram word
constexpr unsigned long long kMassMask = kOne - 1;

__device__ __forceinline__ unsigned long long shfl_up_u64(unsigned long long v, int o) {
  const unsigned lo = __shfl_up((unsigned)v, o, kWave);
  const unsigned hi = __shfl_up((unsigned)(v >> 32), o, kWave);
  return ((unsigned long long)hi << 32) | lo;
}
__device__ __forceinline__ unsigned long long shfl_u64(unsigned long long v, int l) {
  const unsigned lo = __shfl((unsigned)v, l, kWave);
  const unsigned hi = __shfl((unsigned)(v >> 32), l, kWave);
  return ((unsigned long long)hi << 32) | lo;
}

struct Pick {
  unsigned long long before;  // packed (count, mass) of the elements ranked before the chosen bin
  unsigned long long in_bin;  // packed (count, mass) of the chosen bin
  int bin;
};

// Wave 0: scan the 256 bins in order (bin 0 = best scores) on top of `base`
// and find the first bin at which the cumulative count (by_mass false) or
// mass (by_mass true) reaches the target.  Also returns the grand total.
__device__ __forceinline__ Pick scan_bins(const unsigned long long* hist, unsigned long long base, bool by_mass,
                                          double target, unsigned long long* total) {
  const int lane = threadIdx.x & (kWave - 1);
  unsigned long long h[4];
  unsigned long long s = 0;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    h[j] = hist[4 * lane + j];
    s += h[j];
  }
  unsigned long long incl = s;
#pragma unroll
  for (int o = 1; o < kWave; o <<= 1) {
    const unsigned long long y = shfl_up_u64(incl, o);
    if (lane >= o) incl += y;
  }
  *total = shfl_u64(incl, kWave - 1);
  unsigned long long run = base + incl - s;
  int jc = -1;
  unsigned long long before = 0;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const unsigned long long after = run + h[j];
    const double v = by_mass ? (double)(after & kMassMask) : (double)(after >> 51);
    if (jc < 0 && v >= target) {
      jc = j;
      before = run;
    }
    run = after;
  }
  const unsigned long long has = __ballot(jc >= 0);
  Pick p;
  if (has == 0ull) {  // target not reached (rounding of p * Z): the last bin
    p.bin = kBins - 1;
    p.before = shfl_u64(run - h[3], kWave - 1);
    p.in_bin = shfl_u64(h[3], kWave - 1);
    return p;
  }
  const int l0 = __ffsll((long long)has) - 1;
  const int j0 = __shfl(jc, l0, kWave);
  p.bin = 4 * l0 + j0;
  p.before = shfl_u64(before, l0);
  unsigned long long hj = h[0];
#pragma unroll
  for (int j = 1; j < 4; ++j) hj = j0 == j ? h[j] : hj;
  p.in_bin = shfl_u64(hj, l0);
  return p;
}

template <int EPT>
__global__ void __launch_bounds__(kThreads) select_hist_kernel(SelectArgs a) {
  __shared__ unsigned long long hist[kBins];
  __shared__ unsigned mask[kMaxBlocksH / 32];
  __shared__ int iscratch[2 * kWaves];
  __shared__ unsigned long long pick_before, pick_inbin;
  __shared__ int pick_bin;

  const int row = blockIdx.x;
  const int b = row / a.M;
  const int i = row - b * a.M;
  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wid = tid / kWave;
  const int nKb = a.nKb;
  const RowRange rr = row_range(a, b, i);
  const int n_cand = rr.n_cand, c0 = rr.c0;

  // candidates tid*EPT .. tid*EPT+EPT-1 (blocks c0 + r), loaded over the whole row
  const int32_t* srow = a.scores + (size_t)row * nKb;
  int sc[EPT];
#pragma unroll
  for (int e = 0; e < EPT; ++e) {
    const int r = tid * EPT + e;
    sc[e] = c0 + r < nKb ? srow[c0 + r] : 0;
  }
  for (int t = tid; t < kMaxBlocksH / 32; t += kThreads) mask[t] = 0u;
  int lmax = INT32_MIN, nlmin = INT32_MIN;
#pragma unroll
  for (int e = 0; e < EPT; ++e)
    if (tid * EPT + e < n_cand) {
      lmax = max(lmax, sc[e]);
      nlmin = max(nlmin, -sc[e]);
    }
  for (int o = 1; o < kWave; o <<= 1) {
    lmax = max(lmax, __shfl_xor(lmax, o, kWave));
    nlmin = max(nlmin, __shfl_xor(nlmin, o, kWave));
  }
  if (lane == 0) {
    iscratch[2 * wid] = lmax;
    iscratch[2 * wid + 1] = nlmin;
  }
  __syncthreads();
  int smax = iscratch[0], nsmin = iscratch[1];
  for (int w = 1; w < kWaves; ++w) {
    smax = max(smax, iscratch[2 * w]);
    nsmin = max(nsmin, iscratch[2 * w + 1]);
  }
  const int smin = -nsmin;

  // d = s_max - s (0 = best), fixed-point masses
  const bool topp = a.mode != 0;
  unsigned dd[EPT];
  unsigned long long word[EPT];
#pragma unroll
  for (int e = 0; e < EPT; ++e) {
    dd[e] = (unsigned)((long long)smax - (long long)sc[e]);
    unsigned long long mf = 0;
    if (topp && tid * EPT + e < n_cand) {
      const float m = expf(a.beta * (float)((long long)sc[e] - smax));
      mf = (unsigned long long)__float2ull_rn(m * 0x1p38f);
    }
    word[e] = kOne | mf;
  }
  const unsigned range = n_cand > 0 ? (unsigned)((long long)smax - (long long)smin) : 0u;
  int levels = 1;
  while (levels < 4 && (range >> (8 * levels)) != 0u) ++levels;

  // Radix search for the rank-k threshold: by_mass finds the first rank whose
  // cumulative mass reaches target, else the rank `target` by count.  Returns
  // the threshold d and the counts/masses before it and at it.
  auto search = [&](bool by_mass, double target, unsigned& d_thr, unsigned long long& before,
                    unsigned long long& at) {
    unsigned prefix = 0;
    unsigned long long base = 0;
    for (int lv = levels - 1; lv >= 0; --lv) {
      const int shift = 8 * lv;
      if (tid < kBins) hist[tid] = 0ull;
      __syncthreads();
#pragma unroll
      for (int e = 0; e < EPT; ++e)
        if (tid * EPT + e < n_cand && (unsigned)((unsigned long long)dd[e] >> (shift + 8)) == prefix)
          atomicAdd(&hist[(dd[e] >> shift) & 255u], word[e]);
      __syncthreads();
      if (wid == 0) {
        unsigned long long tot;
        const Pick pk = scan_bins(hist, base, by_mass, target, &tot);
        if (lane == 0) {
          pick_bin = pk.bin;
          pick_before = pk.before;
          pick_inbin = pk.in_bin;
        }
      }
      __syncthreads();
      prefix = (prefix << 8) | (unsigned)pick_bin;
      base = pick_before;
      at = pick_inbin;
    }
    d_thr = prefix;
    before = base;
  };

  int k_sel = 0;         // candidates kept
  unsigned d_f = 0;      // threshold d of the kept set
  int t_f = 0;           // ties at d_f kept (lowest indices); -1: every candidate
  bool found = false;    // d_f and t_f known
  if (n_cand > 0) {
    if (topp) {
      // Z, the total mass, by a block reduction
      unsigned long long zl = 0;
#pragma unroll
      for (int e = 0; e < EPT; ++e)
        if (tid * EPT + e < n_cand) zl += word[e] & kMassMask;
      for (int o = 1; o < kWave; o <<= 1) zl += (unsigned long long)__shfl_xor((long long)zl, o, kWave);
      if (lane == 0) hist[wid] = zl;  // hist is free until the first search level clears it
      __syncthreads();
      unsigned long long Z = 0;
      for (int w = 0; w < kWaves; ++w) Z += hist[w];
      __syncthreads();
      const double thr = (double)a.p * (double)Z;
      unsigned d1;
      unsigned long long bef, at;
      search(true, thr, d1, bef, at);
      // t: ties at d1 needed for the cumulative mass to reach thr
      const unsigned long long cnt_b = bef >> 51, n_g = at >> 51;
      const unsigned long long m_b = bef & kMassMask, m_g_tot = at & kMassMask;
      const unsigned long long m_g = n_g ? m_g_tot / n_g : 0;  // equal scores, equal masses
      long long t = 1;
      if (m_g > 0) {
        const double need = thr - (double)m_b;
        t = need <= 0.0 ? 1 : (long long)ceil(need / (double)m_g);
      }
      t = t < 1 ? 1 : (t > (long long)n_g ? (long long)n_g : t);
      const int kp = (int)(cnt_b + t);
      k_sel = min(n_cand, max(a.k_min, min(kp, a.k_max)));
      if (k_sel == kp) {
        d_f = d1;
        t_f = (int)t;
        found = true;
      }
    } else {
      k_sel = min(a.k, n_cand);
    }
    if (k_sel > 0 && !found) {
      if (k_sel == n_cand) {
        d_f = range;
        t_f = -1;  // everything
      } else {
        unsigned long long bef, at;
        search(false, (double)k_sel, d_f, bef, at);
        t_f = k_sel - (int)(bef >> 51);
      }
    }
  }

  // ties at d_f in index order: block-wide exclusive count
  int my_ties = 0;
  if (k_sel > 0 && t_f >= 0) {
#pragma unroll
    for (int e = 0; e < EPT; ++e) my_ties += (tid * EPT + e < n_cand && dd[e] == d_f) ? 1 : 0;
  }
  int x = my_ties;
  for (int o = 1; o < kWave; o <<= 1) {
    const int y = __shfl_up(x, o, kWave);
    if (lane >= o) x += y;
  }
  if (lane == kWave - 1) iscratch[wid] = x;
  __syncthreads();
  int tie_rank = x - my_ties;
  for (int w = 0; w < wid; ++w) tie_rank += iscratch[w];

  // mark kept and reserved blocks
  if (k_sel > 0) {
#pragma unroll
    for (int e = 0; e < EPT; ++e) {
      const int r = tid * EPT + e;
      if (r >= n_cand) continue;
      bool keep;
      if (t_f < 0) {
        keep = true;
      } else if (dd[e] < d_f) {
        keep = true;
      } else if (dd[e] == d_f) {
        keep = tie_rank < t_f;
        ++tie_rank;
      } else {
        keep = false;
      }
      if (keep) atomicOr(&mask[(c0 + r) >> 5], 1u << ((c0 + r) & 31));
    }
  }
  for (int j = tid; j < rr.sink_end; j += kThreads) atomicOr(&mask[j >> 5], 1u << (j & 31));
  for (int j = rr.loc0 + tid; j < rr.loc1; j += kThreads) atomicOr(&mask[j >> 5], 1u << (j & 31));
  if (tid == 0 && rr.diag >= 0) atomicOr(&mask[rr.diag >> 5], 1u << (rr.diag & 31));
  __syncthreads();

  // ascending output: wave 0, one 32-block word per lane and pass
  if (wid != 0) return;
  const int nwords = (nKb + 31) >> 5;
  int32_t* out = a.idx + (size_t)row * a.cap;
  int written = 0;
  for (int w0 = 0; w0 < nwords; w0 += kWave) {
    const int wdx = w0 + lane;
    const unsigned m = wdx < nwords ? mask[wdx] : 0u;
    const int c = __popc(m);
    int incl = c;
#pragma unroll
    for (int o = 1; o < kWave; o <<= 1) {
      const int y = __shfl_up(incl, o, kWave);
      if (lane >= o) incl += y;
    }
    int pos = written + incl - c;
    unsigned mm = m;
    while (mm) {
      const int bit = __ffs(mm) - 1;
      mm &= mm - 1;
      if (pos < a.cap) out[pos] = (wdx << 5) + bit;
      ++pos;
    }
    written += __shfl(incl, kWave - 1, kWave);
  }
  for (int t = written + lane; t < a.cap; t += kWave) out[t] = -1;
  if (lane == 0) a.count[row] = min(written, a.cap);
}

}  // namespace

hipError_t launch_select_hist(const SelectArgs& a, hipStream_t s) {
  const int grid = a.B * a.M;
  if (a.nKb <= 512)
    select_hist_kernel<1><<<grid, kThreads, 0, s>>>(a);
  else if (a.nKb <= 1024)
    select_hist_kernel<2><<<grid, kThreads, 0, s>>>(a);
  else if (a.nKb <= 2048)
    select_hist_kernel<4><<<grid, kThreads, 0, s>>>(a);
  else
    select_hist_kernel<8><<<grid, kThreads, 0, s>>>(a);
  return hipGetLastError();
}

}  // namespace spa
