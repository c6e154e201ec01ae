// Global key importance from a proxy query block, and the importance-sorted
// segment permutation.
//
// PBS-Attn page, §3 "Permutación de Claves Basada en Importancia Global": the
// last query block stands in for all queries; the mean of its attention
// probabilities gives one importance per key; inside each permutation segment
// (§2) the keys are ordered by descending importance, so the keys that draw
// the most attention fill the segment's first blocks.
//
// Work: the proxy block is at most 64 queries per head, so one wave holds a
// head's whole proxy block as MFMA operands and streams the key rows of its KV
// head.  The softmax needs each query row's maximum and sum before any
// probability is final, so the keys are read twice:
//   pass 1  S^T = K.Q^T (v_mfma_f32_32x32x16_bf16, K rows as the A operand):
//           a lane's accumulators hold 16 keys of one query, so the running
//           maximum and sum per query need no cross-lane work;
//   merge   per (head, query) the chunk statistics combine into the log-sum
//           c = m + log2(l) (one small kernel);
//   pass 2  S = Q.K^T (the same registers with the operands swapped): a lane
//           holds 16 queries of one key, so exp2(x - c) summed over the lane
//           plus its partner lane is that key's probability mass over the
//           head's proxy block, written once per (head, key);
//   sort    per (sequence, segment): the heads' masses are added in head order
//           and divided by Hq * n (the importance), then the segment's keys are
//           sorted by a 64-bit key (~bits(importance), position) with a
//           bitonic network in LDS; keys at or past seq_len sort last in their
//           own order.
// The dot product over d is invariant under any permutation of d applied to
// both operands, so lane half `hi` takes the contiguous d range
// [64*hi + 8*ks, +8) at k-step ks: each lane reads one contiguous half row.
#include "bitonic.h"
#include "spa_internal.h"

namespace spa {

namespace {

typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kD = 128;        // head dimension
constexpr int kProxyMax = 64;  // proxy queries per head (two 32-row MFMA halves)
constexpr int kImpChunk = 1024;  // keys per workgroup and head
constexpr int kImpTile = 32;     // keys per MFMA tile
constexpr int kSortThreads = 1024;
constexpr int kSortEPT = 4;
constexpr int kSortMax = kSortThreads * kSortEPT;  // longest segment the sort handles (4096)

__device__ __forceinline__ bf16x8 as_bf16x8(const uint4& u) { return __builtin_bit_cast(bf16x8, u); }

template <int N>
struct IC {
  static constexpr int value = N;
};

__host__ __device__ inline size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

struct ImpWs {
  float2* stats;  // [B, Hq, nch, 64] running (max, sum) per chunk, log2 domain
  float* cval;    // [B, Hq, 64] log2-sum-exp per proxy query (+inf for padding rows)
  float* part;    // [B, Hq/W, T] probability mass of each key per workgroup head group
};

__host__ __device__ inline size_t imp_ws_parts(int B, int Hq, int T, size_t* off_c, size_t* off_p) {
  const int nch = (T + kImpChunk - 1) / kImpChunk;
  const size_t s = align256((size_t)B * Hq * nch * kProxyMax * sizeof(float2));
  const size_t c = align256((size_t)B * Hq * kProxyMax * sizeof(float));
  const size_t p = align256((size_t)B * Hq * T * sizeof(float));
  if (off_c) *off_c = s;
  if (off_p) *off_p = s + c;
  return s + c + p;
}

__device__ __forceinline__ ImpWs imp_ws(void* ws, int B, int Hq, int T) {
  size_t oc, op;
  imp_ws_parts(B, Hq, T, &oc, &op);
  char* base = static_cast<char*>(ws);
  return ImpWs{reinterpret_cast<float2*>(base), reinterpret_cast<float*>(base + oc),
               reinterpret_cast<float*>(base + op)};
}

struct ImpArgs {
  const uint16_t* q;  // [B, Hq, T, 128] bf16
  const uint16_t* k;  // [B, Hkv, T, 128] bf16
  int B, Hq, Hkv, T;
  const int32_t* seq_len;  // [B] or null (= T)
  int proxy;
  float scale_log2;  // scale * log2(e)
  int seg;
  float* imp;     // [B, T]
  int32_t* perm;  // [B, T]
  void* ws;
};

// The wave's proxy block as MFMA operands: qf[half][ks] holds query row
// 32*half + (lane & 31), d range [64*hi + 8*ks, +8); rows at or past n are 0.
__device__ __forceinline__ void load_proxy(const ImpArgs& a, int b, int h, int u0, int n, bf16x8 (&qf)[2][8]) {
  const int lane = threadIdx.x & (kWave - 1);
  const int l32 = lane & 31, hi = lane >> 5;
#pragma unroll
  for (int half = 0; half < 2; ++half) {
    const int row = 32 * half + l32;
    const uint16_t* src = a.q + (((size_t)b * a.Hq + h) * a.T + (size_t)(u0 + max(min(row, n - 1), 0))) * kD + 64 * hi;
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) {
      const uint4 v = row < n ? *reinterpret_cast<const uint4*>(src + 8 * ks) : uint4{0, 0, 0, 0};
      qf[half][ks] = as_bf16x8(v);
    }
  }
}

// LDS byte offset of 16-byte chunk c (0..15) of tile row r: the chunk index is
// XOR-swizzled with the row, so the 16 rows one quarter-wave reads at a fixed
// chunk fall on 16 different chunk slots (all 64 banks, no conflict).
__device__ __forceinline__ int tile_off(int r, int c) { return r * 256 + 16 * (c ^ (r & 15)); }

// W waves per workgroup share one KV head; the 32-row key tile (8 KB) is
// loaded once per workgroup, U = 8 / W 16-byte units per thread, with D tiles
// in flight in a register ring (at most 32 VGPRs), and staged through LDS.
template <int W>
struct Stage {
  static constexpr int U = 8 / W;
  static constexpr int D = W == 1 ? 1 : 2;
};

// Issue the loads of the tile at tok0 (rows at or past c1 read row c1 - 1).
template <int W>
__device__ __forceinline__ void stage_load(const uint16_t* kbase, int tok0, int c1, u32x4 (&r)[Stage<W>::U]) {
#pragma unroll
  for (int u = 0; u < Stage<W>::U; ++u) {
    const int e = u * (64 * W) + (int)threadIdx.x;  // 16-byte unit of the tile
    const int row = e >> 4, c = e & 15;
    r[u] = *reinterpret_cast<const u32x4*>(kbase + (size_t)min(tok0 + row, c1 - 1) * kD + 8 * c);
  }
}

template <int W>
__device__ __forceinline__ void stage_store(char* buf, const u32x4 (&r)[Stage<W>::U]) {
#pragma unroll
  for (int u = 0; u < Stage<W>::U; ++u) {
    const int e = u * (64 * W) + (int)threadIdx.x;
    *reinterpret_cast<u32x4*>(buf + tile_off(e >> 4, e & 15)) = r[u];
  }
}

// This lane's key operands of the staged tile: row l32, d range [64*hi + 8*ks, +8);
// rows at or past c1 read as 0.
__device__ __forceinline__ void tile_operands(const char* buf, int tok0, int c1, bf16x8 (&kf)[8]) {
  const int lane = threadIdx.x & (kWave - 1);
  const int l32 = lane & 31, hi = lane >> 5;
  const bool in = tok0 + l32 < c1;
#pragma unroll
  for (int ks = 0; ks < 8; ++ks) {
    const uint4 v = *reinterpret_cast<const uint4*>(buf + tile_off(l32, 8 * hi + ks));
    kf[ks] = as_bf16x8(in ? v : uint4{0, 0, 0, 0});
  }
}

// grid (nch, Hq / W, B), block 64*W: wave w handles query head W*blockIdx.y + w
// over keys [chunk*kImpChunk, +kImpChunk) of its sequence; the W heads share
// one KV head (W divides Hq / Hkv).
//   PASS 1 writes the per-chunk (max, sum) of every proxy query;
//   PASS 2 merges them into c = max + log2(sum) per query, then writes, per
//          key, the probability mass summed over the workgroup's W heads and
//          all proxy queries into part[b, blockIdx.y, t].
template <int PASS, int W>
__global__ void __launch_bounds__(64 * W) importance_pass_kernel(ImpArgs a) {
  constexpr int D = Stage<W>::D;
  __shared__ __attribute__((aligned(16))) char kbuf[2][kImpTile * 256];
  __shared__ float red[2][W][kImpTile];
  __shared__ float cs[W][kProxyMax];
  const int chunk = blockIdx.x, b = blockIdx.z;
  const int wv = (int)(threadIdx.x >> 6);
  const int h = blockIdx.y * W + wv;
  const int lane = threadIdx.x & (kWave - 1);
  const int l32 = lane & 31, hi = lane >> 5;
  const int L = a.seq_len ? a.seq_len[b] : a.T;
  const int n = min(a.proxy, L);
  const int u0 = L - n;
  const int g = h / (a.Hq / a.Hkv);
  const int nch = gridDim.x;
  ImpWs ws = imp_ws(a.ws, a.B, a.Hq, a.T);
  const int c0 = chunk * kImpChunk;
  const int c1 = min(c0 + kImpChunk, L);
  const int ntiles = c1 > c0 ? (c1 - c0 + kImpTile - 1) / kImpTile : 0;  // same for the whole workgroup
  const uint16_t* kbase = a.k + ((size_t)b * a.Hkv + g) * (size_t)a.T * kD;

  bf16x8 qf[2][8];
  load_proxy(a, b, h, u0, n, qf);

  // PASS 1 state: lane holds query j = 32*half + l32 over keys i = 8*(v/4) + 4*hi + v%4
  float m[2] = {-INFINITY, -INFINITY}, l[2] = {0.f, 0.f};
  // PASS 2 state: c of the queries i = 32*half + 8*(v/4) + 4*hi + v%4 this lane meets
  float creg[2][16];
  if constexpr (PASS == 2) {
    // merge this head's chunk statistics (lane j = query j), chunk order
    const int nval = (L + kImpChunk - 1) / kImpChunk;
    const float2* st = ws.stats + ((size_t)b * a.Hq + h) * nch * kProxyMax + lane;
    float M = -INFINITY, S = 0.f;
    for (int c = 0; c < nval; c += 8) {
      float2 ml[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) ml[e] = c + e < nval ? st[(size_t)(c + e) * kProxyMax] : float2{-INFINITY, 0.f};
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        if (ml[e].x == -INFINITY) continue;
        const float Mn = fmaxf(M, ml[e].x);
        S = S * __builtin_amdgcn_exp2f(M - Mn) + ml[e].y * __builtin_amdgcn_exp2f(ml[e].x - Mn);
        M = Mn;
      }
    }
    // padding rows get +inf, so their terms below are exp2(-inf) = 0
    cs[wv][lane] = (lane < n && S > 0.f) ? M + __log2f(S) : INFINITY;
    __syncthreads();
#pragma unroll
    for (int half = 0; half < 2; ++half)
#pragma unroll
      for (int v = 0; v < 16; ++v) creg[half][v] = cs[wv][32 * half + 8 * (v >> 2) + 4 * hi + (v & 3)];
  }
  float* part = ws.part + ((size_t)b * gridDim.y + blockIdx.y) * a.T;

  // prologue: tiles 0 .. D-1 in flight, tile 0 staged, tile D refilling slot 0
  u32x4 ring[D][Stage<W>::U];
  if (0 < ntiles) stage_load<W>(kbase, c0, c1, ring[0]);
  if constexpr (D > 1) {
    if (1 < ntiles) stage_load<W>(kbase, c0 + kImpTile, c1, ring[1]);
  }
  if (ntiles > 0) {
    stage_store<W>(kbuf[0], ring[0]);
    if (D < ntiles) stage_load<W>(kbase, c0 + D * kImpTile, c1, ring[0]);
  }
  __syncthreads();

  // one tile: compute on kbuf[i & 1], stage tile i + 1 from ring slot NXT into
  // the other buffer and refill that slot with tile i + 1 + D; the slot is a
  // compile-time constant so the ring stays in registers
  auto tile = [&](int i, auto nxt_slot) __attribute__((always_inline)) {
    constexpr int NXT = decltype(nxt_slot)::value;
    if (i >= ntiles) return;  // uniform over the workgroup
    const int tok0 = c0 + i * kImpTile;
    const char* cur = kbuf[i & 1];
    bf16x8 kf[8];
    tile_operands(cur, tok0, c1, kf);
    f32x16 s[2] = {f32x16{}, f32x16{}};
    // every key of the tile is valid and visible to every proxy query (all but
    // the last tiles of a sequence): no per-element mask
    const bool full = tok0 + kImpTile <= c1 && tok0 + kImpTile - 1 <= u0;
    if constexpr (PASS == 1) {
#pragma unroll
      for (int ks = 0; ks < 8; ++ks) {
        s[0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[ks], qf[0][ks], s[0], 0, 0, 0);
        s[1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[ks], qf[1][ks], s[1], 0, 0, 0);
      }
      if (full) {
        // scale > 0: the largest logit comes from the largest raw dot product
#pragma unroll
        for (int half = 0; half < 2; ++half) {
          float smax = s[half][0];
#pragma unroll
          for (int v = 1; v < 16; ++v) smax = fmaxf(smax, s[half][v]);
          const float mn = fmaxf(m[half], smax * a.scale_log2);
          float sum = 0.f;
#pragma unroll
          for (int v = 0; v < 16; ++v) sum += __builtin_amdgcn_exp2f(__builtin_fmaf(s[half][v], a.scale_log2, -mn));
          l[half] = l[half] * __builtin_amdgcn_exp2f(m[half] - mn) + sum;
          m[half] = mn;
        }
      } else {
#pragma unroll
      for (int half = 0; half < 2; ++half) {
        const int qpos = u0 + 32 * half + l32;
        float x[16];
        float tmax = -INFINITY;
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int t = tok0 + 8 * (v >> 2) + 4 * hi + (v & 3);
          x[v] = (t < c1 && t <= qpos) ? s[half][v] * a.scale_log2 : -INFINITY;
          tmax = fmaxf(tmax, x[v]);
        }
        const float mn = fmaxf(m[half], tmax);
        if (mn != -INFINITY) {
          float sum = 0.f;
#pragma unroll
          for (int v = 0; v < 16; ++v) sum += __builtin_amdgcn_exp2f(x[v] - mn);
          l[half] = l[half] * __builtin_amdgcn_exp2f(m[half] - mn) + sum;
          m[half] = mn;
        }
      }
      }
    } else {
#pragma unroll
      for (int ks = 0; ks < 8; ++ks) {
        s[0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qf[0][ks], kf[ks], s[0], 0, 0, 0);
        s[1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qf[1][ks], kf[ks], s[1], 0, 0, 0);
      }
      const int t = tok0 + l32;
      float psum = 0.f;
      if (full) {
#pragma unroll
        for (int half = 0; half < 2; ++half)
#pragma unroll
          for (int v = 0; v < 16; ++v)
            psum += __builtin_amdgcn_exp2f(__builtin_fmaf(s[half][v], a.scale_log2, -creg[half][v]));
      } else {
#pragma unroll
        for (int half = 0; half < 2; ++half)
#pragma unroll
          for (int v = 0; v < 16; ++v) {
            const int qpos = u0 + 32 * half + 8 * (v >> 2) + 4 * hi + (v & 3);
            const float e = __builtin_amdgcn_exp2f(s[half][v] * a.scale_log2 - creg[half][v]);
            psum += t <= qpos ? e : 0.f;
          }
      }
      psum += lane_swap_f<32>(psum);
      if (hi == 0) red[i & 1][wv][l32] = psum;
      // the previous tile's per-head sums are complete (barrier below it):
      // add them in head order and write once for the workgroup
      if (i > 0 && wv == 0 && hi == 0) {
        float v = 0.f;
#pragma unroll
        for (int w = 0; w < W; ++w) v += red[(i - 1) & 1][w][l32];
        part[tok0 - kImpTile + l32] = v;
      }
    }
    if (i + 1 < ntiles) {
      stage_store<W>(kbuf[(i + 1) & 1], ring[NXT]);
      if (i + 1 + D < ntiles) stage_load<W>(kbase, c0 + (i + 1 + D) * kImpTile, c1, ring[NXT]);
    }
    __syncthreads();
  };
  for (int base = 0; base < ntiles; base += D) {
    tile(base, IC<1 % D>{});
    if constexpr (D > 1) tile(base + 1, IC<2 % D>{});
  }

  if constexpr (PASS == 1) {
#pragma unroll
    for (int half = 0; half < 2; ++half) {
      // the partner lane (lane ^ 32) covered the other keys of the same query
      const float m2 = lane_swap_f<32>(m[half]);
      const float l2 = lane_swap_f<32>(l[half]);
      const float M = fmaxf(m[half], m2);
      const float S = M == -INFINITY ? 0.f
                                     : l[half] * __builtin_amdgcn_exp2f(m[half] - M) +
                                           l2 * __builtin_amdgcn_exp2f(m2 - M);
      if (hi == 0)
        ws.stats[(((size_t)b * a.Hq + h) * nch + chunk) * kProxyMax + 32 * half + l32] = float2{M, S};
    }
  } else if (ntiles > 0 && wv == 0 && hi == 0) {
    const int tp = c0 + (ntiles - 1) * kImpTile + l32;
    float v = 0.f;
#pragma unroll
    for (int w = 0; w < W; ++w) v += red[(ntiles - 1) & 1][w][l32];
    if (tp < c1) part[tp] = v;
  }
}

// grid (ceil(T/256), B), block 256: importance of key t = the part rows added
// in order, divided by Hq * n (0 at or past seq_len).
__global__ void __launch_bounds__(256) importance_sum_kernel(ImpArgs a, int nparts) {
  const int b = blockIdx.y;
  const int t = blockIdx.x * 256 + (int)threadIdx.x;
  if (t >= a.T) return;
  const int L = a.seq_len ? a.seq_len[b] : a.T;
  float v = 0.f;
  if (t < L) {
    const float* part = imp_ws(a.ws, a.B, a.Hq, a.T).part + (size_t)b * nparts * a.T + t;
    for (int p = 0; p < nparts; ++p) v += part[(size_t)p * a.T];
    v = v / ((float)a.Hq * (float)min(a.proxy, L));
  }
  a.imp[(size_t)b * a.T + t] = v;
}

// grid (ceil(T/seg), B), block kSortThreads (1024, four keys each): a
// descending register bitonic sort of the segment's 64-bit keys
// (bits(importance) << 32) | ~position -- the largest importance first, equal
// importances by lower position, keys at or past seq_len (importance part 0)
// after every valid key and in their own order, padding (key 0, position all
// ones) last -- then the permutation.
__global__ void __launch_bounds__(kSortThreads) importance_sort_kernel(ImpArgs a) {
  __shared__ unsigned long long lds[kSortMax];
  const int b = blockIdx.y;
  const int s0 = blockIdx.x * a.seg;
  const int len = min(a.seg, a.T - s0);
  const int L = a.seq_len ? a.seq_len[b] : a.T;
  const float* imp = a.imp + (size_t)b * a.T + s0;
  unsigned long long x[kSortEPT];
#pragma unroll
  for (int i = 0; i < kSortEPT; ++i) {
    const int e = (int)threadIdx.x * kSortEPT + i;
    const int t = s0 + e;
    x[i] = e < len ? ((unsigned long long)(t < L ? __float_as_uint(imp[e]) : 0u) << 32) | (unsigned)~t : 0ull;
  }
  bitonic64s<kSortEPT, kSortMax>(x, lds, (int)threadIdx.x);
#pragma unroll
  for (int i = 0; i < kSortEPT; ++i) {
    const int e = (int)threadIdx.x * kSortEPT + i;
    if (e < len) a.perm[(size_t)b * a.T + s0 + e] = (int32_t)~(unsigned)x[i];
  }
}

}  // namespace

size_t importance_ws_bytes(int B, int Hq, int T) { return imp_ws_parts(B, Hq, T, nullptr, nullptr); }

int importance_max_proxy() { return kProxyMax; }
int importance_max_seg() { return kSortMax; }

hipError_t launch_importance(const void* q, const void* k, int B, int Hq, int Hkv, int T,
                             const int32_t* seq_len, int proxy, float scale, int seg, float* imp,
                             int32_t* perm, void* ws, hipStream_t s) {
  ImpArgs a;
  a.q = static_cast<const uint16_t*>(q);
  a.k = static_cast<const uint16_t*>(k);
  a.B = B;
  a.Hq = Hq;
  a.Hkv = Hkv;
  a.T = T;
  a.seq_len = seq_len;
  a.proxy = proxy;
  a.scale_log2 = scale * 1.4426950408889634f;
  a.seg = seg;
  a.imp = imp;
  a.perm = perm;
  a.ws = ws;
  const int nch = (T + kImpChunk - 1) / kImpChunk;
  const int G = Hq / Hkv;
  const int W = G % 4 == 0 ? 4 : (G % 2 == 0 ? 2 : 1);  // waves per workgroup, all on one KV head
  const dim3 grid(nch, Hq / W, B);
  hipError_t e;
  if (W == 4) {
    importance_pass_kernel<1, 4><<<grid, 256, 0, s>>>(a);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    importance_pass_kernel<2, 4><<<grid, 256, 0, s>>>(a);
  } else if (W == 2) {
    importance_pass_kernel<1, 2><<<grid, 128, 0, s>>>(a);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    importance_pass_kernel<2, 2><<<grid, 128, 0, s>>>(a);
  } else {
    importance_pass_kernel<1, 1><<<grid, 64, 0, s>>>(a);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    importance_pass_kernel<2, 1><<<grid, 64, 0, s>>>(a);
  }
  if ((e = hipGetLastError()) != hipSuccess) return e;
  importance_sum_kernel<<<dim3((T + 255) / 256, B), 256, 0, s>>>(a, Hq / W);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  importance_sort_kernel<<<dim3((T + seg - 1) / seg, B), kSortThreads, 0, s>>>(a);
  return hipGetLastError();
}

}  // namespace spa
