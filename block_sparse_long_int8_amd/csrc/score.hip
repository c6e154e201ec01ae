// Indexer scoring kernels.
//
// Score of a query row against key block t (SpotAttention page, §1
// "Arquitectura del Selector"): sum over indexer heads h of
// w_h * ReLU(qI_h . kI_{h,t}); the vectors are int8 of rank r (RTPurbo page,
// §2) and every product is accumulated exactly in int32.
//
//  * decode: one lane per (key block, head) for r = 16 (a 16-byte load, four
//    v_dot4 of 4 MACs each, then a lane-move sum over the block's heads); a
//    thread-per-block loop handles other r.  With per-group selection (SparDA
//    page, §2 "Indexador de Pronóstico Compacto") the heads split into
//    consecutive equal groups and each group's sum is a score row of its own.
//  * prefill: int8 MFMA 32x32x16 -- one MFMA per indexer head covers 32 query
//    blocks x 32 key blocks with K = r = 16, so no MAC is padding; ReLU and the
//    head weights are applied per head in the epilogue (the ReLU sits inside
//    the head sum, so heads cannot be folded into the K dimension).
//  * pooling: per-token vectors averaged per block and rounded to
//    floor(mean + 1/2) (PBS-Attn page, §4: block importance by mean pooling).
//  * int4 selector cache (SpotAttention page, §4 "Cuantización"): each key
//    vector is stored as 16 int4 codes plus one power-of-two scale 2^e, so the
//    dequantised key code * 2^e is an exact integer and so is every score.
#include "spa_internal.h"

namespace spa {

namespace {

constexpr int INT32_MIN_V = (int)0x80000000;

__device__ __forceinline__ int floor_div_pos(int a, int b) {  // b > 0
  int q = a / b;
  return (a % b != 0 && a < 0) ? q - 1 : q;
}

// ---------------------------------------------------------------- decode ----
// scores [B, groups, nKb]; group g sums heads g*H/groups .. (g+1)*H/groups-1.
// grid: (ceil(nKb / 256), B); block 256.
__global__ void __launch_bounds__(256) score_decode_kernel(const int8_t* __restrict__ qI,
                                                           const int8_t* __restrict__ kI,
                                                           const int8_t* __restrict__ w, int H,
                                                           int r, int groups, int nKb,
                                                           const int32_t* __restrict__ seq_len,
                                                           int blk, int32_t* __restrict__ scores) {
  __shared__ int q_words[256];  // H*r/4 <= 256
  __shared__ int w_s[256];
  const int b = blockIdx.y;
  const int HR = H * r;
  const int nw = HR >> 2;
  const int* q_src = reinterpret_cast<const int*>(qI + (size_t)b * HR);
  for (int t = threadIdx.x; t < nw; t += blockDim.x) q_words[t] = q_src[t];
  for (int t = threadIdx.x; t < H; t += blockDim.x) w_s[t] = w[(size_t)b * H + t];
  __syncthreads();

  const int j = blockIdx.x * blockDim.x + threadIdx.x;
  if (j >= nKb) return;
  const int L = seq_len[b];
  const int nbv = min(nKb, (L + blk - 1) / blk);
  int32_t* dst = scores + (size_t)b * groups * nKb + j;
  if (j >= nbv) {
    for (int g = 0; g < groups; ++g) dst[(size_t)g * nKb] = INT32_MIN_V;
    return;
  }
  const int hpg = H / groups;
  const int wpr = r >> 2;  // words per head
  const int8_t* row = kI + ((size_t)b * nKb + j) * HR;
  int total = 0;
  if ((HR & 15) == 0) {
    const int4* row4 = reinterpret_cast<const int4*>(row);
    int h = 0, in_head = 0, dot = 0;
    for (int c = 0; c < (HR >> 4); ++c) {
      const int4 kv = row4[c];
      const int kw[4] = {kv.x, kv.y, kv.z, kv.w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        dot = __builtin_amdgcn_sdot4(q_words[c * 4 + e], kw[e], dot, false);
        if (++in_head == wpr) {
          total += w_s[h] * max(dot, 0);
          ++h;
          in_head = 0;
          dot = 0;
          if (h % hpg == 0) {
            dst[(size_t)(h / hpg - 1) * nKb] = total;
            total = 0;
          }
        }
      }
    }
  } else {
    const int* roww = reinterpret_cast<const int*>(row);
    for (int h = 0; h < H; ++h) {
      int dot = 0;
      for (int e = 0; e < wpr; ++e) dot = __builtin_amdgcn_sdot4(q_words[h * wpr + e], roww[h * wpr + e], dot, false);
      total += w_s[h] * max(dot, 0);
      if ((h + 1) % hpg == 0) {
        dst[(size_t)(h / hpg) * nKb] = total;
        total = 0;
      }
    }
  }
}

// Sum over each aligned run of 2^log2hpg lanes (log2hpg <= 6), by register
// lane moves; every lane of the wave must call it.
__device__ __forceinline__ int group_sum(int v, int log2hpg) {
  if (log2hpg >= 1) v += (int)lane_xor<1>((unsigned)v);
  if (log2hpg >= 2) v += (int)lane_xor<2>((unsigned)v);
  if (log2hpg >= 3) v += (int)lane_xor<4>((unsigned)v);
  if (log2hpg >= 4) v += (int)lane_xor<8>((unsigned)v);
  if (log2hpg >= 5) v += (int)lane_xor<16>((unsigned)v);
  if (log2hpg >= 6) v += (int)lane_xor<32>((unsigned)v);
  return v;
}

// Fast decode path for r == 16 and a power-of-two H <= 64: one lane per
// (block, head) loads that head's 16 bytes (the wave reads 1 KB contiguous),
// four v_dot4 give the head dot, ReLU * w, and each group's 2^log2hpg
// neighbouring lanes sum their heads with register lane moves.  The sequence
// is the grid's y index, so no lane divides by nKb.  (Two or four lanes per
// thread, with their loads issued together, were slower: fewer waves hide
// less of the load latency.)
// grid: (ceil(nKb*H / 256), B); block 256.
__global__ void __launch_bounds__(256) score_decode_r16_kernel(const int8_t* __restrict__ qI,
                                                               const int8_t* __restrict__ kI,
                                                               const int8_t* __restrict__ w, int H,
                                                               int log2H, int log2hpg, int nKb,
                                                               const int32_t* __restrict__ seq_len,
                                                               int blk, int32_t* __restrict__ scores) {
  const int b = blockIdx.y;
  const int n = nKb * H;  // (block, head) lanes of this sequence
  const int t = blockIdx.x * 256 + threadIdx.x;
  const int h = t & (H - 1);
  const int j = t >> log2H;
  // every (block, head) below nKb is addressable: the loads go out together
  // with seq_len's, and the sequence end only masks the result
  const int4 kv = t < n ? *reinterpret_cast<const int4*>(kI + ((size_t)b * n + t) * 16) : int4{0, 0, 0, 0};
  const int4 qv = *reinterpret_cast<const int4*>(qI + ((size_t)b * H + h) * 16);
  const int wt = w[(size_t)b * H + h];
  const int L = seq_len[b];
  const bool valid = t < n && j < min(nKb, (L + blk - 1) / blk);
  int dot = __builtin_amdgcn_sdot4(qv.x, kv.x, 0, false);
  dot = __builtin_amdgcn_sdot4(qv.y, kv.y, dot, false);
  dot = __builtin_amdgcn_sdot4(qv.z, kv.z, dot, false);
  dot = __builtin_amdgcn_sdot4(qv.w, kv.w, dot, false);
  const int v = group_sum(valid ? wt * max(dot, 0) : 0, log2hpg);
  if (t < n && (h & ((1 << log2hpg) - 1)) == 0) {
    const int groups = H >> log2hpg;
    scores[((size_t)b * groups + (h >> log2hpg)) * nKb + j] = valid ? v : INT32_MIN_V;
  }
}

// ------------------------------------------------------- int4 selector keys --
// One lane per 16-element key vector: e is the smallest exponent for which the
// largest and the smallest element (the rounding is monotonic, so they bound
// every code) give codes floor(x / 2^e + 1/2) in [-8, 7]; the codes are
// packed two per byte, element 2c in the low nibble.
__global__ void __launch_bounds__(256) quantize_keys_kernel(const int8_t* __restrict__ kI, long n_vec,
                                                            uint8_t* __restrict__ codes,
                                                            uint8_t* __restrict__ exps) {
  const long i = (long)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n_vec) return;
  const int4 v = *reinterpret_cast<const int4*>(kI + i * 16);
  const int w[4] = {v.x, v.y, v.z, v.w};
  int x[16];
#pragma unroll
  for (int k = 0; k < 16; ++k) x[k] = (int)(int8_t)(w[k >> 2] >> (8 * (k & 3)));
  int vmax = x[0], vmin = x[0];
#pragma unroll
  for (int k = 1; k < 16; ++k) {
    vmax = max(vmax, x[k]);
    vmin = min(vmin, x[k]);
  }
  int e = 0;
  while (((2 * vmax + (1 << e)) >> (e + 1)) > 7 || ((2 * vmin + (1 << e)) >> (e + 1)) < -8) ++e;
  uint32_t packed[2] = {0u, 0u};
#pragma unroll
  for (int k = 0; k < 16; ++k) {
    const uint32_t c = (uint32_t)((2 * x[k] + (1 << e)) >> (e + 1)) & 0xFu;
    packed[k >> 3] |= c << (4 * (k & 7));
  }
  *reinterpret_cast<uint2*>(codes + i * 8) = uint2{packed[0], packed[1]};
  exps[i] = (uint8_t)e;
}

// Decode scores from int4 keys, r == 16 and a power-of-two H <= 64: one lane
// per (block, head) loads its 8 bytes of codes (the wave reads 512 B
// contiguous) and its exponent.  Shifting each nibble to the top of a byte
// gives 16 * code as int8, so four v_dot4 against the query bytes regrouped
// into even and odd elements give 16 * (q . code) exactly; >> 4 and << e
// give q . (code * 2^e).  ReLU, weight and the group sums as for int8 keys.
// grid: ceil(B*nKb*H / 256); block 256.
__global__ void __launch_bounds__(256) score_decode_q4_kernel(const int8_t* __restrict__ qI,
                                                              const uint8_t* __restrict__ codes,
                                                              const uint8_t* __restrict__ exps,
                                                              const int8_t* __restrict__ w, int H,
                                                              int log2H, int log2hpg, int nKb, int B,
                                                              const int32_t* __restrict__ seq_len,
                                                              int blk, int32_t* __restrict__ scores) {
  const long t = (long)blockIdx.x * blockDim.x + threadIdx.x;
  const long total = (long)B * nKb * H;
  const bool in = t < total;
  const long bj = in ? (t >> log2H) : 0;
  const int h = (int)(t & (H - 1));
  const int b = (int)(bj / nKb);
  const int j = (int)(bj - (long)b * nKb);
  int v = 0;
  bool valid = false;
  if (in) {
    const uint2 c = *reinterpret_cast<const uint2*>(codes + (size_t)t * 8);
    const int e = exps[t];
    const int4 q = *reinterpret_cast<const int4*>(qI + ((size_t)b * H + h) * 16);
    const int wt = w[(size_t)b * H + h];
    const int L = seq_len[b];
    valid = j < min(nKb, (L + blk - 1) / blk);
    {
      // even / odd elements of each 8-element half of the query
      const int qe0 = (int)__builtin_amdgcn_perm((unsigned)q.y, (unsigned)q.x, 0x06040200u);
      const int qo0 = (int)__builtin_amdgcn_perm((unsigned)q.y, (unsigned)q.x, 0x07050301u);
      const int qe1 = (int)__builtin_amdgcn_perm((unsigned)q.w, (unsigned)q.z, 0x06040200u);
      const int qo1 = (int)__builtin_amdgcn_perm((unsigned)q.w, (unsigned)q.z, 0x07050301u);
      int dot = __builtin_amdgcn_sdot4(qe0, (int)((c.x << 4) & 0xF0F0F0F0u), 0, false);
      dot = __builtin_amdgcn_sdot4(qo0, (int)(c.x & 0xF0F0F0F0u), dot, false);
      dot = __builtin_amdgcn_sdot4(qe1, (int)((c.y << 4) & 0xF0F0F0F0u), dot, false);
      dot = __builtin_amdgcn_sdot4(qo1, (int)(c.y & 0xF0F0F0F0u), dot, false);
      v = valid ? wt * max((dot >> 4) << (e & 7), 0) : 0;
    }
  }
  v = group_sum(v, log2hpg);
  if (in && (h & ((1 << log2hpg) - 1)) == 0) {
    const int groups = H >> log2hpg;
    scores[((size_t)b * groups + (h >> log2hpg)) * nKb + j] = valid ? v : INT32_MIN_V;
  }
}

// --------------------------------------------------------------- pooling ----
// Both per-token tensors of a prefill scoring call are pooled by one launch:
// grid (max(nblocks), B, 2), z = 0 the query chunk, z = 1 the keys.  One
// workgroup pools one block: with r = 16 a token's vector of head h is the
// 16-byte chunk h of its row, thread (token lane tl, head c) loads chunk c of
// the block's tokens tl, tl + TL, ... (TL = 256 / H lanes) and sums its 16
// signed bytes; the TL partial sums of each byte meet in LDS.  Slot t of a
// block is row t - row_off of the tensor, or row tok_pos[b, t] when the
// tensors are in original token order (the segment permutation is applied by
// this gather).  Tokens at or past the slot limit are left out of the mean.
struct PoolJob {
  const int8_t* x;  // [B, rows, H*16]
  int rows;         // rows per sequence
  int slot0;        // slot of the first token of block 0
  int row_off;      // row = slot - row_off without tok_pos
  int nblocks;
  int8_t* out;      // [B, nblocks, H*16]
};

constexpr int kPoolThreads = 256;

__global__ void __launch_bounds__(kPoolThreads) pool_kernel(PoolJob jq, PoolJob jk, int H, int blk,
                                                           const int32_t* __restrict__ seq_len,
                                                           const int32_t* __restrict__ tok_pos, int npos) {
  __shared__ int part[kPoolThreads * 16];
  const PoolJob& j = blockIdx.z ? jk : jq;
  const int jb = blockIdx.x;
  if (jb >= j.nblocks) return;
  const int b = blockIdx.y;
  const int tid = threadIdx.x;
  const int TL = kPoolThreads / H;
  const int c = tid % H, tl = tid / H;
  const int a0 = j.slot0 + jb * blk;
  int lim = j.slot0 + j.nblocks * blk;
  if (!tok_pos) lim = min(lim, j.row_off + j.rows);
  if (seq_len) lim = min(lim, seq_len[b]);
  const int n = max(0, min(a0 + blk, lim) - a0);
  int acc[16];
#pragma unroll
  for (int e = 0; e < 16; ++e) acc[e] = 0;
  if (tl < TL) {
    for (int t = tl; t < n; t += TL) {
      const int slot = a0 + t;
      const int row = tok_pos ? tok_pos[(size_t)b * npos + slot] : slot - j.row_off;
      const uint4 v = *reinterpret_cast<const uint4*>(j.x + ((size_t)b * j.rows + row) * (size_t)(H * 16) + c * 16);
      const unsigned w4[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int x = (int)w4[q];
        acc[4 * q + 0] += (int)(int8_t)(x & 0xFF);
        acc[4 * q + 1] += (int)(int8_t)((x >> 8) & 0xFF);
        acc[4 * q + 2] += (int)(int8_t)((x >> 16) & 0xFF);
        acc[4 * q + 3] += x >> 24;  // arithmetic shift keeps the sign of the top byte
      }
    }
  }
#pragma unroll
  for (int e = 0; e < 16; ++e) part[e * kPoolThreads + tid] = acc[e];
  __syncthreads();
  // thread o < 16H finishes byte e = o / H of head ch = o % H (neighbouring
  // threads read neighbouring LDS words)
  int8_t* ob = j.out + ((size_t)b * j.nblocks + jb) * (size_t)(H * 16);
  for (int o = tid; o < H * 16; o += kPoolThreads) {
    const int e = o / H, ch = o - e * H;
    int sum = 0;
    for (int l = 0; l < TL; ++l) sum += part[e * kPoolThreads + l * H + ch];
    ob[ch * 16 + e] = n > 0 ? (int8_t)floor_div_pos(2 * sum + n, 2 * n) : 0;
  }
}

// ------------------------------------------------------- prefill (MFMA) ----
// One wave computes a 32 (query blocks) x 32 (key blocks) tile for all heads.
// v_mfma_i32_32x32x16_i8 operands: lane l supplies row/col (l % 32) and the 8
// K-elements 8*(l/32)..+7; the result gives lane l column (l % 32) and rows
// 8*(v/4) + 4*(l/32) + (v%4), v = 0..15.
// grid: (ceil(nKb/32), ceil(Mq/32), B); block 64.
__global__ void __launch_bounds__(64) score_prefill_kernel(const int8_t* __restrict__ qIb,
                                                          const int8_t* __restrict__ kIb,
                                                          const int8_t* __restrict__ w, int H,
                                                          int Mq, int nKb, int q_blk0,
                                                          const int32_t* __restrict__ seq_len,
                                                          int blk, int32_t* __restrict__ scores) {
  const int lane = threadIdx.x;
  const int j0 = blockIdx.x * 32;
  const int i0 = blockIdx.y * 32;
  const int b = blockIdx.z;
  const int col = j0 + (lane & 31);
  const int half = lane >> 5;
  const int nbv = seq_len ? min(nKb, (seq_len[b] + blk - 1) / blk) : nKb;

  int acc[16];
#pragma unroll
  for (int v = 0; v < 16; ++v) acc[v] = 0;

  // the whole tile lies on or above the diagonal: nothing to compute
  const bool any = j0 < q_blk0 + min(i0 + 32, Mq) - 1 && j0 < nbv;
  if (any) {
    const int arow = i0 + (lane & 31);
    for (int h = 0; h < H; ++h) {
      long a = 0, bb = 0;
      if (arow < Mq) a = *reinterpret_cast<const long*>(qIb + (((size_t)b * Mq + arow) * H + h) * 16 + half * 8);
      if (col < nKb) bb = *reinterpret_cast<const long*>(kIb + (((size_t)b * nKb + col) * H + h) * 16 + half * 8);
      i32x16 d = {0};
      d = __builtin_amdgcn_mfma_i32_32x32x16_i8(a, bb, d, 0, 0, 0);
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int row = i0 + 8 * (v >> 2) + 4 * half + (v & 3);
        const int wv = row < Mq ? (int)w[((size_t)b * Mq + row) * H + h] : 0;
        acc[v] += wv * max(d[v], 0);
      }
    }
  }
  if (col >= nKb) return;
#pragma unroll
  for (int v = 0; v < 16; ++v) {
    const int row = i0 + 8 * (v >> 2) + 4 * half + (v & 3);
    if (row >= Mq) continue;
    const bool valid = col < q_blk0 + row && col < nbv;
    scores[((size_t)b * Mq + row) * nKb + col] = valid ? acc[v] : INT32_MIN_V;
  }
}

}  // namespace

hipError_t launch_score_decode(const int8_t* qI, const int8_t* kI, const int8_t* w, int B, int H,
                               int r, int groups, int nKb, const int32_t* seq_len, int blk,
                               int32_t* scores, hipStream_t s) {
  if (r == 16 && H <= kWave && (H & (H - 1)) == 0 && B <= 65535 && (long)nKb * H <= 0x7FFFFF00L) {
    // groups divides a power of two, so the heads per group are one too
    int log2H = 0, log2hpg = 0;
    while ((1 << log2H) < H) ++log2H;
    while ((1 << log2hpg) < H / groups) ++log2hpg;
    const dim3 grid((unsigned)(((long)nKb * H + 255) / 256), (unsigned)B);
    score_decode_r16_kernel<<<grid, 256, 0, s>>>(qI, kI, w, H, log2H, log2hpg, nKb, seq_len, blk, scores);
    return hipGetLastError();
  }
  dim3 grid((nKb + 255) / 256, B);
  score_decode_kernel<<<grid, 256, 0, s>>>(qI, kI, w, H, r, groups, nKb, seq_len, blk, scores);
  return hipGetLastError();
}

hipError_t launch_quantize_keys(const int8_t* kI, long n_vec, uint8_t* codes, uint8_t* exps, hipStream_t s) {
  quantize_keys_kernel<<<(unsigned)((n_vec + 255) / 256), 256, 0, s>>>(kI, n_vec, codes, exps);
  return hipGetLastError();
}

hipError_t launch_score_decode_q4(const int8_t* qI, const uint8_t* codes, const uint8_t* exps, const int8_t* w,
                                  int B, int H, int groups, int nKb, const int32_t* seq_len, int blk,
                                  int32_t* scores, hipStream_t s) {
  int log2H = 0, log2hpg = 0;
  while ((1 << log2H) < H) ++log2H;
  while ((1 << log2hpg) < H / groups) ++log2hpg;
  const long total = (long)B * nKb * H;
  score_decode_q4_kernel<<<(unsigned)((total + 255) / 256), 256, 0, s>>>(qI, codes, exps, w, H, log2H, log2hpg, nKb,
                                                                          B, seq_len, blk, scores);
  return hipGetLastError();
}

hipError_t launch_pool_pair(const int8_t* q_tok, int q_rows, int q_slot0, int q_row_off, int Mq,
                            const int8_t* k_tok, int k_rows, int nKb, int B, int H, int blk,
                            const int32_t* seq_len, const int32_t* tok_pos, int npos, int8_t* q_out,
                            int8_t* k_out, hipStream_t s) {
  const PoolJob jq{q_tok, q_rows, q_slot0, q_row_off, Mq, q_out};
  const PoolJob jk{k_tok, k_rows, 0, 0, nKb, k_out};
  dim3 grid(Mq > nKb ? Mq : nKb, B, 2);
  pool_kernel<<<grid, kPoolThreads, 0, s>>>(jq, jk, H, blk, seq_len, tok_pos, npos);
  return hipGetLastError();
}

hipError_t launch_score_prefill(const int8_t* qIb, const int8_t* kIb, const int8_t* w, int B,
                                int H, int Mq, int nKb, int q_blk0, const int32_t* seq_len,
                                int blk, int32_t* scores, hipStream_t s) {
  dim3 grid((nKb + 31) / 32, (Mq + 31) / 32, B);
  score_prefill_kernel<<<grid, 64, 0, s>>>(qIb, kIb, w, H, Mq, nKb, q_blk0, seq_len, blk, scores);
  return hipGetLastError();
}

}  // namespace spa
