// Block-sparse causal prefill attention over per-query-block key-block lists.
//
// PBS-Attn page: block-sparse attention computes only the key blocks of a
// precomputed list ("Declaración del Problema"); tokens may be permuted inside
// segments, with causality enforced on the original positions (§2).  HGA
// page: the softmax is exact over the selected tokens.
//
// One workgroup = one (sequence, 16 query slots of a 64-slot block, 4 query
// heads of one KV head); one wave = one query head x 16 query slots.  For
// each selected key block the wave walks two 32-key tiles:
//   S^T[32 keys, 16 queries] = K . Q^T   (2 x 4 MFMA 16x16x32 bf16)
//   O^T[128, 16 queries]    += V^T . P^T (8 MFMA 16x16x32 bf16)
// with the same operand scheme as the decode kernel: K rows feed the A operand
// directly, V rows are transposed in registers, and S^T's accumulator layout
// is already the P^T operand layout.  Keys are masked with
// k_pos <= q_pos (original positions) and t < T.  One register buffer each
// for K and V: the next tile's K loads start once QK^T has consumed K, its V
// loads once PV has consumed V, so memory and MFMA work overlap.
#include "spa_internal.h"

namespace spa {

namespace {

constexpr int D = 128;
constexpr int BLK = 64;
constexpr int NT = 1;         // query n-tiles (of 16) per wave: 16 query slots
constexpr int QW = NT * 16;   // query slots per wave
constexpr int NSUB = BLK / QW;  // query sub-blocks per 64-slot block
constexpr int kWaves = 4;     // 4 query heads of one KV head
constexpr int kTile = 32;
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

__device__ __forceinline__ bf16x8 as_bf16x8(const uint4& u) { return __builtin_bit_cast(bf16x8, u); }
__device__ __forceinline__ uint32_t word_of(const uint4& u, int i) {
  return i == 0 ? u.x : i == 1 ? u.y : i == 2 ? u.z : u.w;
}

// K tile as A operands: lane (row m, group g4) holds 16 bytes of token m per k-step.
__device__ __forceinline__ void load_k(const uint16_t* __restrict__ kb, int tok0, int nvalid, int lane,
                                       uint4* kr) {
  const int m = lane & 15, g4 = lane >> 4;
#pragma unroll
  for (int mt = 0; mt < 2; ++mt) {
    const int tau = min(16 * mt + m, nvalid - 1);
    const uint16_t* row = kb + (size_t)(tok0 + tau) * D;
#pragma unroll
    for (int j = 0; j < 4; ++j) kr[mt * 4 + j] = *reinterpret_cast<const uint4*>(row + 8 * (4 * j + g4));
  }
}

// V tile: the 16 lanes of group g4 read token 16*(i/4) + 4*g4 + i%4 whole.
__device__ __forceinline__ void load_v(const uint16_t* __restrict__ vb, int tok0, int nvalid, int lane,
                                       uint4* vr) {
  const int m = lane & 15, g4 = lane >> 4;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int tau = min(16 * (i >> 2) + 4 * g4 + (i & 3), nvalid - 1);
    vr[i] = *reinterpret_cast<const uint4*>(vb + (size_t)(tok0 + tau) * D + 8 * m);
  }
}

struct State {
  float m[NT];
  float l[NT];
  f32x4 o[8][NT];
};

// grid: (Mq * NSUB, Hkv * ceil(G/4), B); block 256 (4 waves).
__global__ void __launch_bounds__(kWaves * kWave, 2) prefill_kernel(PrefillArgs a) {
  const int lane = threadIdx.x & (kWave - 1);
  const int wv = threadIdx.x / kWave;
  const int i = blockIdx.x / NSUB;
  const int qh = blockIdx.x - i * NSUB;  // which 16-slot part of the query block
  const int G = a.Hq / a.Hkv;
  const int zg = (G + 3) / 4;
  const int g = blockIdx.y / zg;
  const int hg = (blockIdx.y - g * zg) * 4 + wv;
  const int b = blockIdx.z;
  if (hg >= G) return;
  const int h = g * G + hg;
  const int m = lane & 15, g4 = lane >> 4;
  const float scale_log2 = a.scale * kLog2e;
  const int Mq = (a.Tq + BLK - 1) / BLK;

  const uint16_t* qb = (const uint16_t*)a.q + ((size_t)b * a.Hq + h) * (size_t)a.Tq * D;
  const size_t kv_off = ((size_t)b * a.Hkv + g) * (size_t)a.T * D;
  const uint16_t* kb = (const uint16_t*)a.k + kv_off;
  const uint16_t* vb = (const uint16_t*)a.v + kv_off;
  const int32_t* kpos = a.k_pos ? a.k_pos + (size_t)b * a.T : nullptr;

  bf16x8 qreg[NT][4];
  int qp[NT];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    const int row = i * BLK + qh * QW + 16 * nt + m;  // local query row of the chunk
    const int slot = a.q_blk0 * BLK + row;
    qp[nt] = row < a.Tq ? (a.q_pos ? a.q_pos[(size_t)b * a.T + slot] : slot) : -1;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      uint4 qv = {0u, 0u, 0u, 0u};
      if (row < a.Tq) qv = *reinterpret_cast<const uint4*>(qb + (size_t)row * D + 8 * (4 * j + g4));
      qreg[nt][j] = as_bf16x8(qv);
    }
  }
  State st;
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    st.m[nt] = -INFINITY;
    st.l[nt] = 0.f;
#pragma unroll
    for (int jj = 0; jj < 8; ++jj) st.o[jj][nt] = f32x4{0.f, 0.f, 0.f, 0.f};
  }

  const int32_t* lst = a.idx + ((size_t)b * Mq + i) * a.cap;
  const int nsel = a.count[(size_t)b * Mq + i];
  const int ntiles = nsel * (BLK / kTile);
  auto tinfo = [&](int u, int& tok0, int& nv) {
    const int j = lst[u >> 1];
    tok0 = j * BLK + (u & 1) * kTile;
    nv = min(kTile, a.T - tok0);
  };
  uint4 kr[8], vr[8];
  int tok = 0, nv = 0;
  if (ntiles > 0) {
    tinfo(0, tok, nv);
    if (nv > 0) {
      load_k(kb, tok, nv, lane, kr);
      load_v(vb, tok, nv, lane, vr);
    }
  }
  for (int u = 0; u < ntiles; ++u) {
    int tokn = 0, nvn = 0;
    const bool more = u + 1 < ntiles;
    if (more) tinfo(u + 1, tokn, nvn);
    if (nv <= 0) {
      if (more && nvn > 0) {
        load_k(kb, tokn, nvn, lane, kr);
        load_v(vb, tokn, nvn, lane, vr);
      }
      tok = tokn;
      nv = nvn;
      continue;
    }
    // ---- S^T = K . Q^T for both query n-tiles
    f32x4 s[2][NT];
#pragma unroll
    for (int nt = 0; nt < NT; ++nt)
#pragma unroll
      for (int mt = 0; mt < 2; ++mt) {
        s[mt][nt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int j = 0; j < 4; ++j)
          s[mt][nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(kr[mt * 4 + j]), qreg[nt][j],
                                                              s[mt][nt], 0, 0, 0);
      }
    // key positions of this lane's 8 rows
    int kp[8];
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int tau = 16 * mt + 4 * g4 + r;
        kp[mt * 4 + r] = tau < nv ? (kpos ? kpos[tok + tau] : tok + tau) : 0x7FFFFFFF;
      }
    // K registers are free: start the next tile's K loads
    if (more && nvn > 0) load_k(kb, tokn, nvn, lane, kr);
    // ---- online softmax per query column
    bf16x8 pb[NT];
    float corr[NT];
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      float x[8];
      float tmax = -INFINITY;
#pragma unroll
      for (int mt = 0; mt < 2; ++mt)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const float v = kp[mt * 4 + r] <= qp[nt] ? s[mt][nt][r] * scale_log2 : -INFINITY;
          x[mt * 4 + r] = v;
          tmax = fmaxf(tmax, v);
        }
      tmax = fmaxf(tmax, shfl_xor_f(tmax, 16));
      tmax = fmaxf(tmax, shfl_xor_f(tmax, 32));
      const float m_new = fmaxf(st.m[nt], tmax);
      const float base = m_new == -INFINITY ? 0.f : m_new;
      corr[nt] = exp2f(st.m[nt] - base);
      float p[8];
      float psum = 0.f;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        p[e] = exp2f(x[e] - base);
        psum += p[e];
      }
      st.l[nt] = st.l[nt] * corr[nt] + psum;
      st.m[nt] = m_new;
      pb[nt] = as_bf16x8(uint4{pack_bf16x2(p[0], p[1]), pack_bf16x2(p[2], p[3]),
                               pack_bf16x2(p[4], p[5]), pack_bf16x2(p[6], p[7])});
    }
    // ---- O^T += V^T . P^T; V^T rows d = 8m + jj come from an in-register transpose
#pragma unroll
    for (int jj = 0; jj < 8; ++jj) {
      const int wsel = jj >> 1;
      uint32_t a4[4];
#pragma unroll
      for (int aa = 0; aa < 4; ++aa) {
        const uint32_t lo = word_of(vr[2 * aa], wsel);
        const uint32_t hi = word_of(vr[2 * aa + 1], wsel);
        a4[aa] = (jj & 1) ? ((lo >> 16) | (hi & 0xFFFF0000u)) : ((lo & 0xFFFFu) | (hi << 16));
      }
      const bf16x8 vt = as_bf16x8(uint4{a4[0], a4[1], a4[2], a4[3]});
#pragma unroll
      for (int nt = 0; nt < NT; ++nt)
        st.o[jj][nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vt, pb[nt], st.o[jj][nt] * corr[nt], 0, 0, 0);
    }
    if (more && nvn > 0) load_v(vb, tokn, nvn, lane, vr);
    tok = tokn;
    nv = nvn;
  }

  // epilogue: normalise and store
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    float lt = st.l[nt];
    lt += shfl_xor_f(lt, 16);
    lt += shfl_xor_f(lt, 32);
    const int row = i * BLK + qh * QW + 16 * nt + m;
    if (row >= a.Tq) continue;
    const bool empty = st.m[nt] == -INFINITY || lt <= 0.f;
    const float inv = empty ? 0.f : 1.f / lt;
    const size_t obase = (((size_t)b * a.Hq + h) * a.Tq + row) * D + 32 * g4;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      float v8[8];
#pragma unroll
      for (int jj = 0; jj < 8; ++jj) v8[jj] = st.o[jj][nt][r] * inv;
      if (a.out_bf16) {
        uint4 pk = {pack_bf16x2(v8[0], v8[1]), pack_bf16x2(v8[2], v8[3]), pack_bf16x2(v8[4], v8[5]),
                    pack_bf16x2(v8[6], v8[7])};
        *reinterpret_cast<uint4*>((uint16_t*)a.out + obase + 8 * r) = pk;
      } else {
        float* o = (float*)a.out + obase + 8 * r;
        *reinterpret_cast<float4*>(o) = float4{v8[0], v8[1], v8[2], v8[3]};
        *reinterpret_cast<float4*>(o + 4) = float4{v8[4], v8[5], v8[6], v8[7]};
      }
    }
    if (a.lse && g4 == 0)
      a.lse[((size_t)b * a.Hq + h) * a.Tq + row] = empty ? -INFINITY : (st.m[nt] + log2f(lt)) * kLn2;
  }
}

}  // namespace

hipError_t launch_prefill(const PrefillArgs& a, hipStream_t s) {
  const int G = a.Hq / a.Hkv;
  const int Mq = (a.Tq + BLK - 1) / BLK;
  dim3 grid(Mq * NSUB, a.Hkv * ((G + 3) / 4), a.B);
  prefill_kernel<<<grid, kWaves * kWave, 0, s>>>(a);
  return hipGetLastError();
}

}  // namespace spa
