// Block-sparse causal prefill attention over per-query-block key-block lists.
//
// PBS-Attn page: block-sparse attention computes only the key blocks of a
// precomputed list ("Declaración del Problema"); tokens may be permuted inside
// segments, with causality enforced on the original positions (§2).  HGA
// page: the softmax is exact over the selected tokens.  Query rows are read,
// and output rows written, either in the chunk's slot order or at each
// query's original position; K and V rows are read either in slot order or
// at each key's original position.  The original orders take the
// permutations of Q, K and V and the inverse permutation of O off the
// pipeline: the kernel applies them as it reads and writes.
//
// One workgroup = one (sequence, KV head, query block of 64 slots) and up to
// four query heads of that KV head: eight waves, wave w owns query head
// 4*quad + (w & 3) and query slots 32*(w >> 2) .. +31.  The four heads share
// every key block of the list, so each 64-key block is staged once per
// workgroup into LDS (direct global->LDS 16-byte loads, 16-byte chunks
// XOR-swizzled by row so that the MFMA operand reads are free of bank
// conflicts) and read by all eight waves.  K, V and key positions are
// double-buffered: tile u+1 streams in while tile u is computed, and the
// block number and K/V source rows of tile u+2 are loaded meanwhile.  The
// operand fragments of the two products are read from LDS one step ahead of
// the MFMAs that consume them.
//
// The two buffers are separate LDS arrays and the tile loop is unrolled by
// two, so every LDS read names its buffer at compile time.  The compiler
// must otherwise assume that a read may overlap a global->LDS load still in
// flight and waits for all of them (vmcnt(0)) before it: with one array
// indexed by u & 1, each tile's V and position reads waited for the next
// tile's loads to land, which serialised the prefetch with the compute.
//
// Per 64-key tile a wave computes, with v_mfma_f32_32x32x16_bf16:
//   S^T[64 keys, 32 queries] = K . Q^T      (2 x 8 MFMA)
//   O^T[128, 32 queries]    += V^T . P^T    (4 x 4 MFMA)
// K rows are the A operand as stored; V^T fragments come from the LDS
// transpose read (ds_read_b64_tr_b16), whose key order matches the order in
// which S^T's accumulator registers hold the keys, so P^T is packed straight
// from S^T.  Two waves share each SIMD, so one wave's softmax (VALU) runs
// while the other's products (MFMA) do.
//
// The running maximum is rescaled lazily: O and the normaliser keep the old
// reference until a tile's maximum exceeds it by more than 2^8 in the exp2
// domain, so the O rescale (64 multiplies per lane) runs only on the rare
// tiles that raise the maximum that much.  The result is the same softmax;
// only the reference point of the partial sums differs.  The largest
// probability is then 2^x rather than 1, and the bf16 P operand rounds it to
// 8 significant bits, so O is normalised by the sum of the probabilities as
// rounded (v_dot2 against ones, 16 instructions per tile): O is an exact
// convex combination of V rows with the bf16 weights, and a row that a few
// keys dominate stays within rounding of the exact output.  The log-sum-exp
// keeps the exact fp32 sum.  (Normalised by the exact sum, that rounding
// alone moved such rows by up to 0.4 % of |v|; rescaling at every new
// maximum fixes it too, at 5 % of the kernel's time against 3 % here.)
//
// Keys are masked with k_pos <= q_pos (original positions) and t < T; the
// masks are skipped for tiles whose key positions all lie below the block's
// smallest query position (every block of an earlier segment), which one
// wave vote decides.
#include "spa_internal.h"

namespace spa {

namespace {

constexpr int D = 128;
constexpr int BLK = 64;
constexpr int kWaves = 8;
constexpr int ROWB = D * 2;          // bytes of one K/V row
constexpr int TILEB = BLK * ROWB;    // bytes of one 64-key K or V tile
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kLazy = 8.f;

typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void_t;
typedef __attribute__((address_space(3))) s16x4 lds_s16x4_t;

// the two staging buffers, as distinct objects (see above)
__shared__ __attribute__((aligned(16))) uint8_t lds_k0[TILEB];
__shared__ __attribute__((aligned(16))) uint8_t lds_k1[TILEB];
__shared__ __attribute__((aligned(16))) uint8_t lds_v0[TILEB];
__shared__ __attribute__((aligned(16))) uint8_t lds_v1[TILEB];
__shared__ __attribute__((aligned(16))) int32_t lds_p0[BLK];
__shared__ __attribute__((aligned(16))) int32_t lds_p1[BLK];

template <int S> struct Slot {
  static constexpr int value = S;
  static __device__ __forceinline__ uint8_t* k() { return S ? lds_k1 : lds_k0; }
  static __device__ __forceinline__ uint8_t* v() { return S ? lds_v1 : lds_v0; }
  static __device__ __forceinline__ int32_t* pos() { return S ? lds_p1 : lds_p0; }
};

// byte offset of 16-byte chunk c of row r inside a swizzled tile
__device__ __forceinline__ int swz(int r, int c) { return r * ROWB + ((c ^ (r & 15)) << 4); }
__device__ __forceinline__ int vsw(int r) { return 4 * (r & 3) + 2 * ((r >> 1) & 1); }
__device__ __forceinline__ int swz_v(int r, int c) { return r * ROWB + ((c ^ vsw(r)) << 4); }

__device__ __forceinline__ bf16x8 as_bf16x8(const uint4& u) { return __builtin_bit_cast(bf16x8, u); }

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
// two floats to a bf16 pair, round to nearest even (one v_cvt_pk_bf16_f32)
__device__ __forceinline__ uint32_t cvt_pk_bf16(float lo, float hi) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2_t{lo, hi}, bf16x2_t));
}

__device__ __forceinline__ int wave_min_i(int v) {
#pragma unroll
  for (int o = 1; o < kWave; o <<= 1) v = min(v, shfl_xor_i(v, o));
  return v;
}

// Stage key block tok0 (K, V rows and positions) into buffer S.  Wave w
// moves rows 8w..8w+7 of K and of V: each instruction writes 1 KB (4 rows) at
// LDS base + 16*lane, so lane l fetches the global chunk that the swizzle
// places at its slot.  Rows past T re-read row T-1 (masked later).
// src[n4] is the row of K and V that holds this lane's slot of the tile: the
// slot itself, or with K/V in original order its original position.
template <int S>
__device__ __forceinline__ void stage(const uint16_t* __restrict__ kb, const uint16_t* __restrict__ vb,
                                      const int32_t* __restrict__ kpos, int tok0, int T, int w, int lane,
                                      const int (&src)[2]) {
  const int cpos = lane & 15;
#pragma unroll
  for (int n4 = 0; n4 < 2; ++n4) {
    const int r0 = 8 * w + 4 * n4;
    const int r = r0 + (lane >> 4);
    const size_t row = (size_t)src[n4] * D;
    __builtin_amdgcn_global_load_lds(kb + row + 8 * (cpos ^ (r & 15)), (lds_void_t*)(Slot<S>::k() + r0 * ROWB), 16, 0, 0);
    __builtin_amdgcn_global_load_lds(vb + row + 8 * (cpos ^ vsw(r)), (lds_void_t*)(Slot<S>::v() + r0 * ROWB), 16, 0, 0);
  }
  if (w == 0) {
    if (kpos)
      __builtin_amdgcn_global_load_lds(kpos + min(tok0 + lane, T - 1), (lds_void_t*)Slot<S>::pos(), 4, 0, 0);
    else
      Slot<S>::pos()[lane] = tok0 + lane < T ? tok0 + lane : 0x7FFFFFFF;  // past T: masked by position
  }
}

// grid: (Mq * B * Hkv * ceil(G/4)); block 512 (8 waves).  Workgroups are
// ordered (query block descending, then sequence/KV head/quad), so that
// consecutive workgroups -- which the dispatcher spreads over the XCDs --
// work on different KV heads and the longest lists start first.
__global__ void __launch_bounds__(kWaves * kWave, 1) prefill_kernel(PrefillArgs a) {
  const int lane = threadIdx.x & (kWave - 1);
  const int w = threadIdx.x / kWave;
  const int G = a.Hq / a.Hkv;
  const int zq = (G + 3) / 4;
  const int NG = a.B * a.Hkv * zq;
  const int Mq = (a.Tq + BLK - 1) / BLK;
  const int gid = blockIdx.x % NG;
  const int i = Mq - 1 - (int)(blockIdx.x / NG);
  const int b = gid / (a.Hkv * zq);
  const int g = (gid / zq) % a.Hkv;
  const int hg = (gid % zq) * 4 + (w & 3);
  const bool active = hg < G;
  const int h = g * G + min(hg, G - 1);
  const int l32 = lane & 31, hi = lane >> 5;
  const int row = i * BLK + 32 * (w >> 2) + l32;  // this lane's query slot (local to the chunk)
  const bool row_ok = row < a.Tq;
  const float c2 = a.scale * kLog2e;

  const int32_t* lst = a.idx + ((size_t)b * Mq + i) * a.cap;
  const int nsel = a.count[(size_t)b * Mq + i];

  // query position; the smallest over the whole query block decides which tiles need masks
  int qp = -1, qmin = 0x7FFFFFFF;
  {
    const int slot = a.q_blk0 * BLK + row;
    if (row_ok) qp = a.q_pos ? a.q_pos[(size_t)b * a.T + slot] : slot;
    const int r2 = i * BLK + lane;  // every slot of the block, one per lane
    if (r2 < a.Tq) {
      const int s2 = a.q_blk0 * BLK + r2;
      qmin = a.q_pos ? a.q_pos[(size_t)b * a.T + s2] : s2;
    }
    qmin = wave_min_i(qmin);
  }
  const bool force_mask = (i + 1) * BLK > a.Tq;

  // this lane's row of q, out and lse: its slot in the chunk, or in original
  // order its query's position (q rows read and O rows written where they
  // belong, which makes the permutation of Q and the inverse permutation of O
  // unnecessary)
  const size_t qrow0 = a.orig_order ? (((size_t)b * a.Hq + h) * (size_t)a.T + (row_ok ? qp : 0))
                                    : (((size_t)b * a.Hq + h) * (size_t)a.Tq + (row_ok ? row : 0));
  if (nsel <= 0) {
    if (active && row_ok) {
      for (int d0 = 64 * hi; d0 < 64 * hi + 64; d0 += 8) {
        if (a.out_bf16) {
          *reinterpret_cast<uint4*>((uint16_t*)a.out + qrow0 * D + d0) = uint4{0u, 0u, 0u, 0u};
        } else {
          float* o = (float*)a.out + qrow0 * D + d0;
          *reinterpret_cast<float4*>(o) = float4{0.f, 0.f, 0.f, 0.f};
          *reinterpret_cast<float4*>(o + 4) = float4{0.f, 0.f, 0.f, 0.f};
        }
      }
      if (a.lse && hi == 0) a.lse[qrow0] = -INFINITY;
    }
    return;
  }

  const size_t kv_off = ((size_t)b * a.Hkv + g) * (size_t)a.T * D;
  const uint16_t* kb = (const uint16_t*)a.k + kv_off;
  const uint16_t* vb = (const uint16_t*)a.v + kv_off;
  const int32_t* kpos = a.k_pos ? a.k_pos + (size_t)b * a.T : nullptr;

  // K/V rows of this lane's two staging slots in the tile at tok (loaded from
  // k_pos when K and V are in original order, so a tile's rows are known one
  // tile before it is staged)
  auto kv_src = [&](int tok, int (&src)[2]) __attribute__((always_inline)) {
#pragma unroll
    for (int n4 = 0; n4 < 2; ++n4) {
      const int t = min(tok + 8 * w + 4 * n4 + (lane >> 4), a.T - 1);
      src[n4] = a.kv_orig && kpos ? kpos[t] : t;
    }
  };
  // block list, 64 entries per register chunk (read back with readlane); the
  // chunk holds the entry two tiles ahead, tk0/tk1 the token offsets of tiles
  // u and u+1
  int chunk = lane < nsel ? lst[lane] : 0;
  int tk0 = __builtin_amdgcn_readfirstlane(chunk) * BLK;
  int tk1 = nsel > 1 ? __builtin_amdgcn_readlane(chunk, 1) * BLK : 0;
  int src1[2], src2[2] = {0, 0};
  kv_src(tk0, src1);
  stage<0>(kb, vb, kpos, tk0, a.T, w, lane, src1);
  kv_src(tk1, src1);

  // Q^T fragments (B operand): lane holds query slot row, d = 16ks + 8hi .. +7
  bf16x8 qf[8];
  {
    const uint16_t* qb = (const uint16_t*)a.q + qrow0 * D;
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) {
      uint4 v = *reinterpret_cast<const uint4*>(qb + 16 * ks + 8 * hi);
      if (!row_ok) v = uint4{0u, 0u, 0u, 0u};
      qf[ks] = as_bf16x8(v);
    }
  }

  f32x16 o[4];
#pragma unroll
  for (int dt = 0; dt < 4; ++dt)
#pragma unroll
    for (int e = 0; e < 16; ++e) o[dt][e] = 0.f;
  float mrun = -INFINITY, lsum = 0.f, lsum_r = 0.f;  // exact and as-rounded probability sums
  const int grp = lane >> 4, s16 = lane & 15;

  // one tile: compute tile u from buffer S while tile u+1 streams into the other
  auto tile = [&](auto slot_tag, const int u) __attribute__((always_inline)) {
    constexpr int S = decltype(slot_tag)::value;
    const int tok0 = tk0;
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): this wave's loads of tile u have landed
    __syncthreads();
    // keys at or past T (the tail of the last block) take position INT_MAX so
    // that the position test alone masks them; loaded positions are patched
    // once they have landed, behind one more barrier (at most one tile per list)
    if (kpos && tok0 + BLK > a.T) {
      if (w == 0 && tok0 + lane >= a.T) Slot<S>::pos()[lane] = 0x7FFFFFFF;
      __syncthreads();
    }
    // tile u+2's entry and rows first: a wait they may need then comes before
    // the next tile's loads are issued
    int tk2 = 0;
    if (u + 2 < nsel) {
      if (((u + 2) & 63) == 0) chunk = u + 2 + lane < nsel ? lst[u + 2 + lane] : 0;
      tk2 = __builtin_amdgcn_readlane(chunk, (u + 2) & 63) * BLK;
      kv_src(tk2, src2);
    }
    if (u + 1 < nsel) stage<S ^ 1>(kb, vb, kpos, tk1, a.T, w, lane, src1);
    tk0 = tk1;
    tk1 = tk2;
    src1[0] = src2[0];
    src1[1] = src2[1];
    const bool need_mask = force_mask || __any((int)(Slot<S>::pos()[lane] > qmin));
    if (!active) return;

    // ---- S^T = K . Q^T
    f32x16 s[2];
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
      for (int e = 0; e < 16; ++e) s[mt][e] = 0.f;
    const uint8_t* kt = Slot<S>::k();
    bf16x8 kf[8][2];
#pragma unroll
    for (int ks = 0; ks < 8; ++ks)
#pragma unroll
      for (int mt = 0; mt < 2; ++mt)
        kf[ks][mt] = as_bf16x8(*reinterpret_cast<const uint4*>(kt + swz(32 * mt + l32, 2 * ks + hi)));
#pragma unroll
    for (int ks = 0; ks < 8; ++ks)
#pragma unroll
      for (int mt = 0; mt < 2; ++mt) s[mt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[ks][mt], qf[ks], s[mt], 0, 0, 0);
    // reads of d-step ks+1 are issued before the products of d-step ks
    __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
#pragma unroll
    for (int ks = 0; ks < 7; ++ks) {
      __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
    }
    __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
    // ---- mask: this lane holds keys 32mt + 8a + 4hi + r (keys past T carry
    // position INT_MAX, so the position test covers them)
    if (need_mask) {
#pragma unroll
      for (int mt = 0; mt < 2; ++mt)
#pragma unroll
        for (int aa = 0; aa < 4; ++aa) {
          const int key0 = 32 * mt + 8 * aa + 4 * hi;
          const int4 kp4 = *reinterpret_cast<const int4*>(&Slot<S>::pos()[key0]);
          const int kpv[4] = {kp4.x, kp4.y, kp4.z, kp4.w};
#pragma unroll
          for (int r = 0; r < 4; ++r)
            if (!(kpv[r] <= qp)) s[mt][4 * aa + r] = -INFINITY;
        }
    }
    // ---- online softmax (exp2 domain, lazy reference)
    float tm = -INFINITY;
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
      for (int e = 0; e < 16; ++e) tm = fmaxf(tm, s[mt][e]);
    tm = fmaxf(tm, lane_swap_f<32>(tm));
    const float tmc = tm * c2;
    const bool resc = tmc > mrun + kLazy;
    if (__any((int)resc)) {
      const float mnew = resc ? tmc : mrun;
      const float corr = resc ? exp2f(mrun - mnew) : 1.f;
#pragma unroll
      for (int dt = 0; dt < 4; ++dt) o[dt] *= corr;
      lsum *= corr;
      lsum_r *= corr;
      mrun = mnew;
    }
    const float nb = mrun == -INFINITY ? 0.f : -mrun;
    bf16x8 pf[4];
    float ps[4] = {0.f, 0.f, 0.f, 0.f};  // four partial sums: no 32-long dependent chain
#pragma unroll
    for (int kb4 = 0; kb4 < 4; ++kb4) {
      float p[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        p[e] = __builtin_amdgcn_exp2f(fmaf(s[kb4 >> 1][8 * (kb4 & 1) + e], c2, nb));
        ps[e & 3] += p[e];
      }
      pf[kb4] = as_bf16x8(uint4{cvt_pk_bf16(p[0], p[1]), cvt_pk_bf16(p[2], p[3]), cvt_pk_bf16(p[4], p[5]),
                                cvt_pk_bf16(p[6], p[7])});
    }
    lsum += (ps[0] + ps[1]) + (ps[2] + ps[3]);
    {
      const bf16x2_t one2 = __builtin_bit_cast(bf16x2_t, 0x3F803F80u);  // (1, 1)
      float pr = 0.f;
#pragma unroll
      for (int kb4 = 0; kb4 < 4; ++kb4) {
        const uint4 pu = __builtin_bit_cast(uint4, pf[kb4]);
        pr = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, pu.x), one2, pr, false);
        pr = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, pu.y), one2, pr, false);
        pr = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, pu.z), one2, pr, false);
        pr = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, pu.w), one2, pr, false);
      }
      lsum_r += pr;
    }
    // ---- O^T += V^T . P^T
    const uint8_t* vt = Slot<S>::v();
    bf16x8 vf[4][4];
#pragma unroll
    for (int kb4 = 0; kb4 < 4; ++kb4)
#pragma unroll
      for (int dt = 0; dt < 4; ++dt) {
        s16x4 x[2];
#pragma unroll
        for (int t = 0; t < 2; ++t) {
          const int r = 16 * kb4 + 4 * (grp >> 1) + 8 * t + (s16 >> 2);
          const int c = 4 * dt + 2 * (grp & 1) + ((s16 & 3) >> 1);
          x[t] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t*)(vt + swz_v(r, c) + 8 * (s16 & 1)));
        }
        vf[kb4][dt] = __builtin_bit_cast(bf16x8, __builtin_shufflevector(x[0], x[1], 0, 1, 2, 3, 4, 5, 6, 7));
      }
#pragma unroll
    for (int kb4 = 0; kb4 < 4; ++kb4)
#pragma unroll
      for (int dt = 0; dt < 4; ++dt) o[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf[kb4][dt], pf[kb4], o[dt], 0, 0, 0);
    // fragment reads run two steps ahead of the products that use them
    __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
#pragma unroll
    for (int j = 0; j < 14; ++j) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
    }
    __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
  };
  for (int u = 0; u < nsel; u += 2) {
    tile(Slot<0>{}, u);
    if (u + 1 < nsel) tile(Slot<1>{}, u + 1);
  }
  if (!active || !row_ok) return;

  // ---- epilogue: normalise and store; lane holds d = 32dt + 8a + 4hi + r of its query slot
  const float lt = lsum + shfl_xor_f(lsum, 32);
  const float lr = lsum_r + shfl_xor_f(lsum_r, 32);  // >= 1 when lt > 0: the row maximum's weight is >= 1
  const bool empty = !(lt > 0.f);
  const float inv = empty ? 0.f : 1.f / lr;
  const size_t obase = qrow0 * D + 4 * hi;
#pragma unroll
  for (int dt = 0; dt < 4; ++dt)
#pragma unroll
    for (int aa = 0; aa < 4; ++aa) {
      const float v0 = o[dt][4 * aa] * inv, v1 = o[dt][4 * aa + 1] * inv;
      const float v2 = o[dt][4 * aa + 2] * inv, v3 = o[dt][4 * aa + 3] * inv;
      const size_t off = obase + 32 * dt + 8 * aa;
      if (a.out_bf16)
        *reinterpret_cast<uint2*>((uint16_t*)a.out + off) = uint2{cvt_pk_bf16(v0, v1), cvt_pk_bf16(v2, v3)};
      else
        *reinterpret_cast<float4*>((float*)a.out + off) = float4{v0, v1, v2, v3};
    }
  if (a.lse && hi == 0) a.lse[qrow0] = empty ? -INFINITY : (mrun + log2f(lt)) * kLn2;
}

}  // namespace

hipError_t launch_prefill(const PrefillArgs& a, hipStream_t s) {
  const int G = a.Hq / a.Hkv;
  const int Mq = (a.Tq + BLK - 1) / BLK;
  const long n = (long)Mq * a.B * a.Hkv * ((G + 3) / 4);
  if (n <= 0) return hipSuccess;
  prefill_kernel<<<dim3((unsigned)n), kWaves * kWave, 0, s>>>(a);
  return hipGetLastError();
}

}  // namespace spa
