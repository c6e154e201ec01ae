// Internal declarations shared by the HIP kernels and the C-ABI layer.
// gfx950 only: 64-wide waves, MFMA builtins of CDNA4.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace spa {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef int i32x16 __attribute__((ext_vector_type(16)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

// 16-byte load with the non-temporal (streaming) hint: data read once from
// HBM does not displace reusable lines in the caches.
__device__ __forceinline__ uint4 load_nt16(const void* p) {
  const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
  return uint4{v.x, v.y, v.z, v.w};
}

constexpr int kWave = 64;

// ---- bf16 bit helpers (bf16 is carried as uint16 bit patterns) ----------
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }
__device__ __forceinline__ uint32_t f32_to_bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return f32_to_bf16_rne(lo) | (f32_to_bf16_rne(hi) << 16);
}

// ---- cross-lane helpers ---------------------------------------------------
__device__ __forceinline__ float shfl_xor_f(float v, int m) { return __shfl_xor(v, m, kWave); }
__device__ __forceinline__ int shfl_xor_i(int v, int m) { return __shfl_xor(v, m, kWave); }

// Value of lane (l ^ M) for a compile-time M: DPP lane moves for M <= 8
// (quad permutes and row / half-row mirrors), a swizzle for 16, a permute for 32.
template <int M>
__device__ __forceinline__ unsigned lane_xor(unsigned v) {
  const int x = (int)v;
  if constexpr (M == 1) {
    return (unsigned)__builtin_amdgcn_mov_dpp(x, 0xB1, 0xF, 0xF, true);   // quad_perm [1,0,3,2]
  } else if constexpr (M == 2) {
    return (unsigned)__builtin_amdgcn_mov_dpp(x, 0x4E, 0xF, 0xF, true);   // quad_perm [2,3,0,1]
  } else if constexpr (M == 4) {
    const int h = __builtin_amdgcn_mov_dpp(x, 0x141, 0xF, 0xF, true);     // half-row mirror: l ^ 7
    return (unsigned)__builtin_amdgcn_mov_dpp(h, 0x1B, 0xF, 0xF, true);   // quad_perm [3,2,1,0]: ^ 3
  } else if constexpr (M == 8) {
    const int r = __builtin_amdgcn_mov_dpp(x, 0x140, 0xF, 0xF, true);     // row mirror: l ^ 15
    return (unsigned)__builtin_amdgcn_mov_dpp(r, 0x141, 0xF, 0xF, true);  // half-row mirror: ^ 7
  } else if constexpr (M == 16) {
    return (unsigned)__builtin_amdgcn_ds_swizzle(x, 0x401F);              // bitmask mode, xor 16
  } else {
    return (unsigned)__shfl_xor(x, M, kWave);
  }
}

// Wave-wide inclusive prefix sum in registers: row shifts by 1, 2, 4 and 8
// lanes scan each 16-lane row, then the last lane of row 0 is added to row 1
// and of row 2 to row 3 (row broadcast 15), and the last lane of row 1 to
// rows 2 and 3 (row broadcast 31).  Lanes with no source get the identity.
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ int dpp_or_zero(int v) {
  return __builtin_amdgcn_update_dpp(0, v, CTRL, ROW_MASK, 0xf, true);
}
__device__ __forceinline__ int wave_incl_scan_int(int x) {
  x += dpp_or_zero<0x111, 0xf>(x);  // row_shr:1
  x += dpp_or_zero<0x112, 0xf>(x);  // row_shr:2
  x += dpp_or_zero<0x114, 0xf>(x);  // row_shr:4
  x += dpp_or_zero<0x118, 0xf>(x);  // row_shr:8
  x += dpp_or_zero<0x142, 0xa>(x);  // row_bcast:15 into rows 1 and 3
  x += dpp_or_zero<0x143, 0xc>(x);  // row_bcast:31 into rows 2 and 3
  return x;
}
__device__ __forceinline__ float wave_incl_scan_float(float x) {
#define SPA_FSTEP(C, R) x += __builtin_bit_cast(float, dpp_or_zero<C, R>(__builtin_bit_cast(int, x)))
  SPA_FSTEP(0x111, 0xf);
  SPA_FSTEP(0x112, 0xf);
  SPA_FSTEP(0x114, 0xf);
  SPA_FSTEP(0x118, 0xf);
  SPA_FSTEP(0x142, 0xa);
  SPA_FSTEP(0x143, 0xc);
#undef SPA_FSTEP
  return x;
}

// Value of lane (l ^ M), M = 16 or 32, through the gfx950 lane swaps (VALU
// only, no LDS round trip; for a single dependent reduction step, where the
// swizzle or permute latency would show).  v_permlane16_swap exchanges 16-lane
// rows 1 and 3 of its first operand with rows 0 and 2 of its second, and
// v_permlane32_swap the upper half of the first with the lower half of the
// second; with both operands v, lane l finds lane l ^ M's value in the first
// result when bit M of l is set, else in the second.  All lanes of the wave
// must be active.
template <int M>
__device__ __forceinline__ float lane_swap_f(float v) {
  static_assert(M == 16 || M == 32, "lane_swap_f: lane distance 16 or 32");
  const unsigned u = __float_as_uint(v);
  if constexpr (M == 16) {
    const auto r = __builtin_amdgcn_permlane16_swap(u, u, false, false);
    return __uint_as_float((__lane_id() & 16) ? r[0] : r[1]);
  } else {
    const auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
    return __uint_as_float((__lane_id() & 32) ? r[0] : r[1]);
  }
}

// ---- launch plumbing --------------------------------------------------------
struct LaunchStatus {
  int code;  // 0 ok, else hipError_t value
};

// Score kernels (score.hip)
hipError_t launch_score_decode(const int8_t* qI, const int8_t* kI, const int8_t* w, int B, int H,
                               int r, int groups, int nKb, const int32_t* seq_len, int blk,
                               int32_t* scores, hipStream_t s);
hipError_t launch_quantize_keys(const int8_t* kI, long n_vec, uint8_t* codes, uint8_t* exps, hipStream_t s);
hipError_t launch_score_decode_q4(const int8_t* qI, const uint8_t* codes, const uint8_t* exps, const int8_t* w,
                                  int B, int H, int groups, int nKb, const int32_t* seq_len, int blk,
                                  int32_t* scores, hipStream_t s);
// Mean-pools per-token int8 vectors (r = 16, H heads) of the query chunk (Mq
// blocks from slot q_slot0) and of the keys (nKb blocks from slot 0), both in
// one launch.  Slot t is row t - row_off of its tensor (q_row_off for the
// queries, 0 for the keys), or row tok_pos[b, t] (tok_pos [B, npos]) if given.
hipError_t launch_pool_pair(const int8_t* q_tok, int q_rows, int q_slot0, int q_row_off, int Mq,
                            const int8_t* k_tok, int k_rows, int nKb, int B, int H, int blk,
                            const int32_t* seq_len, const int32_t* tok_pos, int npos, int8_t* q_out,
                            int8_t* k_out, hipStream_t s);
hipError_t launch_score_prefill(const int8_t* qIb, const int8_t* kIb, const int8_t* w, int B,
                                int H, int Mq, int nKb, int q_blk0, const int32_t* seq_len,
                                int blk, int32_t* scores, hipStream_t s);

// Selection kernels (select.hip)
struct SelectArgs {
  const int32_t* scores;
  int B, M, nKb, q_blk0;
  const int32_t* seq_len;
  int blk, n_sink, n_local, prefill;
  int mode;  // 0 top-k, 1 top-p
  int k;
  float beta, p;
  int k_min, k_max;
  int32_t* idx;
  int32_t* count;
  int cap;
  // fused decode scoring (scores == nullptr): int8 indexer inputs, r == 16
  const int8_t* qI;
  const int8_t* kI;
  const int8_t* w;
  int H;
  int32_t* scores_out;  // optional copy of every block's score
};
hipError_t launch_select(const SelectArgs& a, hipStream_t s);       // bitonic sort of the candidates
hipError_t launch_select_hist(const SelectArgs& a, hipStream_t s);  // radix threshold search, no sort
int select_max_blocks();

// Block ranges of selection row (b, i): valid blocks, reserved sink / local /
// diagonal blocks and the candidate range [c0, c1).
struct RowRange {
  int nbv, sink_end, loc0, loc1, diag, c0, c1, n_cand;
};
__device__ __forceinline__ RowRange row_range(const SelectArgs& a, int b, int i) {
  RowRange r;
  const int nKb = a.nKb;
  r.nbv = a.seq_len ? min(nKb, (a.seq_len[b] + a.blk - 1) / a.blk) : nKb;
  if (!a.prefill) {
    r.sink_end = min(a.n_sink, r.nbv);
    r.loc0 = max(0, r.nbv - a.n_local);
    r.loc1 = r.nbv;
    r.diag = -1;
    r.c0 = a.n_sink;
    r.c1 = r.nbv - a.n_local;
  } else {
    const int qa = a.q_blk0 + i;
    r.sink_end = min(min(a.n_sink, qa + 1), nKb);
    r.loc0 = max(0, qa - a.n_local);
    r.loc1 = min(qa, nKb);
    r.diag = qa < nKb ? qa : -1;
    r.c0 = a.n_sink;
    r.c1 = min(min(qa, r.nbv), qa - a.n_local);
  }
  r.n_cand = max(0, r.c1 - r.c0);
  return r;
}

// Decode attention (decode_attn.hip)
struct DecodeArgs {
  const void* q;
  const void* k;
  const void* v;
  int io_bf16;
  const int32_t* seq_len;
  const int32_t* idx;    // [B, cap], or [B, Hkv, cap] when per_group
  const int32_t* count;  // [B], or [B, Hkv] when per_group
  int cap, blk;
  int per_group;         // one block list per (sequence, KV head)
  const uint8_t* head_mode;
  int sink_tok, window_tok;
  int B, Hq, Hkv, d, Tcap;
  float scale;
  void* out;
  int out_bf16;
  float* lse;
  void* ws;
};
size_t decode_ws_bytes(int B, int Hq, int Hkv, int d, int workers);
int decode_workers();  // persistent workers (waves) for the current device
// The library's own decode workspace on the current device (a file-scope device
// array of decode_scratch_bytes(); its address is looked up once per device).
size_t decode_scratch_bytes();
hipError_t decode_scratch(void** ptr);
hipError_t launch_decode(const DecodeArgs& a, hipStream_t s);

// Key importance and importance-sorted segment permutation (importance.hip)
size_t importance_ws_bytes(int B, int Hq, int T);
int importance_max_proxy();
int importance_max_seg();
hipError_t launch_importance(const void* q, const void* k, int B, int Hq, int Hkv, int T,
                             const int32_t* seq_len, int proxy, float scale, int seg, float* imp,
                             int32_t* perm, void* ws, hipStream_t s);

// Block-sparse prefill (prefill_attn.hip)
struct PrefillArgs {
  const void* q;
  int q_blk0, Tq;
  const void* k;
  const void* v;
  const int32_t* q_pos;
  const int32_t* k_pos;
  const int32_t* idx;
  const int32_t* count;
  int cap, blk, B, Hq, Hkv, d, T;
  float scale;
  void* out;
  int out_bf16;
  float* lse;
  int orig_order;  // q, out, lse indexed by original position q_pos[b, slot] ([.., T, ..]) instead of slot
  int kv_orig;     // k, v in original order: slot t's row is k_pos[b, t]
};
hipError_t launch_prefill(const PrefillArgs& a, hipStream_t s);

// Segment permutation (permute.hip)
hipError_t launch_permute(const void* src, void* dst, int64_t outer, int T, size_t row_bytes,
                          const int32_t* perm, int inverse, hipStream_t s);

// rate probes of the device (probes.hip)
hipError_t launch_probe_read(const void* buf, size_t bytes, int workgroups, unsigned* sink, hipStream_t s);
hipError_t launch_probe_mfma_bf16(int workgroups, int iters, float* sink, hipStream_t s);


// ---- optional device-side checks (debug_checks.hip) ------------------------
// Each launches a check kernel on s that records violations in one device word;
// dbg_fetch copies the word back and synchronises s (all ones = no violation,
// else (code << 40) | element index).
hipError_t dbg_reset(hipStream_t s);
hipError_t dbg_range_i32(const int32_t* v, long long n, long long lo, long long hi, int code, hipStream_t s);
hipError_t dbg_range_u8(const uint8_t* v, long long n, long long lo, long long hi, int code, hipStream_t s);
hipError_t dbg_lists(const int32_t* idx, const int32_t* count, long long rows, int cap, int rows_per_seq,
                     const int32_t* seq_len, int blk, int nb, hipStream_t s);
hipError_t dbg_perm(const int32_t* perm, int T, int seg, hipStream_t s);
hipError_t dbg_fetch(unsigned long long* word, hipStream_t s);

}  // namespace spa
