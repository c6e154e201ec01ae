// Sparse flash-decode over the selected tokens, split over waves, merged by
// log-sum-exp.
//
// HGA page, "Atención Exacta de Token": the output is a standard softmax over
// exactly the selected tokens.  RTPurbo page §1: retrieval heads attend the
// selected blocks, local heads attend attention-sink tokens plus a sliding
// window; §5 of the same page motivates a bandwidth-first decode kernel.
//
// Work decomposition (MI355X: 256 CUs, HBM-bound gather):
//   * an "item" is one (sequence b, KV head g); its tokens are cut into 32-token
//     tiles (a selected 64-token block is two tiles);
//   * all items' tiles are laid end to end and split over a persistent grid
//     of waves in contiguous ranges (at least 2 tiles per wave for bf16; the
//     waves of each compute unit's second workgroup take 80 % of a first-slot
//     wave's share, see make_split), so load balance does not depend on how
//     budgets vary per sequence (dual top-p gives 21..185 blocks per
//     sequence);
//   * a wave writes one partial (unnormalised o, running max m, running sum l)
//     per item it touched, into slot item + wave; a second kernel merges the
//     partials of item i (slots i + w for the waves w whose ranges hold its
//     first to last tile) by log-sum-exp.  (Merging inside the main kernel
//     would need a device-scope release per wave, which on this chip writes
//     back and invalidates the whole L2 of the XCD: far slower than a launch.)
//
// bf16 tile (d = 128 shown; d = 64 halves the d-steps and the V^T rows; up to
// 16 query heads per KV head, GQA sharing: K/V are read once per KV head for
// all its query heads):
//   S^T[32 tok, 16 heads] = K[32, 128] . Q^T     (2 x 4 MFMA 16x16x32 bf16)
//   O^T[128, 16 heads]   += V^T[128, 32] . P^T   (8 MFMA 16x16x32 bf16)
//   - K feeds the A operand straight from HBM: lane (row m, group g4) loads 16
//     bytes of token m; the d-order of the contraction is permuted identically
//     in Q, so no transposition is needed.
//   - V is loaded so that the 16 lanes of a group read one token's whole
//     256-byte row; each lane then holds 8 tokens x 8 dims and an in-register
//     8x8 transpose (byte permutes) forms the V^T operands whose rows are
//     d = 8m + jj.  No LDS round trip.
//   - P^T needs no data movement: the C layout of S^T already puts each
//     lane's 8 token probabilities where the B operand wants them.
//   - each wave walks its tile range in one flat loop with two tiles in
//     flight (register ring), prefetching across item boundaries; tile
//     descriptors (item, first token, valid count) are computed 64 at a time,
//     one per lane, so no tile waits on a dependent index load.
// fp32 tile (d in {64, 128}): plain VALU version of the same online softmax.
#include <algorithm>
#include <atomic>
#include <mutex>

#include "spa_internal.h"

namespace spa {

namespace {

constexpr int kWPB = 4;
constexpr int kThreads = kWPB * kWave;
constexpr int kMaxItems = 4096;
constexpr int kTile = 32;
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
// two floats to a bf16 pair, round to nearest even (one v_cvt_pk_bf16_f32)
__device__ __forceinline__ uint32_t cvt_pk_bf16(float lo, float hi) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2_t{lo, hi}, bf16x2_t));
}
constexpr size_t kHeader = 256;
constexpr int kQCache = 2;  // items whose Q a wave keeps in LDS
constexpr int kOcc = 2;     // bf16 workgroups (4 waves each) resident per CU
#ifndef SPA_SLOW_PCT
#define SPA_SLOW_PCT 80
#endif
constexpr int kSlowPct = SPA_SLOW_PCT;  // tiles of a second-slot wave per 100 of a first-slot wave

struct WsLayout {
  int* hdr;         // [0] total tiles, [1] workers, [2..5] the wave split (s1, s2, t1, half)
  int* item_start;  // [n_items + 1] first tile of each item (copy of the plan)
  float* part_ml;  // [slots][G][2]
  float* part_o;   // [slots][G][d]
};

__host__ __device__ inline size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

__host__ __device__ inline WsLayout ws_layout(void* ws, int n_items, int workers, int G, int d) {
  char* p = (char*)ws;
  WsLayout L;
  L.hdr = (int*)p;
  L.item_start = (int*)(p + kHeader);
  size_t off = kHeader + align256((size_t)(n_items + 1) * sizeof(int));
  const size_t slots = (size_t)n_items + workers;
  L.part_ml = (float*)(p + off);
  off += align256(slots * G * 2 * sizeof(float));
  L.part_o = (float*)(p + off);
  return L;
}

__host__ __device__ inline size_t ws_total(int n_items, int workers, int G, int d) {
  const size_t slots = (size_t)n_items + workers;
  return kHeader + align256((size_t)(n_items + 1) * sizeof(int)) + align256(slots * G * 2 * sizeof(float)) +
         align256(slots * G * d * sizeof(float));
}

// The persistent waves' tile ranges, in wave order: waves w < half take s1
// tiles each from tile 0, the others s2 each from tile t1 = half * s1 (the
// last ranges may be short or empty).  Every wave takes at least min_share
// tiles, so that small steps (few sequences) do not scatter into one-tile
// partials whose merge costs more than the attention itself.  slow_pct sets
// s2 relative to s1: the second half of the waves sit in each compute unit's
// second workgroup slot, and while both slots stream, the older workgroup's
// waves win the SIMDs' issue arbitration; measured per-wave timestamps put
// the second slot's tile rate at about two thirds of the first's, so an even
// split leaves the first slot idle for the last third of the kernel.  While
// both slots stream, HBM is the bound, so the gain is the tail only (1-2 %
// of the 128K decode attention at 80 %).
struct Split {
  int s1, s2, t1, half;
};

__host__ __device__ inline Split make_split(int total, int workers, int min_share, int slow_pct) {
  Split sp{0, 0, 0, workers / 2};
  if (total <= 0) return sp;
  const int rest = workers - sp.half;
  const long den = (long)sp.half * 100 + (long)rest * slow_pct;
  const long num = (long)total * 100 + den - 1;
  // a 32-bit division when it fits (the 64-bit one is a long instruction sequence)
  sp.s1 = max(min_share, num <= 0x7FFFFFFF ? (int)num / (int)den : (int)(num / den));
  sp.s2 = max(min_share, sp.s1 * slow_pct / 100);
  while ((long)sp.half * sp.s1 + (long)rest * sp.s2 < total) {
    ++sp.s1;
    sp.s2 = max(min_share, sp.s1 * slow_pct / 100);
  }
  sp.t1 = sp.half * sp.s1;
  return sp;
}
__device__ __forceinline__ int split_begin(const Split& sp, int w) {
  return w < sp.half ? w * sp.s1 : sp.t1 + (w - sp.half) * sp.s2;
}
__device__ __forceinline__ int split_len(const Split& sp, int w) { return w < sp.half ? sp.s1 : sp.s2; }
// the wave whose range holds tile t
__device__ __forceinline__ int split_wave(const Split& sp, int t) {
  return t < sp.t1 ? t / sp.s1 : sp.half + (t - sp.t1) / sp.s2;
}
// the split travels from the main kernel to the merge in the workspace header
__device__ __forceinline__ void store_split(const WsLayout& ws, int total, int workers, const Split& sp) {
  ws.hdr[0] = total;
  ws.hdr[1] = workers;
  ws.hdr[2] = sp.s1;
  ws.hdr[3] = sp.s2;
  ws.hdr[4] = sp.t1;
  ws.hdr[5] = sp.half;
}
__device__ __forceinline__ Split load_split(const WsLayout& ws) {
  return Split{ws.hdr[2], ws.hdr[3], ws.hdr[4], ws.hdr[5]};
}

__device__ __forceinline__ void wave_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// Row of idx / count that lists item (b, g)'s blocks: one list per sequence,
// or one per (sequence, KV head) with per-group selection.
__device__ __forceinline__ int list_row(const DecodeArgs& a, int b, int g) {
  return a.per_group ? b * a.Hkv + g : b;
}

// Number of 32-token tiles of item (b, g).  The head mode, the sequence
// length and the list count are loaded unconditionally (every row of count
// exists), so the three loads share one round trip.
__device__ __forceinline__ int item_tiles(const DecodeArgs& a, int b, int g, int tpb) {
  const int local = a.head_mode ? (int)a.head_mode[g] : 0;
  const int L = a.seq_len[b];
  const int cnt = a.count[list_row(a, b, g)];
  const int ns = min(a.sink_tok, L);
  const int wstart = max(ns, L - a.window_tok);
  const int local_tiles = (ns + kTile - 1) / kTile + (L - wstart + kTile - 1) / kTile;
  return local ? local_tiles : cnt * tpb;
}

// Block indices of a retrieval item, 64 at a time in the lanes of a wave, so
// a tile's address needs no dependent global load.
struct IdxWindow {
  int base;  // first block slot held
  int val;   // lane l holds the list entry base + l
};

__device__ __forceinline__ void load_window(const DecodeArgs& a, int row, int base, int cnt, IdxWindow& win) {
  const int l = threadIdx.x & (kWave - 1);
  win.base = base;
  win.val = base + l < cnt ? a.idx[(size_t)row * a.cap + base + l] : 0;
}

// First token and number of valid tokens of tile u of item (b, g).
__device__ __forceinline__ void tile_info(const DecodeArgs& a, int b, int g, int u, int tpb, int L,
                                          bool local, int cnt, IdxWindow& win, int& tok0, int& nvalid) {
  if (local) {
    const int ns = min(a.sink_tok, L);
    const int wstart = max(ns, L - a.window_tok);
    const int nst = (ns + kTile - 1) / kTile;
    if (u < nst) {
      tok0 = u * kTile;
      nvalid = min(kTile, ns - tok0);
    } else {
      tok0 = wstart + (u - nst) * kTile;
      nvalid = min(kTile, L - tok0);
    }
  } else {
    const int slot = u / tpb;
    if (slot - win.base >= kWave) load_window(a, list_row(a, b, g), slot, cnt, win);
    const int j = __builtin_amdgcn_readlane(win.val, slot - win.base);
    const int sub = u - slot * tpb;
    tok0 = j * a.blk + sub * kTile;
    nvalid = min(min(kTile, a.blk - sub * kTile), L - tok0);
  }
}

// Block-wide: item_start[] = exclusive prefix of item tile counts (in LDS),
// returns the total.  Every thread of the block must call it.
__device__ int build_plan(const DecodeArgs& a, int n_items, int* item_start, int* scratch) {
  const int tpb = (a.blk + kTile - 1) / kTile;
  const int tid = threadIdx.x;
  const int per = (n_items + kThreads - 1) / kThreads;
  const int i0 = tid * per;
  const int i1 = min(n_items, i0 + per);
  int local = 0;
  for (int it = i0; it < i1; ++it) {
    const int len = item_tiles(a, it / a.Hkv, it % a.Hkv, tpb);
    item_start[it] = local;  // provisional: offset inside this thread's run
    local += len;
  }
  // exclusive scan of per-thread totals
  const int lane = tid & (kWave - 1), wid = tid / kWave;
  const int x = wave_incl_scan_int(local);
  if (lane == kWave - 1) scratch[wid] = x;
  __syncthreads();
  int off = 0, tot = 0;
#pragma unroll
  for (int w = 0; w < kWPB; ++w) {
    off += (w < wid) ? scratch[w] : 0;
    tot += scratch[w];
  }
  off += x - local;
  for (int it = i0; it < i1; ++it) item_start[it] += off;
  if (tid == 0) item_start[n_items] = tot;
  __syncthreads();
  return tot;
}

// largest it in [0, n_items) with item_start[it] <= t
__device__ __forceinline__ int find_item(const int* item_start, int n_items, int t) {
  int lo = 0, hi = n_items - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (item_start[mid] <= t) lo = mid; else hi = mid - 1;
  }
  return lo;
}

// The same for a wave-uniform t (item_start[0] == 0 <= t), searched by the
// whole wave in two steps instead of a chain of dependent LDS reads: lane l
// compares the first item of segment l (segments of ceil(n_items / 64)
// items), then the items of the last segment that starts at or below t.
// Every lane of the wave must call it; n_items <= 4096.
__device__ __forceinline__ int find_item_wave(const int* item_start, int n_items, int t) {
  const int lane = threadIdx.x & (kWave - 1);
  const int seg = (n_items + kWave - 1) / kWave;
  const int i1 = lane * seg;
  const int c1 = __popcll(__ballot(i1 < n_items && item_start[i1] <= t));  // >= 1: item_start[0] = 0
  const int i2 = (c1 - 1) * seg + lane;
  const int c2 = __popcll(__ballot(lane < seg && i2 < n_items && item_start[i2] <= t));
  return (c1 - 1) * seg + c2 - 1;
}

// ------------------------------------------------------------- merging ----
// Items without any token (no selected block, empty window): out = 0, lse = -inf.
// Called by workgroup 0 after the plan; every thread of it must call.
__device__ void write_empty_items(const DecodeArgs& a, const int* item_start, int n_items, int G, int d,
                                  int* flag) {
  if (threadIdx.x == 0) *flag = 0;
  __syncthreads();
  for (int it = threadIdx.x; it < n_items; it += blockDim.x)
    if (item_start[it + 1] == item_start[it]) *flag = 1;
  __syncthreads();
  if (*flag == 0) return;
  const int per_item = G * d;
  for (long e = threadIdx.x; e < (long)n_items * per_item; e += blockDim.x) {
    const int it = (int)(e / per_item);
    if (item_start[it + 1] != item_start[it]) continue;
    const int r = (int)(e - (long)it * per_item);
    const int h = r / d, c = r - h * d;
    const int b = it / a.Hkv, g = it - (it / a.Hkv) * a.Hkv;
    const size_t orow = ((size_t)b * a.Hq + g * G + h) * d + c;
    if (a.out_bf16)
      ((uint16_t*)a.out)[orow] = 0;
    else
      ((float*)a.out)[orow] = 0.f;
    if (a.lse && c == 0) a.lse[(size_t)b * a.Hq + g * G + h] = -INFINITY;
  }
}

// ------------------------------------------------------------ bf16 path ----
// Head dimension DD = 128 or 64.  Per 32-token tile, with 16x16x32 MFMAs:
// S^T[32 tokens, 16 heads] = K . Q^T in 2 x DD/32 products (lane (m, g4)
// holds key row m of each 16-token half and d = 8 (4 j + g4) .. +7 of d-step
// j, the same d order as the Q operand), and O^T[DD, 16 heads] += V^T . P^T in
// VW = DD/16 products, lane m holding d = VW m .. VW m + VW-1 of 8 tokens.
template <int DD> struct Bf16Shape {
  static constexpr int KS = DD / 32;  // 32-wide d-steps of the score products
  static constexpr int VW = DD / 16;  // d values per lane of a V row: 8 (16 bytes) or 4 (8 bytes)
  static constexpr int VWORDS = VW / 2;
};

template <int DD>
struct TileRegs {
  uint4 k[2 * Bf16Shape<DD>::KS];            // [mt * KS + j]
  uint32_t v[8][Bf16Shape<DD>::VWORDS];      // [i][word]: VW bf16 of one token row
};

// Same operand layout through raw buffer loads on the (b, g) slab.  An offset
// past num_records returns zeros without touching memory, so a tile can be
// "loaded" as a placeholder at no cost: every loop iteration then issues the
// same number of loads, which keeps the compiler's in-order wait counts exact.
constexpr int kBufOOB = 0x7FFFFFF0;
constexpr int kBufNT = 2;  // cache policy: non-temporal

__device__ __forceinline__ uint4 buf_ld16(__amdgpu_buffer_rsrc_t r, int off) {
  const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, kBufNT);
  return uint4{v.x, v.y, v.z, v.w};
}

typedef unsigned u32x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint2 buf_ld8(__amdgpu_buffer_rsrc_t r, int off) {
  const u32x2 v = __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, kBufNT);
  return uint2{v.x, v.y};
}

template <int DD>
__device__ __forceinline__ void load_tile_buf(__amdgpu_buffer_rsrc_t rk, __amdgpu_buffer_rsrc_t rv, int tok0,
                                              int nvalid, bool real, int lane, TileRegs<DD>& t) {
  using SH = Bf16Shape<DD>;
  const int m = lane & 15, g4 = lane >> 4;
  const int nv = real ? nvalid : 1;
#pragma unroll
  for (int mt = 0; mt < 2; ++mt) {
    const int tau = min(16 * mt + m, nv - 1);
    const int row = real ? (tok0 + tau) * (DD * 2) : kBufOOB;
#pragma unroll
    for (int j = 0; j < SH::KS; ++j) t.k[mt * SH::KS + j] = buf_ld16(rk, row + (real ? 16 * (4 * j + g4) : 0));
  }
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int tau = min(16 * (i >> 2) + 4 * g4 + (i & 3), nv - 1);
    const int off = real ? (tok0 + tau) * (DD * 2) + 2 * SH::VW * m : kBufOOB;
    if constexpr (SH::VW == 8) {
      const uint4 u = buf_ld16(rv, off);
      t.v[i][0] = u.x;
      t.v[i][1] = u.y;
      t.v[i][2] = u.z;
      t.v[i][3] = u.w;
    } else {
      const uint2 u = buf_ld8(rv, off);
      t.v[i][0] = u.x;
      t.v[i][1] = u.y;
    }
  }
}

__device__ __forceinline__ bf16x8 as_bf16x8(const uint4& u) { return __builtin_bit_cast(bf16x8, u); }

template <int DD>
struct HeadState {
  float m;                           // running max of scaled logits (log2 domain), per column
  float l;                           // lane-partial running sum
  f32x4 o[Bf16Shape<DD>::VW];        // O^T accumulators, [jj] -> rows d = VW (4 g4 + r) + jj
};

template <int DD>
__device__ __forceinline__ void tile_math(const TileRegs<DD>& t, const bf16x8* qreg, int nvalid,
                                          float scale_log2, int lane, HeadState<DD>& st) {
  using SH = Bf16Shape<DD>;
  const int g4 = lane >> 4;
  f32x4 s[2];
#pragma unroll
  for (int mt = 0; mt < 2; ++mt) {
    s[mt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int j = 0; j < SH::KS; ++j)
      s[mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(t.k[mt * SH::KS + j]), qreg[j], s[mt], 0, 0, 0);
  }
  float x[8];
  float tmax = -INFINITY;
#pragma unroll
  for (int mt = 0; mt < 2; ++mt)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int tau = 16 * mt + 4 * g4 + r;
      const float v = tau < nvalid ? s[mt][r] * scale_log2 : -INFINITY;
      x[mt * 4 + r] = v;
      tmax = fmaxf(tmax, v);
    }
  tmax = fmaxf(tmax, lane_swap_f<16>(tmax));
  tmax = fmaxf(tmax, lane_swap_f<32>(tmax));
  // the running maximum is the reference of every probability: O and the
  // normaliser are rescaled whenever a tile raises it, so the largest
  // probability of the row so far is exp2(0) = 1, exact in the bf16 P
  // operand.  (A lazy reference that tolerated growth up to 2^8 left the
  // dominant weight at 2^x, rounded to 8 significant bits: on rows that a few
  // keys dominate, that rounding alone moved the output by up to 0.4 % of
  // |v|.  The extra rescales cost nothing measurable here: the kernel waits
  // on HBM.)
  const bool resc = tmax > st.m;
  const float m_new = resc ? tmax : st.m;
  // m_new is -inf only if every token seen so far is masked: nothing to add
  const float base = m_new == -INFINITY ? 0.f : m_new;
  const float corr = resc ? exp2f(st.m - base) : 1.f;
  float p[8];
  float psum = 0.f;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    p[e] = __builtin_amdgcn_exp2f(x[e] - base);
    psum += p[e];
  }
  st.l = st.l * corr + psum;
  st.m = m_new;
  if (__any((int)resc)) {
#pragma unroll
    for (int jj = 0; jj < SH::VW; ++jj) st.o[jj] *= corr;
  }
  // P^T operand: k index 8*g4 + e <-> token 16*(e/4) + 4*g4 + (e%4)
  const uint4 pu = {cvt_pk_bf16(p[0], p[1]), cvt_pk_bf16(p[2], p[3]), cvt_pk_bf16(p[4], p[5]),
                    cvt_pk_bf16(p[6], p[7])};
  const bf16x8 pb = as_bf16x8(pu);
#pragma unroll
  for (int jj = 0; jj < SH::VW; ++jj) {
    // V^T operand of output rows d = VW m + jj: element jj of each of the 8 token rows
    const int wsel = jj >> 1;
    uint32_t a4[4];
#pragma unroll
    for (int aa = 0; aa < 4; ++aa) {
      const uint32_t lo = t.v[2 * aa][wsel];
      const uint32_t hi = t.v[2 * aa + 1][wsel];
      a4[aa] = (jj & 1) ? ((lo >> 16) | (hi & 0xFFFF0000u)) : ((lo & 0xFFFFu) | (hi << 16));
    }
    const uint4 au = {a4[0], a4[1], a4[2], a4[3]};
    st.o[jj] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(au), pb, st.o[jj], 0, 0, 0);
  }
}

// Per-lane descriptors of 64 consecutive tiles of a wave's range: lane l
// describes tile base + l (its item, first token and valid-token count), so
// the tile loop only reads lanes (no dependent global loads per tile).
struct TileWindow {
  int base;
  int item, tok0, nvalid;
};

// it_lo is an item at or before the one holding tile base.  Lane l holds the
// next item boundary item_start[it_lo + 1 + l]: the item of tile base + l is
// it_lo plus the number of boundaries at or below it, counted over the
// boundaries inside the window (usually a few).  When all 64 boundaries lie
// inside the window (items of one tile or none), each lane searches.
// Every lane of the wave must call it.
__device__ __forceinline__ void fill_window(const DecodeArgs& a, const int* item_start, int n_items,
                                            int total, int tpb, int base, int it_lo, TileWindow& win) {
  const int lane = threadIdx.x & (kWave - 1);
  const int tt = base + lane;
  win.base = base;
  win.item = 0;
  win.tok0 = 0;
  win.nvalid = 0;
  const int bnd = item_start[min(it_lo + 1 + lane, n_items)];  // item_start[n_items] = total
  const int nb = __popcll(__ballot(bnd <= base + kWave - 1));
  int it_scan = it_lo;
  for (int k = 0; k < nb && nb < kWave; ++k) it_scan += __builtin_amdgcn_readlane(bnd, k) <= tt ? 1 : 0;
  if (tt < total) {
    const int it = nb < kWave ? it_scan : find_item(item_start, n_items, tt);
    const int u = tt - item_start[it];
    const int b = it / a.Hkv, g = it - (it / a.Hkv) * a.Hkv;
    // the list entry is loaded before the head mode is known (a local head's
    // tile reads a clamped, in-bounds entry and ignores it): one round trip
    const int slot = u / tpb;
    const int sub = u - slot * tpb;
    const int local = a.head_mode ? (int)a.head_mode[g] : 0;
    const int L = a.seq_len[b];
    const int j = a.idx[(size_t)list_row(a, b, g) * a.cap + min(slot, a.cap - 1)];
    win.item = it;
    if (local) {
      const int ns = min(a.sink_tok, L);
      const int wstart = max(ns, L - a.window_tok);
      const int nst = (ns + kTile - 1) / kTile;
      if (u < nst) {
        win.tok0 = u * kTile;
        win.nvalid = min(kTile, ns - win.tok0);
      } else {
        win.tok0 = wstart + (u - nst) * kTile;
        win.nvalid = min(kTile, L - win.tok0);
      }
    } else {
      win.tok0 = j * a.blk + sub * kTile;
      win.nvalid = min(min(kTile, a.blk - sub * kTile), L - win.tok0);
    }
  }
}

// grid: workers / 4 workgroups of 4 waves (kOcc per CU).  Each wave walks its
// tile range with two register buffers: the loads of tile t + 1 are issued
// before the math of tile t, across item boundaries; the Q operands of the
// wave's items are staged in LDS up front.  Two workgroups per CU (two waves per SIMD, <= 256 registers
// each) let one wave's math overlap the other's loads.
template <int OCC, int DD>
__global__ void __launch_bounds__(kThreads, OCC) decode_bf16_kernel(DecodeArgs a, int n_items, int workers) {
  using SH = Bf16Shape<DD>;
  constexpr int D = DD;
  __shared__ int item_start[kMaxItems + 1];
  __shared__ int scratch[kWPB];
  __shared__ uint4 qcache[kWPB][kQCache][4][kWave];  // Q operands of a wave's first items
  __shared__ int4 tdesc[kWPB][kWave];                 // descriptors of 64 consecutive tiles
  const int total = build_plan(a, n_items, item_start, scratch);
  const Split sp = make_split(total, workers, 2, kSlowPct);
  const int G = a.Hq / a.Hkv;
  WsLayout ws = ws_layout(a.ws, n_items, workers, G, D);
  if (blockIdx.x == 0) {
    for (int t = threadIdx.x; t <= n_items; t += kThreads) ws.item_start[t] = item_start[t];
    if (threadIdx.x == 0) store_split(ws, total, workers, sp);
    write_empty_items(a, item_start, n_items, G, D, &scratch[0]);
  }
  if (sp.s1 == 0) return;
  const int lane = threadIdx.x & (kWave - 1);
  const int w = blockIdx.x * kWPB + threadIdx.x / kWave;
  const int t0 = split_begin(sp, w);
  const int t1 = min(total, t0 + split_len(sp, w));
  if (t0 >= t1) return;

  const int tpb = (a.blk + kTile - 1) / kTile;
  const int m = lane & 15, g4 = lane >> 4;
  const float scale_log2 = a.scale * kLog2e;
  const uint16_t* q = (const uint16_t*)a.q;
  const uint16_t* kc = (const uint16_t*)a.k;
  const uint16_t* vc = (const uint16_t*)a.v;

  const int wv = threadIdx.x / kWave;
  const int it_first = find_item_wave(item_start, n_items, t0);
  // Tile descriptors sit in LDS: reading one is an LDS access, so it never
  // waits behind the K/V loads in flight (global loads complete in order).
  int win_base = t0;
  auto refill = [&](int base, int it_lo) {
    TileWindow win;
    fill_window(a, item_start, n_items, total, tpb, base, it_lo, win);
    wave_sync();
    tdesc[wv][lane] = int4{win.item, win.tok0, win.nvalid, 0};
    wave_sync();
    win_base = base;
  };
  refill(t0, it_first);
  // the wave's last item, from the window when the range fits in it
  const int it_last = t1 - t0 <= kWave ? __builtin_amdgcn_readfirstlane(tdesc[wv][t1 - 1 - t0].x)
                                       : find_item(item_start, n_items, t1 - 1);
  auto desc = [&](int t, int& it, int& tok0, int& nv) {
    // a later window starts at t: the item of tile t - 1 (the old window's
    // last lane) is a lower bound of t's
    if (t - win_base >= kWave) refill(t, __builtin_amdgcn_readfirstlane(tdesc[wv][kWave - 1].x));
    const int4 dd = tdesc[wv][t - win_base];
    it = __builtin_amdgcn_readfirstlane(dd.x);
    tok0 = __builtin_amdgcn_readfirstlane(dd.y);
    nv = __builtin_amdgcn_readfirstlane(dd.z);
  };
  auto load_q = [&](int it, uint4* qr) {
    const int b = it / a.Hkv, g = it - (it / a.Hkv) * a.Hkv;
#pragma unroll
    for (int j = 0; j < SH::KS; ++j) {
      uint4 qv = {0u, 0u, 0u, 0u};
      if (m < G) qv = *reinterpret_cast<const uint4*>(q + ((size_t)b * a.Hq + g * G + m) * D + 8 * (4 * j + g4));
      qr[j] = qv;
    }
  };
  bf16x8 qcur[SH::KS];
  auto set_q = [&](int it) {
    const int c = it - it_first;
    uint4 qr[SH::KS];
    if (c < kQCache) {
#pragma unroll
      for (int j = 0; j < SH::KS; ++j) qr[j] = qcache[wv][c][j][lane];
    } else {
      load_q(it, qr);
    }
#pragma unroll
    for (int j = 0; j < SH::KS; ++j) qcur[j] = as_bf16x8(qr[j]);
  };
  // (b, g) slab of the K and V caches as buffer resources
  const unsigned slab_bytes = (unsigned)((size_t)a.Tcap * D * 2);
  auto rsrc = [&](const uint16_t* base, int it) {
    it = __builtin_amdgcn_readfirstlane(it);  // the item is wave-uniform
    // item = b * Hkv + g is also the index of its [Tcap, d] slab
    const uintptr_t p = (uintptr_t)(base + (size_t)it * a.Tcap * D);
    const unsigned lo = __builtin_amdgcn_readfirstlane((unsigned)p);
    const unsigned hi = __builtin_amdgcn_readfirstlane((unsigned)(p >> 32));
    void* up = (void*)(((uintptr_t)hi << 32) | lo);
    return __builtin_amdgcn_make_buffer_rsrc(up, 0, slab_bytes, 0x00020000);
  };
  // placeholder loads (real == false) fetch nothing; a tile with no valid token
  // is one of them and its math is fully masked
  auto load_kv = [&](int it, int tok0, int nv, bool real, TileRegs<DD>& tr) {
    load_tile_buf<DD>(rsrc(kc, it), rsrc(vc, it), tok0, nv, real && nv > 0, lane, tr);
  };

  HeadState<DD> st;
  auto reset = [&]() {
    st.m = -INFINITY;
    st.l = 0.f;
#pragma unroll
    for (int jj = 0; jj < SH::VW; ++jj) st.o[jj] = f32x4{0.f, 0.f, 0.f, 0.f};
  };
  auto flush = [&](int item) {
    const size_t slot = (size_t)item + w;
    float lt = st.l;
    lt += lane_swap_f<16>(lt);
    lt += lane_swap_f<32>(lt);
    if (m < G) {
      // this lane's rows d = VW (4 g4 + r) + jj: VW consecutive d per r
      float* po = ws.part_o + (slot * G + m) * D + 4 * SH::VW * g4;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
#pragma unroll
        for (int q4 = 0; q4 < SH::VW / 4; ++q4) {
          const float4 o4 = {st.o[4 * q4][r], st.o[4 * q4 + 1][r], st.o[4 * q4 + 2][r], st.o[4 * q4 + 3][r]};
          *reinterpret_cast<float4*>(po + SH::VW * r + 4 * q4) = o4;
        }
      }
      if (g4 == 0) {
        ws.part_ml[(slot * G + m) * 2 + 0] = st.m;
        ws.part_ml[(slot * G + m) * 2 + 1] = lt;
      }
    }
  };

  // Two register buffers: tile t + 1 (or a placeholder after the last tile)
  // is requested before the math of tile t.
  TileRegs<DD> A, Bt;
  int itA, tokA, nvA, itB = 0, tokB = 0, nvB = 0;
  desc(t0, itA, tokA, nvA);
  // the first tile's K and V are requested before Q: the loads overlap, and
  // the wait for Q (loads complete in order) then covers the tile as well
  load_kv(itA, tokA, nvA, true, A);
  // Q of the wave's first kQCache items goes to LDS once, so an item switch
  // inside the tile loop reads LDS instead of waiting on a global load
  // (global loads complete in order, so that wait would drain the prefetch)
  {
    for (int c = 0; c < kQCache && it_first + c <= it_last; ++c) {
      uint4 qr[SH::KS];
      load_q(it_first + c, qr);
#pragma unroll
      for (int j = 0; j < SH::KS; ++j) qcache[wv][c][j][lane] = qr[j];
    }
  }
  set_q(itA);
  int cur = itA;
  reset();
  int t = t0;
  while (true) {
    const bool moreB = t + 1 < t1;
    if (moreB) desc(t + 1, itB, tokB, nvB);
    load_kv(moreB ? itB : itA, tokB, nvB, moreB, Bt);
    __builtin_amdgcn_sched_barrier(0);  // keep the prefetch ahead of the math
    tile_math(A, qcur, nvA, scale_log2, lane, st);
    if (!moreB) break;
    ++t;
    if (itB != cur) {
      flush(cur);
      cur = itB;
      reset();
      set_q(cur);
    }
    const bool moreA = t + 1 < t1;
    if (moreA) desc(t + 1, itA, tokA, nvA);
    load_kv(moreA ? itA : itB, tokA, nvA, moreA, A);
    __builtin_amdgcn_sched_barrier(0);
    tile_math(Bt, qcur, nvB, scale_log2, lane, st);
    if (!moreA) break;
    ++t;
    if (itA != cur) {
      flush(cur);
      cur = itA;
      reset();
      set_q(cur);
    }
  }
  flush(cur);
}

// ------------------------------------------------------------ fp32 path ----
// One wave per worker.  Scores: lane (tau, half) computes q_h . k_tau for the
// heads h = 2*hh + half.  The running max of every head is kept replicated in
// all lanes; probabilities and new maxima go through per-wave LDS, then every
// lane accumulates P.V for its d values.
template <int DD>
__global__ void __launch_bounds__(kThreads) decode_f32_kernel(DecodeArgs a, int n_items,
                                                              int workers) {
  __shared__ int item_start[kMaxItems + 1];
  __shared__ int scratch[kWPB];
  __shared__ float q_s[kWPB][16 * DD];
  __shared__ float p_s[kWPB][16][kTile];
  __shared__ float mnew_s[kWPB][16];
  const int total = build_plan(a, n_items, item_start, scratch);
  const Split sp = make_split(total, workers, 1, 100);  // an even split
  const int G = a.Hq / a.Hkv;
  WsLayout ws = ws_layout(a.ws, n_items, workers, G, DD);
  if (blockIdx.x == 0) {
    for (int t = threadIdx.x; t <= n_items; t += kThreads) ws.item_start[t] = item_start[t];
    if (threadIdx.x == 0) store_split(ws, total, workers, sp);
    write_empty_items(a, item_start, n_items, G, DD, &scratch[0]);
  }
  if (sp.s1 == 0) return;
  const int lane = threadIdx.x & (kWave - 1);
  const int wv = threadIdx.x / kWave;
  const int w = blockIdx.x * kWPB + wv;
  int t = split_begin(sp, w);
  const int t_end = min(total, t + split_len(sp, w));
  if (t >= t_end) return;
  const int tpb = (a.blk + kTile - 1) / kTile;
  const float scale_log2 = a.scale * kLog2e;
  const float* q = (const float*)a.q;
  const float* kc = (const float*)a.k;
  const float* vc = (const float*)a.v;
  constexpr int NDL = DD / kWave;  // d values per lane in P.V
  const int tau = lane & 31, half = lane >> 5;

  int item = find_item(item_start, n_items, t);
  while (t < t_end) {
    while (item_start[item + 1] <= t) ++item;
    const int seg_end = min(t_end, item_start[item + 1]);
    const int b = item / a.Hkv, g = item - (item / a.Hkv) * a.Hkv;
    const size_t kv_off = ((size_t)b * a.Hkv + g) * (size_t)a.Tcap * DD;
    // the sequence length, head mode, list count and first list window are
    // requested with Q: one round trip (window entries are clamped in bounds;
    // those past the count, and a local head's, go unused)
    const int row = list_row(a, b, g);
    const int L = a.seq_len[b];
    // (without head modes the byte is read from seq_len[b] and ignored, so the
    // load needs no branch that would wait for it at once)
    const uint8_t* hmp = a.head_mode ? a.head_mode + g : reinterpret_cast<const uint8_t*>(a.seq_len + b);
    const int hm_raw = *hmp;
    const int cnt_all = a.count[row];
    IdxWindow win;
    win.base = (t - item_start[item]) / tpb;
    win.val = a.idx[(size_t)row * a.cap + min(win.base + lane, a.cap - 1)];
    // Q of the item's G heads (contiguous, G * DD floats), every float4 of a
    // lane loaded before any is stored.  Indices past the end are clamped to
    // the last float4, so those lanes load and store it again (same value).
    constexpr int kQ4 = 16 * DD / 4 / kWave;  // float4 per lane for 16 heads
    const int nq4 = G * DD / 4;
    const f32x4* q4 = reinterpret_cast<const f32x4*>(q + ((size_t)b * a.Hq + g * G) * DD);
    f32x4 qv[kQ4];
#pragma unroll
    for (int j = 0; j < kQ4; ++j) qv[j] = q4[min(lane + kWave * j, nq4 - 1)];
    wave_sync();
#pragma unroll
    for (int j = 0; j < kQ4; ++j) reinterpret_cast<f32x4*>(q_s[wv])[min(lane + kWave * j, nq4 - 1)] = qv[j];
    wave_sync();
    const bool local = a.head_mode && hm_raw != 0;
    const int cnt = local ? 0 : cnt_all;
    float mrun[16], lrun[16], acc[16][NDL];
#pragma unroll
    for (int h = 0; h < 16; ++h) {
      mrun[h] = -INFINITY;
      lrun[h] = 0.f;
#pragma unroll
      for (int c = 0; c < NDL; ++c) acc[h][c] = 0.f;
    }
    for (int u = t - item_start[item]; u < seg_end - item_start[item]; ++u) {
      int tok0, nvalid;
      tile_info(a, b, g, u, tpb, L, local, cnt, win, tok0, nvalid);
      if (nvalid <= 0) continue;
      // the V values of every token of the tile are requested with the K rows,
      // before the scores: one round trip per tile.  Tokens past nvalid re-read
      // the last valid row; their probabilities are 0.
      const float* vbase = vc + kv_off + (size_t)tok0 * DD + lane;
      float vv[kTile][NDL];
#pragma unroll
      for (int tt = 0; tt < kTile; ++tt)
#pragma unroll
        for (int c = 0; c < NDL; ++c) vv[tt][c] = vbase[(size_t)min(tt, nvalid - 1) * DD + kWave * c];
      const float* krow = kc + kv_off + (size_t)(tok0 + min(tau, nvalid - 1)) * DD;
      float sc[8];
#pragma unroll
      for (int hh = 0; hh < 8; ++hh) sc[hh] = 0.f;
      for (int c = 0; c < DD; c += 4) {
        const float4 kv = *reinterpret_cast<const float4*>(krow + c);
#pragma unroll
        for (int hh = 0; hh < 8; ++hh) {
          const int h = 2 * hh + half;
          if (h < G) {
            const float* qh = &q_s[wv][h * DD + c];
            sc[hh] += qh[0] * kv.x + qh[1] * kv.y + qh[2] * kv.z + qh[3] * kv.w;
          }
        }
      }
#pragma unroll
      for (int hh = 0; hh < 8; ++hh) {
        const int h = 2 * hh + half;
        const float x = tau < nvalid ? sc[hh] * scale_log2 : -INFINITY;
        float mx = x;  // maximum over the 32 tokens of this half, by register lane moves
        mx = fmaxf(mx, __uint_as_float(lane_xor<1>(__float_as_uint(mx))));
        mx = fmaxf(mx, __uint_as_float(lane_xor<2>(__float_as_uint(mx))));
        mx = fmaxf(mx, __uint_as_float(lane_xor<4>(__float_as_uint(mx))));
        mx = fmaxf(mx, __uint_as_float(lane_xor<8>(__float_as_uint(mx))));
        mx = fmaxf(mx, __uint_as_float(lane_xor<16>(__float_as_uint(mx))));
        if (h < G) {
          const float m_new = fmaxf(mrun[h], mx);
          const float base = m_new == -INFINITY ? 0.f : m_new;
          p_s[wv][h][tau] = exp2f(x - base);
          if (tau == 0) mnew_s[wv][h] = m_new;
        }
      }
      wave_sync();
#pragma unroll
      for (int h = 0; h < 16; ++h) {
        if (h < G) {
          const float m_new = mnew_s[wv][h];
          const float base = m_new == -INFINITY ? 0.f : m_new;
          const float corr = exp2f(mrun[h] - base);
          mrun[h] = m_new;
#pragma unroll
          for (int c = 0; c < NDL; ++c) acc[h][c] *= corr;
          // every token of the tile in order (probability 0 past nvalid, which
          // leaves both sums unchanged)
          float ps = 0.f;
#pragma unroll
          for (int tt = 0; tt < kTile; ++tt) {
            const float pv = p_s[wv][h][tt];
            ps += pv;
#pragma unroll
            for (int c = 0; c < NDL; ++c) acc[h][c] += pv * vv[tt][c];
          }
          lrun[h] = lrun[h] * corr + ps;
        }
      }
      wave_sync();
    }
    const size_t slot = (size_t)item + w;
#pragma unroll
    for (int h = 0; h < 16; ++h)
      if (h < G) {
#pragma unroll
        for (int c = 0; c < NDL; ++c) ws.part_o[(slot * G + h) * DD + lane + kWave * c] = acc[h][c];
        if (lane == 0) {
          ws.part_ml[(slot * G + h) * 2 + 0] = mrun[h];
          ws.part_ml[(slot * G + h) * 2 + 1] = lrun[h];
        }
      }
    t = seg_end;
  }
}

// ----------------------------------------------------------------- merge ----
// One workgroup of 256 threads per (item, pair of query heads), so the merge
// spreads over all compute units (one workgroup per item, 1024 threads, took
// 60 % longer).  Thread (sub, pair) owns one float4 of one head and every
// nsub-th partial; it loads its partials BATCH (eight) at a time before
// combining them, so those loads are in flight together, and the nsub sums are added by
// log-sum-exp in LDS.  Items with no tile were written by workgroup 0 of the
// main kernel.  When the pair grid would leave most compute units idle and
// items have many partials (one sequence at 32K: 16 workgroups, up to 69
// partials each), one query head per workgroup with sixteen loads in flight
// spreads the same reads over twice the compute units.
constexpr int kMergeThreads = 256;

template <int GH, int BATCH>  // query heads per workgroup, partial loads of a thread in flight together
__global__ void __launch_bounds__(kMergeThreads) decode_merge_kernel(DecodeArgs a, int n_items, int workers) {
  __shared__ float Ms_all[kMergeThreads];
  __shared__ float red[kMergeThreads];
  __shared__ float4 acc_s[kMergeThreads];
  const int G = a.Hq / a.Hkv;
  const int d = a.d;
  const int hgroups = (G + GH - 1) / GH;
  const int item = blockIdx.x / hgroups;
  const int hg = blockIdx.x - item * hgroups;
  WsLayout ws = ws_layout(a.ws, n_items, workers, G, d);
  const Split sp = load_split(ws);
  const int s0 = ws.item_start[item], s1 = ws.item_start[item + 1];
  if (s1 <= s0 || sp.s1 <= 0) return;
  const int w0 = split_wave(sp, s0);
  const int nparts = split_wave(sp, s1 - 1) - w0 + 1;
  const int per_head = d / 4;
  const int pairs = GH * per_head;  // <= 256 (GH * d <= 1024)
  const int nsub = kMergeThreads / pairs;
  const int tid = threadIdx.x;
  const int sub = tid / pairs;
  const int pair = tid - sub * pairs;
  const int hl = pair / per_head;
  const int h = hg * GH + hl;
  const int c4 = pair - hl * per_head;
  const bool active = sub < nsub && h < G;
  float M = -INFINITY, L = 0.f;
  float4 acc = {0.f, 0.f, 0.f, 0.f};
  if (active) {
    for (int p0 = sub; p0 < nparts; p0 += BATCH * nsub) {
      float2 ml[BATCH];
      float4 ow[BATCH];
#pragma unroll
      for (int e = 0; e < BATCH; ++e) {
        const int p = p0 + e * nsub;
        if (p < nparts) {
          const size_t slot = (size_t)item + w0 + p;
          ml[e] = *reinterpret_cast<const float2*>(ws.part_ml + (slot * G + h) * 2);
          ow[e] = *reinterpret_cast<const float4*>(ws.part_o + (slot * G + h) * d + 4 * c4);
        } else {
          ml[e] = float2{-INFINITY, 0.f};
          ow[e] = float4{0.f, 0.f, 0.f, 0.f};
        }
      }
      float Mc = M;
#pragma unroll
      for (int e = 0; e < BATCH; ++e) Mc = fmaxf(Mc, ml[e].x);
      if (Mc != -INFINITY) {
        const float sc = exp2f(M - Mc);  // 0 while M is -inf
        L *= sc;
        acc.x *= sc;
        acc.y *= sc;
        acc.z *= sc;
        acc.w *= sc;
#pragma unroll
        for (int e = 0; e < BATCH; ++e) {
          if (ml[e].x == -INFINITY) continue;
          const float f = exp2f(ml[e].x - Mc);
          L += f * ml[e].y;
          acc.x += f * ow[e].x;
          acc.y += f * ow[e].y;
          acc.z += f * ow[e].z;
          acc.w += f * ow[e].w;
        }
        M = Mc;
      }
    }
  }
  Ms_all[tid] = M;
  red[tid] = L;
  acc_s[tid] = acc;
  __syncthreads();
  if (sub != 0 || !active) return;
  const int b = item / a.Hkv, g = item - (item / a.Hkv) * a.Hkv;
  for (int u = 1; u < nsub; ++u) M = fmaxf(M, Ms_all[u * pairs + pair]);
  if (M != -INFINITY) {
    const float f0 = exp2f(Ms_all[pair] - M);
    L *= f0;
    acc.x *= f0;
    acc.y *= f0;
    acc.z *= f0;
    acc.w *= f0;
    for (int u = 1; u < nsub; ++u) {
      const float mu = Ms_all[u * pairs + pair];
      if (mu == -INFINITY) continue;
      const float f = exp2f(mu - M);
      L += f * red[u * pairs + pair];
      const float4 o2 = acc_s[u * pairs + pair];
      acc.x += f * o2.x;
      acc.y += f * o2.y;
      acc.z += f * o2.z;
      acc.w += f * o2.w;
    }
  }
  float4 o = {0.f, 0.f, 0.f, 0.f};
  float lse_v = -INFINITY;
  if (M != -INFINITY && L > 0.f) {
    const float inv = 1.f / L;
    o = {acc.x * inv, acc.y * inv, acc.z * inv, acc.w * inv};
    lse_v = (M + log2f(L)) * kLn2;
  }
  const size_t orow = ((size_t)b * a.Hq + g * G + h) * d + 4 * c4;
  if (a.out_bf16) {
    const uint2 pk = {pack_bf16x2(o.x, o.y), pack_bf16x2(o.z, o.w)};
    *reinterpret_cast<uint2*>((uint16_t*)a.out + orow) = pk;
  } else {
    *reinterpret_cast<float4*>((float*)a.out + orow) = o;
  }
  if (a.lse && c4 == 0) a.lse[(size_t)b * a.Hq + g * G + h] = lse_v;
}

// Decode workspace for callers that cannot allocate (spa_sparse_decode_attn_noalloc):
// one file-scope device array per GPU the library runs on, held until the
// process ends.  Host code never passes the array's name to a kernel (on the
// host it is only a stand-in for the symbol); it looks up the array's device
// address once per device, with that device current, and uses that address.
// The decode kernels need nothing in it cleared: workgroup 0 writes the plan
// header and item offsets, every wave writes the partials it produces, and
// the merge reads only those.
constexpr size_t kScratchBytes = (size_t)16 << 20;
__device__ __align__(256) unsigned char scratch[kScratchBytes];
std::mutex g_scratch_lock;
void* g_scratch_addr[64];  // per device, guarded by g_scratch_lock

// Persistent decode workers per device, filled on first use.  Threads that
// race on the first call compute the same value, and the atomic makes the
// race well defined.  Devices past kMaxDevices are queried on every call.
constexpr int kMaxDevices = 64;
std::atomic<int> g_workers[kMaxDevices];

}  // namespace

int decode_workers() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) dev = 0;
  std::atomic<int>* slot = dev < kMaxDevices ? &g_workers[dev] : nullptr;
  if (slot) {
    const int cached = slot->load(std::memory_order_relaxed);
    if (cached > 0) return cached;
  }
  int cus = 256, v = 0;
  if (hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && v > 0) cus = v;
  // kOcc 4-wave workgroups per CU
  const int workers = cus * kOcc * kWPB;
  if (slot) slot->store(workers, std::memory_order_relaxed);
  return workers;
}

size_t decode_scratch_bytes() { return kScratchBytes; }

hipError_t decode_scratch(void** ptr) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= (int)(sizeof(g_scratch_addr) / sizeof(g_scratch_addr[0]))) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_lock);
  if (!g_scratch_addr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    g_scratch_addr[dev] = p;
  }
  *ptr = g_scratch_addr[dev];
  return hipSuccess;
}

size_t decode_ws_bytes(int B, int Hq, int Hkv, int d, int workers) {
  return ws_total(B * Hkv, workers, Hq / Hkv, d);
}

hipError_t launch_decode(const DecodeArgs& a, hipStream_t s) {
  const int n_items = a.B * a.Hkv;
  const int workers = decode_workers();
  const int blocks = workers / kWPB;
  if (a.io_bf16 && a.d == 64) {
    decode_bf16_kernel<kOcc, 64><<<blocks, kThreads, 0, s>>>(a, n_items, workers);
  } else if (a.io_bf16) {
    decode_bf16_kernel<kOcc, 128><<<blocks, kThreads, 0, s>>>(a, n_items, workers);
  } else if (a.d == 64) {
    decode_f32_kernel<64><<<blocks, kThreads, 0, s>>>(a, n_items, workers);
  } else {
    decode_f32_kernel<128><<<blocks, kThreads, 0, s>>>(a, n_items, workers);
  }
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int G = a.Hq / a.Hkv;
  // most partials an item can have: its most tiles (a full list, or the sink
  // and window of a local head) over the smallest wave share
  const int tpb = (a.blk + kTile - 1) / kTile;
  const int local_tiles = a.head_mode ? (a.sink_tok + a.window_tok) / kTile + 2 : 0;
  const int max_parts = std::max(a.cap * tpb, local_tiles) / (a.io_bf16 ? 2 : 1) + 1;
  if ((long)n_items * ((G + 1) / 2) < 64 && max_parts > 16) {
    decode_merge_kernel<1, 16><<<n_items * G, kMergeThreads, 0, s>>>(a, n_items, workers);
  } else {
    decode_merge_kernel<2, 8><<<n_items * ((G + 1) / 2), kMergeThreads, 0, s>>>(a, n_items, workers);
  }
  return hipGetLastError();
}

}  // namespace spa
