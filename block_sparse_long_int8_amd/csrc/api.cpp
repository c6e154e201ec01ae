// C ABI of the block-sparse attention library: argument validation, workspace
// sizing and kernel launches.  Every check runs on the host before anything is
// enqueued; a failed check launches nothing.  See include/spa.h for the
// contract of each entry point.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <mutex>
#include <string>

#include "../../include/spa.h"
#include "../../include/spa_probe.h"
#include "spa_internal.h"

namespace {

thread_local std::string g_last_error;

spa_status fail(spa_status code, const char* fn, const char* fmt, ...) __attribute__((format(printf, 3, 4)));
spa_status fail(spa_status code, const char* fn, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = std::string(fn) + ": " + buf;
  return code;
}

spa_status ok() {
  g_last_error.clear();
  return SPA_OK;
}

spa_status from_hip(hipError_t e, const char* fn) {
  if (e == hipSuccess) return ok();
  return fail(SPA_ERR_HIP, fn, "HIP launch error %d (%s)", (int)e, hipGetErrorString(e));
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

#define REQUIRE(cond, code, ...)                    \
  do {                                              \
    if (!(cond)) return fail(code, fn, __VA_ARGS__); \
  } while (0)

// ---- device-side checks ------------------------------------------------------

std::atomic<int> g_checks{-1};  // -1: not yet read from the environment
std::mutex g_checks_lock;       // one checked call at a time: they share the device word
thread_local int g_check_code = SPA_DBG_NONE;

bool checks_on() {
  int v = g_checks.load(std::memory_order_relaxed);
  if (v < 0) {
    const char* e = std::getenv("SPA_DEBUG_CHECKS");
    int want = e && e[0] == '1' && e[1] == 0;
    g_checks.compare_exchange_strong(v, want);
    v = g_checks.load(std::memory_order_relaxed);
  }
  return v == 1;
}

const char* check_name(int code) {
  switch (code) {
    case SPA_DBG_SEQ_LEN: return "seq_len outside its range";
    case SPA_DBG_COUNT: return "count outside [0, cap]";
    case SPA_DBG_IDX_RANGE: return "listed block outside its valid range";
    case SPA_DBG_IDX_ORDER: return "block list not strictly ascending";
    case SPA_DBG_HEAD_MODE: return "head_mode neither 0 nor 1";
    case SPA_DBG_Q_POS: return "q_pos outside [0, T)";
    case SPA_DBG_K_POS: return "k_pos outside [0, T)";
    case SPA_DBG_PERM_RANGE: return "perm value outside its segment";
    case SPA_DBG_PERM_DUP: return "perm value repeated in its segment";
    case SPA_DBG_TOK_POS: return "tok_pos outside [0, nKb*blk)";
    default: return "unknown violation";
  }
}

// With the checks on: run the call's check kernels (launch(s) enqueues them),
// wait, and turn a violation into SPA_ERR_INVALID_ARG.  With them off: SPA_OK.
template <class F>
spa_status device_checks(const char* fn, void* stream, F&& launch) {
  if (!checks_on()) return SPA_OK;
  g_check_code = SPA_DBG_NONE;
  hipStream_t s = (hipStream_t)stream;
  hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
  if (hipStreamIsCapturing(s, &cs) != hipSuccess || cs != hipStreamCaptureStatusNone)
    return fail(SPA_ERR_INVALID_ARG, fn, "device-side checks are on: the call waits for them and cannot be captured");
  std::lock_guard<std::mutex> lock(g_checks_lock);
  unsigned long long word = ~0ull;
  hipError_t e = spa::dbg_reset(s);
  if (e == hipSuccess) e = launch(s);
  if (e == hipSuccess) e = spa::dbg_fetch(&word, s);
  if (e != hipSuccess) return from_hip(e, fn);
  if (word == ~0ull) return SPA_OK;
  g_check_code = (int)(word >> 40);
  return fail(SPA_ERR_INVALID_ARG, fn, "device-side check: %s (element %llu)", check_name(g_check_code),
              word & ((1ull << 40) - 1));
}

#define DEVICE_CHECKS(...)                                                               \
  do {                                                                                   \
    const spa_status st_ = device_checks(fn, stream, [&](hipStream_t s_) -> hipError_t { \
      hipError_t e_ = hipSuccess;                                                        \
      __VA_ARGS__;                                                                       \
      return e_;                                                                         \
    });                                                                                  \
    if (st_ != SPA_OK) return st_;                                                       \
  } while (0)
#define CHECK_STEP(call) \
  if (e_ == hipSuccess) e_ = (call)

}  // namespace

extern "C" {

const char* spa_status_string(spa_status s) {
  switch (s) {
    case SPA_OK: return "SPA_OK";
    case SPA_ERR_INVALID_ARG: return "SPA_ERR_INVALID_ARG";
    case SPA_ERR_UNSUPPORTED: return "SPA_ERR_UNSUPPORTED";
    case SPA_ERR_WORKSPACE: return "SPA_ERR_WORKSPACE";
    case SPA_ERR_HIP: return "SPA_ERR_HIP";
    default: return "SPA_ERR_UNKNOWN";
  }
}

const char* spa_last_error(void) { return g_last_error.c_str(); }

int spa_version(void) { return 100; }

void spa_set_debug_checks(int on) { g_checks.store(on ? 1 : 0); }

int spa_debug_checks(void) { return checks_on() ? 1 : 0; }

int spa_debug_error(void) { return g_check_code; }

// ------------------------------------------------------------------ scores --

size_t spa_index_score_workspace_size(int B, int H_idx, int r, int Mq, int nKb, int mode) {
  if (mode != SPA_SCORE_PREFILL_TOKENS || B <= 0 || H_idx <= 0 || r <= 0) return 0;
  const size_t hr = (size_t)H_idx * r;
  return align256((size_t)B * (size_t)(Mq > 0 ? Mq : 0) * hr) + align256((size_t)B * (size_t)(nKb > 0 ? nKb : 0) * hr);
}

spa_status spa_index_score(const int8_t* qI, const int8_t* kI, const int8_t* w, int B, int H_idx,
                           int r, int Mq, int nKb, int q_blk0, const int32_t* seq_len,
                           const int32_t* tok_pos, int blk, int mode, int32_t* scores, void* ws,
                           size_t ws_bytes, void* stream) {
  const char* fn = "spa_index_score";
  REQUIRE(mode == SPA_SCORE_DECODE || mode == SPA_SCORE_PREFILL_POOLED || mode == SPA_SCORE_PREFILL_TOKENS ||
              mode == SPA_SCORE_DECODE_GROUPED,
          SPA_ERR_INVALID_ARG, "unknown mode %d", mode);
  REQUIRE(B >= 0 && Mq >= 0 && nKb >= 0 && q_blk0 >= 0, SPA_ERR_INVALID_ARG,
          "negative size (B=%d Mq=%d nKb=%d q_blk0=%d)", B, Mq, nKb, q_blk0);
  REQUIRE(H_idx >= 1 && r >= 4 && r % 4 == 0, SPA_ERR_INVALID_ARG, "need H_idx >= 1 and r a positive multiple of 4 (H_idx=%d r=%d)", H_idx, r);
  REQUIRE((long)H_idx * r <= 1024, SPA_ERR_INVALID_ARG, "H_idx*r = %ld exceeds 1024 (int32 scores could overflow)", (long)H_idx * r);
  REQUIRE(blk >= 1, SPA_ERR_INVALID_ARG, "blk must be >= 1 (got %d)", blk);
  if (mode == SPA_SCORE_DECODE) REQUIRE(Mq == 1, SPA_ERR_INVALID_ARG, "decode mode needs Mq == 1 (got %d)", Mq);
  if (mode == SPA_SCORE_DECODE_GROUPED)
    REQUIRE(Mq >= 1 && H_idx % Mq == 0, SPA_ERR_INVALID_ARG, "grouped decode needs Mq groups dividing H_idx (Mq=%d H_idx=%d)",
            Mq, H_idx);
  if (tok_pos) {
    REQUIRE(mode == SPA_SCORE_PREFILL_TOKENS, SPA_ERR_INVALID_ARG, "tok_pos needs mode SPA_SCORE_PREFILL_TOKENS");
    REQUIRE(!seq_len, SPA_ERR_UNSUPPORTED, "tok_pos with seq_len is not supported");
    REQUIRE((long)q_blk0 + Mq <= nKb, SPA_ERR_INVALID_ARG, "query blocks [%d, %ld) exceed nKb = %d with tok_pos",
            q_blk0, (long)q_blk0 + Mq, nKb);
    REQUIRE((long)nKb * blk <= 0x7FFFFFFFL, SPA_ERR_UNSUPPORTED, "nKb*blk exceeds the int32 range");
  }
  if (B == 0 || Mq == 0 || nKb == 0) return ok();
  REQUIRE(qI && kI && w && scores, SPA_ERR_INVALID_ARG, "null tensor pointer");
  REQUIRE(aligned16(qI) && aligned16(kI) && aligned16(scores), SPA_ERR_INVALID_ARG, "qI, kI and scores must be 16-byte aligned");
  hipStream_t s = (hipStream_t)stream;
  if (mode == SPA_SCORE_DECODE || mode == SPA_SCORE_DECODE_GROUPED)
    REQUIRE(seq_len, SPA_ERR_INVALID_ARG, "decode mode needs seq_len");
  if (mode != SPA_SCORE_DECODE && mode != SPA_SCORE_DECODE_GROUPED)
    REQUIRE(r == 16, SPA_ERR_UNSUPPORTED, "prefill scoring supports r == 16 only (got %d)", r);
  if (mode == SPA_SCORE_PREFILL_TOKENS) {
    const size_t need = spa_index_score_workspace_size(B, H_idx, r, Mq, nKb, mode);
    REQUIRE(ws && ws_bytes >= need, SPA_ERR_WORKSPACE, "workspace of %zu bytes needed, %zu given", need, ws_bytes);
    REQUIRE(aligned16(ws), SPA_ERR_INVALID_ARG, "workspace must be 16-byte aligned");
  }
  // every host-side check above; the device-side checks (when on) below
  if (seq_len) DEVICE_CHECKS(CHECK_STEP(spa::dbg_range_i32(seq_len, B, 1, (long long)nKb * blk, SPA_DBG_SEQ_LEN, s_)));
  if (tok_pos)
    DEVICE_CHECKS(CHECK_STEP(
        spa::dbg_range_i32(tok_pos, (long long)B * nKb * blk, 0, (long long)nKb * blk - 1, SPA_DBG_TOK_POS, s_)));
  if (mode == SPA_SCORE_DECODE || mode == SPA_SCORE_DECODE_GROUPED) {
    return from_hip(spa::launch_score_decode(qI, kI, w, B, H_idx, r, Mq, nKb, seq_len, blk, scores, s), fn);
  }
  const int8_t* qb = qI;
  const int8_t* kb = kI;
  if (mode == SPA_SCORE_PREFILL_TOKENS) {
    int8_t* pq = (int8_t*)ws;
    int8_t* pk = pq + align256((size_t)B * Mq * H_idx * r);
    const int npos = nKb * blk;
    hipError_t e = spa::launch_pool_pair(qI, tok_pos ? npos : Mq * blk, q_blk0 * blk, q_blk0 * blk, Mq, kI, npos, nKb,
                                         B, H_idx, blk, seq_len, tok_pos, npos, pq, pk, s);
    if (e != hipSuccess) return from_hip(e, fn);
    qb = pq;
    kb = pk;
  }
  return from_hip(spa::launch_score_prefill(qb, kb, w, B, H_idx, Mq, nKb, q_blk0, seq_len, blk, scores, s), fn);
}

spa_status spa_quantize_selector_keys(const int8_t* kI, int64_t n_vec, int r, uint8_t* codes, uint8_t* exps,
                                      void* stream) {
  const char* fn = "spa_quantize_selector_keys";
  REQUIRE(n_vec >= 0, SPA_ERR_INVALID_ARG, "negative vector count");
  REQUIRE(r == 16, SPA_ERR_UNSUPPORTED, "int4 selector keys support r == 16 only (got %d)", r);
  if (n_vec == 0) return ok();
  REQUIRE(kI && codes && exps, SPA_ERR_INVALID_ARG, "null tensor pointer");
  REQUIRE(aligned16(kI) && aligned16(codes), SPA_ERR_INVALID_ARG, "kI and codes must be 16-byte aligned");
  return from_hip(spa::launch_quantize_keys(kI, (long)n_vec, codes, exps, (hipStream_t)stream), fn);
}

spa_status spa_index_score_q4(const int8_t* qI, const uint8_t* codes, const uint8_t* exps, const int8_t* w, int B,
                              int H_idx, int r, int Mq, int nKb, const int32_t* seq_len, int blk, int mode,
                              int32_t* scores, void* stream) {
  const char* fn = "spa_index_score_q4";
  REQUIRE(mode == SPA_SCORE_DECODE || mode == SPA_SCORE_DECODE_GROUPED, SPA_ERR_INVALID_ARG,
          "int4 keys support the decode modes only (got mode %d)", mode);
  REQUIRE(B >= 0 && Mq >= 0 && nKb >= 0, SPA_ERR_INVALID_ARG, "negative size (B=%d Mq=%d nKb=%d)", B, Mq, nKb);
  REQUIRE(blk >= 1, SPA_ERR_INVALID_ARG, "blk must be >= 1 (got %d)", blk);
  REQUIRE(H_idx >= 1, SPA_ERR_INVALID_ARG, "H_idx must be >= 1");
  if (mode == SPA_SCORE_DECODE) REQUIRE(Mq == 1, SPA_ERR_INVALID_ARG, "decode mode needs Mq == 1 (got %d)", Mq);
  else
    REQUIRE(Mq >= 1 && H_idx % Mq == 0, SPA_ERR_INVALID_ARG, "grouped decode needs Mq groups dividing H_idx (Mq=%d H_idx=%d)",
            Mq, H_idx);
  REQUIRE(r == 16 && H_idx <= 32 && (H_idx & (H_idx - 1)) == 0, SPA_ERR_UNSUPPORTED,
          "int4 scoring supports r == 16 and a power-of-two H_idx <= 32 (got r=%d, H_idx=%d)", r, H_idx);
  if (B == 0 || nKb == 0) return ok();
  REQUIRE(qI && codes && exps && w && scores && seq_len, SPA_ERR_INVALID_ARG, "null tensor pointer");
  REQUIRE(aligned16(qI) && aligned16(codes) && aligned16(scores), SPA_ERR_INVALID_ARG,
          "qI, codes and scores must be 16-byte aligned");
  DEVICE_CHECKS(CHECK_STEP(spa::dbg_range_i32(seq_len, B, 1, (long long)nKb * blk, SPA_DBG_SEQ_LEN, s_)));
  return from_hip(spa::launch_score_decode_q4(qI, codes, exps, w, B, H_idx, Mq, nKb, seq_len, blk, scores,
                                              (hipStream_t)stream),
                  fn);
}

// --------------------------------------------------------------- selection --

static spa_status select_common(const char* fn, const int32_t* scores, int B, int M, int nKb,
                                int q_blk0, const int32_t* seq_len, int blk, int n_sink, int n_local,
                                int prefill, int mode, int k, float beta, float p, int k_min,
                                int k_max, int32_t* idx, int32_t* count, int cap, void* stream,
                                const int8_t* qI = nullptr, const int8_t* kI = nullptr,
                                const int8_t* w = nullptr, int H = 0, int32_t* scores_out = nullptr,
                                bool hist = false) {
  REQUIRE(prefill == 0 || prefill == 1, SPA_ERR_INVALID_ARG, "prefill must be 0 or 1 (got %d)", prefill);
  REQUIRE(B >= 0 && M >= 0 && nKb >= 0 && q_blk0 >= 0, SPA_ERR_INVALID_ARG, "negative size");
  REQUIRE(blk >= 1 && n_sink >= 0 && n_local >= 0, SPA_ERR_INVALID_ARG, "need blk >= 1, n_sink >= 0, n_local >= 0");
  if (!prefill && !scores) REQUIRE(M == 1, SPA_ERR_INVALID_ARG, "fused decode selection needs M == 1 (got %d)", M);
  const int budget = mode == 0 ? k : k_max;
  if (mode == 0) {
    REQUIRE(k >= 0, SPA_ERR_INVALID_ARG, "k must be >= 0 (got %d)", k);
  } else {
    REQUIRE(std::isfinite(p) && p > 0.f && p <= 1.f, SPA_ERR_INVALID_ARG, "need 0 < p <= 1 (got %g)", (double)p);
    REQUIRE(std::isfinite(beta) && beta >= 0.f, SPA_ERR_INVALID_ARG, "need finite beta >= 0 (got %g)", (double)beta);
    REQUIRE(k_min >= 0 && k_min <= k_max, SPA_ERR_INVALID_ARG, "need 0 <= k_min <= k_max (got %d, %d)", k_min, k_max);
  }
  // a row lists distinct blocks below nKb: reserved + budget, at most nKb of them
  const long need_cap = std::min((long)nKb, (long)n_sink + n_local + budget + (prefill ? 1 : 0));
  REQUIRE(cap >= 1 && (long)cap >= need_cap, SPA_ERR_INVALID_ARG, "cap %d < min(nKb, reserved + budget) = %ld", cap,
          need_cap);
  REQUIRE(nKb <= spa::select_max_blocks(), SPA_ERR_UNSUPPORTED, "nKb %d exceeds %d", nKb, spa::select_max_blocks());
  if (B == 0 || M == 0) return ok();
  REQUIRE((scores || (qI && kI && w)) && idx && count, SPA_ERR_INVALID_ARG, "null tensor pointer");
  if (!prefill) REQUIRE(seq_len, SPA_ERR_INVALID_ARG, "decode selection needs seq_len");
  REQUIRE(aligned16(scores) && aligned16(idx) && aligned16(count) && aligned16(qI) && aligned16(kI) &&
              aligned16(scores_out),
          SPA_ERR_INVALID_ARG, "scores, idx, count, qI, kI and scores_out must be 16-byte aligned");
  if (seq_len) DEVICE_CHECKS(CHECK_STEP(spa::dbg_range_i32(seq_len, B, 1, (long long)nKb * blk, SPA_DBG_SEQ_LEN, s_)));
  spa::SelectArgs a;
  a.scores = scores;
  a.B = B;
  a.M = M;
  a.nKb = nKb;
  a.q_blk0 = q_blk0;
  a.seq_len = seq_len;
  a.blk = blk;
  a.n_sink = n_sink;
  a.n_local = n_local;
  a.prefill = prefill;
  a.mode = mode;
  a.k = k;
  a.beta = beta;
  a.p = p;
  a.k_min = k_min;
  a.k_max = k_max;
  a.idx = idx;
  a.count = count;
  a.cap = cap;
  a.qI = qI;
  a.kI = kI;
  a.w = w;
  a.H = H;
  a.scores_out = scores_out;
  return from_hip(hist ? spa::launch_select_hist(a, (hipStream_t)stream) : spa::launch_select(a, (hipStream_t)stream),
                  fn);
}

spa_status spa_score_select_decode(const int8_t* qI, const int8_t* kI, const int8_t* w, int B, int H_idx,
                                   int r, int nKb, const int32_t* seq_len, int blk, int n_sink,
                                   int n_local, int mode, int k, float beta, float p, int k_min,
                                   int k_max, int32_t* scores_out, int32_t* idx, int32_t* count,
                                   int cap, void* stream) {
  const char* fn = "spa_score_select_decode";
  REQUIRE(mode == 0 || mode == 1, SPA_ERR_INVALID_ARG, "mode must be 0 (top-k) or 1 (top-p), got %d", mode);
  REQUIRE(H_idx >= 1 && r >= 4 && r % 4 == 0, SPA_ERR_INVALID_ARG, "need H_idx >= 1 and r a positive multiple of 4 (H_idx=%d r=%d)", H_idx, r);
  REQUIRE(r == 16 && H_idx <= 64 && (H_idx & (H_idx - 1)) == 0, SPA_ERR_UNSUPPORTED,
          "fused scoring supports r == 16 and a power-of-two H_idx <= 64 (got r=%d, H_idx=%d)", r, H_idx);
  if (B > 0) REQUIRE(qI && kI && w, SPA_ERR_INVALID_ARG, "null indexer pointer");
  return select_common(fn, nullptr, B, 1, nKb, 0, seq_len, blk, n_sink, n_local, 0, mode, k, beta, p, k_min,
                       k_max, idx, count, cap, stream, qI, kI, w, H_idx, scores_out);
}

spa_status spa_select_topk(const int32_t* scores, int B, int M, int nKb, int q_blk0,
                           const int32_t* seq_len, int blk, int n_sink, int n_local, int prefill,
                           int k, int32_t* idx, int32_t* count, int cap, void* ws, size_t ws_bytes,
                           void* stream) {
  (void)ws;
  (void)ws_bytes;
  return select_common("spa_select_topk", scores, B, M, nKb, q_blk0, seq_len, blk, n_sink, n_local,
                       prefill, 0, k, 0.f, 1.f, 0, 0, idx, count, cap, stream);
}

spa_status spa_select_topp(const int32_t* scores, int B, int M, int nKb, int q_blk0,
                           const int32_t* seq_len, int blk, int n_sink, int n_local, int prefill,
                           float beta, float p, int k_min, int k_max, int32_t* idx, int32_t* count,
                           int cap, void* ws, size_t ws_bytes, void* stream) {
  (void)ws;
  (void)ws_bytes;
  return select_common("spa_select_topp", scores, B, M, nKb, q_blk0, seq_len, blk, n_sink, n_local,
                       prefill, 1, 0, beta, p, k_min, k_max, idx, count, cap, stream);
}

spa_status spa_select_topk_hist(const int32_t* scores, int B, int M, int nKb, int q_blk0,
                                const int32_t* seq_len, int blk, int n_sink, int n_local,
                                int prefill, int k, int32_t* idx, int32_t* count, int cap, void* ws,
                                size_t ws_bytes, void* stream) {
  (void)ws;
  (void)ws_bytes;
  return select_common("spa_select_topk_hist", scores, B, M, nKb, q_blk0, seq_len, blk, n_sink, n_local,
                       prefill, 0, k, 0.f, 1.f, 0, 0, idx, count, cap, stream, nullptr, nullptr, nullptr, 0,
                       nullptr, true);
}

spa_status spa_select_topp_hist(const int32_t* scores, int B, int M, int nKb, int q_blk0,
                                const int32_t* seq_len, int blk, int n_sink, int n_local,
                                int prefill, float beta, float p, int k_min, int k_max,
                                int32_t* idx, int32_t* count, int cap, void* ws, size_t ws_bytes,
                                void* stream) {
  (void)ws;
  (void)ws_bytes;
  return select_common("spa_select_topp_hist", scores, B, M, nKb, q_blk0, seq_len, blk, n_sink, n_local,
                       prefill, 1, 0, beta, p, k_min, k_max, idx, count, cap, stream, nullptr, nullptr, nullptr,
                       0, nullptr, true);
}

// ---------------------------------------------------------- decode attention --

size_t spa_sparse_decode_attn_workspace_size(int B, int Hq, int Hkv, int d) {
  if (B <= 0 || Hkv <= 0 || Hq <= 0 || d <= 0 || Hq % Hkv) return 0;
  return spa::decode_ws_bytes(B, Hq, Hkv, d, spa::decode_workers());
}

static spa_status decode_common(const char* fn, int per_group, const void* q, const void* k_cache,
                                const void* v_cache, int io_dtype, const int32_t* seq_len,
                                const int32_t* idx, const int32_t* count, int cap, int blk,
                                const uint8_t* head_mode, int local_sink_tok, int local_window_tok,
                                int B, int Hq, int Hkv, int d, int Tcap, float scale, void* out,
                                int out_dtype, float* lse, void* ws, size_t ws_bytes, void* stream) {
  REQUIRE(io_dtype == SPA_F32 || io_dtype == SPA_BF16, SPA_ERR_INVALID_ARG, "unknown io_dtype %d", io_dtype);
  REQUIRE(out_dtype == SPA_F32 || out_dtype == SPA_BF16, SPA_ERR_INVALID_ARG, "unknown out_dtype %d", out_dtype);
  REQUIRE(B >= 0 && Hq >= 1 && Hkv >= 1 && d >= 1 && Tcap >= 1, SPA_ERR_INVALID_ARG, "bad sizes (B=%d Hq=%d Hkv=%d d=%d Tcap=%d)", B, Hq, Hkv, d, Tcap);
  REQUIRE(Hq % Hkv == 0, SPA_ERR_INVALID_ARG, "Hq %d not a multiple of Hkv %d", Hq, Hkv);
  REQUIRE(cap >= 1 && local_sink_tok >= 0 && local_window_tok >= 0, SPA_ERR_INVALID_ARG, "need cap >= 1 and non-negative local sizes");
  REQUIRE(std::isfinite(scale), SPA_ERR_INVALID_ARG, "scale must be finite");
  REQUIRE(blk == 16 || blk == 32 || blk == 64 || blk == 128, SPA_ERR_UNSUPPORTED, "blk %d not in {16,32,64,128}", blk);
  REQUIRE(Hq / Hkv <= 16, SPA_ERR_UNSUPPORTED, "more than 16 query heads per KV head (%d)", Hq / Hkv);
  REQUIRE(d == 64 || d == 128, SPA_ERR_UNSUPPORTED, "decode supports d in {64,128} (got %d)", d);
  REQUIRE((long)B * Hkv <= 4096, SPA_ERR_UNSUPPORTED, "B*Hkv = %ld exceeds 4096", (long)B * Hkv);
  if (B == 0) return ok();
  REQUIRE(q && k_cache && v_cache && out && seq_len && idx && count, SPA_ERR_INVALID_ARG, "null tensor pointer");
  REQUIRE(aligned16(q) && aligned16(k_cache) && aligned16(v_cache) && aligned16(out) && aligned16(idx),
          SPA_ERR_INVALID_ARG, "tensor pointers must be 16-byte aligned");
  const size_t need = spa_sparse_decode_attn_workspace_size(B, Hq, Hkv, d);
  REQUIRE(ws && ws_bytes >= need, SPA_ERR_WORKSPACE, "workspace of %zu bytes needed, %zu given", need, ws_bytes);
  REQUIRE(aligned16(ws), SPA_ERR_INVALID_ARG, "workspace must be 16-byte aligned");
  DEVICE_CHECKS({
    CHECK_STEP(spa::dbg_range_i32(seq_len, B, 1, Tcap, SPA_DBG_SEQ_LEN, s_));
    if (head_mode) CHECK_STEP(spa::dbg_range_u8(head_mode, Hkv, 0, 1, SPA_DBG_HEAD_MODE, s_));
    const int rows_per_seq = per_group ? Hkv : 1;
    CHECK_STEP(spa::dbg_lists(idx, count, (long long)B * rows_per_seq, cap, rows_per_seq, seq_len, blk, 0, s_));
  });
  spa::DecodeArgs a;
  a.q = q;
  a.k = k_cache;
  a.v = v_cache;
  a.io_bf16 = io_dtype == SPA_BF16;
  a.seq_len = seq_len;
  a.idx = idx;
  a.count = count;
  a.cap = cap;
  a.blk = blk;
  a.per_group = per_group;
  a.head_mode = head_mode;
  a.sink_tok = local_sink_tok;
  a.window_tok = local_window_tok;
  a.B = B;
  a.Hq = Hq;
  a.Hkv = Hkv;
  a.d = d;
  a.Tcap = Tcap;
  a.scale = scale;
  a.out = out;
  a.out_bf16 = out_dtype == SPA_BF16;
  a.lse = lse;
  a.ws = ws;
  return from_hip(spa::launch_decode(a, (hipStream_t)stream), fn);
}

spa_status spa_sparse_decode_attn(const void* q, const void* k_cache, const void* v_cache,
                                  int io_dtype, const int32_t* seq_len, const int32_t* idx,
                                  const int32_t* count, int cap, int blk, const uint8_t* head_mode,
                                  int local_sink_tok, int local_window_tok, int B, int Hq, int Hkv,
                                  int d, int Tcap, float scale, void* out, int out_dtype,
                                  float* lse, void* ws, size_t ws_bytes, void* stream) {
  return decode_common("spa_sparse_decode_attn", 0, q, k_cache, v_cache, io_dtype, seq_len, idx, count,
                       cap, blk, head_mode, local_sink_tok, local_window_tok, B, Hq, Hkv, d, Tcap, scale,
                       out, out_dtype, lse, ws, ws_bytes, stream);
}

spa_status spa_sparse_decode_attn_grouped(const void* q, const void* k_cache, const void* v_cache,
                                          int io_dtype, const int32_t* seq_len, const int32_t* idx,
                                          const int32_t* count, int cap, int blk,
                                          const uint8_t* head_mode, int local_sink_tok,
                                          int local_window_tok, int B, int Hq, int Hkv, int d,
                                          int Tcap, float scale, void* out, int out_dtype, float* lse,
                                          void* ws, size_t ws_bytes, void* stream) {
  return decode_common("spa_sparse_decode_attn_grouped", 1, q, k_cache, v_cache, io_dtype, seq_len, idx,
                       count, cap, blk, head_mode, local_sink_tok, local_window_tok, B, Hq, Hkv, d, Tcap,
                       scale, out, out_dtype, lse, ws, ws_bytes, stream);
}

spa_status spa_sparse_decode_attn_noalloc(const void* q, const void* k_cache, const void* v_cache,
                                          int io_dtype, const int32_t* seq_len, const int32_t* idx,
                                          const int32_t* count, int cap, int blk,
                                          const uint8_t* head_mode, int local_sink_tok,
                                          int local_window_tok, int B, int Hq, int Hkv, int d,
                                          int Tcap, float scale, void* out, int out_dtype, float* lse,
                                          void* stream) {
  const char* fn = "spa_sparse_decode_attn_noalloc";
  const size_t need = spa_sparse_decode_attn_workspace_size(B, Hq, Hkv, d);
  const size_t have = spa::decode_scratch_bytes();
  REQUIRE(need <= have, SPA_ERR_UNSUPPORTED,
          "B=%d Hq=%d Hkv=%d d=%d needs %zu bytes of decode workspace; the library's own scratch holds %zu "
          "(use spa_sparse_decode_attn with a workspace)", B, Hq, Hkv, d, need, have);
  void* ws = nullptr;
  const hipError_t e = spa::decode_scratch(&ws);
  if (e != hipSuccess) return fail(SPA_ERR_HIP, fn, "scratch address lookup failed: %d (%s)", (int)e, hipGetErrorString(e));
  return decode_common(fn, 0, q, k_cache, v_cache, io_dtype, seq_len, idx, count, cap, blk, head_mode,
                       local_sink_tok, local_window_tok, B, Hq, Hkv, d, Tcap, scale, out, out_dtype, lse, ws, have,
                       stream);
}

// ----------------------------------------------------------------- prefill --

spa_status spa_block_sparse_prefill(const void* q, int q_blk0, int Tq, const void* k,
                                    const void* v, const int32_t* q_pos, const int32_t* k_pos,
                                    const int32_t* idx, const int32_t* count, int cap, int blk,
                                    int B, int Hq, int Hkv, int d, int T, float scale, void* out,
                                    int out_dtype, float* lse, int order, void* ws, size_t ws_bytes,
                                    void* stream) {
  const char* fn = "spa_block_sparse_prefill";
  (void)ws;
  (void)ws_bytes;
  REQUIRE(out_dtype == SPA_F32 || out_dtype == SPA_BF16, SPA_ERR_INVALID_ARG, "unknown out_dtype %d", out_dtype);
  REQUIRE(order >= 0 && order <= (SPA_ORDER_ORIGINAL | SPA_ORDER_KV_ORIGINAL), SPA_ERR_INVALID_ARG,
          "unknown order flags %d", order);
  REQUIRE(B >= 0 && Tq >= 0 && q_blk0 >= 0 && Hq >= 1 && Hkv >= 1 && d >= 1 && T >= 1 && cap >= 1,
          SPA_ERR_INVALID_ARG, "bad sizes");
  REQUIRE(Hq % Hkv == 0, SPA_ERR_INVALID_ARG, "Hq %d not a multiple of Hkv %d", Hq, Hkv);
  REQUIRE(std::isfinite(scale), SPA_ERR_INVALID_ARG, "scale must be finite");
  REQUIRE(blk == 64, SPA_ERR_UNSUPPORTED, "prefill supports blk == 64 only (got %d)", blk);
  REQUIRE(d == 128, SPA_ERR_UNSUPPORTED, "prefill supports d == 128 only (got %d)", d);
  REQUIRE((long)q_blk0 * blk + Tq <= T, SPA_ERR_INVALID_ARG, "query slots [%ld, %ld) exceed T = %d",
          (long)q_blk0 * blk, (long)q_blk0 * blk + Tq, T);
  if (B == 0 || Tq == 0) return ok();
  REQUIRE(q && k && v && idx && count && out, SPA_ERR_INVALID_ARG, "null tensor pointer");
  REQUIRE(aligned16(q) && aligned16(k) && aligned16(v) && aligned16(out), SPA_ERR_INVALID_ARG,
          "tensor pointers must be 16-byte aligned");
  DEVICE_CHECKS({
    const long long Mq = (Tq + blk - 1) / blk;
    CHECK_STEP(spa::dbg_lists(idx, count, (long long)B * Mq, cap, (int)Mq, nullptr, blk, (T + blk - 1) / blk, s_));
    if (q_pos && (order & SPA_ORDER_ORIGINAL))
      CHECK_STEP(spa::dbg_range_i32(q_pos, (long long)B * T, 0, T - 1, SPA_DBG_Q_POS, s_));
    if (k_pos && (order & SPA_ORDER_KV_ORIGINAL))
      CHECK_STEP(spa::dbg_range_i32(k_pos, (long long)B * T, 0, T - 1, SPA_DBG_K_POS, s_));
  });
  spa::PrefillArgs a;
  a.q = q;
  a.q_blk0 = q_blk0;
  a.Tq = Tq;
  a.k = k;
  a.v = v;
  a.q_pos = q_pos;
  a.k_pos = k_pos;
  a.idx = idx;
  a.count = count;
  a.cap = cap;
  a.blk = blk;
  a.B = B;
  a.Hq = Hq;
  a.Hkv = Hkv;
  a.d = d;
  a.T = T;
  a.scale = scale;
  a.out = out;
  a.out_bf16 = out_dtype == SPA_BF16;
  a.lse = lse;
  a.orig_order = (order & SPA_ORDER_ORIGINAL) != 0;
  a.kv_orig = (order & SPA_ORDER_KV_ORIGINAL) != 0;
  return from_hip(spa::launch_prefill(a, (hipStream_t)stream), fn);
}

// ------------------------------------------------------------- permutation --

size_t spa_importance_permutation_workspace_size(int B, int Hq, int T) {
  if (B <= 0 || Hq <= 0 || T <= 0) return 0;
  return spa::importance_ws_bytes(B, Hq, T);
}

spa_status spa_importance_permutation(const void* q, const void* k, int B, int Hq, int Hkv, int T, int d,
                                      const int32_t* seq_len, int proxy, float scale, int seg, float* imp,
                                      int32_t* perm, void* ws, size_t ws_bytes, void* stream) {
  const char* fn = "spa_importance_permutation";
  REQUIRE(B >= 0 && Hq >= 1 && Hkv >= 1 && d >= 1 && T >= 1, SPA_ERR_INVALID_ARG, "bad sizes (B=%d Hq=%d Hkv=%d d=%d T=%d)",
          B, Hq, Hkv, d, T);
  REQUIRE(Hq % Hkv == 0, SPA_ERR_INVALID_ARG, "Hq %d not a multiple of Hkv %d", Hq, Hkv);
  REQUIRE(std::isfinite(scale) && scale > 0.f, SPA_ERR_INVALID_ARG, "scale must be finite and positive");
  REQUIRE(seg >= 1, SPA_ERR_INVALID_ARG, "seg must be >= 1 (got %d)", seg);
  REQUIRE(proxy >= 1, SPA_ERR_INVALID_ARG, "proxy must be >= 1 (got %d)", proxy);
  REQUIRE(d == 128, SPA_ERR_UNSUPPORTED, "importance supports d == 128 only (got %d)", d);
  REQUIRE(proxy <= spa::importance_max_proxy(), SPA_ERR_UNSUPPORTED, "proxy %d exceeds %d queries", proxy,
          spa::importance_max_proxy());
  REQUIRE(seg <= spa::importance_max_seg(), SPA_ERR_UNSUPPORTED, "seg %d exceeds %d", seg, spa::importance_max_seg());
  REQUIRE(B <= 65535, SPA_ERR_UNSUPPORTED, "B %d exceeds 65535", B);
  if (B == 0) return ok();
  REQUIRE(q && k && imp && perm, SPA_ERR_INVALID_ARG, "null tensor pointer");
  REQUIRE(aligned16(q) && aligned16(k) && aligned16(imp) && aligned16(perm), SPA_ERR_INVALID_ARG,
          "tensor pointers must be 16-byte aligned");
  const size_t need = spa_importance_permutation_workspace_size(B, Hq, T);
  REQUIRE(ws && ws_bytes >= need, SPA_ERR_WORKSPACE, "workspace of %zu bytes needed, %zu given", need, ws_bytes);
  REQUIRE(aligned16(ws), SPA_ERR_INVALID_ARG, "workspace must be 16-byte aligned");
  if (seq_len) DEVICE_CHECKS(CHECK_STEP(spa::dbg_range_i32(seq_len, B, 1, T, SPA_DBG_SEQ_LEN, s_)));
  return from_hip(spa::launch_importance(q, k, B, Hq, Hkv, T, seq_len, proxy, scale, seg, imp, perm, ws,
                                         (hipStream_t)stream),
                  fn);
}

spa_status spa_segment_permute(const void* src, void* dst, int64_t outer, int T, size_t row_bytes,
                               const int32_t* perm, int seg, int inverse, void* stream) {
  const char* fn = "spa_segment_permute";
  REQUIRE(outer >= 0 && T >= 0 && row_bytes >= 1 && seg >= 1, SPA_ERR_INVALID_ARG, "bad sizes");
  REQUIRE(inverse == 0 || inverse == 1, SPA_ERR_INVALID_ARG, "inverse must be 0 or 1");
  REQUIRE(outer <= 65535, SPA_ERR_UNSUPPORTED, "outer %ld exceeds 65535", (long)outer);
  if (outer == 0 || T == 0) return ok();
  REQUIRE(src && dst && perm, SPA_ERR_INVALID_ARG, "null pointer");
  const uintptr_t s0 = (uintptr_t)src, d0 = (uintptr_t)dst;
  const uintptr_t n = (uintptr_t)outer * (uintptr_t)T * row_bytes;
  REQUIRE(s0 + n <= d0 || d0 + n <= s0, SPA_ERR_INVALID_ARG, "src and dst overlap");
  DEVICE_CHECKS(CHECK_STEP(spa::dbg_perm(perm, T, seg, s_)));
  return from_hip(spa::launch_permute(src, dst, outer, T, row_bytes, perm, inverse, (hipStream_t)stream), fn);
}

spa_status spa_probe_read(const void* buf, size_t bytes, int workgroups, uint32_t* sink, void* stream) {
  const char* fn = "spa_probe_read";
  REQUIRE(buf && sink, SPA_ERR_INVALID_ARG, "null pointer");
  REQUIRE(aligned16(buf), SPA_ERR_INVALID_ARG, "buf must be 16-byte aligned");
  REQUIRE(bytes > 0 && bytes % 16 == 0, SPA_ERR_INVALID_ARG, "bytes must be a positive multiple of 16 (got %zu)", bytes);
  REQUIRE(workgroups >= 1 && workgroups <= (1 << 20), SPA_ERR_INVALID_ARG, "workgroups %d outside 1..2^20", workgroups);
  return from_hip(spa::launch_probe_read(buf, bytes, workgroups, sink, (hipStream_t)stream), fn);
}

spa_status spa_probe_mfma_bf16(int workgroups, int iters, float* sink, void* stream) {
  const char* fn = "spa_probe_mfma_bf16";
  REQUIRE(sink, SPA_ERR_INVALID_ARG, "null pointer");
  REQUIRE(workgroups >= 1 && workgroups <= (1 << 20), SPA_ERR_INVALID_ARG, "workgroups %d outside 1..2^20", workgroups);
  REQUIRE(iters >= 1 && iters <= (1 << 24), SPA_ERR_INVALID_ARG, "iters %d outside 1..2^24", iters);
  return from_hip(spa::launch_probe_mfma_bf16(workgroups, iters, sink, (hipStream_t)stream), fn);
}

}  // extern "C"
