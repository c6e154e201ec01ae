/*
 * spa.h -- C ABI of the block-sparse long-context attention library (gfx950).
 *
 * One decode step of query-dependent block-sparse attention is
 *     spa_index_score -> spa_select_topk | spa_select_topp -> spa_sparse_decode_attn
 * (with one selection per KV group: spa_index_score (SPA_SCORE_DECODE_GROUPED)
 * -> spa_select_* with M = Hkv rows per sequence -> spa_sparse_decode_attn_grouped;
 * with the int4 selector cache, spa_index_score_q4 in place of spa_index_score,
 * the cache written by spa_quantize_selector_keys when keys enter it; the
 * spa_select_*_hist variants select without sorting)
 * and one permuted block-sparse prefill is
 *     [spa_importance_permutation ->] spa_index_score (prefill, tok_pos = the
 *     permutation) -> spa_select_topk (prefill) -> spa_block_sparse_prefill,
 *     every tensor in the original token order (the kernels apply the
 *     permutation; spa_segment_permute does it for other tensors)
 *
 * Conventions shared by every entry point:
 *   - Every tensor pointer is a DEVICE pointer to a dense row-major array with
 *     the layout stated at the call; the caller owns all buffers.  The library
 *     never allocates device memory: temporaries live in a caller-provided
 *     workspace sized by the matching *_workspace_size function.
 *   - Calls are asynchronous on the caller's stream (a hipStream_t passed as
 *     void*; NULL is the default stream).  Nothing synchronises, unless the
 *     device-side checks are on.
 *   - Arguments are validated on the host before anything is enqueued; on any
 *     error the function returns a negative status and launches nothing.
 *     Values inside device arrays (idx, count, perm, positions, seq_len) are
 *     trusted: they must satisfy the stated ranges.  The optional device-side
 *     checks (spa_set_debug_checks) verify them before a call's kernels run.
 *   - Pointers to bf16/fp32/int tensors must be 16-byte aligned.
 *   - The only process-wide state is a per-device cache of each GPU's
 *     compute-unit count, taken atomically on first use on that device (it
 *     sets the decode work split and so the decode workspace size; size and
 *     call with the same device current), and the on/off switch of the
 *     device-side checks.  Calls from several host threads, and calls on
 *     different streams, may run concurrently as long as their workspaces do
 *     not overlap.
 *   - bf16 is passed as its 16-bit pattern (uint16 storage).
 */
#ifndef SPA_H_
#define SPA_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef int spa_status;
#define SPA_OK 0
#define SPA_ERR_INVALID_ARG (-1) /* bad shape, null pointer, misalignment, cap too small */
#define SPA_ERR_UNSUPPORTED (-2) /* valid request outside what the kernels implement     */
#define SPA_ERR_WORKSPACE (-3)   /* workspace missing or smaller than required            */
#define SPA_ERR_HIP (-4)         /* the HIP runtime reported an error at launch           */

/* element types of attention inputs/outputs */
#define SPA_F32 0
#define SPA_BF16 1

/* row orders of spa_block_sparse_prefill (the two flags combine) */
#define SPA_ORDER_SLOT 0        /* every tensor in slot (permuted) order              */
#define SPA_ORDER_ORIGINAL 1    /* q, out, lse: the whole sequence, original order    */
#define SPA_ORDER_KV_ORIGINAL 2 /* k, v: original order, slot t's row is k_pos[b, t]  */

/* spa_index_score modes */
#define SPA_SCORE_DECODE 0         /* one query row per sequence against its key blocks  */
#define SPA_SCORE_PREFILL_POOLED 1 /* query blocks x key blocks, block vectors given     */
#define SPA_SCORE_PREFILL_TOKENS 2 /* as POOLED, per-token vectors pooled by the library */
#define SPA_SCORE_DECODE_GROUPED 3 /* as DECODE, one score row per group of indexer heads */

/* Human-readable name of a status code (static storage). */
const char* spa_status_string(spa_status s);

/* Detail of the last error returned on the calling host thread ("" if none). */
const char* spa_last_error(void);

/* Library version as major*10000 + minor*100 + patch. */
int spa_version(void);

/*
 * Device-side checks of the values inside device arrays.
 *
 * The entry points trust the contents of their device arrays (the host cannot
 * read them without waiting).  With the checks on, a call that reads such
 * arrays first launches check kernels over them on its stream, waits for them
 * (the call then blocks the host and cannot be captured into a graph: under
 * capture it returns SPA_ERR_INVALID_ARG) and, if a value breaks the call's
 * stated ranges, returns SPA_ERR_INVALID_ARG without launching anything else;
 * spa_last_error() names the violation and spa_debug_error() returns its code.
 * What is checked:
 *   seq_len       -- spa_index_score, spa_index_score_q4, spa_select_*,
 *                    spa_score_select_decode: 1 <= seq_len[b] <= nKb*blk;
 *                    spa_sparse_decode_attn*: 1 <= seq_len[b] <= Tcap;
 *                    spa_importance_permutation: 1 <= seq_len[b] <= T;
 *   block lists   -- spa_sparse_decode_attn* and spa_block_sparse_prefill:
 *                    0 <= count <= cap and the first count entries of each
 *                    row strictly ascending in [0, ceil(seq_len[b]/blk))
 *                    (decode) or [0, ceil(T/blk)) (prefill);
 *   head_mode     -- spa_sparse_decode_attn*: every entry 0 or 1;
 *   positions     -- spa_block_sparse_prefill: q_pos with SPA_ORDER_ORIGINAL,
 *                    k_pos with SPA_ORDER_KV_ORIGINAL, in [0, T);
 *                    spa_index_score: tok_pos in [0, nKb*blk);
 *   perm          -- spa_segment_permute: each perm[t] in t's segment and,
 *                    for seg <= 262144, no value twice in a segment.
 * The checks share one device word per GPU and run one call at a time in the
 * process (a lock); stream and current device must be the same GPU.
 * Off by default; the environment variable SPA_DEBUG_CHECKS=1 at the first
 * call switches them on, spa_set_debug_checks switches them at any time.
 */
#define SPA_DBG_NONE 0
#define SPA_DBG_SEQ_LEN 1    /* seq_len outside the call's range          */
#define SPA_DBG_COUNT 2      /* count outside [0, cap]                    */
#define SPA_DBG_IDX_RANGE 3  /* a listed block outside its valid range    */
#define SPA_DBG_IDX_ORDER 4  /* a list not strictly ascending             */
#define SPA_DBG_HEAD_MODE 5  /* head_mode neither 0 nor 1                 */
#define SPA_DBG_Q_POS 6      /* q_pos used as a row number, outside [0, T) */
#define SPA_DBG_K_POS 7      /* k_pos used as a row number, outside [0, T) */
#define SPA_DBG_PERM_RANGE 8 /* perm[t] outside t's segment              */
#define SPA_DBG_PERM_DUP 9   /* a value twice in one segment of perm      */
#define SPA_DBG_TOK_POS 10   /* tok_pos outside [0, nKb*blk)               */

/* Switch the device-side checks on (1) or off (0) for the whole process. */
void spa_set_debug_checks(int on);

/* 1 if the device-side checks are on, else 0. */
int spa_debug_checks(void);

/* Code (SPA_DBG_*) of the violation behind the last call on the calling host
   thread that ran the device-side checks; SPA_DBG_NONE if it found none. */
int spa_debug_error(void);

/*
 * spa_index_score -- int8 indexer block scores, exact in int32.
 *
 * Defined by the SpotAttention page, §1 "Arquitectura del Selector": a query
 * row's score for key block t is sum_h w_h * ReLU(qI_h . kI_{h,t}) over H_idx
 * indexer heads, with per-head projections of rank r (r = 16 on the RTPurbo
 * page, §2) given here as int8 vectors.  Products are accumulated exactly in
 * int32; the host rejects H_idx*r > 1024 so no score can overflow.
 *
 * mode SPA_SCORE_DECODE (Mq must be 1):
 *   qI [B, H_idx, r], kI [B, nKb, H_idx, r], w [B, H_idx]  ->  scores [B, nKb].
 *   Blocks j >= ceil(seq_len[b]/blk) get INT32_MIN.  seq_len [B] is required.
 * mode SPA_SCORE_DECODE_GROUPED (Mq = number of groups, dividing H_idx):
 *   per-KV-group selection (SparDA page, §2 "Indexador de Pronóstico
 *   Compacto": one forecast head set per GQA group).  Inputs as DECODE;
 *   group g sums only heads g*H_idx/Mq .. (g+1)*H_idx/Mq - 1 ->
 *   scores [B, Mq, nKb], the groups' rows adding up to the DECODE score.
 * mode SPA_SCORE_PREFILL_POOLED:
 *   qI [B, Mq, H_idx, r] are the pooled vectors of query blocks q_blk0..q_blk0+Mq-1,
 *   kI [B, nKb, H_idx, r] the pooled key-block vectors, w [B, Mq, H_idx]
 *   -> scores [B, Mq, nKb], defined for key blocks j < q_blk0 + i (strictly
 *   before the query block, and j < ceil(seq_len[b]/blk) when seq_len is given);
 *   INT32_MIN elsewhere.  seq_len may be NULL.
 * mode SPA_SCORE_PREFILL_TOKENS:
 *   per-token vectors; block i's vector is the mean of its blk slots' vectors
 *   (slots below seq_len), rounded to floor(mean + 1/2) (block importance by
 *   mean pooling, PBS-Attn page §4); the blocks are then scored as in POOLED
 *   mode.  Needs spa_index_score_workspace_size bytes.
 *   tok_pos == NULL: the tensors are in slot order, qI [B, Mq*blk, H_idx, r]
 *     the chunk's slots (its first row is block q_blk0's first slot) and kI
 *     [B, nKb*blk, H_idx, r] every key slot.
 *   tok_pos [B, nKb*blk] int32: the tensors are in the original token order,
 *     qI and kI [B, nKb*blk, H_idx, r], and slot t's vector is row
 *     tok_pos[b, t] (values in [0, nKb*blk)), so the segment permutation of
 *     PBS-Attn §2 happens inside the pooling.  Needs q_blk0 + Mq <= nKb and
 *     seq_len == NULL (else SPA_ERR_UNSUPPORTED).
 * tok_pos must be NULL in the other modes.
 * Supported: r % 4 == 0, 1 <= H_idx, H_idx*r <= 1024; PREFILL modes need r == 16.
 */
spa_status spa_index_score(const int8_t* qI, const int8_t* kI, const int8_t* w, int B, int H_idx,
                           int r, int Mq, int nKb, int q_blk0, const int32_t* seq_len,
                           const int32_t* tok_pos, int blk, int mode, int32_t* scores, void* ws,
                           size_t ws_bytes, void* stream);
size_t spa_index_score_workspace_size(int B, int H_idx, int r, int Mq, int nKb, int mode);

/*
 * spa_quantize_selector_keys / spa_index_score_q4 -- the selector key cache in
 * micro-scaled int4.
 *
 * SpotAttention page, §4 "Cuantización": the selector's key cache, separate
 * from the attention K/V cache, can be held in micro-scaled int4, cutting its
 * footprint without touching the attention path.  Here each r = 16 key vector
 * (one key block and indexer head) is one micro-block: codes c in [-8, 7] and
 * one power-of-two scale 2^e, e the smallest exponent for which every element
 * x gives floor(x / 2^e + 1/2) within [-8, 7] (that value is its code).  The
 * dequantised key c * 2^e is an exact integer, so scores stay exact int32.
 *
 * spa_quantize_selector_keys: kI [n_vec, 16] int8 (any leading layout, e.g.
 *   [B, nKb, H_idx, 16]) -> codes [n_vec, 8] uint8 (element 2i in the low
 *   nibble of byte i, 2i+1 in the high nibble, 4-bit two's complement) and
 *   exps [n_vec] uint8 (0..5).  Run when keys enter the cache.
 * spa_index_score_q4: spa_index_score's decode modes (SPA_SCORE_DECODE with
 *   Mq == 1, SPA_SCORE_DECODE_GROUPED with Mq groups) on the int4 cache:
 *   qI [B, H_idx, 16], codes [B, nKb, H_idx, 8], exps [B, nKb, H_idx] (as written
 *   above; exps are trusted to be those values), w [B, H_idx], seq_len [B]
 *   -> scores [B, Mq, nKb] with the dequantised keys in place of kI.
 * Supported: r == 16; scoring needs a power-of-two H_idx <= 32 (so no score can
 * overflow int32).  No workspace.
 */
spa_status spa_quantize_selector_keys(const int8_t* kI, int64_t n_vec, int r, uint8_t* codes, uint8_t* exps,
                                      void* stream);
spa_status spa_index_score_q4(const int8_t* qI, const uint8_t* codes, const uint8_t* exps, const int8_t* w, int B,
                              int H_idx, int r, int Mq, int nKb, const int32_t* seq_len, int blk, int mode,
                              int32_t* scores, void* stream);

/*
 * spa_select_topk -- static top-k block selection with reserved blocks.
 *
 * RTPurbo page §3 (fixed top-k budget) with the reserved blocks of the
 * SpotAttention page §3 (sink prefix and recency suffix always kept) and the
 * always-visible current chunk of the HGA page ("Mecanismo Central").
 * Per row, candidates are ranked by (score descending, block index ascending)
 * and the first min(k, #candidates) are kept.
 *
 * scores [B, M, nKb] int32 (as written by spa_index_score).
 * prefill == 0 (decode): with e = ceil(seq_len[b]/blk) valid blocks,
 *   reserved = {0..n_sink-1} and {e-n_local..e-1}; candidates = the other valid blocks.
 *   M is 1, or the number of KV groups with per-group scores: the M rows of
 *   sequence b (row b*M + g) all use seq_len[b].
 * prefill == 1: row i is query block a = q_blk0 + i; reserved = {0..n_sink-1} (those <= a),
 *   {a-n_local..a-1} and the diagonal {a}; candidates = the other blocks j < a.
 *   seq_len may be NULL (then every block below nKb is valid).
 * Output: idx [B, M, cap] int32, ascending block indices of reserved + chosen,
 *   padded with -1; count [B, M] int32 = number of valid entries.
 * Errors: SPA_ERR_INVALID_ARG if cap < min(nKb, n_sink + n_local + k (+1 in
 *   prefill)): no list is longer than that.
 * Supported: nKb <= 4096.  No workspace needed (ws may be NULL).
 */
spa_status spa_select_topk(const int32_t* scores, int B, int M, int nKb, int q_blk0,
                           const int32_t* seq_len, int blk, int n_sink, int n_local, int prefill,
                           int k, int32_t* idx, int32_t* count, int cap, void* ws, size_t ws_bytes,
                           void* stream);

/*
 * spa_select_topp -- dual top-p block selection.
 *
 * RTPurbo page §3 and SpotAttention page §3: the reserved sink / recency
 * blocks are always kept; over the remaining candidates (the residual
 * distribution) the masses softmax(beta * score) are accumulated in rank order
 * (score descending, index ascending) until the cumulative mass reaches p; the
 * prefix length is clamped to [k_min, k_max] (k_min is the floor of the
 * SpotAttention page, k_max a cap on the workspace of the attention step) and
 * to the number of candidates.  Masses are computed in fp32 on the device.
 * Arguments and outputs as spa_select_topk; cap >= min(nKb, n_sink + n_local +
 * k_max (+1 in prefill)).  0 < p <= 1, beta >= 0, 0 <= k_min <= k_max.
 */
spa_status spa_select_topp(const int32_t* scores, int B, int M, int nKb, int q_blk0,
                           const int32_t* seq_len, int blk, int n_sink, int n_local, int prefill,
                           float beta, float p, int k_min, int k_max, int32_t* idx, int32_t* count,
                           int cap, void* ws, size_t ws_bytes, void* stream);

/*
 * spa_select_topk_hist / spa_select_topp_hist -- the same selections without a
 * sort (arguments, outputs, limits and errors as spa_select_topk /
 * spa_select_topp).
 *
 * RTPurbo page §5 motivates a sort-free threshold for speed.  Rank order is
 * (score descending, index ascending), so the kept set of size k is every
 * candidate scoring above the rank-k score plus the lowest-index candidates
 * scoring equal to it.  Integer scores let a radix search over 256-bin LDS
 * histograms find that score exactly; top-p accumulates the softmax masses in
 * fixed point (38 fraction bits per mass, exact sums) and finds the rank at
 * which the cumulative mass first reaches p times the total.  Top-k lists are
 * identical to spa_select_topk's; top-p lists can differ from
 * spa_select_topp's only where a cumulative mass lies within fp32 rounding of
 * p (the two accumulate in different arithmetic).
 */
spa_status spa_select_topk_hist(const int32_t* scores, int B, int M, int nKb, int q_blk0,
                                const int32_t* seq_len, int blk, int n_sink, int n_local,
                                int prefill, int k, int32_t* idx, int32_t* count, int cap, void* ws,
                                size_t ws_bytes, void* stream);
spa_status spa_select_topp_hist(const int32_t* scores, int B, int M, int nKb, int q_blk0,
                                const int32_t* seq_len, int blk, int n_sink, int n_local,
                                int prefill, float beta, float p, int k_min, int k_max,
                                int32_t* idx, int32_t* count, int cap, void* ws, size_t ws_bytes,
                                void* stream);

/*
 * spa_score_select_decode -- spa_index_score (decode) and spa_select_topk /
 * spa_select_topp fused into one launch.
 *
 * Same definitions as the two calls it replaces (SpotAttention page §1 for the
 * score, RTPurbo page §3 and SpotAttention page §3 for the selection): each
 * sequence's workgroup computes its blocks' scores from qI [B, H_idx, 16],
 * kI [B, nKb, H_idx, 16] and w [B, H_idx] and selects from them directly, so
 * the scores never travel through HBM.  mode 0 = top-k (uses k), 1 = top-p
 * (uses beta, p, k_min, k_max); one row per sequence (no per-group mode).
 * scores_out [B, nKb] may be NULL; when given it
 * receives every block's score exactly as spa_index_score writes it.
 * Outputs and errors as spa_select_topk / spa_select_topp (decode rows).
 * Supported: r == 16, H_idx a power of two <= 64, nKb <= 4096.
 */
spa_status spa_score_select_decode(const int8_t* qI, const int8_t* kI, const int8_t* w, int B, int H_idx,
                                   int r, int nKb, const int32_t* seq_len, int blk, int n_sink,
                                   int n_local, int mode, int k, float beta, float p, int k_min,
                                   int k_max, int32_t* scores_out, int32_t* idx, int32_t* count,
                                   int cap, void* stream);

/*
 * spa_sparse_decode_attn -- exact softmax attention over the selected tokens.
 *
 * HGA page, "Atención Exacta de Token": a standard softmax over exactly the
 * selected token set.  RTPurbo page §1: retrieval heads read the selected
 * blocks, local heads read attention-sink tokens plus a sliding window.
 * Split over the selected tokens (each split keeps a running max and sum),
 * then a log-sum-exp merge.
 *
 * q [B, Hq, d]; k_cache, v_cache [B, Hkv, Tcap, d] (io_dtype SPA_BF16 or
 * SPA_F32); query head h reads KV head h / (Hq/Hkv).  The query is the token at
 * position seq_len[b]-1, already in the cache.
 * head_mode [Hkv] uint8 (NULL = all 0): 0 = retrieval head, attends the tokens
 *   of blocks idx[b, 0..count[b]-1] (idx [B, cap], count [B]) below seq_len;
 *   1 = local head, attends tokens [0, local_sink_tok) and
 *   [seq_len-local_window_tok, seq_len).
 * scale multiplies q.k (normally 1/sqrt(d)).
 * out [B, Hq, d] (out_dtype SPA_F32 or SPA_BF16); lse [B, Hq] fp32 natural-log
 * log-sum-exp of the scaled logits (may be NULL).  A head with no token gets
 * out = 0 and lse = -inf.
 * Supported: d in {64, 128} (bf16 or f32); Hq % Hkv == 0, Hq/Hkv <= 16;
 * blk in {16, 32, 64, 128}; B*Hkv <= 4096.
 * Workspace: spa_sparse_decode_attn_workspace_size bytes (depends on the
 * current device's compute-unit count).
 */
spa_status spa_sparse_decode_attn(const void* q, const void* k_cache, const void* v_cache,
                                  int io_dtype, const int32_t* seq_len, const int32_t* idx,
                                  const int32_t* count, int cap, int blk, const uint8_t* head_mode,
                                  int local_sink_tok, int local_window_tok, int B, int Hq, int Hkv,
                                  int d, int Tcap, float scale, void* out, int out_dtype,
                                  float* lse, void* ws, size_t ws_bytes, void* stream);
size_t spa_sparse_decode_attn_workspace_size(int B, int Hq, int Hkv, int d);

/*
 * spa_sparse_decode_attn_grouped -- spa_sparse_decode_attn with one block list
 * per KV head.
 *
 * SparDA page, §2 "Indexador de Pronóstico Compacto": each GQA group selects
 * its own blocks, so the query heads of KV head g attend the tokens of blocks
 * idx[b, g, 0..count[b, g]-1] (idx [B, Hkv, cap], count [B, Hkv], as
 * spa_select_* writes them for M = Hkv rows per sequence).  Every other
 * argument, the outputs, limits, errors and the workspace are those of
 * spa_sparse_decode_attn.
 */
spa_status spa_sparse_decode_attn_grouped(const void* q, const void* k_cache, const void* v_cache,
                                          int io_dtype, const int32_t* seq_len, const int32_t* idx,
                                          const int32_t* count, int cap, int blk,
                                          const uint8_t* head_mode, int local_sink_tok,
                                          int local_window_tok, int B, int Hq, int Hkv, int d,
                                          int Tcap, float scale, void* out, int out_dtype, float* lse,
                                          void* ws, size_t ws_bytes, void* stream);

/*
 * spa_sparse_decode_attn_noalloc -- spa_sparse_decode_attn for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation): no workspace argument.
 *
 * Arguments, outputs, limits and the arithmetic are those of
 * spa_sparse_decode_attn (the same kernels).  The workspace is a 16 MiB device
 * array that the library holds on each GPU it runs on until the process ends;
 * its address is looked up on the first call on each device (with that device
 * current).  The call allocates nothing and frees nothing.
 * Errors: SPA_ERR_UNSUPPORTED if spa_sparse_decode_attn_workspace_size(B, Hq,
 * Hkv, d) exceeds 16 MiB (about B*Hkv + 2048 <= 4032 partial slots at 8 query
 * heads per KV head); otherwise as spa_sparse_decode_attn.
 * Every call on one GPU shares that GPU's array: calls ordered on one stream are
 * fine, but two calls that may overlap in time on one GPU (different streams, or
 * different host threads without ordering) race and give undefined results.
 */
spa_status spa_sparse_decode_attn_noalloc(const void* q, const void* k_cache, const void* v_cache,
                                          int io_dtype, const int32_t* seq_len, const int32_t* idx,
                                          const int32_t* count, int cap, int blk,
                                          const uint8_t* head_mode, int local_sink_tok,
                                          int local_window_tok, int B, int Hq, int Hkv, int d,
                                          int Tcap, float scale, void* out, int out_dtype, float* lse,
                                          void* stream);

/*
 * spa_block_sparse_prefill -- causal attention of a query chunk over selected key blocks.
 *
 * PBS-Attn page: block-sparse attention that skips key blocks outside a
 * precomputed block list ("Declaración del Problema"), on token orders
 * permuted inside segments with causality kept on the original positions
 * (§2); HGA page: exact softmax over the selected tokens.
 *
 * The chunk is query slots q_blk0*blk .. q_blk0*blk+Tq-1.  q_pos, k_pos [B, T]
 * int32 give each slot's original position (NULL = identity).  Query slot u in block a = q_blk0 + i attends the
 * key slots t of blocks idx[b, i, 0..count[b,i]-1] (idx [B, Mq, cap], Mq =
 * ceil(Tq/blk), count [B, Mq]) with t < T and k_pos[t] <= q_pos[u].
 * order (flags) selects where rows are read and written:
 *   queries -- without SPA_ORDER_ORIGINAL, q [B, Hq, Tq, d], out [B, Hq, Tq, d]
 *     and lse [B, Hq, Tq] hold row u - q_blk0*blk for slot u; with it, q [B,
 *     Hq, T, d], out [B, Hq, T, d] and lse [B, Hq, T] are in the original token
 *     order, row q_pos[b, u] for slot u (only the chunk's rows are read and
 *     written);
 *   keys -- without SPA_ORDER_KV_ORIGINAL, k, v [B, Hkv, T, d] hold slot t in
 *     row t; with it, in row k_pos[b, t] (the original order).
 * With both flags the caller permutes nothing: the permutation of Q, K, V and
 * the inverse permutation of O (PBS-Attn §2) happen inside the kernel.  The
 * positions used as row numbers (q_pos with SPA_ORDER_ORIGINAL, k_pos with
 * SPA_ORDER_KV_ORIGINAL) must lie in [0, T): they live on the device and are
 * not checked.
 * out is SPA_F32 or SPA_BF16; lse fp32 (may be NULL).  A query with no visible
 * key gets out = 0 and lse = -inf.
 * Supported: bf16 inputs, d == 128, blk == 64, Hq % Hkv == 0.  No workspace.
 */
spa_status spa_block_sparse_prefill(const void* q, int q_blk0, int Tq, const void* k,
                                    const void* v, const int32_t* q_pos, const int32_t* k_pos,
                                    const int32_t* idx, const int32_t* count, int cap, int blk,
                                    int B, int Hq, int Hkv, int d, int T, float scale, void* out,
                                    int out_dtype, float* lse, int order, void* ws, size_t ws_bytes,
                                    void* stream);

/*
 * spa_importance_permutation -- importance-sorted segment permutation of the keys.
 *
 * PBS-Attn page, §3 "Permutación de Claves Basada en Importancia Global": the
 * last query block is a proxy for all queries; its attention probabilities,
 * mean-pooled over the proxy queries and all query heads, give one global
 * importance per key; inside each segment of seg tokens (§2) the keys are
 * ordered by descending importance, so heavy-hitter keys fill the first
 * blocks of their segment.
 *
 * q [B, Hq, T, d] and k [B, Hkv, T, d] bf16 in natural token order; query head h
 * reads KV head h / (Hq/Hkv).  With L = seq_len[b] (NULL = T for every
 * sequence; 1 <= L <= T) the proxy rows are the n = min(proxy, L) queries at
 * positions L-n .. L-1, each attending keys at positions <= its own with
 * softmax(scale * q.k).
 * Outputs: imp [B, T] fp32, the mean probability of each key over the Hq*n
 * proxy rows (0 for keys at or past L; a sequence's importances sum to 1);
 * perm [B, T] int32, for segment s the keys s*seg .. below L in order of
 * importance (descending, equal importances by position), then the keys at or
 * past L in their own order -- perm[b] maps every segment onto itself and is
 * the forward permutation of spa_segment_permute.
 * The order is decided on the fp32 importances as written to imp.
 * scale > 0 multiplies q.k (normally 1/sqrt(d)).
 * Supported: d == 128, 1 <= proxy <= 64, 1 <= seg <= 4096.
 * Workspace: spa_importance_permutation_workspace_size(B, Hq, T) bytes.
 */
spa_status spa_importance_permutation(const void* q, const void* k, int B, int Hq, int Hkv, int T, int d,
                                      const int32_t* seq_len, int proxy, float scale, int seg, float* imp,
                                      int32_t* perm, void* ws, size_t ws_bytes, void* stream);
size_t spa_importance_permutation_workspace_size(int B, int Hq, int T);

/*
 * spa_segment_permute -- gather or scatter rows through a segment-wise permutation.
 *
 * PBS-Attn page §1 (keys/values permuted in pairs leave the output unchanged,
 * permuted queries permute the output, the inverse restores the order) and §2
 * (permutations stay inside contiguous segments of seg tokens).
 * src and dst are viewed as [outer, T, row_bytes].  inverse == 0:
 * dst[o, t] = src[o, perm[t]]; inverse == 1: dst[o, perm[t]] = src[o, t].
 * perm [T] int32 must map every segment [s*seg, (s+1)*seg) onto itself
 * (checked only by the device-side checks).  src and dst must not overlap.  Pointers need 16-byte alignment
 * only when row_bytes % 16 == 0 (the fast path); otherwise any alignment.
 */
spa_status spa_segment_permute(const void* src, void* dst, int64_t outer, int T, size_t row_bytes,
                               const int32_t* perm, int seg, int inverse, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* SPA_H_ */
