/*
 * csa.h -- C ABI of libcsa, the MI355X (gfx950) compressed-sparse-attention
 * decode path: lightning-indexer scoring, causal top-k, gather, and shared-KV
 * MQA attention (plus the dense HCA variant), as described by the
 * nvfp4-megamoe-kernel design notes "ARCHITECTURE & MEMORY AUDIT" (post-probe
 * rewrite and the earlier 1M-context-viability audit) and "PART A -- Next
 * Session Clues".
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * - bf16 tensors are passed as uint16_t bit patterns.
 * - Every tensor pointer is a DEVICE pointer owned by the caller; layouts are
 *   row-major with the last index fastest and no padding.  Pointers to bf16
 *   and fp32 tensors must be 16-byte aligned.
 * - Per-token metadata arrays (pos, seq_kv, n_comp, ...) are device arrays of
 *   length T.  Caches of several sequences are concatenated ("packed"); token
 *   t's sequence starts at row seq_kv[t].
 * - Visible blocks of token t: n_vis[t] = min(floor(pos[t] / ratio), n_comp[t])
 *   -- a decode query sees only compressed blocks strictly before its own,
 *   incomplete block (PART A, suspect 3).
 * - Calls are asynchronous on `stream` (a hipStream_t; NULL = default stream).
 *   The library never allocates, frees or synchronises; it holds no global
 *   mutable state and is reentrant.  Scratch memory is the caller's `ws`.
 * - Host-side validation happens before any launch and returns CSA_EINVAL /
 *   CSA_EUNSUPPORTED / CSA_EWORKSPACE without touching the GPU.  A failed launch
 *   returns CSA_EHIP.  Conditions that only the device can see (a row index
 *   outside its buffer, more visible blocks than `ld`, ...) never cause an
 *   out-of-bounds access: the kernel skips or clamps the offending item and ORs
 *   a CSA_DERR_* bit into *err (a device uint32 word, may be NULL; never
 *   cleared by the library).
 * - There is no silent fallback: an unsupported shape is an error.
 */
#ifndef CSA_H_
#define CSA_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum csa_status {
  CSA_OK = 0,
  CSA_EINVAL = 1,        /* null required pointer, negative size, bad value   */
  CSA_EUNSUPPORTED = 2,  /* shape outside the compiled set (see each call)    */
  CSA_EWORKSPACE = 3,    /* ws NULL, misaligned (256 B) or smaller than needed */
  CSA_EHIP = 4,          /* the HIP runtime rejected a launch                  */
  CSA_ESCRATCH = 5       /* csa_decode_step_noalloc: workspace need above
                            CSA_NOALLOC_SCRATCH_BYTES                          */
} csa_status;

/* Device-side error bits ORed into *err. */
#define CSA_DERR_VIS_OVER_LD   0x1u  /* n_vis[t] > ld: only the first ld scores kept      */
#define CSA_DERR_KEY_RANGE     0x2u  /* seq_kv[t]+n_vis[t] > k_rows: token scored as 0 blocks */
#define CSA_DERR_BAD_META      0x4u  /* pos, n_comp or seq_kv < 0; one_sequence broken    */
#define CSA_DERR_ROW_RANGE     0x8u  /* gather/attend row outside its buffer: row zeroed / skipped */
#define CSA_DERR_COUNT_RANGE   0x10u /* count > top_k or swa_len > window: clamped        */
#define CSA_DERR_ROWS_OVER_MAX 0x20u /* a_len+b_len > max_rows: rows beyond max_rows ignored */

/* Human-readable name of a csa_status value. */
const char* csa_status_str(int status);

/* Version of this ABI (bumped on any signature change). */
int csa_abi_version(void);

/*
 * S1 -- lightning-indexer scores (post-probe audit, F1 and F3; eq. 16 of
 * DeepSeek-V4 sec. 2.3.1 as restated there):
 *     scores[t, s] = sum_{h < n_ih} w[t,h] * max(0, sum_{d < ihd} q_idx[t,h,d] * k_idx[seq_kv[t]+s, d])
 * for s < n_vis[t].  One key per block, shared by every indexer head.
 *   q_idx  [T, n_ih, ihd] bf16     w [T, n_ih] fp32
 *   k_idx  [k_rows, ihd] bf16      (packed keys of all sequences)
 *   scores [T, ld] fp32            entries s >= n_vis[t] are not written
 * bf16 products are accumulated in fp32 (MFMA); ReLU, weighting and the head
 * sum are fp32.  Supported: ihd in {32, 64, 128}; 1 <= n_ih <= 128;
 * ratio >= 1; ld >= 1; T >= 0 (T == 0 is a no-op).
 */
csa_status csa_index_score(const uint16_t* q_idx, const float* w,
                           const uint16_t* k_idx, int64_t k_rows,
                           const int64_t* pos, const int64_t* seq_kv, const int32_t* n_comp,
                           int T, int n_ih, int ihd, int ratio,
                           float* scores, int64_t ld, uint32_t* err, void* stream);

/*
 * S1 with narrow keys (post-probe audit, C4; 1M-context audit, M1/A2: indexer
 * keys and queries stored and multiplied in an 8-bit floating-point format).
 * q_idx [T, n_ih, ihd] and k_idx [k_rows, ihd] are OCP FP8 E4M3 codes (one
 * byte each: sign, 4 exponent bits with bias 7, 3 mantissa bits) with one
 * power-of-two scale per query head, q_scale [T, n_ih] fp32, and per key
 * block, k_scale [k_rows] fp32 (as csa_quantize_e4m3 makes them).  The score
 * is S1's formula on the dequantised values:
 *     scores[t, s] = sum_h w[t,h] * max(0, (q_scale[t,h] q[t,h]) . (k_scale[r] k[r])),
 *     r = seq_kv[t] + s,
 * computed as k_scale[r] * sum_h (w[t,h] q_scale[t,h]) * max(0, q[t,h] . k[r]) with
 * FP8 matrix products (exact products, fp32 sums).  Everything else --
 * visibility, layout of scores, errors, supported shapes -- is as for
 * csa_index_score; q_idx and k_idx must be 16-byte aligned.  The key stream
 * is half the bf16 one.
 */
csa_status csa_index_score_e4m3(const uint8_t* q_idx, const float* q_scale, const float* w,
                                const uint8_t* k_idx, const float* k_scale, int64_t k_rows,
                                const int64_t* pos, const int64_t* seq_kv, const int32_t* n_comp,
                                int T, int n_ih, int ihd, int ratio,
                                float* scores, int64_t ld, uint32_t* err, void* stream);

/*
 * Quantisation of bf16 rows to E4M3 codes for csa_index_score_e4m3 (the
 * post-probe audit's C4 cache format; the write side of the indexer-key
 * cache).  For each row i of src [rows, d]: scale[i] = 2**e for the smallest
 * e with max_j |src[i,j]| * 2**-e <= 448 (E4M3's largest finite value;
 * 1 for a zero row), and codes[i, j] = src[i, j] * 2**-e rounded to the
 * nearest E4M3 value, ties to even (subnormals included).  The codes are a
 * function of the inputs alone (a power-of-two scale is exact).
 *   src [rows, d] bf16   codes [rows, d] uint8   scale [rows] fp32
 * Supported: 1 <= d <= 512, rows >= 0.
 */
csa_status csa_quantize_e4m3(const uint16_t* src, int64_t rows, int d, uint8_t* codes,
                             float* scale, void* stream);

/*
 * S2 -- causal top-k (post-probe audit, F3: tk = min(top_k, n_comp), topk over
 * the scores; PART A suspect 3: only blocks before the query's own block).
 * For each token, k_eff = min(top_k, n_vis[t]) indices s < n_vis[t] of the
 * largest scores[t, s] are written to idx[t, 0:k_eff] in ascending block order;
 * idx[t, k_eff:top_k] = -1; count[t] = k_eff.  Among equal scores the lower
 * block index wins, so the result is deterministic.  Comparison is on the fp32
 * values (-0.0 == +0.0).  NaN scores are not supported.
 *   scores [T, ld] fp32 (entries s < n_vis[t] read)
 *   idx    [T, top_k] int32      count [T] int32
 *   ws     >= csa_topk_workspace_bytes(T, ld, top_k) bytes, 256-B aligned;
 *          contents on entry are irrelevant.
 * Supported: 1 <= top_k <= 2048, ld >= 1.
 */
size_t csa_topk_workspace_bytes(int T, int64_t ld, int top_k);
csa_status csa_topk(const float* scores, int64_t ld,
                    const int64_t* pos, const int32_t* n_comp,
                    int T, int ratio, int top_k,
                    int32_t* idx, int32_t* count,
                    void* ws, size_t ws_bytes, uint32_t* err, void* stream);

/*
 * S3 -- gather into one preallocated buffer (post-probe audit, B1/B2 and C2;
 * 1M-context audit, D3/D5): row j < count[t] of all_kv[t] is
 * comp_kv[seq_kv[t] + idx[t,j]]; rows count[t] .. count[t]+swa_len[t]-1 are
 * swa[swa_row0[t] + i].  n_kv[t] = count[t] + swa_len[t].  Rows of all_kv[t]
 * at or beyond n_kv[t] are left untouched.  Bit-exact copy.
 *   comp_kv [comp_rows, head_dim] bf16     swa [swa_rows, head_dim] bf16
 *   idx [T, top_k] int32   count [T] int32   swa_row0 [T] int64  swa_len [T] int32
 *   all_kv  [T, top_k + window, head_dim] bf16     n_kv [T] int32
 * Supported: head_dim in {64, 128, 256, 512}; top_k >= 0; window >= 0.
 */
csa_status csa_gather(const uint16_t* comp_kv, int64_t comp_rows, const int64_t* seq_kv,
                      const int32_t* idx, const int32_t* count, int top_k,
                      const uint16_t* swa, int64_t swa_rows,
                      const int64_t* swa_row0, const int32_t* swa_len, int window,
                      int T, int head_dim,
                      uint16_t* all_kv, int32_t* n_kv, uint32_t* err, void* stream);

/*
 * S4 -- shared-KV MQA softmax attention (post-probe audit, F3 "shared key-value
 * MQA"; 1M-context audit, D4 for the dense HCA row set and D6 for the sink).
 * Token t attends over segment A rows kv_a[a_row0[t] .. a_row0[t]+a_len[t]-1]
 * followed by segment B rows kv_b[b_row0[t] .. +b_len[t]-1]; each row is both
 * key and value:
 *     z_j = scale * q[t,h] . row_j
 *     out[t,h] = sum_j e^{z_j} row_j / (sum_j e^{z_j} + [sink] e^{sink[h]})
 *     lse[t,h] = log(sum_j e^{z_j} + [sink] e^{sink[h]})
 * bf16 MFMA products, fp32 softmax and accumulation, bf16 output.  An empty row
 * set without sink gives out = 0 and lse = -inf.
 *   q [T, n_heads, head_dim] bf16   out [T, n_heads, head_dim] bf16
 *   lse [T, n_heads] fp32 or NULL   sink [n_heads] fp32 or NULL
 *   kv_b, b_row0, b_len may all be NULL (one segment).
 *   max_rows: host bound on a_len[t] + b_len[t] (sizes the split grid).
 *   ws >= csa_attend_workspace_bytes(T, n_heads, head_dim, max_rows), 256-B aligned.
 * Supported: head_dim in {64, 128, 256, 512}; 1 <= n_heads <= 128; max_rows >= 0.
 */
size_t csa_attend_workspace_bytes(int T, int n_heads, int head_dim, int max_rows);
csa_status csa_mqa_attend(const uint16_t* q, int T, int n_heads, int head_dim,
                          float scale, const float* sink,
                          const uint16_t* kv_a, int64_t a_rows,
                          const int64_t* a_row0, const int32_t* a_len,
                          const uint16_t* kv_b, int64_t b_rows,
                          const int64_t* b_row0, const int32_t* b_len,
                          int max_rows, uint16_t* out, float* lse,
                          void* ws, size_t ws_bytes, uint32_t* err, void* stream);

/*
 * S5 -- one decode step of one attention layer, all stages enqueued on one
 * stream with no host synchronisation (capturable in a HIP graph).
 *
 * mode CSA_MODE_CSA: S1 -> S2 -> S3 -> S4 over the selected compressed rows,
 *   then the SWA rows.  Requires q_idx, w, k_idx.  The rows are read in place
 *   (the selected ones through their block indices); all_kv, when given,
 *   also receives them in that order -- the preallocated gather buffer of the
 *   post-probe audit's C2 -- and may be NULL (1M-context audit, M5/A9: the
 *   attention reads the two buffers directly).
 *   With idx_e4m3 = 1, S1 scores E4M3 copies of the indexer queries and keys
 *   (post-probe audit, C4: narrow storage paired with narrow products; the
 *   1M-context audit's A2 gates it on top-k recall against a full-precision
 *   indexer) and S2 keeps the best C of them, whose bf16 scores then decide
 *   the top_k (see the idx_e4m3 fields).
 * mode CSA_MODE_HCA (1M-context audit, D4): no indexer; S4 over the entire
 *   visible compressed history comp_kv[seq_kv[t] .. +n_vis[t]-1] followed by
 *   the SWA rows, read in place (no concatenation).
 *
 * Optional outputs (NULL = kept in the workspace): scores [T, max_vis],
 * idx [T, top_k], count [T], n_kv [T], lse [T, n_heads].
 * max_vis is the host bound on n_vis[t] over the batch.
 */
enum { CSA_MODE_CSA = 0, CSA_MODE_HCA = 1 };

typedef struct csa_step_args {
  int mode;
  int T, n_ih, ihd, ratio, top_k, window, n_heads, head_dim;
  int64_t max_vis;
  float scale;
  const uint16_t* q_idx;    /* [T, n_ih, ihd] bf16   (CSA) */
  const float* w;           /* [T, n_ih]             (CSA) */
  const uint16_t* k_idx;    /* [k_rows, ihd] bf16    (CSA) */
  int64_t k_rows;
  const uint16_t* comp_kv;  /* [comp_rows, head_dim] */
  int64_t comp_rows;
  const uint16_t* swa;      /* [swa_rows, head_dim]  */
  int64_t swa_rows;
  const uint16_t* q;        /* [T, n_heads, head_dim] */
  const float* sink;        /* [n_heads] or NULL     */
  const int64_t* pos;       /* [T] */
  const int64_t* seq_kv;    /* [T] */
  const int32_t* n_comp;    /* [T] */
  const int64_t* swa_row0;  /* [T] */
  const int32_t* swa_len;   /* [T] */
  uint16_t* all_kv;         /* [T, top_k + window, head_dim] or NULL  (CSA) */
  uint16_t* out;            /* [T, n_heads, head_dim] (required) */
  float* lse;               /* [T, n_heads] or NULL  */
  float* scores;            /* [T, max_vis] or NULL  */
  int32_t* idx;             /* [T, top_k] or NULL    */
  int32_t* count;           /* [T] or NULL           */
  int32_t* n_kv;            /* [T] or NULL           */
  uint32_t* err;            /* device word or NULL   */
  /* CSA mode, idx_e4m3 = 1: the indexer streams E4M3 copies of its queries
     and keys instead (q_idx8 [T, n_ih, ihd] with q_idx_scale [T, n_ih],
     k_idx8 [k_rows, ihd] with k_idx_scale [k_rows]; see csa_quantize_e4m3)
     and keeps the C = min(top_k + top_k/2, 4096) blocks with the largest
     E4M3 scores (lower index first on ties); the top_k of those C by their
     bf16 scores (q_idx, k_idx: still required) are selected.  `scores`
     receives the E4M3 scores.  idx_e4m3 = 0: the five fields are ignored. */
  int idx_e4m3;
  const uint8_t* q_idx8;
  const float* q_idx_scale;
  const uint8_t* k_idx8;
  const float* k_idx_scale;
  /* 1: every token's key rows start at the same seq_kv (one sequence, e.g. a
     prefill chunk), which lets S1 score the tokens as one GEMM whose key
     tiles serve several tokens at once.  That form is taken for the bf16
     indexer with T >= 64, n_ih <= 64, ihd 64 or 128, per-wave candidate
     lists (not merged per workgroup), and rows too long for the batch
     indexer (which takes up to 512 tokens whose rows fit one tile a wave);
     otherwise the promise changes nothing.  Under the GEMM form a token
     whose seq_kv differs from that of the first token of its group of
     eight (tokens 8g .. 8g+7) scores no block, selects nothing, and raises
     CSA_DERR_BAD_META.  0: no assumption.  Other values: CSA_EINVAL. */
  int one_sequence;
} csa_step_args;

size_t csa_decode_step_workspace_bytes(const csa_step_args* a);
csa_status csa_decode_step(const csa_step_args* a, void* ws, size_t ws_bytes, void* stream);

/*
 * Producer side of one decode step: the compressors and the cache append
 * (1M-context audit, D1/D2: a main and an indexer-key compressor of the form
 * Compressor(ratio, width, H), projecting the hidden state to 2 x width per
 * token, compressed rows width wide; its closing assessment: overlapped
 * 2m-token windows with softmax weights; D5: the sliding-window ring).  For
 * each token t, of sequence s = seq[t] (the tokens of one call belong to
 * distinct sequences) at position p = pos[t]:
 *   y = [w_kv; w_ik] . x[t]                       (fp32: c_kv | z_kv | c_ik | z_ik)
 *   ring[s, p mod 2*ratio] = y
 *   swa[s, swa_head[s]] = bf16(c_kv); swa_head[s] = (swa_head[s] + 1) mod window;
 *   swa_len[s] = min(swa_len[s] + 1, window)
 *   if (p + 1) mod ratio == 0, block i = (p + 1)/ratio - 1 is complete:
 *     per channel, softmax over tokens j in [max(0, (i-1)*ratio), (i+1)*ratio)
 *     of z_j weighting c_j (read from the ring), in bf16 to
 *     comp_kv[seq_kv[s] + i] (width hd) and k_idx[seq_kv[s] + i] (width ihd);
 *     n_comp[s] = i + 1.
 * Reading of the pages: the projection's two halves are values and scores;
 * the window row of a token is its main value half.
 *   x [T, H] bf16; w_kv [2*hd, H], w_ik [2*ihd, H] bf16, one output channel per
 *   row; ring [S, 2*ratio, 2*hd + 2*ihd] fp32 (the last 2*ratio tokens'
 *   projections, kept between calls); swa [S, window, hd] bf16;
 *   swa_head, swa_len, n_comp [S] int32; seq [T] int32; pos [T] int64;
 *   seq_kv [S] int64, the row of each sequence's block 0 (only the row
 *   written, seq_kv[s] + i, must lie in [0, comp_rows)); comp_kv
 *   [comp_rows, hd] and k_idx [comp_rows, ihd] bf16.
 *   ws >= csa_compress_append_workspace_bytes(T, H, hd, ihd), 256-B aligned.
 * Device errors (in *err): CSA_DERR_BAD_META for a sequence id, position or
 * ring head out of range, or n_comp[s] != i at a block end (the row is still
 * written); CSA_DERR_KEY_RANGE for a compressed row outside comp_rows (not
 * written).
 * Supported: H a multiple of 256; hd, ihd multiples of 16 (hd <= 1024,
 * ihd <= 512); ratio a power of two up to 16; window <= 1024.
 */
size_t csa_compress_append_workspace_bytes(int T, int H, int hd, int ihd);
csa_status csa_compress_append(const uint16_t* x, int T, int H, const uint16_t* w_kv, int hd,
                               const uint16_t* w_ik, int ihd, const int32_t* seq,
                               const int64_t* pos, int S, int ratio, int window, float* ring,
                               uint16_t* swa, int32_t* swa_head, int32_t* swa_len,
                               uint16_t* comp_kv, uint16_t* k_idx, const int64_t* seq_kv,
                               int32_t* n_comp, int64_t comp_rows, void* ws, size_t ws_bytes,
                               uint32_t* err, void* stream);

/*
 * One stage of csa_decode_step, for callers that schedule other work between
 * the indexer and the rest of the step, or time the stages apart.
 *   stage CSA_STAGE_INDEX: S1 -- the indexer scores and the candidate lists
 *     of the top-k, left in ws (and in `scores` when given);
 *   stage CSA_STAGE_REST: S2 .. S4, reading them from the same ws.
 * The two in this order on one stream, with the same arguments and ws,
 * compute exactly what csa_decode_step computes.  In HCA mode the INDEX stage
 * does nothing.  Same validation and workspace size as csa_decode_step; any
 * other stage value gives CSA_EINVAL.
 */
enum { CSA_STAGE_INDEX = 1, CSA_STAGE_REST = 2 };
csa_status csa_decode_step_stage(const csa_step_args* a, int stage, void* ws, size_t ws_bytes,
                                 void* stream);

/*
 * Allocation-free decode step, for callers that cannot allocate device
 * memory: code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc.  Same arguments, computation and results as
 * csa_decode_step; its workspace is a fixed array of
 * CSA_NOALLOC_SCRATCH_BYTES (64 MiB) in the memory of each GPU the library
 * runs on, held until the process ends.  The call itself allocates nothing.
 *   Runs on the current device; `stream` must belong to it (NULL: its null
 *     stream).  The first call on a device looks the array's address up.
 *   Returns CSA_ESCRATCH, before any launch, when
 *     csa_decode_step_workspace_bytes(a) exceeds the array (the 1M-token and
 *     32 x 16K..128K decode steps need about 2 and 42 MiB).
 *   Every call on one GPU uses that GPU's one array: calls that may overlap
 *     in time on one GPU (other streams, other host threads) race and must be
 *     serialised by the caller.  Each step writes every workspace word it
 *     reads before reading it, so nothing needs clearing between calls.
 */
#define CSA_NOALLOC_SCRATCH_BYTES (64u << 20)
csa_status csa_decode_step_noalloc(const csa_step_args* a, void* stream);

#ifdef __cplusplus
}
#endif
#endif /* CSA_H_ */
