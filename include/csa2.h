/*
 * csa2.h -- C ABI of the CSA2 layer-step library for AMD Instinct MI355X (gfx950).
 *
 * One CSA2 (Compressed Sparse Attention 2) layer step is
 *   (1) an indexer that scores every causally visible compressed main-KV entry
 *       with FP4 indexer Q/K,
 *   (2) a Top-K (K = 512) selection per query, and
 *   (3) sparse attention over the selected entries, dequantised from the FP4 main-KV
 *       cache, merged in one softmax with the layer's own FP8 sliding window.
 * Full layers run (1)-(3); Reindex layers run (1)-(3) on a borrowed cache, optionally
 * inside a candidate pool; Reuse layers borrow the index set and run (3) only.
 *
 * Sources, cited by page and section:
 *   [W] shibing624.github.io walkthrough "一个 token 只花 890 字节：DeepSeek-V4.1-Flash 把
 *       KV 缓存压到了什么程度": "CSA2：跨层复用，能借就不自己算" (Figure 4),
 *       "分层稀疏索引器" (Figure 5), "FP4 与 SWA Bounded Replay".
 *   [J] jdon.com article "557亿参数只唤醒80亿！DeepSeek把AI记忆砍掉437倍还拿了第一！":
 *       "缓存压缩真的是越大越好吗".
 *   [L] m.lsln.cn summary of the report: "4.3 消融实验", "五、相关工作".
 *   [MX] OCP Microscaling Formats v1.0; [FP8] OCP 8-bit floating point (E4M3, no inf).
 *
 * Conventions (all calls):
 *   - Every data pointer is caller-owned DEVICE memory; the library never allocates or
 *     frees on these calls.  Scratch space comes in through `workspace`, sized by the
 *     matching *_workspace_bytes() helper.
 *   - `stream` is a hipStream_t (NULL = the default stream).  Calls are asynchronous,
 *     stream-ordered, stateless and re-entrant; overlapping calls on different streams
 *     must not share a workspace.
 *   - Arguments are validated on the host before anything is launched; on failure the
 *     call returns a negative csa2 status and launches nothing.  CSA2_ERR_HIP means the
 *     runtime rejected a launch; csa2_last_error() then holds its text (per thread).
 *   - Values read from device arrays (positions, counts, indices) are clamped or skipped
 *     in-kernel so that no access leaves the buffers the sizes describe.
 *   - A kernel cannot return a status; where one meets a condition its outputs cannot show
 *     (a bounded wait that gave up) it stores a code into the device status word, and the
 *     next call on the host returns CSA2_ERR_DEVICE (csa2_device_status).
 *   - Inputs are finite; NaN/Inf inputs are outside the contract.
 *   - Code arrays (codes, q_codes, k_codes, kv_codes, swa), q and out must start on a
 *     16-byte boundary and kv_scales on an 8-byte one (CSA2_ERR_SHAPE otherwise); row
 *     sizes keep every row aligned.
 *
 * Cache layouts.  Every cache is addressed through its base pointers and byte strides, so
 * the codes and scales of a cache may be separate arrays or one interleaved record (the main
 * KV's 288-byte entry: scales = codes + 256, both entry strides 288):
 *   entry e of sequence b   codes  + b*codes_seq_stride  + e*codes_stride
 *                           scales + b*scales_seq_stride + e*scales_stride
 * A stride of 0 means dense: an entry stride of the row's own size and a sequence stride of
 * seq_cap entries.  Entry strides are at least the row size; code strides are multiples of
 * 16, main-KV scale strides multiples of 4 and NVFP4 indexer scale strides multiples of 2
 * (CSA2_ERR_SHAPE otherwise).  Distinct (sequence, entry) pairs must address disjoint bytes.
 *   main-KV cache   codes  D/2 bytes per entry: E2M1 pairs, channel 2i in the low nibble
 *                          of byte i
 *                   scales D/16 bytes per entry: E4M3, one per 16 channels
 *   indexer-K cache codes  d/2 bytes per entry: E2M1 pairs
 *                   scales d/32 bytes per entry (MXFP4: E8M0 per 32 channels) or d/16
 *                          (CSA2_FMT_NVFP4: E4M3 per 16 channels)
 *   indexer Q       q_codes [n_q, H_I, d/2], q_scales [n_q, H_I, d/32 or d/16] (dense)
 *   SWA cache       row r of sequence b: D bytes of E4M3 at swa + b*swa_seq_stride +
 *                   r*swa_row_stride (0: dense, D and swa_cap*D); token p of sequence b sits
 *                   in row (p - swa_base[b]) mod swa_cap
 *   index sets      idx [n_q, k] int32 positions, ascending, -1 padded
 */
#ifndef CSA2_H
#define CSA2_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* ---- status codes ---- */
#define CSA2_OK 0
#define CSA2_ERR_NULL (-1)         /* a required pointer is NULL */
#define CSA2_ERR_SHAPE (-2)        /* a size, count or shape argument is out of range */
#define CSA2_ERR_UNSUPPORTED (-3)  /* argument combination not supported (format, dtype, device) */
#define CSA2_ERR_HIP (-4)          /* the HIP runtime reported an error */
#define CSA2_ERR_WORKSPACE (-5)    /* workspace missing or smaller than required */
#define CSA2_ERR_DEVICE (-6)       /* a kernel of an earlier call stored a device status code
                                      (csa2_last_error names it); nothing was launched */

/* ---- device status codes (csa2_device_status) ---- */
#define CSA2_STATUS_ATTN_WAIT 1    /* an attention kernel's bounded wait for its partner wave
                                      gave up: that call's out and lse are invalid */

/* ---- storage formats ---- */
#define CSA2_FMT_NVFP4 0  /* main KV: E2M1 + one E4M3 scale per 16 channels, no global scale
                             ([W] "FP4 与 SWA Bounded Replay"; [L] 4.3, 5) */
#define CSA2_FMT_MXFP4 1  /* indexer Q/K: E2M1 + one E8M0 scale per 32 channels ([MX];
                             [W] "FP4 与 SWA Bounded Replay": indexer Q/K in FP4) */
#define CSA2_FMT_FP8 2    /* sliding-window KV: unscaled E4M3 ([J] "缓存压缩真的是越大越好吗") */
/* fmt of the indexer scoring calls that take it (csa2_index_score, csa2_index_topk,
   csa2_index_segments, csa2_index_topk_pool): the indexer K in MXFP4 and the indexer Q
   given unquantised, [n_q, n_heads, 128] f32 or bf16 in q_codes (16-byte aligned, finite;
   q_scales unused, may be NULL); every workgroup quantises its query's Q to MXFP4 itself by
   the csa2_quantize_kv rule, so the results equal csa2_quantize_kv (CSA2_FMT_MXFP4) followed
   by the same call with CSA2_FMT_MXFP4 on its codes, and a layer step needs no quantise
   launch before scoring ([W] "FP4 与 SWA Bounded Replay": indexer Q in FP4) */
#define CSA2_FMT_MXFP4_Q_F32 3
#define CSA2_FMT_MXFP4_Q_BF16 4

/* ---- element types of dense inputs / outputs ---- */
#define CSA2_DT_F32 0
#define CSA2_DT_BF16 1

/* ---- fixed limits ---- */
#define CSA2_MAX_TOPK 2048         /* k of csa2_topk, max_blocks of csa2_build_pool */
#define CSA2_MAX_INDEX_HEADS 16    /* H_I of csa2_index_score */
#define CSA2_INDEX_DIM 128         /* d of csa2_index_score */
#define CSA2_MAX_INDEX_ENTRIES (1 << 26)  /* seq_cap of csa2_index_score / csa2_index_topk */
#define CSA2_MAIN_DIM 512          /* D of csa2_sparse_attn */
#define CSA2_MAX_WINDOW 1024       /* window of csa2_sparse_attn */
#define CSA2_MAX_ATTN_ENTRIES (1 << 24)   /* seq_cap of csa2_sparse_attn */
#define CSA2_MAX_WINDOW_ROWS (1 << 23)    /* swa_cap of csa2_sparse_attn */

/* Library version (major*10000 + minor*100 + patch). */
int csa2_version(void);

/* Checks that the current HIP device is a gfx950 (MI355X) and that the library's code
 * objects load on it, and (once per process) allocates the library's 4-byte device status
 * word in pinned, mapped host memory.  Returns CSA2_OK, CSA2_ERR_UNSUPPORTED (other
 * device) or CSA2_ERR_HIP (no device / runtime error).  Calls made before csa2_init work,
 * but their kernels have no status word to report into. */
int csa2_init(void);

/* The device status word: 0, or the CSA2_STATUS_* code a kernel stored since it was last
 * cleared (clear != 0 clears it).  Every compute call first reads it on the host (no device
 * synchronisation); if it is nonzero the call clears it, puts its text in csa2_last_error,
 * launches nothing and returns CSA2_ERR_DEVICE.  A status stored by a kernel that is still
 * running when the next call starts is reported by a later call. */
uint32_t csa2_device_status(int clear);

/* Testing aid for the status path: sets how many times the attention kernel polls its
 * partner's flag before giving up (default 2^22; a negative value restores it) and returns
 * the previous bound.  With 0 every exchange gives up at once: the kernel still completes,
 * its output is wrong, and the status word is set.  Only the split-channel attention kernel,
 * which csa2_sparse_attn* run for a window wider than 128 keys, has such an exchange; with a
 * window of at most 128 keys no wave waits for another and the bound has no effect. */
int csa2_debug_set_wait_limit(int polls);

/* Static text for a status code; never NULL. */
const char* csa2_status_string(int status);

/* Text of the last HIP error seen by a csa2 call on this thread ("" if none). */
const char* csa2_last_error(void);

/*
 * csa2_quantize_kv -- quantise rows and scatter them into a cache.
 * [W] "FP4 与 SWA Bounded Replay" (main KV: E2M1 with an E4M3 scale per 16 channels,
 * quantised after RoPE); [L] 4.3 and 5 (no second-level global scale, after RoPE);
 * [MX] (indexer Q/K); [J] "缓存压缩真的是越大越好吗" (SWA KV in FP8).
 *
 *   src        [rows, dim] f32 or bf16 (src_dtype), the post-RoPE latents
 *   fmt        CSA2_FMT_NVFP4: per 16 channels, scale = E4M3 nearest to amax/6
 *                (saturating at 448); element = E2M1 nearest to x/scale (saturating at
 *                6), sign kept; a scale of 0 stores signed zeros.
 *              CSA2_FMT_MXFP4: per 32 channels, scale = 2^E, E = floor(log2 amax) - 2
 *                clamped to [-127, 127], code E+127 (0 for an all-zero group); element =
 *                E2M1 nearest to x/2^E, saturating at 6.
 *              CSA2_FMT_FP8: element = E4M3 nearest to x, saturating at +-448.
 *              Nearest = round to nearest, ties to the even code (bit-exact).
 *   dst_row    [rows] int64 destination row of each source row (NULL: row r -> r);
 *              rows whose destination is outside [0, dst_rows) are skipped
 *   codes      destination row d at codes + d*codes_stride: dim/2 bytes (FP4) or dim (FP8);
 *              codes_stride 0 = dense (dim/2 or dim), else >= that and a multiple of 16
 *   scales     destination row d at scales + d*scales_stride: dim/16 bytes (NVFP4) or dim/32
 *              (MXFP4); scales_stride 0 = dense; unused for FP8
 *              (an interleaved main-KV record: codes = rec, scales = rec + 256, both strides 288)
 * Errors: NULL src/codes (or scales for FP4) -> CSA2_ERR_NULL; rows < 0, dim <= 0, dim not
 * a multiple of the group (16 / 32 / 8 for FP8), dim > 8192, or a stride below the row size
 * or (codes) not a multiple of 16 -> CSA2_ERR_SHAPE; unknown fmt or src_dtype ->
 * CSA2_ERR_UNSUPPORTED.  rows == 0 launches nothing (src, codes and scales may then be NULL).
 */
int csa2_quantize_kv(const void* src, int src_dtype, int64_t rows, int dim, int fmt,
                     const int64_t* dst_row, int64_t dst_rows, uint8_t* codes, int64_t codes_stride,
                     uint8_t* scales, int64_t scales_stride, void* stream);

/*
 * csa2_quantize_kv_multi -- several csa2_quantize_kv jobs in one launch (a decode step's
 * appends: the new main-KV entry, indexer-K entry and window entry of every sequence, and
 * the queries' indexer Q).  Each job has the arguments and semantics of csa2_quantize_kv.
 *   jobs    host array of n_jobs descriptors, read during the call; n_jobs in 0..8.
 * The jobs must not write overlapping destinations.  Errors: those of csa2_quantize_kv for
 * any job (nothing is launched), CSA2_ERR_SHAPE for n_jobs out of range.
 */
#define CSA2_MAX_QUANT_JOBS 8
typedef struct {
  const void* src;
  int src_dtype;
  int64_t rows;
  int dim;
  int fmt;
  const int64_t* dst_row;
  int64_t dst_rows;
  uint8_t* codes;
  int64_t codes_stride;
  uint8_t* scales;
  int64_t scales_stride;
} csa2_quant_job;
int csa2_quantize_kv_multi(const csa2_quant_job* jobs, int n_jobs, void* stream);

/*
 * csa2_index_score -- indexer scores of each query over its sequence's entries.
 * [W] "CSA2：跨层复用，能借就不自己算" (a lightweight indexer scores the global main KV with
 * indexer Q/K), "分层稀疏索引器" (later layers score only inside the pool);
 * [W] "FP4 与 SWA Bounded Replay" (indexer Q/K in FP4; the page does not fix the indexer's
 * scale format, so both readings are served).
 *
 *   score(q, j) = sum_h w[q,h] * max(0, sum_c Q[q,h,c] K[seq(q), j, c])
 * with Q and K the exact FP4 values; products are exact, sums are fp32.
 *
 *   fmt               the indexer format of Q and K: CSA2_FMT_MXFP4 (E8M0 per 32 channels,
 *                     the scaled FP4 matrix-core path) or CSA2_FMT_NVFP4 (E4M3 per 16
 *                     channels, as the main KV; dequantised exactly to fp16 matrix cores);
 *                     CSA2_FMT_MXFP4_Q_F32 / _Q_BF16: MXFP4 with Q given unquantised
 *   q_codes/q_scales  [n_q, n_heads, dim/2] / [n_q, n_heads, dim/32 (MXFP4) or dim/16]
 *                     (q_codes 16-byte aligned); with CSA2_FMT_MXFP4_Q_*: q_codes the
 *                     [n_q, n_heads, dim] f32 / bf16 Q, q_scales unused
 *   w                 [n_q, n_heads] f32
 *   n_heads           1..16;  dim == 128
 *   k_codes, k_scales and their strides   the indexer-K cache (see Cache layouts)
 *   q_seq             [n_q] int32 sequence of each query (queries with q_seq outside
 *                     [0, n_seq) get no scores)
 *   n_vis             [n_q] int64 visible entries of each query (clamped to seq_cap)
 *   cand_blocks       NULL: score positions j in [0, n_vis), written to scores[q, j];
 *                     positions past n_vis are not written.
 *                     else [n_q, max_cand_blocks] int32 block ids with n_cand_blocks [n_q]
 *                     valid ones: slot s in [0, max_cand_blocks*block) holds position
 *                     cand_blocks[q, s/block]*block + s%block and is written to
 *                     scores[q, s]; slots past n_cand_blocks*block, with a negative block
 *                     id or with an invisible position get -inf.
 *   block             positions per pool block (1..64) when cand_blocks is given
 *   scores            [n_q, scores_stride] f32
 * Errors: CSA2_ERR_NULL, CSA2_ERR_SHAPE (n_q < 0, n_heads not in 1..16, dim != 128,
 * seq_cap outside 0..CSA2_MAX_INDEX_ENTRIES, n_seq < 1, scores_stride too small for
 * seq_cap or max_cand_blocks*block).
 */
int csa2_index_score(const uint8_t* q_codes, const uint8_t* q_scales, const float* w, int n_q,
                     int n_heads, int dim, int fmt, const uint8_t* k_codes, int64_t k_codes_stride,
                     int64_t k_codes_seq_stride, const uint8_t* k_scales, int64_t k_scales_stride,
                     int64_t k_scales_seq_stride, int64_t seq_cap, int n_seq, const int32_t* q_seq,
                     const int64_t* n_vis, const int32_t* cand_blocks, const int32_t* n_cand_blocks,
                     int block, int max_cand_blocks, float* scores, int64_t scores_stride,
                     void* stream);

/*
 * csa2_index_score_q -- csa2_index_score with the indexer Q given unquantised: every
 * workgroup quantises its query's Q to MXFP4 itself (the csa2_quantize_kv rule, bit for
 * bit), so a layer step that appends nothing (Reindex) needs no quantise launch before
 * scoring.  [W] "FP4 与 SWA Bounded Replay" (indexer Q in FP4 after RoPE);
 * [W] "分层稀疏索引器" (Reindex inside the pool).
 *
 *   q        [n_q, n_heads, 128] f32 (q_dtype CSA2_DT_F32) or bf16 (CSA2_DT_BF16),
 *            16-byte aligned, finite; read only
 *   others   as csa2_index_score
 * The scores equal those of csa2_quantize_kv (CSA2_FMT_MXFP4) followed by
 * csa2_index_score on its codes.  fmt must be CSA2_FMT_MXFP4.  Errors: as csa2_index_score;
 * CSA2_ERR_UNSUPPORTED for another q_dtype or fmt.
 */
int csa2_index_score_q(const void* q, int q_dtype, const float* w, int n_q, int n_heads, int dim,
                       int fmt, const uint8_t* k_codes, int64_t k_codes_stride,
                       int64_t k_codes_seq_stride, const uint8_t* k_scales, int64_t k_scales_stride,
                       int64_t k_scales_seq_stride, int64_t seq_cap, int n_seq,
                       const int32_t* q_seq, const int64_t* n_vis, const int32_t* cand_blocks,
                       const int32_t* n_cand_blocks, int block, int max_cand_blocks, float* scores,
                       int64_t scores_stride, void* stream);

/*
 * csa2_index_score_grouped -- csa2_index_score (without a pool) for query rows that come in
 * groups sharing one sequence, reading each group's indexer K once.  For the tokens of a
 * sequence scored together: several decode tokens verified at once, or the rows of a
 * prefill chunk ([W] "CSA2：跨层复用，能借就不自己算": every query row is scored by the
 * indexer against the sequence's visible entries; here rows of one sequence share the pass).
 *
 * Arguments as csa2_index_score with cand_blocks = NULL, plus
 *   group   1..8: rows [g*group, (g+1)*group) form group g (the last one may be shorter)
 *           and read the indexer K of the sequence of the group's first row.
 * Every row's scores are written exactly as csa2_index_score writes them (bit-identical:
 * the same arithmetic per row and entry); positions past a row's n_vis are not written.  A
 * row whose q_seq differs from its group's first row, or lies outside [0, n_seq), gets no
 * scores.  fmt must be CSA2_FMT_MXFP4.  Errors: those of csa2_index_score, CSA2_ERR_SHAPE for
 * group out of range, CSA2_ERR_UNSUPPORTED for another fmt.
 */
int csa2_index_score_grouped(const uint8_t* q_codes, const uint8_t* q_scales, const float* w,
                             int n_q, int n_heads, int dim, int fmt, const uint8_t* k_codes,
                             int64_t k_codes_stride, int64_t k_codes_seq_stride,
                             const uint8_t* k_scales, int64_t k_scales_stride,
                             int64_t k_scales_seq_stride, int64_t seq_cap, int n_seq,
                             const int32_t* q_seq, const int64_t* n_vis, int group, float* scores,
                             int64_t scores_stride, void* stream);

/*
 * csa2_index_topk_grouped -- csa2_index_score_grouped followed by csa2_topk, without the
 * score array: for query rows that come in groups sharing one sequence (the rows of a prefill
 * chunk, several decode tokens of a sequence), each group's indexer K is read once and every
 * row keeps only its running best candidates.  [W] "CSA2：跨层复用，能借就不自己算" (every
 * query row's indexer scores, then its Top-K), "分层稀疏索引器" (the scoring of the whole
 * visible range is the cost that matters).
 *
 * Arguments up to n_vis and `group` are those of csa2_index_score_grouped; k, idx_out and
 * count_out are those of csa2_topk.  For every row whose q_seq equals its group's first
 * row's (and lies in [0, n_seq)), idx_out / count_out are exactly what csa2_index_score_grouped
 * followed by csa2_topk (no pool, n_vis as given) returns: the same fp32 scores in the same
 * ranking (score descending, position ascending), ascending positions, -1 padded.  Any other
 * row gets count 0 and an all -1 row.
 *   k in 1..CSA2_MAX_GROUPED_TOPK; n_q <= 65535 * group.
 *   Workspace: csa2_index_topk_grouped_workspace_bytes(n_q, seq_cap, k, group) bytes (each
 *   row's best k of every range of its entries: at most 8,192 keys per row).
 * fmt must be CSA2_FMT_MXFP4.  Errors: those of csa2_index_score_grouped; CSA2_ERR_NULL
 * (idx_out, count_out);
 * CSA2_ERR_SHAPE (k, n_q); CSA2_ERR_WORKSPACE.
 */
#define CSA2_MAX_GROUPED_TOPK 704
int csa2_index_topk_grouped(const uint8_t* q_codes, const uint8_t* q_scales, const float* w,
                            int n_q, int n_heads, int dim, int fmt, const uint8_t* k_codes,
                            int64_t k_codes_stride, int64_t k_codes_seq_stride,
                            const uint8_t* k_scales, int64_t k_scales_stride,
                            int64_t k_scales_seq_stride, int64_t seq_cap, int n_seq,
                            const int32_t* q_seq, const int64_t* n_vis, int group, int k,
                            int32_t* idx_out, int32_t* count_out, void* workspace,
                            size_t workspace_bytes, void* stream);
size_t csa2_index_topk_grouped_workspace_bytes(int n_q, int64_t seq_cap, int k, int group);

/*
 * csa2_append -- new cache entries that a fused scoring call (csa2_index_topk without a pool,
 * csa2_index_segments, csa2_index_topk_pool) writes itself, for decode steps whose Full
 * layer would otherwise make a quantise launch first: each query's new entry of its own
 * sequence, its main-KV row in NVFP4 and its indexer-K row in MXFP4 (the csa2_quantize_kv
 * rules, bit for bit).  [W] "FP4 与 SWA Bounded Replay" (new entries in FP4 after RoPE).
 * The call's scores see the new indexer-K entry, so the results (and the caches afterwards)
 * equal csa2_quantize_kv of the two rows followed by the same call without an append.
 *   row        [n_q] int64: the row of query q's new entry in sequence q_seq[q]; no append
 *              for q when row[q] is outside [0, seq_cap) or q_seq[q] outside [0, n_seq).
 *              Queries with an append must be of distinct sequences (no other query of the
 *              call may read that sequence: its row is written while the call runs).
 *   main       [n_q, 512] latents of the new main-KV rows (f32 or bf16, 16-byte aligned),
 *              or NULL: no main-KV append
 *   index      [n_q, 128] latents of the new indexer-K rows, or NULL: no indexer-K append;
 *              written into the call's own indexer-K cache (k_codes / k_scales)
 *   dtype      CSA2_DT_F32 or CSA2_DT_BF16, of both latents
 *   kv_*       the main-KV cache and its strides (see Cache layouts; 0 = dense), written;
 *              unused without `main`
 * A NULL csa2_append pointer: nothing is appended.  Errors of the calls that take it:
 * CSA2_ERR_NULL (row, or the main-KV cache with `main`), CSA2_ERR_SHAPE (alignment, strides),
 * CSA2_ERR_UNSUPPORTED (dtype; an NVFP4 indexer; an append to csa2_index_topk inside a pool).
 */
typedef struct csa2_append {
  const int64_t* row;
  const void* main;
  const void* index;
  int dtype;
  uint8_t* kv_codes;
  int64_t kv_codes_stride, kv_codes_seq_stride;
  uint8_t* kv_scales;
  int64_t kv_scales_stride, kv_scales_seq_stride;
} csa2_append;

/*
 * csa2_index_topk -- csa2_index_score followed by csa2_topk in one pass, without the score
 * array.  [W] "CSA2：跨层复用，能借就不自己算" (indexer scores, then Top-K, K = 512),
 * "分层稀疏索引器" (inside the pool).
 *
 * Arguments up to max_cand_blocks are those of csa2_index_score; k, idx_out and count_out
 * are those of csa2_topk.  The result (idx_out, count_out) is identical to calling
 * csa2_index_score and then csa2_topk with the same arguments: the same fp32 scores in
 * the same ranking (score descending, position ascending).
 *   k in 1..2048; n_q <= 65535.
 *   Workspace: csa2_index_topk_workspace_bytes(n_q, n_slots, k, in_pool) bytes, with
 *   n_slots = seq_cap and in_pool = 0 (no pool), or n_slots = max_cand_blocks*block and
 *   in_pool = 1.  Without a pool no score array exists: each workgroup scores 8,192 slots
 *   and keeps its best k in registers.  Inside a pool (at most a few thousand blocks) the
 *   scores go through the workspace, which lets the block-id gather spread over many
 *   workgroups.
 *   append     NULL, or the new entries the call writes first (csa2_append; not inside a pool)
 * Errors: those of csa2_index_score (except the score array's), CSA2_ERR_NULL (idx_out,
 * count_out), CSA2_ERR_SHAPE (k, n_q), CSA2_ERR_WORKSPACE; those of csa2_append.
 */
int csa2_index_topk(const uint8_t* q_codes, const uint8_t* q_scales, const float* w, int n_q,
                    int n_heads, int dim, int fmt, const uint8_t* k_codes, int64_t k_codes_stride,
                    int64_t k_codes_seq_stride, const uint8_t* k_scales, int64_t k_scales_stride,
                    int64_t k_scales_seq_stride, int64_t seq_cap, int n_seq, const int32_t* q_seq,
                    const int64_t* n_vis, const int32_t* cand_blocks, const int32_t* n_cand_blocks,
                    int block, int max_cand_blocks, int k, int32_t* idx_out, int32_t* count_out,
                    void* workspace, size_t workspace_bytes, const csa2_append* append,
                    void* stream);
size_t csa2_index_topk_workspace_bytes(int n_q, int64_t n_slots, int k, int in_pool);

/*
 * csa2_index_segments -- the first half of csa2_index_topk without a pool: scores every
 * visible entry (as csa2_index_score) and keeps, for every run of 8,192 consecutive
 * positions of a query's sequence, the k best of them (score descending, position
 * ascending), as selection keys that csa2_sparse_attn_topk turns into the query's Top-k.
 * [W] "CSA2：跨层复用，能借就不自己算" (indexer scores, then Top-K): the Top-k of a query is
 * the Top-k of the union of its runs' Top-k, so nothing is lost.
 *
 * Arguments up to n_vis are those of csa2_index_score; k in 1..2048; n_q <= 65535.
 *   cand_keys  [n_q, csa2_segment_keys(seq_cap, k)] uint64, caller-owned device memory,
 *              fully overwritten: per run its k keys in position order, then zeros.  The
 *              keys are opaque (0 = no candidate): only csa2_sparse_attn_topk reads them.
 * csa2_segment_keys(n_slots, k) = ceil(n_slots / 8192) * k (at least k; 0 for a bad k).
 *   append     NULL, or the new entries the call writes first (csa2_append)
 * Errors: those of csa2_index_score (except the score array's), CSA2_ERR_NULL (cand_keys),
 * CSA2_ERR_SHAPE (k, n_q); those of csa2_append.
 */
int csa2_index_segments(const uint8_t* q_codes, const uint8_t* q_scales, const float* w, int n_q,
                        int n_heads, int dim, int fmt, const uint8_t* k_codes,
                        int64_t k_codes_stride, int64_t k_codes_seq_stride, const uint8_t* k_scales,
                        int64_t k_scales_stride, int64_t k_scales_seq_stride, int64_t seq_cap,
                        int n_seq, const int32_t* q_seq, const int64_t* n_vis, int k,
                        uint64_t* cand_keys, const csa2_append* append, void* stream);
int64_t csa2_segment_keys(int64_t n_slots, int k);

/*
 * csa2_index_topk_pool -- the decoder's first Full layer in one pass over the indexer-K
 * cache: the Top-K of csa2_index_topk (no pool) and the candidate pool of
 * csa2_build_pool over the same scores.  [W] "CSA2：跨层复用，能借就不自己算" (Top-K),
 * "分层稀疏索引器" and Figure 5 (at most 2,048 blocks of 8 positions by max indexer score).
 *
 * Arguments up to n_vis are those of csa2_index_score without a pool; k, idx_out,
 * count_out as csa2_topk; block (a power of two, 1..64), max_blocks (1..2048), blocks_out
 * [n_q, max_blocks] and blocks_count [n_q] as csa2_build_pool.  Results are identical to
 * csa2_index_score + csa2_topk + csa2_build_pool with the same arguments.  The scoring pass
 * writes only each block's maximum visible score (4 B per block) besides the per-segment
 * Top-K survivors.  A query whose q_seq is outside [0, n_seq) gets count 0 and a pool of
 * its lowest visible block ids (all their scores are -inf).
 *   Workspace: csa2_index_topk_pool_workspace_bytes(n_q, seq_cap, k, block, max_blocks).
 * append: NULL, or the new entries the call writes first (csa2_append).
 * fmt must be CSA2_FMT_MXFP4 or CSA2_FMT_MXFP4_Q_F32 / _Q_BF16.  Errors: as csa2_index_topk;
 * CSA2_ERR_SHAPE for block or max_blocks out of range; CSA2_ERR_UNSUPPORTED for another fmt.
 */
int csa2_index_topk_pool(const uint8_t* q_codes, const uint8_t* q_scales, const float* w, int n_q,
                         int n_heads, int dim, int fmt, const uint8_t* k_codes,
                         int64_t k_codes_stride, int64_t k_codes_seq_stride,
                         const uint8_t* k_scales, int64_t k_scales_stride,
                         int64_t k_scales_seq_stride, int64_t seq_cap, int n_seq,
                         const int32_t* q_seq, const int64_t* n_vis, int k, int32_t* idx_out,
                         int32_t* count_out, int block, int max_blocks, int32_t* blocks_out,
                         int32_t* blocks_count, void* workspace, size_t workspace_bytes,
                         const csa2_append* append, void* stream);
size_t csa2_index_topk_pool_workspace_bytes(int n_q, int64_t n_slots, int k, int block,
                                            int max_blocks);

/*
 * csa2_topk -- the k highest-scoring candidates of each query.
 * [W] "CSA2：跨层复用，能借就不自己算" (Top-K, K = 512).
 *
 * Candidates are ranked by (score descending, position ascending); the first min(k, n)
 * are returned as ascending positions, padded with -1; count_out[q] = their number.
 *   cand_blocks NULL: candidates are positions [0, min(n_vis[q], max_vis)), score of
 *                     position j at scores[q, j].
 *   cand_blocks given: the slot layout of csa2_index_score (slots whose position is
 *                     invalid or invisible are not candidates); with ascending block ids
 *                     (as csa2_build_pool returns them) the output is ascending, otherwise
 *                     it follows slot order.
 *   k in 1..2048.  Workspace: csa2_topk_workspace_bytes(n_q, n_slots, k) bytes, where
 *   n_slots = max_vis (no pool) or max_cand_blocks*block.
 * Errors: CSA2_ERR_NULL, CSA2_ERR_SHAPE, CSA2_ERR_WORKSPACE.
 */
int csa2_topk(const float* scores, int64_t scores_stride, int n_q, const int64_t* n_vis,
              int64_t max_vis, const int32_t* cand_blocks, const int32_t* n_cand_blocks, int block,
              int max_cand_blocks, int k, int32_t* idx_out, int32_t* count_out, void* workspace,
              size_t workspace_bytes, void* stream);
size_t csa2_topk_workspace_bytes(int n_q, int64_t n_slots, int k);

/*
 * csa2_build_pool -- the hierarchical sparse indexer's candidate pool.
 * [W] "分层稀疏索引器" and Figure 5: the decoder's first Full layer keeps at most
 * max_blocks (2,048) aligned blocks of `block` (8) positions, chosen by the block's
 * maximum indexer score; later Reindex layers choose their Top-K inside it.
 *
 *   block score b = max of scores[q, j] over visible j in [b*block, b*block+block)
 *   blocks ranked by (block score descending, block id ascending); the first
 *   min(max_blocks, ceil(n_vis/block)) are returned ascending in blocks_out[q, :],
 *   padded with -1, with count_out[q] their number.
 *   block 1..64, max_blocks 1..2048.
 *   Workspace: csa2_pool_workspace_bytes(n_q, max_vis, block, max_blocks).
 * Errors: CSA2_ERR_NULL, CSA2_ERR_SHAPE, CSA2_ERR_WORKSPACE.
 */
int csa2_build_pool(const float* scores, int64_t scores_stride, int n_q, const int64_t* n_vis,
                    int64_t max_vis, int block, int max_blocks, int32_t* blocks_out,
                    int32_t* count_out, void* workspace, size_t workspace_bytes, void* stream);
size_t csa2_pool_workspace_bytes(int n_q, int64_t max_vis, int block, int max_blocks);

/*
 * csa2_sparse_attn -- attention over the selected main-KV entries and the window.
 * [W] "CSA2：跨层复用，能借就不自己算" (Top-K entries plus the layer's own sliding-window
 * KV; each mode keeps its own Q and window), "FP4 与 SWA Bounded Replay" (FP4 values are
 * dequantised before attention; after a replay from token s, query i sees the window keys
 * [max(s, i-W+1), i]); [J] "缓存压缩真的是越大越好吗" (window KV in FP8).
 *
 * For query row q at token t = q_pos[q] with replay start s = replay_start[q]:
 *   keys  = { main entry idx[q, i] : 0 <= idx < seq_cap }  (others are skipped)
 *         u { window token p : max(s, t-window+1) <= p <= t }   (no de-duplication)
 *   logit = sm_scale * (Q[q,h,:] . key)    with key the exact dequantised value
 *   out[q,h,:] = sum softmax(logit) * key   (V = K: the shared entry)
 *   lse[q,h]   = ln sum exp(logit)           (natural log)
 * A query with no key (only possible when s > t) gets out = 0 and lse = -inf.
 *
 *   q         [n_q, n_heads, dim] bf16;  n_heads a multiple of 16 (<= 256); dim == 512
 *   kv_codes, kv_scales and their strides   the main-KV cache (NVFP4; see Cache layouts)
 *   q_seq     [n_q] int32 (queries with q_seq outside [0, n_seq) get out = 0, lse = -inf)
 *   idx       [n_q, k] int32 positions, any order, -1 (or any value outside
 *             [0, seq_cap)) = empty;  k in 0..2048
 *   swa, swa_row_stride, swa_seq_stride   the window ring (E4M3 rows of dim bytes; see Cache
 *             layouts); swa_base [n_seq] int64; window in 1..1024 and window <= swa_cap <=
 *             CSA2_MAX_WINDOW_ROWS; seq_cap <= CSA2_MAX_ATTN_ENTRIES
 *   new_win   NULL, or [n_q, dim] f32 / bf16 (new_win_dtype; 4-byte aligned): the post-RoPE window latent of
 *             each row's own token t = q_pos[q].  The call appends it first: quantised to
 *             E4M3 exactly as csa2_quantize_kv with CSA2_FMT_FP8 writes it, stored at ring
 *             row (t - swa_base[seq]) mod swa_cap of sequence q_seq[q], and attended as
 *             the window key of token t -- one launch instead of an append call and an
 *             attention call.  Precondition: no two rows of the call belong to the same
 *             sequence (every other window key must already be in the ring).
 *   out       [n_q, n_heads, dim] f32 or bf16 (out_dtype); lse [n_q, n_heads] f32 or NULL
 *   Workspace: csa2_attn_workspace_bytes(n_q, n_heads, dim, k, window).
 * Arithmetic: Q.K and P.V on fp16 matrix cores with fp32 accumulation.  Every key/value
 * (E2M1 x E4M3, or E4M3) is exact in fp16.  Q enters as fp16 after a power-of-two scale per
 * (query, head) that brings the head's largest |q| into [2^14, 2^15): every bf16 value
 * within a factor 2^32 of that maximum is then exact, over the whole bf16 range, and the
 * logits take the scale back exactly.  Softmax in fp32; P rounded to fp16.  With a window
 * of at most 128 keys every wave runs its own key stream over all channels and no wave
 * waits for another; with a wider window the two waves that share a key stream exchange
 * partial logits through one bounded wait, and if it gives up, the call's out and lse are
 * invalid and the next call returns CSA2_ERR_DEVICE.  Batches of at
 * least 1,024 rows with 64 heads, without new_win, run one workgroup per row over all of
 * its heads (each key dequantised once per row; same arithmetic, no wait, no workspace).
 * Errors: CSA2_ERR_NULL, CSA2_ERR_SHAPE, CSA2_ERR_UNSUPPORTED (out_dtype, new_win_dtype),
 * CSA2_ERR_WORKSPACE.
 */
int csa2_sparse_attn(const void* q, int n_q, int n_heads, int dim, const uint8_t* kv_codes,
                     int64_t kv_codes_stride, int64_t kv_codes_seq_stride, const uint8_t* kv_scales,
                     int64_t kv_scales_stride, int64_t kv_scales_seq_stride, int64_t seq_cap,
                     int n_seq, const int32_t* q_seq, const int32_t* idx, int k, uint8_t* swa,
                     int64_t swa_row_stride, int64_t swa_seq_stride, int64_t swa_cap,
                     const int64_t* swa_base, const int64_t* q_pos, const int64_t* replay_start,
                     const void* new_win, int new_win_dtype, int window, float sm_scale, void* out,
                     int out_dtype, float* lse, void* workspace, size_t workspace_bytes,
                     void* stream);
size_t csa2_attn_workspace_bytes(int n_q, int n_heads, int dim, int k, int window);

/*
 * csa2_sparse_attn_noalloc -- csa2_sparse_attn for callers that cannot allocate device
 * memory (code under graph capture, tight serving loops, harnesses that forbid allocation):
 * the same kernels and results, with no workspace argument.  When the key list is split over
 * workgroups, the partial results go to a static device array of the library's own,
 * csa2_sparse_attn_noalloc_max_bytes() = 16 MiB per GPU, held from the library's load until
 * the process ends; csa2_init (or this call's first use on a device) looks up its address
 * once per device.  The call allocates nothing and calls no allocating routine.
 *   Arguments: those of csa2_sparse_attn without workspace / workspace_bytes.
 *   Every call on one GPU shares that GPU's array: calls that overlap in time on one GPU
 *   (different streams, or different threads) race and give undefined results.  No part of
 *   the array needs to start at zero (each call writes every partial it reads).
 * Errors: those of csa2_sparse_attn; CSA2_ERR_WORKSPACE when the call would need more than
 * the static array holds (csa2_attn_workspace_bytes(...) > 16 MiB: the key list is split
 * only while fewer than 256 (query, 16-head group) pairs exist, which keeps every accepted
 * shape within 16 MiB); CSA2_ERR_HIP if the array's address cannot be had.
 */
int csa2_sparse_attn_noalloc(const void* q, int n_q, int n_heads, int dim, const uint8_t* kv_codes,
                             int64_t kv_codes_stride, int64_t kv_codes_seq_stride,
                             const uint8_t* kv_scales, int64_t kv_scales_stride,
                             int64_t kv_scales_seq_stride, int64_t seq_cap, int n_seq,
                             const int32_t* q_seq, const int32_t* idx, int k, uint8_t* swa,
                             int64_t swa_row_stride, int64_t swa_seq_stride, int64_t swa_cap,
                             const int64_t* swa_base, const int64_t* q_pos,
                             const int64_t* replay_start, const void* new_win, int new_win_dtype,
                             int window, float sm_scale, void* out, int out_dtype, float* lse,
                             void* stream);
size_t csa2_sparse_attn_noalloc_max_bytes(void);

/*
 * csa2_sparse_attn_topk -- csa2_sparse_attn whose index set is selected in the same call
 * from csa2_index_segments' keys: the Top-k of the keys (score descending, position
 * ascending), as ascending positions, -1 padded -- exactly what csa2_index_topk returns for
 * the same scoring arguments -- is written to idx_out / count_out (for the Reuse layers
 * that borrow it) and attended over.  [W] "CSA2：跨层复用，能借就不自己算".
 *
 * Arguments are those of csa2_sparse_attn, with idx replaced by
 *   cand_keys   [n_q, cand_per_q] uint64 from csa2_index_segments, cand_per_q =
 *               csa2_segment_keys(seq_cap, k) in 1..8192 (seq_cap up to 131,072 at k = 512)
 *   k           1..2048, the Top-k size given to csa2_index_segments
 *   idx_out     [n_q, k] int32, count_out [n_q] int32 (caller-owned, overwritten)
 * Every workgroup of a query runs the selection itself (the histograms use the LDS of the
 * attention's V buffers before the first tile), so the index set needs no launch of its
 * own and no memory round trip before the gathers.
 * Errors: those of csa2_sparse_attn; CSA2_ERR_NULL (cand_keys, idx_out, count_out);
 * CSA2_ERR_SHAPE (cand_per_q, k).
 */
int csa2_sparse_attn_topk(const void* q, int n_q, int n_heads, int dim, const uint8_t* kv_codes,
                          int64_t kv_codes_stride, int64_t kv_codes_seq_stride,
                          const uint8_t* kv_scales, int64_t kv_scales_stride,
                          int64_t kv_scales_seq_stride, int64_t seq_cap, int n_seq,
                          const int32_t* q_seq, const uint64_t* cand_keys, int cand_per_q, int k,
                          int32_t* idx_out, int32_t* count_out, uint8_t* swa,
                          int64_t swa_row_stride, int64_t swa_seq_stride, int64_t swa_cap,
                          const int64_t* swa_base, const int64_t* q_pos,
                          const int64_t* replay_start, const void* new_win, int new_win_dtype,
                          int window, float sm_scale, void* out, int out_dtype, float* lse,
                          void* workspace, size_t workspace_bytes, void* stream);

/*
 * csa2_sparse_attn_pool_topk -- csa2_sparse_attn for a Reindex layer inside the pool, with
 * the index set selected in the same call from the pool's slot scores: the Top-k of the
 * valid slots (score descending, position ascending), as ascending positions, -1 padded --
 * exactly what csa2_topk returns for the same scores and pool -- is written to idx_out /
 * count_out and attended over.  [W] "分层稀疏索引器" (later layers choose their Top-K inside
 * the pool), "CSA2：跨层复用，能借就不自己算".
 *
 * Arguments are those of csa2_sparse_attn, with idx replaced by
 *   scores, scores_stride   the slot scores csa2_index_score writes with the same pool
 *                           ([n_q, scores_stride] f32, stride >= max_cand_blocks*block)
 *   n_vis, cand_blocks, n_cand_blocks, block, max_cand_blocks   as csa2_topk takes them;
 *                           max_cand_blocks*block <= 16,384 (the pool's 2,048 x 8 slots)
 *   k (1..2048), idx_out [n_q, k] int32, count_out [n_q] int32
 * Every workgroup of a query selects (512 threads x 32 slots, histograms in the V buffers'
 * LDS), so the pool's Top-K needs no launches of its own.
 * Errors: those of csa2_sparse_attn; CSA2_ERR_NULL (scores, n_vis, cand_blocks,
 * n_cand_blocks, idx_out, count_out); CSA2_ERR_SHAPE (block, max_cand_blocks, k, stride).
 */
int csa2_sparse_attn_pool_topk(const void* q, int n_q, int n_heads, int dim,
                               const uint8_t* kv_codes, int64_t kv_codes_stride,
                               int64_t kv_codes_seq_stride, const uint8_t* kv_scales,
                               int64_t kv_scales_stride, int64_t kv_scales_seq_stride,
                               int64_t seq_cap, int n_seq, const int32_t* q_seq,
                               const float* scores, int64_t scores_stride, const int64_t* n_vis,
                               const int32_t* cand_blocks, const int32_t* n_cand_blocks, int block,
                               int max_cand_blocks, int k, int32_t* idx_out, int32_t* count_out,
                               uint8_t* swa, int64_t swa_row_stride, int64_t swa_seq_stride,
                               int64_t swa_cap, const int64_t* swa_base, const int64_t* q_pos,
                               const int64_t* replay_start, const void* new_win, int new_win_dtype,
                               int window, float sm_scale, void* out, int out_dtype, float* lse,
                               void* workspace, size_t workspace_bytes, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* CSA2_H */
