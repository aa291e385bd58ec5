/*
 * wpa.h -- windowed int8 paged prefill attention for AMD Instinct MI355X (gfx950).
 *
 * One operation: causal prefill attention at head_dim 256 over a paged int8 KV
 * pool, with a StreamingLLM sink + window block mask and grouped-query heads.
 * Source of the method: the page "perf(qwen35): int8 tensor-core prefill
 * attention for Qwythos" (sections "Why the attention, and why tensor cores"
 * and "Relation to open PRs"), and for the window semantics the page
 * "perf(qwen35): fp16 shared-memory tiles for windowed prefill attention"
 * (sections "Summary", "Proof of speedup").
 *
 * Conventions shared by every entry point
 *   - head_dim is fixed at 256 (WPA_HEAD_DIM); a KV page holds exactly 16
 *     tokens (WPA_PAGE_TOKENS), the page being the block of the mask.
 *   - All pointers are DEVICE pointers on the current HIP device.  The caller
 *     allocates and frees every buffer; the library allocates nothing, never
 *     synchronizes, and is safe to call from several host threads.  Its only
 *     state is the fixed scratch buffer of wpa_decode_attn_i8_noalloc (a
 *     static device array per GPU and its looked-up address).  Work is enqueued on `stream` (0 = the legacy default stream)
 *     and the call returns at once; buffers must stay alive until the stream
 *     has passed the call.  Calls with no work (n_tokens == 0) return WPA_OK
 *     and enqueue nothing.
 *   - Arguments are validated on the host before anything is enqueued.  On a
 *     nonzero status nothing has been enqueued and no output has been written.
 *     WPA_ERR_LAUNCH reports a failed kernel launch (hipGetLastError).
 *   - Layouts are C-contiguous ("[a][b][c]" = c fastest).
 */
#ifndef WPA_H
#define WPA_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define WPA_HEAD_DIM 256
#define WPA_PAGE_TOKENS 16

typedef enum {
  WPA_OK = 0,
  WPA_ERR_NULL = 1,         /* a required pointer is NULL (with n_tokens > 0)          */
  WPA_ERR_SHAPE = 2,        /* a size, count or scale is out of range                  */
  WPA_ERR_UNSUPPORTED = 3,  /* bad dtype, misaligned pointer, or a limit exceeded      */
  WPA_ERR_LAUNCH = 4,       /* the HIP kernel launch failed                            */
  WPA_ERR_TOO_LARGE = 5     /* more scratch needed than WPA_NOALLOC_SCRATCH_BYTES      */
} wpa_status;

typedef enum { WPA_F32 = 0, WPA_BF16 = 1 } wpa_dtype;

/*
 * Per-row quantization of Q (the method's first step: "one scale per query
 * row", int8 tensor-core prefill attention page, "Why the attention, and why
 * tensor cores").  A row is one (token, head) pair over the 256 channels:
 *     amax = max |q|;   code = clamp(rint(q * (127 / amax)), -127, 127);
 *     scale = amax / 127;           amax == 0 gives scale 0 and all-zero codes.
 * Computed in float32 with IEEE division and round-half-to-even, so the codes
 * are exactly those of that formula.
 *
 *   q        [n_tokens][n_q_heads][256], q_dtype WPA_BF16 or WPA_F32 (values
 *            that are not finite give unspecified codes); 16-byte aligned.
 *   q_i8     out [n_tokens][n_q_heads][256] int8; 16-byte aligned.
 *   q_scale  out [n_tokens][n_q_heads] float32.
 * Errors: NULL pointer -> WPA_ERR_NULL; n_tokens < 0 or n_q_heads <= 0 ->
 * WPA_ERR_SHAPE; other dtype or misalignment -> WPA_ERR_UNSUPPORTED.
 */
wpa_status wpa_quantize_q_rows(const void* q, wpa_dtype q_dtype, int n_tokens, int n_q_heads,
                               int8_t* q_i8, float* q_scale, hipStream_t stream);

/*
 * Prefill attention over the paged int8 KV pool (int8 tensor-core prefill
 * attention page, "Why the attention, and why tensor cores"; window-off rule
 * from its "Relation to open PRs"; StreamingLLM window from the fp16
 * shared-memory tiles page, "Summary").
 *
 * Query row t (token t, prefill from position 0) of query head h attends
 *     A(t) = { j <= t : window_blocks <= 0  or  j/16 < sink_blocks
 *                                           or  j/16 >= rsb(t) },
 *     rsb(t) = max(0, (t + 16)/16 - window_blocks),
 * i.e. the first sink_blocks key blocks plus the last window_blocks blocks up
 * to and including its own, causally; window_blocks <= 0 is full causal
 * attention.  KV head of query head h is h / (n_q_heads / n_kv_heads).
 *     s_j   = (q_i8 . k_i8[j]) * q_scale * k_scale[j] * softmax_scale
 *     P_j   = exp(s_j - max s),  l = sum_{A(t)} P_j
 *     P'_j  = P_j * v_scale[j]; per 16-key block: step ps = max P' / 127,
 *             code_j = rint(P'_j / ps)            (int8, 0..127)
 *     out   = sum_blocks ps * (code . v_i8) / l
 * QK^T and PV run as int8 x int8 -> int32 matrix-core products.  The output
 * matches that formula up to float32 rounding and the rounding of each
 * block's weights ps * code to a 15-bit fixed point relative to a per-row
 * power-of-two reference (below 2e-3 of the largest output magnitude on the
 * tested workloads); which codes a float32 tie flips is not specified.
 *
 *   q_i8, q_scale  from wpa_quantize_q_rows ([n_tokens][n_q_heads][256] int8,
 *                  [n_tokens][n_q_heads] float32); q_i8 16-byte aligned.
 *   k_pool, v_pool [n_pool_pages][16][n_kv_heads][256] int8, 16-byte aligned.
 *   k_scale, v_scale [n_pool_pages][16][n_kv_heads] float32 (per token per KV
 *                  head).  Scales of attended keys must be finite and >= 0,
 *                  v_scale at most 2^64; 0 (what wpa_kv_write_i8 stores for
 *                  an all-zero row) is allowed.
 *   page_table     [ceil(n_tokens/16)] int32, logical block -> physical page.
 *                  Entries should lie in [0, n_pool_pages); the device clamps
 *                  an entry outside into it (a wrong page is read, never
 *                  memory outside the pool), so only the rows that attend
 *                  such a block are wrong.
 *   out            [n_tokens][n_q_heads][256], out_dtype WPA_BF16 (rounded to
 *                  nearest even) or WPA_F32; must not alias any input.
 * Errors: NULL pointer -> WPA_ERR_NULL; n_tokens < 0, heads <= 0,
 * n_q_heads % n_kv_heads != 0, n_pool_pages < ceil(n_tokens/16),
 * sink_blocks < 0, softmax_scale not finite or <= 0 -> WPA_ERR_SHAPE;
 * other dtype or misalignment -> WPA_ERR_UNSUPPORTED.  A row may attend any
 * number of keys (sequence positions stay below 2^31 - 16).
 */
wpa_status wpa_prefill_attn_i8(const int8_t* q_i8, const float* q_scale,
                               const int8_t* k_pool, const int8_t* v_pool,
                               const float* k_scale, const float* v_scale,
                               const int32_t* page_table, int n_pool_pages,
                               int n_tokens, int n_q_heads, int n_kv_heads,
                               int window_blocks, int sink_blocks, float softmax_scale,
                               void* out, wpa_dtype out_dtype, hipStream_t stream);

/*
 * Chunked prefill: the same attention for the query rows at sequence positions
 * q_start .. q_start + n_tokens - 1 over a pool that already holds the keys
 * 0 .. q_start + n_tokens - 1 (the rows before the chunk came from earlier
 * calls).  Row i of q_i8, q_scale and out is position q_start + i; its
 * attended set is A(q_start + i) as defined above, so splitting a prefill
 * into chunks gives bitwise the same rows as one call.  q_start must be a
 * multiple of 16 (the chunk starts on a page, keeping the window start fixed
 * per 16-row tile).  page_table covers ceil((q_start + n_tokens)/16) blocks
 * and n_pool_pages must be at least that.  Other arguments, layouts and
 * errors as wpa_prefill_attn_i8; in addition q_start < 0 -> WPA_ERR_SHAPE and
 * q_start % 16 != 0 -> WPA_ERR_UNSUPPORTED.  (The pages' batched prefill
 * stops at 64k context and hands longer prompts to the token path; int8
 * tensor-core prefill attention page, "Proof of speedup".)
 */
wpa_status wpa_prefill_attn_i8_chunk(const int8_t* q_i8, const float* q_scale,
                                     const int8_t* k_pool, const int8_t* v_pool,
                                     const float* k_scale, const float* v_scale,
                                     const int32_t* page_table, int n_pool_pages,
                                     int q_start, int n_tokens, int n_q_heads, int n_kv_heads,
                                     int window_blocks, int sink_blocks, float softmax_scale,
                                     void* out, wpa_dtype out_dtype, hipStream_t stream);

/*
 * The attention of wpa_prefill_attn_i8_chunk straight from bf16 Q: the
 * attention kernel quantizes each query row as it loads it, with the formula
 * of wpa_quantize_q_rows (one scale per row: int8 tensor-core prefill
 * attention page, "Why the attention, and why tensor cores"), so the output
 * is bitwise that of wpa_quantize_q_rows followed by
 * wpa_prefill_attn_i8_chunk, without the int8 Q round trip through memory.
 *   q        [n_tokens][n_q_heads][256] bf16 (q_dtype must be WPA_BF16),
 *            16-byte aligned.  Row i is sequence position q_start + i; pass
 *            q_start = 0 for a whole prompt.
 * Out must not alias q.  Other arguments, layouts and errors as
 * wpa_prefill_attn_i8_chunk; a q_dtype other than WPA_BF16 ->
 * WPA_ERR_UNSUPPORTED (float32 Q goes through wpa_quantize_q_rows).
 */
wpa_status wpa_prefill_attn_fused_q(const void* q, wpa_dtype q_dtype,
                                    const int8_t* k_pool, const int8_t* v_pool,
                                    const float* k_scale, const float* v_scale,
                                    const int32_t* page_table, int n_pool_pages,
                                    int q_start, int n_tokens, int n_q_heads, int n_kv_heads,
                                    int window_blocks, int sink_blocks, float softmax_scale,
                                    void* out, wpa_dtype out_dtype, hipStream_t stream);

/*
 * counts[t] = |A(t)| for t in [0, n_tokens), computed by walking the same key
 * block list the attention kernel walks (the mask of the int8 tensor-core
 * prefill attention page, "Why the attention, and why tensor cores": window
 * start fixed per 16-row query tile, only the causal bound per row).
 *   counts  out [n_tokens] int32.
 * Errors: NULL -> WPA_ERR_NULL; n_tokens < 0 or sink_blocks < 0 -> WPA_ERR_SHAPE.
 */
wpa_status wpa_mask_counts(int n_tokens, int window_blocks, int sink_blocks, int32_t* counts,
                           hipStream_t stream);

/* counts[i] = |A(q_start + i)| for i in [0, n_tokens): the counts of a chunk
 * (wpa_prefill_attn_i8_chunk).  Errors as wpa_mask_counts, plus q_start < 0
 * -> WPA_ERR_SHAPE. */
wpa_status wpa_mask_counts_chunk(int q_start, int n_tokens, int window_blocks, int sink_blocks,
                                 int32_t* counts, hipStream_t stream);

/*
 * KV-pool writer: quantize new K and V rows and store them into the int8 pool
 * at the given slots.  The pages describe the pool this path reads (int8
 * tensor-core prefill attention page, "Why the attention, and why tensor
 * cores": 16-token pages, rows token-major with stride n_kv_heads*256, one
 * scale per token and KV head) but not how it is filled; each (token, KV head)
 * row of K and of V is quantized with the per-row formula that page gives for
 * Q ("one scale per row"), exactly as wpa_quantize_q_rows does:
 *     amax = max |x|;  code = clamp(rint(x * (127 / amax)), -127, 127);
 *     scale = amax / 127;   amax == 0 gives scale 0 and all-zero codes.
 * Float32 arithmetic, IEEE division, round-half-to-even.
 *
 *   k, v          [n_tokens][n_kv_heads][256], dtype WPA_BF16 or WPA_F32,
 *                 16-byte aligned (values that are not finite give
 *                 unspecified codes).
 *   slots         [n_tokens] int32, device: token t goes to pool slot
 *                 slots[t] = physical page * 16 + position in the page.
 *                 A slot outside [0, 16 * n_pool_pages) is skipped (nothing
 *                 is written for that token); two tokens with the same slot
 *                 race and either row may win.
 *   k_pool, v_pool  [n_pool_pages][16][n_kv_heads][256] int8, 16-byte
 *                 aligned; only the rows of the given slots are written.
 *   k_scale, v_scale  [n_pool_pages][16][n_kv_heads] float32.
 * Errors: NULL pointer -> WPA_ERR_NULL; n_tokens < 0, n_kv_heads <= 0 or
 * n_pool_pages < 0 -> WPA_ERR_SHAPE; other dtype or misalignment ->
 * WPA_ERR_UNSUPPORTED.
 */
wpa_status wpa_kv_write_i8(const void* k, const void* v, wpa_dtype dtype, int n_tokens, int n_kv_heads,
                           const int32_t* slots, int n_pool_pages, int8_t* k_pool, int8_t* v_pool,
                           float* k_scale, float* v_scale, hipStream_t stream);

/*
 * Split-KV decode: one new query token per sequence over the paged int8 pool,
 * with the prefill path's mask and int8 scheme (int8 tensor-core prefill
 * attention page, "Why the attention, and why tensor cores", which credits
 * the scheme to the int8 GQA flash-decode; "Relation to open PRs").  Sequence
 * b has seq_lens[b] tokens in the pool, the last of which is the query:
 * position t = seq_lens[b] - 1 attends A(t) as defined for
 * wpa_prefill_attn_i8, through its own page table.  Per (sequence, head) the
 * output is the same formula (row Q scale, per-token K scale, softmax scale
 * on the int32 QK^T; v_scale folded into P; P quantized per 16-key block;
 * int8 PV; l from the unquantized P), up to float32 rounding.
 *
 *   q_i8, q_scale  [batch][n_q_heads][256] int8 and [batch][n_q_heads] float32
 *                  (wpa_quantize_q_rows with n_tokens = batch); q_i8 16-byte aligned.
 *   k_pool, v_pool, k_scale, v_scale  as for wpa_prefill_attn_i8
 *                  (n_pool_pages pages), pools 16-byte aligned.
 *   page_tables    [batch][max_blocks] int32, device: block -> physical page
 *                  of each sequence.  Entries of attended blocks should lie in
 *                  [0, n_pool_pages); others are clamped into it (a wrong
 *                  entry reads a wrong page, never outside the pool).
 *   seq_lens       [batch] int32, device; a length above 16*max_blocks is
 *                  taken as 16*max_blocks, and a length <= 0 gives a zero row.
 *   n_q_heads / n_kv_heads: any; up to 16 query heads of a KV head share
 *                  each K and V row load (more take one load per 16).
 *   workspace      device scratch of at least wpa_decode_workspace_bytes(...)
 *                  bytes, 16-byte aligned, owned by the caller; its contents
 *                  on entry do not matter.  Calls that share a workspace
 *                  must be ordered on one stream.
 *   out            [batch][n_q_heads][256], WPA_BF16 (rounded to nearest
 *                  even) or WPA_F32.
 * Errors: NULL pointer -> WPA_ERR_NULL; batch < 0, heads <= 0,
 * n_q_heads % n_kv_heads != 0, max_blocks <= 0, n_pool_pages <= 0,
 * sink_blocks < 0, softmax_scale not finite or <= 0, or a workspace smaller
 * than needed -> WPA_ERR_SHAPE; other dtype, misalignment or a grid past
 * 2^31 workgroups -> WPA_ERR_UNSUPPORTED.
 */
size_t wpa_decode_workspace_bytes(int batch, int n_q_heads, int max_blocks, int window_blocks,
                                  int sink_blocks);
wpa_status wpa_decode_attn_i8(const int8_t* q_i8, const float* q_scale,
                              const int8_t* k_pool, const int8_t* v_pool,
                              const float* k_scale, const float* v_scale, int n_pool_pages,
                              const int32_t* page_tables, int max_blocks, const int32_t* seq_lens,
                              int batch, int n_q_heads, int n_kv_heads,
                              int window_blocks, int sink_blocks, float softmax_scale,
                              void* workspace, size_t workspace_bytes,
                              void* out, wpa_dtype out_dtype, hipStream_t stream);

/*
 * wpa_decode_attn_i8 without a workspace argument, for callers that cannot
 * allocate device memory: code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc.  The split rows go to a fixed buffer of
 * WPA_NOALLOC_SCRATCH_BYTES that the library holds on each GPU it runs on
 * until the process ends; its device address is looked up on the first call
 * on a device (with that device current), and the call allocates nothing.
 * Arguments, output and errors are those of wpa_decode_attn_i8; a call whose
 * wpa_decode_workspace_bytes(...) exceeds the buffer returns
 * WPA_ERR_TOO_LARGE before touching the device.  Every call on one GPU uses
 * the same buffer (its contents on entry do not matter): calls that overlap
 * on one GPU, e.g. on two streams, race, and must be ordered by the caller.
 */
#define WPA_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
wpa_status wpa_decode_attn_i8_noalloc(const int8_t* q_i8, const float* q_scale,
                                      const int8_t* k_pool, const int8_t* v_pool,
                                      const float* k_scale, const float* v_scale, int n_pool_pages,
                                      const int32_t* page_tables, int max_blocks, const int32_t* seq_lens,
                                      int batch, int n_q_heads, int n_kv_heads,
                                      int window_blocks, int sink_blocks, float softmax_scale,
                                      void* out, wpa_dtype out_dtype, hipStream_t stream);

/* Static, human-readable name of a status ("WPA_OK", ...; "unknown status"). */
const char* wpa_status_string(wpa_status s);

#ifdef __cplusplus
}
#endif

#endif /* WPA_H */
