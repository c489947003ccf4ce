/*
 * fa.h -- C ABI of the gfx950 tiled online-softmax attention library (libfa.so).
 *
 * The library computes exact scaled-dot-product attention, O = softmax(S) V with
 * S = scale * Q K^T, as one pass over key tiles with an online softmax: a running
 * row max m, a running sum l and an accumulator acc, both rescaled by
 * exp(m_old - m_new) whenever the max moves, so the n x m score matrix never
 * reaches device memory.  The operation is the one stated in section 1 of
 * "手搓 Attention：从三行循环到看懂 FlashAttention" (10100.com): Q has n rows,
 * K has m rows, both of width d; V has m rows of width dv; O has n rows of
 * width dv.  The recurrence is that article's section 7 and the "核心思路"
 * section of the FlashAttention chapter (llminference.xinbetween.com S12).
 *
 * Conventions shared by every entry point:
 *  - Pointers named q, k, v, o, k_cache, v_cache, block_table, seq_lens and
 *    workspace are DEVICE pointers, allocated and owned by the caller.  The
 *    library allocates nothing, frees nothing and keeps no state between calls
 *    except a per-thread text of the last error (fa_last_error).
 *  - Tensors are dense, row-major, with the shapes given below; element pointers
 *    must be 16-byte aligned.  All of q, k, v and o share one dtype.
 *  - Work is enqueued on `stream` (a hipStream_t passed as void*; NULL is the
 *    null stream) and the call returns without synchronising.  Results are
 *    valid once the caller has synchronised that stream.
 *  - Arguments are checked on the host before any HIP call; on any status other
 *    than FA_OK nothing has been launched (FA_ERR_HIP excepted: it reports a
 *    launch failure).  The host never reads device memory: values inside
 *    seq_lens or block_table that break the stated ranges are undefined
 *    behaviour.
 *  - Every call is deterministic: the same inputs give bitwise the same output.
 */
#ifndef FA_H_
#define FA_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  FA_DTYPE_F32 = 0,  /* float32 in and out; scores and the softmax shift in float64 */
  FA_DTYPE_F16 = 1,  /* float16 in and out; MFMA with float32 accumulation        */
  FA_DTYPE_BF16 = 2, /* bfloat16 in and out; MFMA with float32 accumulation       */
  /* Not a dtype.  It makes every int value a valid fa_dtype, so a caller that
   * passes an unknown code gets FA_ERR_INVALID rather than undefined behaviour. */
  FA_DTYPE_MAX_ENUM = 0x7fffffff
} fa_dtype;

typedef enum {
  FA_OK = 0,
  FA_ERR_INVALID = 1,      /* an argument breaks the contract (null, range, shape)   */
  FA_ERR_UNSUPPORTED = 2,  /* valid request this build does not implement            */
  FA_ERR_WORKSPACE = 3,    /* workspace missing or smaller than required             */
  FA_ERR_HIP = 4,          /* the HIP runtime reported an error (see fa_last_error)  */
  FA_STATUS_MAX_ENUM = 0x7fffffff  /* not a status: makes every int a valid fa_status  */
} fa_status;

/*
 * fa_fwd -- batched prefill attention.
 *
 *   q [batch, heads_q,  n, d ]    k [batch, heads_kv, m, d ]
 *   v [batch, heads_kv, m, dv]    o [batch, heads_q,  n, dv]   (o is written)
 *
 * Query head h reads key/value head h / (heads_q / heads_kv) (grouped heads as in
 * the S12 chapter's "它如何与你已经搭好的部分组合" section).
 *
 * scale   : multiplies Q K^T; finite and > 0.  1/sqrt(d) is the usual value (10100.com
 *           section 1, S12 "核心思路"); the 5688vip example uses 1.
 * causal  : nonzero -> query i may attend key j only when j <= i (keys 0..i, the
 *           causal variant of 10100.com section 6).  Requires n == m.
 * seq_lens: NULL, or a device int32[batch] of left-padded lengths 0 <= L_b <= n.
 *           Requires n == m.  Sequence b occupies positions [n - L_b, n) of both
 *           queries and keys; positions before that are padding, are never read
 *           into the arithmetic (they may hold anything, NaN included) and their
 *           output rows are written as 0.  Combined with causal this gives the
 *           ragged causal batch of the S12 NaN note ("exp(-inf - -inf) 是 NaN").
 * A query row with no allowed key gets O = 0 (never NaN).
 *
 * Limits of this build: d == dv, d in {64, 128} (else FA_ERR_UNSUPPORTED).
 * FA_ERR_INVALID: a null tensor pointer (when the tensor is non-empty), negative
 *   sizes, heads_kv == 0 or heads_q % heads_kv != 0, causal or seq_lens with
 *   n != m, a non-finite or non-positive scale, misaligned pointers, an unknown
 *   dtype, or one head of q, k or v (n * d or m * d elements) spanning 2^31
 *   bytes or more.
 * Empty work (batch, heads_q or n zero) returns FA_OK without launching.
 */
fa_status fa_fwd(fa_dtype dt, const void* q, const void* k, const void* v, void* o,
                 int batch, int heads_q, int heads_kv, int n, int m, int d, int dv,
                 float scale, int causal, const int32_t* seq_lens, void* stream);

/*
 * fa_fwd_partial -- fa_fwd restricted to the keys in [key_begin, key_end), with
 * the piece's state exposed so that pieces over disjoint key ranges can be
 * merged (fa_merge).  This is the split of the key loop over workers that the
 * S12 chapter describes for long sequences ("除了快，它还解锁了什么": flash-
 * decoding and ring attention hand each other exactly these partial states)
 * and its exercise 1 merges; here the state (m, l, acc) is given as
 *
 *   o   [batch, heads_q, n, dv] float32 (written): the output normalised over
 *       the row's allowed keys inside the range, acc / l;
 *   lse [batch, heads_q, n]     float32 (written): ln(sum of exp(scale * q.k))
 *       over those keys, i.e. m + ln l with m in natural-log units.
 *
 * A row with no allowed key inside the range (padding, a causal row whose keys
 * all lie at or beyond key_end, an empty range) gets o = 0 and lse = -inf.
 * q, k, v, dtype, scale, causal and seq_lens mean what they mean in fa_fwd
 * (masking and padding apply on top of the range); o must be 16-byte aligned
 * and lse 4-byte aligned.  FA_ERR_INVALID additionally for a range outside
 * 0 <= key_begin <= key_end <= m or a null lse (for non-empty work).
 */
fa_status fa_fwd_partial(fa_dtype dt, const void* q, const void* k, const void* v, float* o,
                         float* lse, int batch, int heads_q, int heads_kv, int n, int m, int d,
                         int dv, float scale, int causal, const int32_t* seq_lens,
                         int key_begin, int key_end, void* stream);

/*
 * fa_fwd_fp8 -- fa_fwd on FP8 inputs.  The S12 chapter's production list
 * names FP8 support only as something FlashAttention-3 added on Hopper; here
 * q, k and v are OCP 8-bit floating point E4M3 codes ("e4m3fn": bias 7, no
 * infinities, 0x7F and 0xFF are NaN, largest finite value 448), one byte per
 * element, each tensor with a float32 descale factor:
 *
 *   real q = q_descale * E4M3(q), real k = k_descale * E4M3(k),
 *   real v = v_descale * E4M3(v),
 *   O = softmax(scale * real_q real_k^T [+ mask]) real_v,
 *
 * written as out_dtype (FA_DTYPE_F32, F16 or BF16; RNE).  Shapes, head
 * grouping, scale, causal and seq_lens mean what they mean in fa_fwd; tensor
 * pointers must be 16-byte aligned.  Scores are exact code products summed in
 * the matrix cores; the softmax weights enter the P.V product rounded to E4M3
 * (about 2^-4 relative each), the one deliberate loss of this path.
 * FA_ERR_INVALID additionally for descales that are not finite and > 0, or
 * whose product with scale underflows float32 (the head-size limit of fa_fwd
 * counts one byte per element here).  Limits: d == dv in {64, 128}
 * (else FA_ERR_UNSUPPORTED).
 */
fa_status fa_fwd_fp8(const void* q, const void* k, const void* v, void* o, fa_dtype out_dtype,
                     int batch, int heads_q, int heads_kv, int n, int m, int d, int dv,
                     float scale, float q_descale, float k_descale, float v_descale, int causal,
                     const int32_t* seq_lens, void* stream);

/*
 * fa_merge -- combine attention pieces over disjoint key ranges (the S12
 * exercise 1 rescale applied to whole pieces): with L = max_s lse_s and
 * w_s = exp(lse_s - L),
 *
 *   O   = sum_s w_s o_s / sum_s w_s          (rounded to out_dtype, RNE)
 *   lse = L + ln(sum_s w_s)                  (if lse_out is not NULL)
 *
 *   o_parts   [parts, rows, dv] float32, lse_parts [parts, rows] float32 (read):
 *             piece s of every row, as written by fa_fwd_partial (rows =
 *             batch * heads_q * n for those tensors);
 *   o         [rows, dv] of out_dtype (written); lse_out [rows] float32 or NULL.
 *
 * Pieces with lse_s = -inf are ignored (their o_s is not read); a row with no
 * finite lse_s gets O = 0 and lse = -inf.  Merging the pieces of a partition
 * of [0, m) reproduces fa_fwd up to rounding.  FA_ERR_INVALID: unknown dtype,
 * parts <= 0, negative rows or dv, rows >= 2^31, null pointers (rows > 0),
 * o_parts or o not 16-byte aligned, lse arrays not 4-byte aligned.
 * FA_ERR_UNSUPPORTED: dv not a multiple of 4, or above 1024.  rows == 0
 * returns FA_OK without launching.
 */
fa_status fa_merge(fa_dtype out_dtype, const float* o_parts, const float* lse_parts, int parts,
                   long long rows, int dv, void* o, float* lse_out, void* stream);

/*
 * fa_paged_prefill -- a chunk of n query tokens per sequence attending over a
 * paged KV cache that already holds the chunk's own keys and values: the
 * prefill counterpart of fa_paged_decode.  The S12 chapter's paged loop walks
 * the block table key block by key block ("实现"), and the chapter notes that
 * each tile of the tiled pass can be such a block; here the K/V tiles of the
 * prefill kernel are gathered through the table.
 *
 *   q           [num_seqs, heads_q, n, d]: query row i of sequence b is its
 *               token L_b - n + i, i.e. the chunk is the last n tokens;
 *   k_cache     [num_blocks, block_size, heads_kv, d ], v_cache likewise with dv;
 *   block_table [num_seqs, max_blocks_per_seq] int32; entries at or past
 *               ceil(L_b / block_size) are never read; used entries must be in
 *               [0, num_blocks);
 *   seq_lens    [num_seqs] int32 total lengths 0 <= L_b <= max_blocks_per_seq *
 *               block_size, chunk included;
 *   o           [num_seqs, heads_q, n, dv] (written).
 *
 * causal: nonzero -> row i attends keys 0 .. L_b - n + i (the mask aligned to
 * the end of the sequence); zero -> all L_b keys.  Rows with L_b - n + i < 0
 * (a chunk longer than its sequence) have no keys and are written as 0.
 * Query head h reads KV head h / (heads_q / heads_kv).  n = 1 with causal is
 * the decode of fa_paged_decode.
 * Limits of this build: f16 or bf16 (f32 -> FA_ERR_UNSUPPORTED), d == dv in
 * {64, 128}, max_blocks_per_seq <= 16384 (else FA_ERR_UNSUPPORTED).
 * FA_ERR_INVALID: as fa_paged_decode, plus a negative n or a chunk of one head
 * (n * d 16-bit values) spanning 2^31 bytes or more.  No workspace.
 */
fa_status fa_paged_prefill(fa_dtype dt, const void* q, const void* k_cache, const void* v_cache,
                           const int32_t* block_table, const int32_t* seq_lens, int block_size,
                           int num_seqs, int heads_q, int heads_kv, int n, int d, int dv,
                           int num_blocks, int max_blocks_per_seq, float scale, int causal,
                           void* o, void* stream);

/*
 * fa_paged_decode_workspace_size -- bytes of device workspace fa_paged_decode needs
 * for these sizes (the split-K partial states).  Depends only on its arguments.
 * Returns 0 for arguments fa_paged_decode would reject.
 */
size_t fa_paged_decode_workspace_size(int num_seqs, int heads_q, int heads_kv, int dv,
                                      int max_blocks_per_seq, int block_size);

/*
 * fa_paged_decode -- one query token per sequence over a paged KV cache, with
 * grouped-query heads, split over key ranges and merged (flash-decoding).
 *
 * Follows the paged loop of the S12 chapter ("实现": walk the block table, the
 * last block holding min(block_size, seq_len - t * block_size) tokens, stop at the
 * first empty block) inside the online-softmax recurrence, with the key ranges
 * spread over workgroups and their (m, l, o) states merged by the same rescale
 * (S12 "除了快，它还解锁了什么" and exercise 1).
 *
 *   q           [num_seqs, heads_q, d]
 *   k_cache     [num_blocks, block_size, heads_kv, d ]
 *   v_cache     [num_blocks, block_size, heads_kv, dv]
 *   block_table [num_seqs, max_blocks_per_seq] int32: physical block of each
 *               logical block; entries at or past ceil(L_b / block_size) are
 *               never read (they may hold -1).  Used entries must be in
 *               [0, num_blocks).
 *   seq_lens    [num_seqs] int32, 0 <= L_b <= max_blocks_per_seq * block_size.
 *               Cache slots past L_b are never read into the arithmetic.  L_b = 0
 *               gives O = 0.
 *   o           [num_seqs, heads_q, dv] (written)
 *   workspace   device buffer of at least fa_paged_decode_workspace_size(...)
 *               bytes, owned by the caller; its contents on entry do not matter.
 *
 * Query head h reads KV head h / (heads_q / heads_kv).
 * Limits of this build: dtype f16 or bf16 (f32 -> FA_ERR_UNSUPPORTED); d == dv,
 * d in {64, 128}; at most 65535 key splits per sequence (768 keys each, fewer
 * when the batch is small), i.e. max_blocks_per_seq * block_size up to about
 * 50 million keys for a large batch (else FA_ERR_UNSUPPORTED).
 * FA_ERR_INVALID: null pointers for non-empty work, non-positive block_size,
 *   num_blocks or max_blocks_per_seq, negative sizes, heads_q % heads_kv != 0,
 *   non-finite or non-positive scale, misaligned pointers, a cache of 2^32 or
 *   more token rows (num_blocks * block_size) or 2^40 or more elements.
 * FA_ERR_WORKSPACE: workspace_bytes below the required size (or a null workspace).
 * Two kernels are enqueued: the split pass and the merge pass.
 */
fa_status fa_paged_decode(fa_dtype dt, const void* q, const void* k_cache, const void* v_cache,
                          const int32_t* block_table, const int32_t* seq_lens, int block_size,
                          int num_seqs, int heads_q, int heads_kv, int d, int dv,
                          int num_blocks, int max_blocks_per_seq, float scale, void* o,
                          void* workspace, size_t workspace_bytes, void* stream);

/*
 * fa_paged_decode_noalloc -- fa_paged_decode for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops, harnesses
 * that forbid allocation): the same computation, arguments and checks, with
 * no workspace argument.  The split states live in a static device array of
 * FA_NOALLOC_SCRATCH_BYTES inside the library, one copy per GPU, held from the
 * moment the library's code is loaded on that GPU until the process ends; the
 * call allocates and frees nothing.
 *
 * Sizes whose split states exceed FA_NOALLOC_SCRATCH_BYTES (see
 * fa_paged_decode_workspace_size) return FA_ERR_WORKSPACE without launching.
 * The 64-sequence, 32-head, 512-block-of-16 decode needs 17 MB of it.
 * Every call on one GPU uses that GPU's one array: calls that overlap on one
 * GPU (other streams, other host threads) race and give undefined results;
 * calls ordered on one stream are safe.  The scratch of the calling thread's
 * current device is used, so `stream` must belong to that device.
 * FA_ERR_HIP also if the scratch address cannot be looked up.
 */
#define FA_NOALLOC_SCRATCH_BYTES (32u << 20)
fa_status fa_paged_decode_noalloc(fa_dtype dt, const void* q, const void* k_cache,
                                  const void* v_cache, const int32_t* block_table,
                                  const int32_t* seq_lens, int block_size, int num_seqs,
                                  int heads_q, int heads_kv, int d, int dv, int num_blocks,
                                  int max_blocks_per_seq, float scale, void* o, void* stream);

/* Static text for a status code. */
const char* fa_status_string(fa_status s);

/* Text of the last error on the calling thread ("" if none). */
const char* fa_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* FA_H_ */
