/*
 * libattn — fused scaled-dot-product attention for AMD Instinct MI355X (gfx950).
 *
 * O = softmax(scale * Q K^T + mask) V, computed tile by tile with online
 * softmax statistics (running max, running sum, output rescaling) so that the
 * T x T score matrix never reaches device memory, plus the per-row
 * log-sum-exp. This is the blockwise attention described on the-ai.news,
 * "Snelle attention-kernels en operatorfusie versnellen AI-modellen",
 * section "FlashAttention-type aandacht en gepagineerde aandacht": per block
 * a part of the scores is computed, the softmax statistics are updated and
 * the output is accumulated on chip. The same section defines the paged KV
 * cache read by attn_decode_paged: fixed-size blocks plus a block table that
 * maps logical positions to physical blocks, 16 tokens per block in its vLLM
 * example.
 *
 * Conventions shared by every call
 *  - Ownership: every array argument is a caller-owned device pointer to a
 *    contiguous, row-major buffer. The library allocates nothing, never
 *    synchronises, and enqueues its kernels asynchronously on `stream`
 *    (0 = the null stream). Calls are therefore stream-ordered and may be
 *    captured in a HIP graph (stable addresses required).
 *  - Errors: every entry point returns an attn_status. Problems visible on the
 *    host (null or misaligned pointers, bad sizes, unsupported head size or
 *    dtype, too small a workspace) return ATTN_ERR_INVALID or
 *    ATTN_ERR_UNSUPPORTED before anything is launched; there is no silent
 *    fallback (the same page notes that hard-coding a backend must fail when
 *    no backend supports the inputs). A failed launch returns ATTN_ERR_HIP.
 *    attn_last_error() returns a per-thread message for the last non-OK status.
 *  - Device-resident lengths (seq_lens, ctx_lens, q_lens, start_pos,
 *    new_lens) are trusted: checking them would need a synchronisation; values
 *    outside the ranges stated below are undefined behaviour.
 *  - Block ids: one rule for every call that takes a block table. An entry
 *    used for a block inside a sequence's context should lie in
 *    [0, num_blocks). Any other value marks an unmapped block: the appends
 *    write nothing to it, and the attention calls read its keys and values as
 *    zeros. No call ever reads or writes memory outside the caches because of
 *    a block id. Entries for blocks past a sequence's context may be loaded
 *    but are never used.
 *  - Alignment: q, k, v, o, k_cache, v_cache must be 16-byte aligned.
 *  - Numerics: products accumulate in fp32; the probabilities are rounded to
 *    the input dtype for the P.V product; O is rounded to the input dtype
 *    (round to nearest even); lse is fp32, natural log.
 */
#ifndef LIBATTN_H
#define LIBATTN_H

#include <stddef.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  ATTN_OK = 0,
  ATTN_ERR_INVALID = 1,      /* malformed argument (null, size, alignment)        */
  ATTN_ERR_UNSUPPORTED = 2,  /* well-formed but not served (head size, dtype ...) */
  ATTN_ERR_HIP = 3           /* the HIP runtime reported an error at launch       */
} attn_status;

typedef enum { ATTN_F16 = 0, ATTN_BF16 = 1 } attn_dtype;

/*
 * Prefill / encoder attention (blockwise attention of the section cited above).
 *
 *  q, o   : [B, Hq, Tq, D] elements of `dtype`.  o may not alias q, k or v.
 *  k, v   : [B, Hkv, Tk, D] elements of `dtype`.
 *  lse    : [B, Hq, Tq] fp32, natural-log log-sum-exp of the scaled, masked
 *           scores of each query row; may be NULL.
 *  Hq % Hkv == 0; query head h reads kv head h / (Hq / Hkv) (grouped-query
 *  attention; Hq == Hkv is multi-head attention).
 *  D in {64, 128}. B, Hq, Hkv, Tq, Tk >= 1; every tensor must hold fewer
 *  than 2^31 elements.
 *  scale  : multiplies q.k before the softmax (any finite value; 1/sqrt(D) is
 *           the usual choice). Applied in fp32 to the fp32 dot products.
 *  causal : nonzero -> key j is visible to query i iff j <= i + (Lk - Lq)
 *           (bottom-right aligned, diagonal included).
 *  seq_lens: NULL, or a device int32 array [B] of valid lengths
 *           (1 <= seq_lens[b] <= Tq) for ragged batches; requires Tq == Tk and
 *           applies to queries and keys alike (Lq = Lk = seq_lens[b]).
 *           Positions >= seq_lens[b] are padding: they are never read into
 *           the result, no work is spent on whole padding tiles, and the
 *           padded output rows receive O = 0 and lse = -inf.
 *  A query row that sees no key (possible only through the causal mask when
 *  Lq > Lk) receives O = 0 and lse = -inf.
 */
attn_status attn_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
                     int B, int Hq, int Hkv, int Tq, int Tk, int D,
                     float scale, int causal, const int* seq_lens,
                     attn_dtype dtype, hipStream_t stream);

/*
 * One-token decode through a paged KV cache (paged attention of the section
 * cited above): the key/value of position t of sequence b live in physical
 * block block_table[b, t / block_size], slot t % block_size.
 *
 *  q, o        : [B, Hq, D] elements of `dtype` (one new token per sequence).
 *  k_cache,
 *  v_cache     : [num_blocks, Hkv, block_size, D] elements of `dtype`, so every
 *                (block, kv head) holds block_size*D contiguous elements.
 *  block_table : device int32 [B, max_blocks_per_seq], 4-byte aligned; block
 *                ids follow the rule above (entries at or beyond
 *                ceil(ctx_lens[b] / block_size) are never used).
 *  ctx_lens    : device int32 [B]; 1 <= ctx_lens[b] <= max_blocks_per_seq *
 *                block_size. It counts every cached token including the new
 *                one, whose key/value are already in the cache: the query sees
 *                positions 0 .. ctx_lens[b]-1. Slots beyond it are never used.
 *  lse         : [B, Hq] fp32 natural-log log-sum-exp; may be NULL; 4-byte
 *                aligned (ctx_lens too).
 *  block_size == 16, D in {64, 128}, Hq % Hkv == 0, Hq / Hkv <= 16.
 *  workspace   : device scratch of at least attn_decode_workspace_bytes(...)
 *                bytes, 256-byte aligned, owned by the caller; contents on
 *                entry are ignored. A long context is split into ranges of 256
 *                tokens handled by different workgroups; the workspace holds
 *                their partial results until a second kernel merges them.
 *                Calls that share a workspace must be ordered on one stream.
 *                May be NULL when max_blocks_per_seq <= 16 (one range only).
 */
attn_status attn_decode_paged(const void* q, const void* k_cache, const void* v_cache,
                              const int* block_table, const int* ctx_lens, void* o, float* lse,
                              int B, int Hq, int Hkv, int D, int block_size,
                              int max_blocks_per_seq, int num_blocks, float scale,
                              attn_dtype dtype, void* workspace, size_t workspace_bytes,
                              hipStream_t stream);

/*
 * Chunked prefill through the paged KV cache: the prefill of the section cited
 * above, with keys/values read through the block table of the paged cache
 * (the address translation attn_decode_paged uses), so that a long prompt can
 * be processed in chunks whose keys/values have already been appended to the
 * cache (attn_cache_append), or one more chunk attends to a cached prefix.
 *
 *  q, o        : [B, Hq, Tq, D] elements of `dtype`. Row i < q_lens[b] of
 *                sequence b is position ctx_lens[b] - q_lens[b] + i: the
 *                newest q_lens[b] positions. Rows >= q_lens[b] are padding and
 *                receive O = 0, lse = -inf.
 *  k_cache,
 *  v_cache     : [num_blocks, Hkv, block_size, D] as for attn_decode_paged;
 *                the keys/values of positions 0 .. ctx_lens[b]-1 must be in
 *                the cache (the chunk's own included).
 *  block_table : device int32 [B, max_blocks_per_seq], 4-byte aligned; block
 *                ids follow the rule above (entries at or beyond
 *                ceil(ctx_lens[b] / block_size) are never used).
 *  ctx_lens    : device int32 [B]; q_lens[b] <= ctx_lens[b] <=
 *                max_blocks_per_seq * block_size.
 *  q_lens      : device int32 [B] with 0 <= q_lens[b] <= Tq, or NULL (every
 *                row is a query: q_lens[b] = Tq).
 *  lse         : [B, Hq, Tq] fp32 natural-log log-sum-exp; may be NULL.
 *  causal      : nonzero -> row i sees keys j <= i + ctx_lens[b] - q_lens[b]
 *                (the bottom-right alignment of attn_fwd); zero -> every row
 *                sees all ctx_lens[b] keys.
 *  block_size == 16, D in {64, 128}, Hq % Hkv == 0,
 *  max_blocks_per_seq <= 2048 (contexts up to 32768 tokens: a workgroup keeps
 *  the sequence's table row in on-chip memory). No workspace.
 */
attn_status attn_fwd_paged(const void* q, const void* k_cache, const void* v_cache,
                           const int* block_table, const int* ctx_lens, const int* q_lens,
                           void* o, float* lse, int B, int Hq, int Hkv, int Tq, int D,
                           int block_size, int max_blocks_per_seq, int num_blocks, float scale,
                           int causal, attn_dtype dtype, hipStream_t stream);

/*
 * Appends new keys/values to the paged KV cache (the block/slot mapping of the
 * paged cache of the section cited above): token i < new_lens[b] of k_new[b]
 * and v_new[b] becomes position p = start_pos[b] + i of sequence b, written to
 * physical block block_table[b, p / block_size], slot p % block_size. Nothing
 * else in the caches changes. Pure data movement (bit-exact copies).
 *
 *  k_new, v_new: [B, Hkv, Tnew, D] elements of `dtype`.
 *  k_cache,
 *  v_cache     : [num_blocks, Hkv, block_size, D], updated in place.
 *  block_table : device int32 [B, max_blocks_per_seq], 4-byte aligned; the
 *                blocks written must be mapped (entries in [0, num_blocks));
 *                a token whose position falls outside the table or on an
 *                unmapped entry is not written (the block-id rule above).
 *  start_pos   : device int32 [B], first position written (>= 0).
 *  new_lens    : device int32 [B] with 0 <= new_lens[b] <= Tnew, or NULL (all
 *                Tnew tokens).
 *  block_size == 16, D in {64, 128}. Two sequences must not map a written slot
 *  to the same physical block (the writes would race).
 */
attn_status attn_cache_append(const void* k_new, const void* v_new, void* k_cache, void* v_cache,
                              const int* block_table, const int* start_pos, const int* new_lens,
                              int B, int Hkv, int Tnew, int D, int block_size,
                              int max_blocks_per_seq, int num_blocks, attn_dtype dtype,
                              hipStream_t stream);

/*
 * FP8 KV cache. The pages name FP8 inference as the next step for LLM serving
 * (comemg.com, "天下苦英偉達久矣！PyTorch免CUDA加速推理，Triton時代要來？", section
 * "未來工作") and the fusion of dequantisation into the consuming product as a
 * standard fusion (the-ai.news page cited above, operator-fusion section);
 * they fix no format. Here the caches hold codes of the E4M3 format of the
 * OCP 8-bit floating point specification (1 byte per element: sign, 4
 * exponent bits with bias 7, 3 mantissa bits; largest finite 448; S.1111.111
 * is NaN) with one float scale per cache: an entry means value(code) * scale.
 *
 * attn_cache_append_fp8: as attn_cache_append, but k_new / v_new (bf16 or
 * fp16, `dtype`) are quantized on the way: code = E4M3(x / scale) with the
 * division in fp32 (correctly rounded), magnitudes above 448 saturating to
 * 448, round to nearest even. k_cache / v_cache are uint8
 * [num_blocks, Hkv, block_size, D]. k_scale, v_scale: finite, > 0.
 */
attn_status attn_cache_append_fp8(const void* k_new, const void* v_new, void* k_cache, void* v_cache,
                                  float k_scale, float v_scale, const int* block_table,
                                  const int* start_pos, const int* new_lens, int B, int Hkv, int Tnew,
                                  int D, int block_size, int max_blocks_per_seq, int num_blocks,
                                  attn_dtype dtype, hipStream_t stream);

/*
 * attn_decode_paged_fp8: as attn_decode_paged over uint8 E4M3 caches
 * [num_blocks, Hkv, block_size, D] with scales k_scale, v_scale (finite,
 * > 0): the result is the decode of the dequantized cache. q, o stay bf16 or
 * fp16 (`dtype`); the products run on that type (E4M3 values are exact in
 * both). Workspace: attn_decode_workspace_bytes, as for attn_decode_paged.
 */
attn_status attn_decode_paged_fp8(const void* q, const void* k_cache, const void* v_cache,
                                  float k_scale, float v_scale, const int* block_table,
                                  const int* ctx_lens, void* o, float* lse, int B, int Hq, int Hkv,
                                  int D, int block_size, int max_blocks_per_seq, int num_blocks,
                                  float scale, attn_dtype dtype, void* workspace,
                                  size_t workspace_bytes, hipStream_t stream);

/*
 * attn_fwd_fp8: prefill attention (attn_fwd) on E4M3 inputs: q, k, v are uint8
 * codes in attn_fwd's layouts with scales q_scale, k_scale, v_scale (finite,
 * > 0); o is `dtype` (bf16 or fp16), lse fp32. Both products run on the fp8
 * matrix cores (v_mfma_scale_f32_32x32x64_f8f6f4), twice the bf16 rate; the
 * scores are exact up to fp32 accumulation. The probabilities enter the P.V
 * product as E4M3 values: the running max moves only once a score exceeds it
 * by more than 1 (log2 units), so p = 2^(x - m) <= 2, and p * 2^7 (<= 2^8) is
 * rounded to nearest; O is divided by the fp32 sum of the unrounded p. Per
 * output element (row i, column d) the error against attention over the
 * dequantized inputs is then at most
 *   2^-4 * sum_j P_ij |v_jd| + 2^-17 * max_j P_ij * sum_j |v_jd|
 * over the row's visible keys j (P the exact softmax: each weight is off by
 * 2^-4 relative in E4M3's normal range, 2^-17 absolute below it), plus the
 * fp32 accumulation and the output rounding. Same masking, ragged and GQA
 * rules as attn_fwd.
 */
attn_status attn_fwd_fp8(const void* q, const void* k, const void* v, float q_scale, float k_scale,
                         float v_scale, void* o, float* lse, int B, int Hq, int Hkv, int Tq, int Tk,
                         int D, float scale, int causal, const int* seq_lens, attn_dtype dtype,
                         hipStream_t stream);

/*
 * attn_fwd_paged_fp8: the chunked prefill of attn_fwd_paged over uint8 E4M3
 * caches with scales k_scale, v_scale (as for attn_decode_paged_fp8): the
 * result is the chunked prefill of the dequantized cache. q, o stay bf16 or
 * fp16 (`dtype`). `rope` (may be NULL) and max_pos: as for
 * attn_fwd_paged_rope below (query rows rotated at their positions).
 */
attn_status attn_fwd_paged_fp8(const void* q, const void* k_cache, const void* v_cache,
                               float k_scale, float v_scale, const float* rope, int max_pos,
                               const int* block_table, const int* ctx_lens, const int* q_lens,
                               void* o, float* lse, int B, int Hq, int Hkv, int Tq, int D,
                               int block_size, int max_blocks_per_seq, int num_blocks, float scale,
                               int causal, attn_dtype dtype, hipStream_t stream);

/*
 * Rotary position embedding fused into the paged path. The Llama3-8B trace of
 * the comemg.com page (section "模型推理") shows RoPE among the small kernels
 * between the products and attention; fusing such a step into its neighbour
 * saves a round trip of the tensor through memory (the-ai.news page cited
 * above, operator-fusion section). The rotation is the half-split rotary
 * embedding of the Llama family: for a row x at position p and i < D/2,
 *   x'[i] = x[i] c - x[i + D/2] s,   x'[i + D/2] = x[i + D/2] c + x[i] s,
 * with c = rope[p, i] and s = rope[p, D/2 + i] from the caller's table
 * `rope`: device fp32 [max_pos, D], 16-byte aligned (cos(p theta_i) in the
 * first half of a row, sin in the second). Computed in fp32, rounded once to
 * the 16-bit type. Positions >= max_pos read row max_pos - 1 (caller error).
 *
 * attn_cache_append_rope: attn_cache_append with each new K row rotated at its
 *   position start_pos[b] + i before it is written (V rows unchanged), so the
 *   cache holds rotated keys.
 * attn_fwd_paged_rope: attn_fwd_paged with query row i rotated at its position
 *   ctx_lens[b] - q_lens[b] + i as it is loaded.
 * attn_decode_paged_rope: attn_decode_paged with the query rotated at position
 *   ctx_lens[b] - 1 as it is loaded.
 */
attn_status attn_cache_append_rope(const void* k_new, const void* v_new, void* k_cache, void* v_cache,
                                   const float* rope, int max_pos, const int* block_table,
                                   const int* start_pos, const int* new_lens, int B, int Hkv, int Tnew,
                                   int D, int block_size, int max_blocks_per_seq, int num_blocks,
                                   attn_dtype dtype, hipStream_t stream);

attn_status attn_fwd_paged_rope(const void* q, const void* k_cache, const void* v_cache,
                                const float* rope, int max_pos, const int* block_table,
                                const int* ctx_lens, const int* q_lens, void* o, float* lse, int B,
                                int Hq, int Hkv, int Tq, int D, int block_size, int max_blocks_per_seq,
                                int num_blocks, float scale, int causal, attn_dtype dtype,
                                hipStream_t stream);

attn_status attn_decode_paged_rope(const void* q, const void* k_cache, const void* v_cache,
                                   const float* rope, int max_pos, const int* block_table,
                                   const int* ctx_lens, void* o, float* lse, int B, int Hq, int Hkv,
                                   int D, int block_size, int max_blocks_per_seq, int num_blocks,
                                   float scale, attn_dtype dtype, void* workspace,
                                   size_t workspace_bytes, hipStream_t stream);

/*
 * Linear-layer matrix product with the reduction (K) dimension split across
 * workers and the pieces summed: the SplitK GEMM that the comemg.com page
 * ("天下苦英偉達久矣！PyTorch免CUDA加速推理，Triton時代要來？", section "Triton
 * SplitK GEMM 內核") uses for the Llama3-8B and Granite-8B linear layers, tuned
 * per weight shape as in its section "GEMM 內核調優":
 *
 *   y[m, n] = sum_k x[m, k] * w[n, k]        (y = x w^T, no bias)
 *
 *  x : device [M, K] elements of `dtype` (activations, one row per token),
 *      16-byte aligned.
 *  w : device [N, K] elements of `dtype` (the weight, out x in features),
 *      16-byte aligned.
 *  y : device [M, N] elements of `dtype`, 2-byte aligned; written.
 *  M, N, K >= 0, K % 8 == 0, K < 2^24. M == 0 or N == 0: nothing is written
 *  (the pointers are not used); K == 0: y = 0 (x and w may be null).
 * Products and sums in fp32, each output rounded once to `dtype`; the
 * summation order depends only on (K, configuration), so results are
 * deterministic. Sized for decode (a few rows of x): each launch covers 64
 * rows of x, so the weight is read ceil(M / 64) times. The K split is made
 * inside a workgroup (its waves sum consecutive K ranges, reduced in on-chip
 * memory): one launch, no workspace.
 *
 * attn_gemm_splitk uses the configuration tuned for (N, K) (the linear
 * layers named above) or a default one; attn_gemm_splitk_cfg takes it:
 *  rows   : weight rows per workgroup, 16 or 32
 *  waves  : waves per workgroup, 1 .. 16, each summing one K range
 *  unroll : k-steps of 32 per round of loads, 1, 2, 4 or 8
 * Errors: ATTN_ERR_INVALID (null pointer with M, N > 0, misalignment, bad
 * configuration), ATTN_ERR_UNSUPPORTED (dtype, K % 8, K too large).
 */
attn_status attn_gemm_splitk(const void* x, const void* w, void* y, int M, int N, int K,
                             attn_dtype dtype, hipStream_t stream);

attn_status attn_gemm_splitk_cfg(const void* x, const void* w, void* y, int M, int N, int K,
                                 attn_dtype dtype, int rows, int waves, int unroll,
                                 hipStream_t stream);

/*
 * attn_decode_paged without a workspace argument, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation). Same arguments and results as
 * attn_decode_paged; the split partials live in a static device array of 32
 * MiB that the library holds on each GPU it runs on until the process ends
 * (its address is looked up on a device's first call, with that device
 * current). Nothing is allocated or freed by the call.
 * Limit: attn_decode_workspace_bytes(B, Hq, Hkv, D, max_blocks_per_seq, 16)
 * <= 32 MiB, else ATTN_ERR_UNSUPPORTED before anything is launched.
 * Every call on one GPU shares that array: calls that overlap in time on one
 * GPU (different streams, or different threads without ordering) race and
 * give undefined results; calls ordered on one stream are safe. The array
 * keeps the last call's contents; nothing needs to start at zero.
 */
attn_status attn_decode_paged_noalloc(const void* q, const void* k_cache, const void* v_cache,
                                      const int* block_table, const int* ctx_lens, void* o, float* lse,
                                      int B, int Hq, int Hkv, int D, int block_size,
                                      int max_blocks_per_seq, int num_blocks, float scale,
                                      attn_dtype dtype, hipStream_t stream);

/* Workspace bytes attn_decode_paged needs for these sizes (0 if they are invalid). */
size_t attn_decode_workspace_bytes(int B, int Hq, int Hkv, int D, int max_blocks_per_seq, int block_size);

/* Static, human-readable name of a status code. */
const char* attn_status_str(attn_status s);

/* Per-thread detail message of the last non-OK status ("" if none). */
const char* attn_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* LIBATTN_H */
