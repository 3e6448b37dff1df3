/* attn.h — C ABI of libattn: exact attention with RoPE on MI355X (gfx950).
 *
 * Operations:
 *   attn_rope_apply       rotary position embedding, in place
 *   attn_prefill          causal (or full) grouped-query attention over a whole sequence
 *   attn_rope_table       (cos, sin) table of the rotary embedding by integer position
 *   attn_prefill_rope     attn_prefill with the rotation of Q fused into the kernel's load of Q
 *   attn_prefill_local_global  causal prefill with a sliding window plus global (leading, periodic) tokens
 *   attn_decode_paged     one query token per sequence against a paged KV cache (split-KV + log-sum-exp combine)
 *   attn_decode_paged_noalloc  attn_decode_paged with library-owned static scratch instead of a workspace
 *   attn_decode_paged_q8  the same over 8-bit (FP8 E4M3 or int8) K/V caches with per-channel scales
 *   attn_mla_decode       multi-head latent attention decode in the absorbed form
 *   attn_mla_decode_q8    the same over an 8-bit (FP8 E4M3 or int8) latent cache with per-channel scales
 *   attn_kv_append_paged  write new tokens' keys (rotated) and values into a paged KV cache
 *   attn_prefill_paged    chunked / variable-length causal prefill of new tokens against a paged KV cache
 *   attn_prefill_paged_rope  the same with RoPE of the queries fused into their load
 *   attn_dsa_indexer      DeepSeek Sparse Attention: lightning-indexer relevance score of every cached token
 *   attn_topk             the indices of the top-k scores of each sequence
 *   attn_mla_sparse_decode  absorbed MLA decode over a list of selected tokens per sequence
 *
 * Every result is the exact softmax attention O = softmax(scale * Q K^T [+ mask]) V. The kernels compute it
 * FlashAttention-style: scores are formed tile by tile on chip, an online softmax keeps a running row max m and
 * a running exp-sum l and rescales the output accumulator whenever m grows, and S and P are never written to
 * memory. (Attention notes, makinaruto.github.io, posts/nlp/llm_learning/attention: sections "FlashAttention"
 * and "online-softmax", update equations for m and l.)
 *
 * Conventions shared by every entry point
 *   - Pointers named as tensors are DEVICE pointers; `stream` is a hipStream_t passed as void* (NULL = the
 *     default stream). Every call only enqueues work on `stream` and returns; it never synchronises, never
 *     allocates or frees device memory, never changes the current device, and keeps no state between calls,
 *     so calls are re-entrant and thread-safe. The caller owns every buffer, including the workspace. The one
 *     exception is attn_decode_paged_noalloc, whose scratch is the library's own (see there).
 *   - Layouts are row-major with the last dimension contiguous. "bf16" is IEEE bfloat16 (results rounded to
 *     nearest even); arithmetic inside the kernels is fp32.
 *   - All validation happens on the host before anything is enqueued: on any error nothing is launched and the
 *     output buffers are untouched. Return value is an attn_status_t:
 *       ATTN_ERR_INVALID_ARG  a required pointer is NULL, a size is negative or inconsistent (Hq % Hkv != 0,
 *                             odd head_dim for RoPE), or the scale is not a finite positive number;
 *       ATTN_ERR_UNSUPPORTED  a valid request this build does not implement (see each function);
 *       ATTN_ERR_WORKSPACE    workspace smaller than the matching *_workspace_size();
 *       ATTN_ERR_HIP          the HIP runtime reported an error at launch. Faults inside a kernel surface
 *                             later, at the caller's synchronisation, as with any HIP kernel.
 *   - Sizes of zero (no tokens, no sequences) are valid and launch nothing.
 */
#ifndef ATTN_H
#define ATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum { ATTN_BF16 = 0, ATTN_FP32 = 1 } attn_dtype_t;

/* 8-bit KV cache element kinds (attn_decode_paged_q8). */
typedef enum { ATTN_KV_FP8_E4M3 = 1, ATTN_KV_INT8 = 2 } attn_kv8_t;

typedef enum {
  ATTN_OK = 0,
  ATTN_ERR_INVALID_ARG = 1,
  ATTN_ERR_UNSUPPORTED = 2,
  ATTN_ERR_WORKSPACE = 3,
  ATTN_ERR_HIP = 4
} attn_status_t;

/* Rotary position embedding, in place.
 * (DeepSeek 32K to 256K long context, tqpw.cn, section 2.1: frequencies theta_i = theta^(-2i/d) and the rotation
 *  [cos -sin; sin cos] applied to pairs of the last dimension; section 2.5: positions are integers, so angles are
 *  taken from the integer position directly rather than accumulated.)
 *   x          [n_tokens, n_heads, head_dim] of `dtype` (ATTN_BF16 or ATTN_FP32), rotated in place. Prefill Q/K in
 *              [B, S, H, D] layout are n_tokens = B*S rows; decode queries [B, H, D] are n_tokens = B rows.
 *   positions  [n_tokens] int32 >= 0, the position of each token row.
 *   theta      RoPE base (10000 for standard RoPE; an NTK-scaled base for stretched contexts), finite, > 1.
 *   interleaved  1: pairs (2i, 2i+1) — the pairing the page prints; 0: pairs (i, i + head_dim/2).
 * For pair i of a token at position p the angle is p * theta^(-2i/head_dim); the angle, its sine and its cosine
 * are evaluated in fp64 and rounded to fp32, the rotation is fp32, and the results are rounded to `dtype`.
 * Errors: INVALID_ARG for NULL x/positions (with n_tokens > 0), odd or non-positive head_dim, n_heads <= 0,
 * theta <= 1 or non-finite; UNSUPPORTED for head_dim > 1024 or another dtype. */
int attn_rope_apply(void* x, attn_dtype_t dtype, int64_t n_tokens, int n_heads, int head_dim,
                    const int32_t* positions, double theta, int interleaved, void* stream);

/* Prefill attention: every query position of a batch of sequences attends to the keys of its own sequence.
 * (Attention notes, makinaruto.github.io: "FlashAttention" — intermediates stay on chip, one read and one write
 *  of HBM; "online-softmax" — running max and exp-sum per block; "Group-Query Attention" derivation table —
 *  query heads share KV heads in consecutive groups.)
 *   q          [batch, seqlen, n_heads_q,  head_dim] of dtype (rotated already, see attn_rope_apply)
 *   k, v       [batch, seqlen, n_heads_kv, head_dim] of dtype
 *   o          [batch, seqlen, n_heads_q,  head_dim] of dtype, written
 *   lse        NULL, or [batch, n_heads_q, seqlen] fp32 written with the natural-log sum-exp of each row's
 *              scaled scores (lse = ln sum_j exp(scale * q.k_j) over the visible keys)
 *   causal     1: key j is visible to query i iff j <= i; 0: every key is visible.
 *   softmax_scale  multiplies q.k inside the softmax (1/sqrt(head_dim) for standard attention).
 * Query head h uses KV head h / (n_heads_q / n_heads_kv).
 * Supported: dtype ATTN_BF16 (bf16 MFMA, fp32 accumulation) or ATTN_FP32 (fp32 throughout), head_dim 64 or
 * 128; anything else is UNSUPPORTED. INVALID_ARG: NULL q/k/v/o (with batch*seqlen > 0), n_heads_q % n_heads_kv
 * != 0, non-positive head counts, bad scale. */
int attn_prefill(const void* q, const void* k, const void* v, void* o, float* lse, attn_dtype_t dtype, int batch,
                 int seqlen, int n_heads_q, int n_heads_kv, int head_dim, int causal, float softmax_scale,
                 void* stream);

/* The rotary embedding's (cos, sin) table by integer position.
 * (DeepSeek 32K to 256K long context, tqpw.cn, section 2.5: cos and sin are precomputed per integer position and
 *  looked up; section 2.1: pair i rotates by the angle position * theta^(-2i/d).)
 *   table        [n_positions, head_dim/2] pairs of fp32 (cos, sin), written: entry (p, i) holds the cosine and
 *                sine of p * theta^(-2i/head_dim), evaluated in fp64 and rounded to fp32 — exactly the values
 *                attn_rope_apply uses, so a rotation read from this table matches attn_rope_apply bit for bit.
 *   theta        RoPE base, finite, > 1.
 * Errors: INVALID_ARG for NULL table (with n_positions > 0), n_positions < 0, odd or non-positive head_dim,
 * bad theta; UNSUPPORTED for head_dim > 1024. */
int attn_rope_table(void* table, int n_positions, int head_dim, double theta, void* stream);

/* attn_prefill (bf16) with RoPE of the queries fused into the kernel: q is NOT rotated; each query is rotated
 * as the kernel loads it, with the cos/sin of its position read from a table made by attn_rope_table, so the
 * separate read and write of Q by attn_rope_apply disappear. Keys must be rotated already (attn_rope_apply): every
 * workgroup of a KV head reads them.
 * (Same passages as attn_rope_apply and attn_prefill.)
 *   q, k, v, o, lse, batch .. softmax_scale   as attn_prefill with dtype ATTN_BF16.
 *   q_positions  NULL (query i of each sequence is at position i) or [batch * seqlen] int32 device positions,
 *                one per query row in q's row order. A position outside [0, rope_table_len) is clamped into it.
 *   rope_table   [rope_table_len, head_dim/2] (cos, sin) fp32 from attn_rope_table with this head_dim, 16-byte
 *                aligned; read only.
 *   interleaved  pairing as attn_rope_apply (1: (2i, 2i+1); 0: (i, i + head_dim/2)).
 * The output equals attn_rope_apply(q) followed by attn_prefill bit for bit (same table values, same fp32
 * rotation arithmetic, same rounding); q itself is left unrotated.
 * Supported: head_dim 64 or 128, and a table under 4 GiB (else UNSUPPORTED). INVALID_ARG: as attn_prefill, plus
 * NULL or misaligned rope_table or rope_table_len <= 0 (with batch*seqlen > 0). */
int attn_prefill_rope(const void* q, const void* k, const void* v, void* o, float* lse, int batch, int seqlen,
                      int n_heads_q, int n_heads_kv, int head_dim, int causal, float softmax_scale,
                      const int32_t* q_positions, const void* rope_table, int rope_table_len, int interleaved,
                      void* stream);

/* Causal prefill with a local + global mask: key j is visible to query i iff j <= i and (i - j < window, or
 * j < n_lead, or anchor_stride > 0 and j % anchor_stride == 0).
 * ("DeepSeek 32K to 256K long context", tqpw.cn, section 4.1: a sliding window keeps the local neighbourhood and a
 *  few global tokens, such as a leading CLS token and periodic anchors at a global sampling rate, keep long-range
 *  links.) window >= S, or anchor_stride 1, gives plain causal attention; window 1 with no globals gives O = V.
 *   q, k, v, o, lse, sizes and scale as attn_prefill (bf16 only, causal by definition).
 *   window >= 1 (keys i-window+1 .. i), n_lead >= 0 leading global tokens, anchor_stride >= 0 (0: no anchors;
 *   otherwise the global sampling rate is 1/anchor_stride and key 0 is an anchor).
 * Work is proportional to window + globals per query, not to i. Unsupported: head_dim other than 64 or 128;
 * anchor_stride * 64 * n_heads_kv * head_dim * 2 >= 2^31. INVALID_ARG as attn_prefill, and for window < 1 or a
 * negative n_lead or anchor_stride. */
int attn_prefill_local_global(const void* q, const void* k, const void* v, void* o, float* lse, int batch, int seqlen,
                              int n_heads_q, int n_heads_kv, int head_dim, int window, int n_lead, int anchor_stride,
                              float softmax_scale, void* stream);

/* Bytes of workspace attn_decode_paged needs for these sizes (0 if any size is non-positive). */
size_t attn_decode_paged_workspace_size(int batch, int n_heads_q, int head_dim, int max_seqlen_kv);

/* Decode over a paged KV cache: one query token per sequence attends to the sequence's seq_lens[b] cached tokens.
 * (Attention notes, makinaruto.github.io: "Page Attention" — the cache is cut into fixed-size pages addressed
 *  through a logical-to-physical map; "online-softmax" — the per-chunk (O, m, l) results merge exactly, so the
 *  keys are split into fixed logical chunks that run in parallel and a second pass combines them by their
 *  log-sum-exp.)
 *   q            [batch, n_heads_q, head_dim] bf16, already rotated (attn_rope_apply at position seq_len-1)
 *   k_cache, v_cache  [num_pages, page_size, n_heads_kv, head_dim] bf16
 *   block_table  [batch, max_pages_per_seq] int32: logical token t of sequence b lives in physical page
 *                block_table[b][t / page_size], slot t % page_size. Only entries t < seq_lens[b] are read,
 *                so unused entries may hold anything (e.g. -1).
 *   seq_lens     [batch] int32 on the device, 0 <= seq_lens[b] <= max_seqlen_kv and
 *                <= max_pages_per_seq * page_size. The library never reads it on the host.
 *   o            [batch, n_heads_q, head_dim] bf16, written; a sequence of length 0 gets O = 0.
 *   lse          NULL or [batch, n_heads_q] fp32 (-inf for a sequence of length 0).
 *   workspace    device buffer of at least attn_decode_paged_workspace_size(batch, n_heads_q, head_dim,
 *                max_seqlen_kv) bytes; its contents need no initialisation and are clobbered.
 * The result does not depend on where pages sit physically: chunk boundaries are logical, so two block tables
 * over the same logical K/V give bitwise identical outputs. A page index outside [0, num_pages) in a used entry
 * is not dereferenced (that chunk of keys is treated as zeros); such a result is meaningless but safe.
 * Supported: head_dim 128 or 64, n_heads_q / n_heads_kv <= 16, page_size a power of two in [16, 1024].
 * Otherwise UNSUPPORTED. INVALID_ARG as above, also for max_seqlen_kv < 0 or num_pages <= 0 (with batch > 0). */
int attn_decode_paged(const void* q, const void* k_cache, const void* v_cache, const int32_t* block_table,
                      const int32_t* seq_lens, void* o, float* lse, int batch, int n_heads_q, int n_heads_kv,
                      int head_dim, int page_size, int max_pages_per_seq, int64_t num_pages, int max_seqlen_kv,
                      float softmax_scale, void* workspace, size_t workspace_bytes, void* stream);

/* Size of the static device scratch behind attn_decode_paged_noalloc (64 MiB per GPU): the largest workspace,
 * as attn_decode_paged_workspace_size reports it, that the no-allocation entry point can serve. */
#define ATTN_DECODE_SCRATCH_BYTES ((size_t)64 << 20)

/* attn_decode_paged without a workspace argument, for callers that cannot allocate device memory: code under HIP
 * graph capture, tight serving loops, harnesses that forbid allocation. The split partials go to a static device
 * array of ATTN_DECODE_SCRATCH_BYTES owned by the library, one copy per GPU, which exists from the moment the
 * library's code is loaded on that GPU until the process ends. The first call on a device looks up that device's
 * copy (hipGetSymbolAddress with the device current); later calls reuse the address. The call itself allocates
 * and frees nothing.
 *   All arguments as attn_decode_paged, without workspace; `stream` must belong to the current device.
 * Errors: as attn_decode_paged, plus ATTN_ERR_WORKSPACE when attn_decode_paged_workspace_size(batch, n_heads_q,
 * head_dim, max_seqlen_kv) exceeds ATTN_DECODE_SCRATCH_BYTES (at head_dim 128 and 64 sequences x 32 query heads,
 * max_seqlen_kv up to 64512 fits), ATTN_ERR_UNSUPPORTED for a device ordinal of 64 or more, and ATTN_ERR_HIP when
 * the device's scratch address cannot be obtained.
 * Every call on one GPU shares that GPU's scratch, which keeps the last call's contents: calls whose executions
 * overlap on one GPU (different streams, or host threads that do not order their streams) race and give wrong
 * results. Calls on one stream are ordered and safe. Nothing in the scratch needs to start at zero: every partial
 * a call reads is written earlier by the same call. Results are bitwise those of attn_decode_paged. */
int attn_decode_paged_noalloc(const void* q, const void* k_cache, const void* v_cache, const int32_t* block_table,
                              const int32_t* seq_lens, void* o, float* lse, int batch, int n_heads_q, int n_heads_kv,
                              int head_dim, int page_size, int max_pages_per_seq, int64_t num_pages,
                              int max_seqlen_kv, float softmax_scale, void* stream);

/* Paged decode over 8-bit K/V caches: attn_decode_paged where each cached value is code * scale[kv_head][channel].
 * ("DeepSeek 32K to 256K long context", tqpw.cn, section 2.5: K and V kept as int8 with per-channel scales;
 *  "7 anti-patterns of DeepSeek attention optimisation", lpnh.cn, section 3.3: FP8 E4M3, largest value 448.)
 *   k_cache, v_cache  [num_pages, page_size, n_heads_kv, head_dim] bytes: OCP FP8 E4M3 codes (kv_kind
 *                ATTN_KV_FP8_E4M3; the NaN code S.1111.111 must not occur) or int8 (ATTN_KV_INT8), 16-byte aligned.
 *   k_scale, v_scale  [n_heads_kv, head_dim] fp32 per-channel scales (16-byte aligned).
 *   Everything else as attn_decode_paged (same workspace size). The K scale is folded into the query, rounded to
 *   bf16 once per query; the V scale multiplies the output channels in fp32.
 * Supported and INVALID_ARG as attn_decode_paged, plus INVALID_ARG for a misaligned pointer and UNSUPPORTED for
 * another kv_kind. */
int attn_decode_paged_q8(const void* q, const void* k_cache, const void* v_cache, const float* k_scale,
                         const float* v_scale, int kv_kind, const int32_t* block_table, const int32_t* seq_lens,
                         void* o, float* lse, int batch, int n_heads_q, int n_heads_kv, int head_dim, int page_size,
                         int max_pages_per_seq, int64_t num_pages, int max_seqlen_kv, float softmax_scale,
                         void* workspace, size_t workspace_bytes, void* stream);

/* Bytes of workspace attn_mla_decode needs for these sizes (0 if any size is non-positive). */
size_t attn_mla_decode_workspace_size(int batch, int n_heads, int kv_lora_rank, int max_seqlen_kv);

/* Multi-head latent attention decode, absorbed form: all heads share one latent cache c_kv and one rope key
 * k_pe; scores are scale * (q_latent . c_kv_t + q_pe . k_pe_t) and the output stays in the latent space,
 * O_latent = softmax(scores) . c_kv.
 * (DeepSeek-V3 attention guide: einsum vs manual optimisation, dksg.cn: the absorb-mode score einsums over
 *  kv_cache and pe_cache; Attention notes, makinaruto.github.io, "Multi-Head Latent Attention": K = C^KV W^K_up
 *  and V = C^KV W^V_up, with W^K_up folded into the query side and W^V_up into W^O; "RoPE" compatibility
 *  section: the rotated part of the key is shared across heads.)
 *   q_latent     [batch, n_heads, kv_lora_rank] bf16 (the no-RoPE query already multiplied by W^K_up)
 *   q_pe         [batch, n_heads, rope_dim] bf16 (rotated)
 *   c_kv         [batch, max_seqlen_kv, kv_lora_rank] bf16
 *   k_pe         [batch, max_seqlen_kv, rope_dim] bf16 (rotated)
 *   seq_lens     [batch] int32 on the device, 0 <= seq_lens[b] <= max_seqlen_kv
 *   o_latent     [batch, n_heads, kv_lora_rank] bf16, written (0 for a sequence of length 0)
 *   lse          NULL or [batch, n_heads] fp32
 *   workspace    >= attn_mla_decode_workspace_size(batch, n_heads, kv_lora_rank, max_seqlen_kv) bytes.
 * Supported: kv_lora_rank 512, rope_dim 64, n_heads 32, 64, 96 or 128 (one wave per 16 heads, all heads of a
 * sequence in one workgroup).
 * Otherwise UNSUPPORTED. INVALID_ARG as above. */
int attn_mla_decode(const void* q_latent, const void* q_pe, const void* c_kv, const void* k_pe,
                    const int32_t* seq_lens, void* o_latent, float* lse, int batch, int n_heads, int kv_lora_rank,
                    int rope_dim, int max_seqlen_kv, float softmax_scale, void* workspace, size_t workspace_bytes,
                    void* stream);

/* MLA decode (as attn_mla_decode) over an 8-bit latent cache: c_kv and k_pe hold 8-bit codes with one fp32 scale
 * per channel, shared by every token and head.
 * ("DeepSeek 32K to 256K long context", tqpw.cn, section 2.5: cached keys and values stored as 8-bit integers with
 *  a per-channel scale; "7 anti-patterns of DeepSeek attention optimisation", lpnh.cn, section 3.3: FP8 E4M3,
 *  largest finite value 448; "DeepSeek-V3 attention guide", dksg.cn: the absorbed scores over the shared latent
 *  cache kv_cache and rope cache pe_cache, served in FP8 as well as BF16.)
 *   c_kv       [batch, max_seqlen_kv, kv_lora_rank] uint8 codes; value = decode(code) * c_scale[channel]
 *   k_pe       [batch, max_seqlen_kv, rope_dim] uint8 codes;     value = decode(code) * pe_scale[channel]
 *   c_scale    [kv_lora_rank] fp32, pe_scale [rope_dim] fp32
 *   kv_kind    ATTN_KV_FP8_E4M3 (OCP E4M3: bias 7, subnormals, no infinities, S.1111.111 is NaN) or ATTN_KV_INT8
 *              (two's complement)
 *   q_latent, q_pe, seq_lens, o_latent, lse, workspace: as attn_mla_decode (same workspace size).
 * The result is the exact attention over the dequantised cache. Codes widen exactly to bf16 for the MFMA; the key
 * scales are folded into the query (one bf16 rounding of q * scale per element), the value scales multiply the
 * output channels in fp32. All of q_latent, q_pe, c_kv, k_pe and both scale arrays must be 16-byte aligned.
 * Errors: as attn_mla_decode, plus INVALID_ARG for a NULL or misaligned scale or tensor, UNSUPPORTED for another
 * kv_kind. */
int attn_mla_decode_q8(const void* q_latent, const void* q_pe, const void* c_kv, const void* k_pe,
                       const float* c_scale, const float* pe_scale, int kv_kind, const int32_t* seq_lens,
                       void* o_latent, float* lse, int batch, int n_heads, int kv_lora_rank, int rope_dim,
                       int max_seqlen_kv, float softmax_scale, void* workspace, size_t workspace_bytes, void* stream);

/* Append new tokens to a paged KV cache, rotating the keys.
 * (Attention notes, makinaruto.github.io, "Page Attention": logical token t of a sequence lives in physical page
 *  block_table[t / page_size], slot t % page_size; DeepSeek 32K to 256K long context, tqpw.cn, sections 2.1 and
 *  2.5: RoPE at the token's integer position.)
 *   k_new, v_new  [total_new, n_heads_kv, head_dim] bf16: the new tokens of all sequences, packed in order; the rows
 *                 of sequence b are cu_new[b] .. cu_new[b+1]-1. 16-byte aligned.
 *   cu_new       [batch + 1] int32, non-decreasing, cu_new[0] = 0, cu_new[batch] = total_new.
 *   cache_lens   [batch] int32 >= 0: tokens already in sequence b's cache. New row r of sequence b goes to
 *                absolute position p = cache_lens[b] + r - cu_new[b]: page block_table[b][p / page_size], slot
 *                p % page_size. Its key is rotated at position p with base `theta` (pairing as attn_rope_apply's
 *                `interleaved`); its value is copied.
 *   k_cache, v_cache  [num_pages, page_size, n_heads_kv, head_dim] bf16, written in place (16-byte aligned).
 *   block_table  [batch, max_pages_per_seq] int32; the entries covering the new positions must name pages in
 *                [0, num_pages). A row whose page entry is out of range, or whose position is past the table, is
 *                not written.
 * Unsupported: head_dim not a multiple of 16 or above 1024, page_size not a power of two. */
int attn_kv_append_paged(const void* k_new, const void* v_new, const int32_t* cu_new, const int32_t* cache_lens,
                         void* k_cache, void* v_cache, const int32_t* block_table, int batch, int total_new,
                         int n_heads_kv, int head_dim, int page_size, int max_pages_per_seq, int64_t num_pages,
                         double theta, int interleaved, void* stream);

/* Chunked / variable-length causal prefill from a paged KV cache.
 * The cache already holds, for each sequence b, its cache_lens[b] earlier tokens followed by its
 * n_b = cu_new[b+1] - cu_new[b] new tokens (attn_kv_append_paged). The new tokens are the queries: query i of
 * sequence b sits at absolute position cache_lens[b] + i and attends keys 0 .. cache_lens[b] + i. With fewer
 * queries than keys the causal mask is aligned to the last query (bottom-right). (Attention notes,
 * makinaruto.github.io: later tokens attend to all earlier ones; "Page Attention" for the cache mapping;
 * "FlashAttention" / "online-softmax" for the computation.)
 *   q            [total_new, n_heads_q, head_dim] bf16, already rotated at the absolute positions.
 *   k_cache, v_cache  [num_pages, page_size, n_heads_kv, head_dim] bf16; block_table [batch, max_pages_per_seq]
 *                int32, entries covering positions 0 .. cache_lens[b] + n_b - 1 in [0, num_pages) (an entry outside
 *                that range, or a position past max_pages_per_seq * page_size, reads as zero keys and values).
 *   cu_new, cache_lens  as for attn_kv_append_paged.
 *   max_new      >= every n_b (and <= total_new): sizes the grid; rows of queries past max_new are not written.
 *   o            [total_new, n_heads_q, head_dim] bf16.
 *   lse          [n_heads_q, total_new] fp32 (natural log) or NULL.
 * Query head h reads KV head h / (n_heads_q / n_heads_kv).
 * Unsupported: head_dim not 64 or 128; page_size not a power of two of at least 64. */
int attn_prefill_paged(const void* q, const void* k_cache, const void* v_cache, const int32_t* block_table,
                       const int32_t* cu_new, const int32_t* cache_lens, void* o, float* lse, int batch, int total_new,
                       int max_new, int n_heads_q, int n_heads_kv, int head_dim, int page_size, int max_pages_per_seq,
                       int64_t num_pages, float softmax_scale, void* stream);

/* attn_prefill_paged with q UNROTATED: each query is rotated as the kernel loads it, by the cos/sin of its position
 * from a table made by attn_rope_table, so the separate rotation pass over q is not needed. (Long-context page,
 * "DeepSeek 32K to 256K long context", tqpw.cn: section 2.1 for the rotation of pairs by position times frequency,
 * section 2.5 for the cos/sin cache indexed by integer position.) The result equals attn_rope_apply of q at the same
 * positions followed by attn_prefill_paged, bit for bit.
 *   q_positions  NULL (query i of sequence b is at its absolute position cache_lens[b] + i) or [total_new] int32
 *                device positions, one per row of q. A position outside [0, rope_table_len) is clamped into it.
 *   rope_table   [rope_table_len, head_dim/2] (cos, sin) fp32 from attn_rope_table with this head_dim, 16-byte
 *                aligned, rope_table_len * head_dim * 4 < 2^32.
 *   interleaved  pairing as attn_rope_apply (1: (2i, 2i+1); 0: (i, i + head_dim/2)).
 * Other arguments, layouts and errors as attn_prefill_paged; also ATTN_ERR_INVALID_ARG for a NULL or misaligned
 * rope_table or rope_table_len <= 0 (with work to do). */
int attn_prefill_paged_rope(const void* q, const void* k_cache, const void* v_cache, const int32_t* block_table,
                            const int32_t* cu_new, const int32_t* cache_lens, void* o, float* lse, int batch,
                            int total_new, int max_new, int n_heads_q, int n_heads_kv, int head_dim, int page_size,
                            int max_pages_per_seq, int64_t num_pages, float softmax_scale, const int32_t* q_positions,
                            const void* rope_table, int rope_table_len, int interleaved, void* stream);

/* DeepSeek Sparse Attention, step 1: lightning-indexer scores for one query token per sequence.
 * (Attention notes, makinaruto.github.io, "Lighting Indexer": each earlier token s is scored by the sum over the
 *  indexer heads j of w_j * ReLU(q_j . k_s); the highest-scoring tokens are the ones attended.)
 *   q_idx     [batch, n_heads_idx, idx_dim] bf16: the indexer queries of the current token (16-byte aligned)
 *   w_idx     [batch, n_heads_idx] fp32: the per-head weights of the current token
 *   k_idx     [batch, max_seqlen_kv, idx_dim] bf16: one indexer key per cached token (16-byte aligned)
 *   seq_lens  [batch] int32 on the device, 0 <= seq_lens[b] <= max_seqlen_kv
 *   scores    [batch, max_seqlen_kv] fp32, written: scores[b][s] = sum_j w_j * max(0, q_j . k_s) for s < seq_lens[b]
 *             (fp32 accumulation of bf16 products), -inf for s >= seq_lens[b].
 * Nothing is scaled or rotated here: any scale or position encoding is already in the inputs.
 * Supported: n_heads_idx 32 or 64, idx_dim 64 or 128; otherwise UNSUPPORTED. */
int attn_dsa_indexer(const void* q_idx, const float* w_idx, const void* k_idx, const int32_t* seq_lens,
                     float* scores, int batch, int n_heads_idx, int idx_dim, int max_seqlen_kv, void* stream);

/* DeepSeek Sparse Attention, step 2: the top-k tokens of each sequence by score ("only the most relevant tokens",
 * Attention notes, "Lighting Indexer").
 *   scores    [batch, max_seqlen_kv] fp32 (e.g. from attn_dsa_indexer); only the first seq_lens[b] of row b are
 *             read. A NaN score (of either sign) ranks below every number, -inf included, and all NaNs tie.
 *   indices   [batch, topk] int32, written: the min(topk, seq_lens[b]) selected token indices in ascending order,
 *             then -1. Selected = the topk largest scores; at equal scores the lower index wins, so the result is
 *             unique (-0 and +0 are equal). A sequence with at most topk tokens keeps all of them.
 * INVALID_ARG for topk <= 0. */
int attn_topk(const float* scores, const int32_t* seq_lens, int32_t* indices, int batch, int max_seqlen_kv, int topk,
              void* stream);

/* Bytes of workspace attn_mla_sparse_decode needs for these sizes (0 if any size is non-positive). */
size_t attn_mla_sparse_decode_workspace_size(int batch, int n_heads, int kv_lora_rank, int topk);

/* DeepSeek Sparse Attention, step 3: absorbed MLA decode (as attn_mla_decode) restricted, for each sequence b, to
 * the tokens indices[b][0 .. topk-1] (Attention notes, "Lighting Indexer": attention over the selected tokens only;
 * the MLA passages as cited for attn_mla_decode).
 *   indices   [batch, topk] int32 on the device: token indices into sequence b's caches. Entries outside
 *             [0, seq_lens[b]) (e.g. the -1 padding of attn_topk) are ignored; a repeated index counts twice.
 *   The other arguments are those of attn_mla_decode; max_seqlen_kv is the caches' token dimension (> 0).
 *   o_latent  0 and lse -inf for a sequence with no valid index.
 *   workspace >= attn_mla_sparse_decode_workspace_size(batch, n_heads, kv_lora_rank, topk) bytes.
 * Only the selected tokens' rows are read. Supported as attn_mla_decode, with max_seqlen_kv * kv_lora_rank * 2
 * <= 2^31. */
int attn_mla_sparse_decode(const void* q_latent, const void* q_pe, const void* c_kv, const void* k_pe,
                           const int32_t* seq_lens, const int32_t* indices, void* o_latent, float* lse, int batch,
                           int n_heads, int kv_lora_rank, int rope_dim, int max_seqlen_kv, int topk,
                           float softmax_scale, void* workspace, size_t workspace_bytes, void* stream);

/* Static, human-readable name of a status code (never NULL). */
const char* attn_status_string(int status);

#ifdef __cplusplus
}
#endif

#endif /* ATTN_H */
