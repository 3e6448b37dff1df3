// kernels.h — internal launchers behind the C ABI (not exported). Arguments are already validated by the
// caller; every launcher only enqueues on `stream` and returns hipGetLastError().
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace attn {

// RoPE, in place. dtype: 0 bf16, 1 fp32.
hipError_t launch_rope(void* x, int dtype, int64_t n_tokens, int n_heads, int head_dim, const int32_t* positions,
                       double theta, int interleaved, hipStream_t stream);

// Prefill. bf16: MFMA path; fp32: VALU path. head_dim 64 or 128.
// rope_table != NULL: Q is rotated as it is loaded ([rope_len, head_dim/2] (cos, sin) fp32 by position; query
// positions from q_positions [batch*seqlen], or 0..seqlen-1 when NULL; clamped into [0, rope_len)).
hipError_t launch_prefill_bf16(const void* q, const void* k, const void* v, void* o, float* lse, int batch,
                               int seqlen, int hq, int hkv, int head_dim, int causal, float scale,
                               hipStream_t stream, const void* rope_table = nullptr, int rope_len = 0,
                               const int32_t* q_positions = nullptr, int rope_interleaved = 0);
// table[p][i] = (cos, sin) of p * theta^(-2i/head_dim), p < n_positions, in fp64 rounded to fp32 (the values the
// rope kernel uses).
hipError_t launch_rope_table(void* table, int n_positions, int head_dim, double theta, hipStream_t stream);
// Causal prefill with a local + global mask: key j visible to query i iff j <= i and (i - j < window or
// j < n_lead or (anchor_stride > 0 and j % anchor_stride == 0)). bf16, head_dim 64 or 128.
hipError_t launch_prefill_window(const void* q, const void* k, const void* v, void* o, float* lse, int batch,
                                 int seqlen, int hq, int hkv, int head_dim, int window, int n_lead, int anchor_stride,
                                 float scale, hipStream_t stream);
// Chunked / variable-length causal prefill from a paged cache (bf16, head_dim 64 or 128, page size a power of two
// that is a multiple of 64).
hipError_t launch_prefill_paged(const void* q, const void* k_cache, const void* v_cache, const int32_t* block_table,
                                const int32_t* cu_new, const int32_t* ctx_lens, void* o, float* lse, int batch,
                                int total_new, int max_new, int hq, int hkv, int head_dim, int page_size,
                                int max_pages_per_seq, int64_t num_pages, float scale, hipStream_t stream,
                                const void* rope_table = nullptr, int rope_len = 0,
                                const int32_t* q_positions = nullptr, int rope_interleaved = 0);
// Append new K (rotated at its absolute positions) and V rows to a paged cache (bf16).
hipError_t launch_kv_append_paged(const void* k_new, const void* v_new, const int32_t* cu_new,
                                  const int32_t* ctx_lens, void* k_cache, void* v_cache, const int32_t* block_table,
                                  int batch, int total_new, int hkv, int head_dim, int page_size, int max_pages_per_seq,
                                  int64_t num_pages, double theta, int interleaved, hipStream_t stream);
hipError_t launch_prefill_fp32(const void* q, const void* k, const void* v, void* o, float* lse, int batch,
                               int seqlen, int hq, int hkv, int head_dim, int causal, float scale,
                               hipStream_t stream);

// Paged decode: split-KV partials into the workspace, then the log-sum-exp combine. head_dim 64 or 128.
#ifndef ATTN_DECODE_CHUNK
#define ATTN_DECODE_CHUNK 1024
#endif
constexpr int kDecodeChunk = ATTN_DECODE_CHUNK;  // keys per split (a multiple of 32); boundaries are logical positions
size_t decode_paged_workspace_bytes(int batch, int hq, int head_dim, int max_seqlen_kv);
hipError_t launch_decode_paged(const void* q, const void* k_cache, const void* v_cache, const int32_t* block_table,
                               const int32_t* seq_lens, void* o, float* lse, int batch, int hq, int hkv,
                               int head_dim, int page_size, int max_pages_per_seq, int64_t num_pages,
                               int max_seqlen_kv, float scale, void* workspace, hipStream_t stream);

// Paged decode over 8-bit K/V caches (fp8 != 0: FP8 E4M3 codes, else int8) with per-(KV head, channel) fp32
// scales [hkv, head_dim]; same workspace as launch_decode_paged. head_dim 64 or 128.
hipError_t launch_decode_paged_q8(int fp8, const void* q, const void* k_cache, const void* v_cache,
                                  const float* k_scale, const float* v_scale, const int32_t* block_table,
                                  const int32_t* seq_lens, void* o, float* lse, int batch, int hq, int hkv,
                                  int head_dim, int page_size, int max_pages_per_seq, int64_t num_pages,
                                  int max_seqlen_kv, float scale, void* workspace, hipStream_t stream);

// MLA absorbed decode: split over tokens, then the log-sum-exp combine.
int mla_num_splits(int batch, int n_heads, int max_seqlen_kv, int target_blocks);
int mla_split_len(int batch, int n_heads, int max_seqlen_kv, int target_blocks);
size_t mla_decode_workspace_bytes(int batch, int n_heads, int kv_lora_rank, int max_seqlen_kv);
size_t mla_sparse_workspace_bytes(int batch, int n_heads, int kv_lora_rank, int topk);
hipError_t launch_mla_decode(const void* q_latent, const void* q_pe, const void* c_kv, const void* k_pe,
                             const int32_t* seq_lens, void* o_latent, float* lse, int batch, int n_heads,
                             int max_seqlen_kv, float scale, void* workspace, hipStream_t stream);
// MLA decode over an 8-bit latent cache: c_kv [batch, max_len, 512] and k_pe [batch, max_len, 64] codes of `kind`
// (1 FP8 E4M3, 2 int8) with per-channel scales c_scale [512], pe_scale [64] (16-byte aligned); workspace as
// mla_decode_workspace_bytes.
hipError_t launch_mla_decode_q8(const void* q_latent, const void* q_pe, const void* c_kv, const void* k_pe,
                                const float* c_scale, const float* pe_scale, int kind, const int32_t* seq_lens,
                                void* o_latent, float* lse, int batch, int n_heads, int max_seqlen_kv, float scale,
                                void* workspace, hipStream_t stream);

// Sparse MLA decode over a [batch, topk] list of token indices per sequence (same workspace layout as the dense
// form with topk in place of max_seqlen_kv).
hipError_t launch_mla_sparse_decode(const void* q_latent, const void* q_pe, const void* c_kv, const void* k_pe,
                                    const int32_t* seq_lens, const int32_t* indices, void* o_latent, float* lse,
                                    int batch, int n_heads, int max_seqlen_kv, int topk, float scale, void* workspace,
                                    hipStream_t stream);

// DeepSeek Sparse Attention selection: lightning-indexer scores [batch, max_seqlen_kv] fp32, then the top-k
// token indices per sequence. Indexer: n_heads_idx 32 or 64, idx_dim 64 or 128, bf16 inputs, fp32 weights.
hipError_t launch_dsa_indexer(const void* q_idx, const float* w_idx, const void* k_idx, const int32_t* seq_lens,
                              float* scores, int batch, int n_heads_idx, int idx_dim, int max_seqlen_kv,
                              hipStream_t stream);
hipError_t launch_topk(const float* scores, const int32_t* seq_lens, int32_t* indices, int batch, int max_seqlen_kv,
                       int k, hipStream_t stream);

}  // namespace attn
