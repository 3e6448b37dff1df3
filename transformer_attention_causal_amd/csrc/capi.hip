// capi.hip — the extern "C" boundary of libattn (declared in include/attn.h).
//
// Each entry point validates its arguments on the host BEFORE touching the HIP runtime, so an invalid call
// returns its status without any device work (and without needing a GPU), then enqueues the kernels on the
// caller's stream. No allocation, no synchronisation, no state kept between calls, except for
// attn_decode_paged_noalloc's per-device scratch address, looked up once per device.
#include <atomic>
#include <cmath>
#include <cstdint>
#include <mutex>

#include "../../include/attn.h"
#include "kernels.h"

#define ATTN_EXPORT extern "C" __attribute__((visibility("default")))

namespace {

bool valid_scale(float s) { return std::isfinite(s) && s > 0.f; }
bool is_pow2(int x) { return x > 0 && (x & (x - 1)) == 0; }
int hip_status(hipError_t e) { return e == hipSuccess ? ATTN_OK : ATTN_ERR_HIP; }

}  // namespace

ATTN_EXPORT const char* attn_status_string(int status) {
  switch (status) {
    case ATTN_OK: return "ATTN_OK";
    case ATTN_ERR_INVALID_ARG: return "ATTN_ERR_INVALID_ARG: invalid argument";
    case ATTN_ERR_UNSUPPORTED: return "ATTN_ERR_UNSUPPORTED: valid request not implemented by this build";
    case ATTN_ERR_WORKSPACE: return "ATTN_ERR_WORKSPACE: workspace too small";
    case ATTN_ERR_HIP: return "ATTN_ERR_HIP: HIP runtime error at launch";
    default: return "unknown attn status";
  }
}

ATTN_EXPORT int attn_rope_apply(void* x, attn_dtype_t dtype, int64_t n_tokens, int n_heads, int head_dim,
                                const int32_t* positions, double theta, int interleaved, void* stream) {
  if (n_tokens < 0 || n_heads <= 0 || head_dim <= 0 || (head_dim & 1)) return ATTN_ERR_INVALID_ARG;
  if (!std::isfinite(theta) || theta <= 1.0) return ATTN_ERR_INVALID_ARG;
  if (dtype != ATTN_BF16 && dtype != ATTN_FP32) return ATTN_ERR_UNSUPPORTED;
  if (head_dim > 1024) return ATTN_ERR_UNSUPPORTED;
  if (n_tokens == 0) return ATTN_OK;
  if (!x || !positions) return ATTN_ERR_INVALID_ARG;
  return hip_status(attn::launch_rope(x, dtype, n_tokens, n_heads, head_dim, positions, theta, interleaved ? 1 : 0,
                                      static_cast<hipStream_t>(stream)));
}

ATTN_EXPORT int attn_prefill(const void* q, const void* k, const void* v, void* o, float* lse, attn_dtype_t dtype,
                             int batch, int seqlen, int n_heads_q, int n_heads_kv, int head_dim, int causal,
                             float softmax_scale, void* stream) {
  if (batch < 0 || seqlen < 0 || n_heads_q <= 0 || n_heads_kv <= 0 || head_dim <= 0) return ATTN_ERR_INVALID_ARG;
  if (n_heads_q % n_heads_kv != 0 || !valid_scale(softmax_scale)) return ATTN_ERR_INVALID_ARG;
  if (dtype != ATTN_BF16 && dtype != ATTN_FP32) return ATTN_ERR_UNSUPPORTED;
  if (head_dim != 64 && head_dim != 128) return ATTN_ERR_UNSUPPORTED;
  if (int64_t(batch) * seqlen == 0) return ATTN_OK;
  if (!q || !k || !v || !o) return ATTN_ERR_INVALID_ARG;
  const hipStream_t s = static_cast<hipStream_t>(stream);
  if (dtype == ATTN_BF16)
    return hip_status(attn::launch_prefill_bf16(q, k, v, o, lse, batch, seqlen, n_heads_q, n_heads_kv, head_dim,
                                                causal ? 1 : 0, softmax_scale, s));
  return hip_status(attn::launch_prefill_fp32(q, k, v, o, lse, batch, seqlen, n_heads_q, n_heads_kv, head_dim,
                                              causal ? 1 : 0, softmax_scale, s));
}

ATTN_EXPORT int attn_rope_table(void* table, int n_positions, int head_dim, double theta, void* stream) {
  if (n_positions < 0 || head_dim <= 0 || (head_dim & 1)) return ATTN_ERR_INVALID_ARG;
  if (!std::isfinite(theta) || theta <= 1.0) return ATTN_ERR_INVALID_ARG;
  if (head_dim > 1024) return ATTN_ERR_UNSUPPORTED;
  if (n_positions == 0) return ATTN_OK;
  if (!table) return ATTN_ERR_INVALID_ARG;
  return hip_status(attn::launch_rope_table(table, n_positions, head_dim, theta, static_cast<hipStream_t>(stream)));
}

ATTN_EXPORT int attn_prefill_rope(const void* q, const void* k, const void* v, void* o, float* lse, int batch,
                                  int seqlen, int n_heads_q, int n_heads_kv, int head_dim, int causal,
                                  float softmax_scale, const int32_t* q_positions, const void* rope_table,
                                  int rope_table_len, int interleaved, void* stream) {
  if (batch < 0 || seqlen < 0 || n_heads_q <= 0 || n_heads_kv <= 0 || head_dim <= 0) return ATTN_ERR_INVALID_ARG;
  if (n_heads_q % n_heads_kv != 0 || !valid_scale(softmax_scale)) return ATTN_ERR_INVALID_ARG;
  if (head_dim != 64 && head_dim != 128) return ATTN_ERR_UNSUPPORTED;
  if (int64_t(batch) * seqlen == 0) return ATTN_OK;
  if (!q || !k || !v || !o || !rope_table || rope_table_len <= 0) return ATTN_ERR_INVALID_ARG;
  if (reinterpret_cast<uintptr_t>(rope_table) % 16 != 0) return ATTN_ERR_INVALID_ARG;
  if (int64_t(rope_table_len) * head_dim * 4 >= (int64_t(1) << 32)) return ATTN_ERR_UNSUPPORTED;   // 32-bit offsets
  return hip_status(attn::launch_prefill_bf16(q, k, v, o, lse, batch, seqlen, n_heads_q, n_heads_kv, head_dim,
                                              causal ? 1 : 0, softmax_scale, static_cast<hipStream_t>(stream),
                                              rope_table, rope_table_len, q_positions, interleaved ? 1 : 0));
}

ATTN_EXPORT int attn_prefill_local_global(const void* q, const void* k, const void* v, void* o, float* lse,
                                          int batch, int seqlen, int n_heads_q, int n_heads_kv, int head_dim,
                                          int window, int n_lead, int anchor_stride, float softmax_scale,
                                          void* stream) {
  if (batch < 0 || seqlen < 0 || n_heads_q <= 0 || n_heads_kv <= 0 || head_dim <= 0) return ATTN_ERR_INVALID_ARG;
  if (n_heads_q % n_heads_kv != 0 || !valid_scale(softmax_scale)) return ATTN_ERR_INVALID_ARG;
  if (window < 1 || n_lead < 0 || anchor_stride < 0) return ATTN_ERR_INVALID_ARG;
  if (head_dim != 64 && head_dim != 128) return ATTN_ERR_UNSUPPORTED;
  // strided anchor tiles address 64 rows of stride anchor_stride within 32-bit offsets
  if (int64_t(anchor_stride) * 64 * n_heads_kv * head_dim * 2 >= (int64_t(1) << 31)) return ATTN_ERR_UNSUPPORTED;
  if (batch == 0 || seqlen == 0) return ATTN_OK;
  if (!q || !k || !v || !o) return ATTN_ERR_INVALID_ARG;
  return hip_status(attn::launch_prefill_window(q, k, v, o, lse, batch, seqlen, n_heads_q, n_heads_kv, head_dim,
                                                window, n_lead, anchor_stride, softmax_scale,
                                                static_cast<hipStream_t>(stream)));
}

ATTN_EXPORT size_t attn_decode_paged_workspace_size(int batch, int n_heads_q, int head_dim, int max_seqlen_kv) {
  return attn::decode_paged_workspace_bytes(batch, n_heads_q, head_dim, max_seqlen_kv);
}

// Static scratch of attn_decode_paged_noalloc: the split partials of one call. Each GPU the library runs on holds
// its own copy at its own address for the life of the process. In host code `scratch` names a host-side stand-in,
// not device memory, so it is never passed to a kernel or a copy: the device address of the current GPU's copy
// comes from hipGetSymbolAddress, looked up once per device and kept in scratch_addr.
static __device__ __align__(256) uint8_t scratch[ATTN_DECODE_SCRATCH_BYTES];

namespace {
// Checks of attn_decode_paged other than the workspace. Returns ATTN_OK with *nothing_to_do set for batch 0.
int check_decode_paged(const void* q, const void* k_cache, const void* v_cache, const int32_t* block_table,
                       const int32_t* seq_lens, void* o, int batch, int n_heads_q, int n_heads_kv, int head_dim,
                       int page_size, int max_pages_per_seq, int64_t num_pages, int max_seqlen_kv,
                       float softmax_scale, bool* nothing_to_do) {
  *nothing_to_do = false;
  if (batch < 0 || n_heads_q <= 0 || n_heads_kv <= 0 || head_dim <= 0 || max_seqlen_kv < 0) return ATTN_ERR_INVALID_ARG;
  if (n_heads_q % n_heads_kv != 0 || !valid_scale(softmax_scale)) return ATTN_ERR_INVALID_ARG;
  if (page_size <= 0 || max_pages_per_seq < 0) return ATTN_ERR_INVALID_ARG;
  if ((head_dim != 128 && head_dim != 64) || n_heads_q / n_heads_kv > 16) return ATTN_ERR_UNSUPPORTED;
  if (!is_pow2(page_size) || page_size < 16 || page_size > 1024) return ATTN_ERR_UNSUPPORTED;
  if (batch == 0) {
    *nothing_to_do = true;
    return ATTN_OK;
  }
  if (!q || !seq_lens || !o) return ATTN_ERR_INVALID_ARG;
  if (max_seqlen_kv > 0 && (!k_cache || !v_cache || !block_table || num_pages <= 0 || max_pages_per_seq <= 0))
    return ATTN_ERR_INVALID_ARG;
  return ATTN_OK;
}

constexpr int kMaxDevices = 64;
std::atomic<void*> scratch_addr[kMaxDevices];
std::mutex scratch_mutex;

// Device address of the current device's scratch (looked up on the first call for that device).
int current_scratch(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) return ATTN_ERR_HIP;
  if (dev < 0 || dev >= kMaxDevices) return ATTN_ERR_UNSUPPORTED;
  void* p = scratch_addr[dev].load(std::memory_order_acquire);
  if (!p) {
    std::lock_guard<std::mutex> lock(scratch_mutex);
    p = scratch_addr[dev].load(std::memory_order_relaxed);
    if (!p) {
      void* addr = nullptr;
      if (hipGetSymbolAddress(&addr, HIP_SYMBOL(scratch)) != hipSuccess || !addr) return ATTN_ERR_HIP;
      scratch_addr[dev].store(addr, std::memory_order_release);
      p = addr;
    }
  }
  *out = p;
  return ATTN_OK;
}
}  // namespace

ATTN_EXPORT int attn_decode_paged_noalloc(const void* q, const void* k_cache, const void* v_cache,
                                          const int32_t* block_table, const int32_t* seq_lens, void* o, float* lse,
                                          int batch, int n_heads_q, int n_heads_kv, int head_dim, int page_size,
                                          int max_pages_per_seq, int64_t num_pages, int max_seqlen_kv,
                                          float softmax_scale, void* stream) {
  bool done = false;
  const int st = check_decode_paged(q, k_cache, v_cache, block_table, seq_lens, o, batch, n_heads_q, n_heads_kv,
                                    head_dim, page_size, max_pages_per_seq, num_pages, max_seqlen_kv,
                                    softmax_scale, &done);
  if (st != ATTN_OK || done) return st;
  const size_t need = attn::decode_paged_workspace_bytes(batch, n_heads_q, head_dim, max(1, max_seqlen_kv));
  if (need > ATTN_DECODE_SCRATCH_BYTES) return ATTN_ERR_WORKSPACE;
  void* ws = nullptr;
  const int sst = current_scratch(&ws);
  if (sst != ATTN_OK) return sst;
  return hip_status(attn::launch_decode_paged(q, k_cache, v_cache, block_table, seq_lens, o, lse, batch, n_heads_q,
                                              n_heads_kv, head_dim, page_size, max_pages_per_seq, num_pages,
                                              max_seqlen_kv, softmax_scale, ws, static_cast<hipStream_t>(stream)));
}

ATTN_EXPORT int attn_decode_paged(const void* q, const void* k_cache, const void* v_cache,
                                  const int32_t* block_table, const int32_t* seq_lens, void* o, float* lse,
                                  int batch, int n_heads_q, int n_heads_kv, int head_dim, int page_size,
                                  int max_pages_per_seq, int64_t num_pages, int max_seqlen_kv,
                                  float softmax_scale, void* workspace, size_t workspace_bytes, void* stream) {
  bool done = false;
  const int st = check_decode_paged(q, k_cache, v_cache, block_table, seq_lens, o, batch, n_heads_q, n_heads_kv,
                                    head_dim, page_size, max_pages_per_seq, num_pages, max_seqlen_kv,
                                    softmax_scale, &done);
  if (st != ATTN_OK || done) return st;
  const size_t need = attn::decode_paged_workspace_bytes(batch, n_heads_q, head_dim, max(1, max_seqlen_kv));
  if (!workspace || workspace_bytes < need) return ATTN_ERR_WORKSPACE;
  return hip_status(attn::launch_decode_paged(q, k_cache, v_cache, block_table, seq_lens, o, lse, batch, n_heads_q,
                                              n_heads_kv, head_dim, page_size, max_pages_per_seq, num_pages,
                                              max_seqlen_kv, softmax_scale, workspace,
                                              static_cast<hipStream_t>(stream)));
}

ATTN_EXPORT int attn_decode_paged_q8(const void* q, const void* k_cache, const void* v_cache, const float* k_scale,
                                     const float* v_scale, int kv_kind, const int32_t* block_table,
                                     const int32_t* seq_lens, void* o, float* lse, int batch, int n_heads_q,
                                     int n_heads_kv, int head_dim, int page_size, int max_pages_per_seq,
                                     int64_t num_pages, int max_seqlen_kv, float softmax_scale, void* workspace,
                                     size_t workspace_bytes, void* stream) {
  if (batch < 0 || n_heads_q <= 0 || n_heads_kv <= 0 || head_dim <= 0 || max_seqlen_kv < 0) return ATTN_ERR_INVALID_ARG;
  if (n_heads_q % n_heads_kv != 0 || !valid_scale(softmax_scale)) return ATTN_ERR_INVALID_ARG;
  if (page_size <= 0 || max_pages_per_seq < 0) return ATTN_ERR_INVALID_ARG;
  if (kv_kind != ATTN_KV_FP8_E4M3 && kv_kind != ATTN_KV_INT8) return ATTN_ERR_UNSUPPORTED;
  if ((head_dim != 128 && head_dim != 64) || n_heads_q / n_heads_kv > 16) return ATTN_ERR_UNSUPPORTED;
  if (!is_pow2(page_size) || page_size < 16 || page_size > 1024) return ATTN_ERR_UNSUPPORTED;
  if (batch == 0) return ATTN_OK;
  if (!q || !seq_lens || !o || !k_scale || !v_scale) return ATTN_ERR_INVALID_ARG;
  if (max_seqlen_kv > 0 && (!k_cache || !v_cache || !block_table || num_pages <= 0 || max_pages_per_seq <= 0))
    return ATTN_ERR_INVALID_ARG;
  const uintptr_t align = reinterpret_cast<uintptr_t>(q) | reinterpret_cast<uintptr_t>(k_cache) |
                          reinterpret_cast<uintptr_t>(v_cache) | reinterpret_cast<uintptr_t>(k_scale) |
                          reinterpret_cast<uintptr_t>(v_scale);
  if (align % 16 != 0) return ATTN_ERR_INVALID_ARG;
  const size_t need = attn::decode_paged_workspace_bytes(batch, n_heads_q, head_dim, max(1, max_seqlen_kv));
  if (!workspace || workspace_bytes < need) return ATTN_ERR_WORKSPACE;
  return hip_status(attn::launch_decode_paged_q8(kv_kind == ATTN_KV_FP8_E4M3 ? 1 : 0, q, k_cache, v_cache, k_scale,
                                                 v_scale, block_table, seq_lens, o, lse, batch, n_heads_q, n_heads_kv,
                                                 head_dim, page_size, max_pages_per_seq, num_pages, max_seqlen_kv, softmax_scale,
                                                 workspace, static_cast<hipStream_t>(stream)));
}

ATTN_EXPORT size_t attn_mla_decode_workspace_size(int batch, int n_heads, int kv_lora_rank, int max_seqlen_kv) {
  return attn::mla_decode_workspace_bytes(batch, n_heads, kv_lora_rank, max_seqlen_kv);
}

ATTN_EXPORT int attn_mla_decode(const void* q_latent, const void* q_pe, const void* c_kv, const void* k_pe,
                                const int32_t* seq_lens, void* o_latent, float* lse, int batch, int n_heads,
                                int kv_lora_rank, int rope_dim, int max_seqlen_kv, float softmax_scale,
                                void* workspace, size_t workspace_bytes, void* stream) {
  if (batch < 0 || n_heads <= 0 || kv_lora_rank <= 0 || rope_dim <= 0 || max_seqlen_kv < 0) return ATTN_ERR_INVALID_ARG;
  if (!valid_scale(softmax_scale)) return ATTN_ERR_INVALID_ARG;
  if (kv_lora_rank != 512 || rope_dim != 64 || n_heads % 32 != 0 || n_heads > 128) return ATTN_ERR_UNSUPPORTED;
  if (batch == 0) return ATTN_OK;
  if (!q_latent || !q_pe || !seq_lens || !o_latent) return ATTN_ERR_INVALID_ARG;
  if (max_seqlen_kv > 0 && (!c_kv || !k_pe)) return ATTN_ERR_INVALID_ARG;
  const size_t need = attn::mla_decode_workspace_bytes(batch, n_heads, kv_lora_rank, max(1, max_seqlen_kv));
  if (!workspace || workspace_bytes < need) return ATTN_ERR_WORKSPACE;
  return hip_status(attn::launch_mla_decode(q_latent, q_pe, c_kv, k_pe, seq_lens, o_latent, lse, batch, n_heads,
                                            max_seqlen_kv, softmax_scale, workspace,
                                            static_cast<hipStream_t>(stream)));
}

ATTN_EXPORT int attn_mla_decode_q8(const void* q_latent, const void* q_pe, const void* c_kv, const void* k_pe,
                                   const float* c_scale, const float* pe_scale, int kv_kind, const int32_t* seq_lens,
                                   void* o_latent, float* lse, int batch, int n_heads, int kv_lora_rank, int rope_dim,
                                   int max_seqlen_kv, float softmax_scale, void* workspace, size_t workspace_bytes,
                                   void* stream) {
  if (batch < 0 || n_heads <= 0 || kv_lora_rank <= 0 || rope_dim <= 0 || max_seqlen_kv < 0) return ATTN_ERR_INVALID_ARG;
  if (!valid_scale(softmax_scale)) return ATTN_ERR_INVALID_ARG;
  if (kv_kind != ATTN_KV_FP8_E4M3 && kv_kind != ATTN_KV_INT8) return ATTN_ERR_UNSUPPORTED;
  if (kv_lora_rank != 512 || rope_dim != 64 || n_heads % 32 != 0 || n_heads > 128) return ATTN_ERR_UNSUPPORTED;
  if (batch == 0) return ATTN_OK;
  if (!q_latent || !q_pe || !seq_lens || !o_latent || !c_scale || !pe_scale) return ATTN_ERR_INVALID_ARG;
  if (max_seqlen_kv > 0 && (!c_kv || !k_pe)) return ATTN_ERR_INVALID_ARG;
  const uintptr_t align = reinterpret_cast<uintptr_t>(q_latent) | reinterpret_cast<uintptr_t>(q_pe) |
                          reinterpret_cast<uintptr_t>(c_kv) | reinterpret_cast<uintptr_t>(k_pe) |
                          reinterpret_cast<uintptr_t>(c_scale) | reinterpret_cast<uintptr_t>(pe_scale);
  if (align % 16 != 0) return ATTN_ERR_INVALID_ARG;
  const size_t need = attn::mla_decode_workspace_bytes(batch, n_heads, kv_lora_rank, max(1, max_seqlen_kv));
  if (!workspace || workspace_bytes < need) return ATTN_ERR_WORKSPACE;
  return hip_status(attn::launch_mla_decode_q8(q_latent, q_pe, c_kv, k_pe, c_scale, pe_scale, kv_kind, seq_lens,
                                               o_latent, lse, batch, n_heads, max_seqlen_kv, softmax_scale,
                                               workspace, static_cast<hipStream_t>(stream)));
}

ATTN_EXPORT int attn_kv_append_paged(const void* k_new, const void* v_new, const int32_t* cu_new,
                                     const int32_t* cache_lens, void* k_cache, void* v_cache,
                                     const int32_t* block_table, int batch, int total_new, int n_heads_kv,
                                     int head_dim, int page_size, int max_pages_per_seq, int64_t num_pages,
                                     double theta, int interleaved, void* stream) {
  if (batch < 0 || total_new < 0 || n_heads_kv <= 0 || head_dim <= 0 || (head_dim & 1)) return ATTN_ERR_INVALID_ARG;
  if (page_size <= 0 || max_pages_per_seq < 0 || num_pages < 0) return ATTN_ERR_INVALID_ARG;
  if (!std::isfinite(theta) || theta <= 1.0) return ATTN_ERR_INVALID_ARG;
  if (head_dim % 16 != 0 || head_dim > 1024 || !is_pow2(page_size)) return ATTN_ERR_UNSUPPORTED;
  if (batch == 0 || total_new == 0) return ATTN_OK;
  if (!k_new || !v_new || !cu_new || !cache_lens || !k_cache || !v_cache || !block_table) return ATTN_ERR_INVALID_ARG;
  if (max_pages_per_seq <= 0 || num_pages <= 0) return ATTN_ERR_INVALID_ARG;
  const uintptr_t align = reinterpret_cast<uintptr_t>(k_new) | reinterpret_cast<uintptr_t>(v_new) |
                          reinterpret_cast<uintptr_t>(k_cache) | reinterpret_cast<uintptr_t>(v_cache);
  if (align % 16 != 0) return ATTN_ERR_INVALID_ARG;
  return hip_status(attn::launch_kv_append_paged(k_new, v_new, cu_new, cache_lens, k_cache, v_cache, block_table,
                                                 batch, total_new, n_heads_kv, head_dim, page_size, max_pages_per_seq,
                                                 num_pages, theta, interleaved ? 1 : 0,
                                                 static_cast<hipStream_t>(stream)));
}

ATTN_EXPORT int attn_prefill_paged(const void* q, const void* k_cache, const void* v_cache, const int32_t* block_table,
                                   const int32_t* cu_new, const int32_t* cache_lens, void* o, float* lse, int batch,
                                   int total_new, int max_new, int n_heads_q, int n_heads_kv, int head_dim,
                                   int page_size, int max_pages_per_seq, int64_t num_pages, float softmax_scale,
                                   void* stream) {
  if (batch < 0 || total_new < 0 || max_new < 0 || n_heads_q <= 0 || n_heads_kv <= 0 || head_dim <= 0)
    return ATTN_ERR_INVALID_ARG;
  if (n_heads_q % n_heads_kv != 0 || !valid_scale(softmax_scale)) return ATTN_ERR_INVALID_ARG;
  if (page_size <= 0 || max_pages_per_seq < 0 || num_pages < 0 || max_new > total_new) return ATTN_ERR_INVALID_ARG;
  if (head_dim != 64 && head_dim != 128) return ATTN_ERR_UNSUPPORTED;
  if (!is_pow2(page_size) || page_size < 64) return ATTN_ERR_UNSUPPORTED;
  if (batch == 0 || total_new == 0 || max_new == 0) return ATTN_OK;
  if (!q || !k_cache || !v_cache || !block_table || !cu_new || !cache_lens || !o) return ATTN_ERR_INVALID_ARG;
  if (max_pages_per_seq <= 0 || num_pages <= 0) return ATTN_ERR_INVALID_ARG;
  return hip_status(attn::launch_prefill_paged(q, k_cache, v_cache, block_table, cu_new, cache_lens, o, lse, batch,
                                               total_new, max_new, n_heads_q, n_heads_kv, head_dim, page_size,
                                               max_pages_per_seq, num_pages, softmax_scale,
                                               static_cast<hipStream_t>(stream)));
}

ATTN_EXPORT int attn_prefill_paged_rope(const void* q, const void* k_cache, const void* v_cache,
                                        const int32_t* block_table, const int32_t* cu_new, const int32_t* cache_lens,
                                        void* o, float* lse, int batch, int total_new, int max_new, int n_heads_q,
                                        int n_heads_kv, int head_dim, int page_size, int max_pages_per_seq,
                                        int64_t num_pages, float softmax_scale, const int32_t* q_positions,
                                        const void* rope_table, int rope_table_len, int interleaved, void* stream) {
  if (batch < 0 || total_new < 0 || max_new < 0 || n_heads_q <= 0 || n_heads_kv <= 0 || head_dim <= 0)
    return ATTN_ERR_INVALID_ARG;
  if (n_heads_q % n_heads_kv != 0 || !valid_scale(softmax_scale)) return ATTN_ERR_INVALID_ARG;
  if (page_size <= 0 || max_pages_per_seq < 0 || num_pages < 0 || max_new > total_new) return ATTN_ERR_INVALID_ARG;
  if (head_dim != 64 && head_dim != 128) return ATTN_ERR_UNSUPPORTED;
  if (!is_pow2(page_size) || page_size < 64) return ATTN_ERR_UNSUPPORTED;
  if (batch == 0 || total_new == 0 || max_new == 0) return ATTN_OK;
  if (!q || !k_cache || !v_cache || !block_table || !cu_new || !cache_lens || !o) return ATTN_ERR_INVALID_ARG;
  if (max_pages_per_seq <= 0 || num_pages <= 0) return ATTN_ERR_INVALID_ARG;
  if (!rope_table || rope_table_len <= 0) return ATTN_ERR_INVALID_ARG;
  if (reinterpret_cast<uintptr_t>(rope_table) % 16 != 0) return ATTN_ERR_INVALID_ARG;
  if (int64_t(rope_table_len) * head_dim * 4 >= (int64_t(1) << 32)) return ATTN_ERR_UNSUPPORTED;   // 32-bit offsets
  return hip_status(attn::launch_prefill_paged(q, k_cache, v_cache, block_table, cu_new, cache_lens, o, lse, batch,
                                               total_new, max_new, n_heads_q, n_heads_kv, head_dim, page_size,
                                               max_pages_per_seq, num_pages, softmax_scale,
                                               static_cast<hipStream_t>(stream), rope_table, rope_table_len,
                                               q_positions, interleaved ? 1 : 0));
}

ATTN_EXPORT int attn_dsa_indexer(const void* q_idx, const float* w_idx, const void* k_idx, const int32_t* seq_lens,
                                 float* scores, int batch, int n_heads_idx, int idx_dim, int max_seqlen_kv,
                                 void* stream) {
  if (batch < 0 || n_heads_idx <= 0 || idx_dim <= 0 || max_seqlen_kv < 0) return ATTN_ERR_INVALID_ARG;
  if ((n_heads_idx != 32 && n_heads_idx != 64) || (idx_dim != 64 && idx_dim != 128)) return ATTN_ERR_UNSUPPORTED;
  if (batch == 0 || max_seqlen_kv == 0) return ATTN_OK;
  if (!q_idx || !w_idx || !k_idx || !seq_lens || !scores) return ATTN_ERR_INVALID_ARG;
  const uintptr_t align = reinterpret_cast<uintptr_t>(q_idx) | reinterpret_cast<uintptr_t>(k_idx);
  if (align % 16 != 0) return ATTN_ERR_INVALID_ARG;
  return hip_status(attn::launch_dsa_indexer(q_idx, w_idx, k_idx, seq_lens, scores, batch, n_heads_idx, idx_dim,
                                             max_seqlen_kv, static_cast<hipStream_t>(stream)));
}

ATTN_EXPORT int attn_topk(const float* scores, const int32_t* seq_lens, int32_t* indices, int batch,
                          int max_seqlen_kv, int topk, void* stream) {
  if (batch < 0 || max_seqlen_kv < 0 || topk <= 0) return ATTN_ERR_INVALID_ARG;
  if (batch == 0) return ATTN_OK;
  if (!seq_lens || !indices || (max_seqlen_kv > 0 && !scores)) return ATTN_ERR_INVALID_ARG;
  return hip_status(attn::launch_topk(scores, seq_lens, indices, batch, max_seqlen_kv, topk,
                                      static_cast<hipStream_t>(stream)));
}

ATTN_EXPORT size_t attn_mla_sparse_decode_workspace_size(int batch, int n_heads, int kv_lora_rank, int topk) {
  return attn::mla_sparse_workspace_bytes(batch, n_heads, kv_lora_rank, topk);
}

ATTN_EXPORT int attn_mla_sparse_decode(const void* q_latent, const void* q_pe, const void* c_kv, const void* k_pe,
                                       const int32_t* seq_lens, const int32_t* indices, void* o_latent, float* lse,
                                       int batch, int n_heads, int kv_lora_rank, int rope_dim, int max_seqlen_kv,
                                       int topk, float softmax_scale, void* workspace, size_t workspace_bytes,
                                       void* stream) {
  if (batch < 0 || n_heads <= 0 || kv_lora_rank <= 0 || rope_dim <= 0 || max_seqlen_kv <= 0 || topk <= 0)
    return ATTN_ERR_INVALID_ARG;
  if (!valid_scale(softmax_scale)) return ATTN_ERR_INVALID_ARG;
  if (kv_lora_rank != 512 || rope_dim != 64 || n_heads % 32 != 0 || n_heads > 128) return ATTN_ERR_UNSUPPORTED;
  if (batch == 0) return ATTN_OK;
  if (!q_latent || !q_pe || !c_kv || !k_pe || !seq_lens || !indices || !o_latent) return ATTN_ERR_INVALID_ARG;
  if (int64_t(max_seqlen_kv) * kv_lora_rank * 2 > (int64_t(1) << 31)) return ATTN_ERR_UNSUPPORTED;
  const size_t need = attn::mla_sparse_workspace_bytes(batch, n_heads, kv_lora_rank, topk);
  if (!workspace || workspace_bytes < need) return ATTN_ERR_WORKSPACE;
  return hip_status(attn::launch_mla_sparse_decode(q_latent, q_pe, c_kv, k_pe, seq_lens, indices, o_latent, lse,
                                                   batch, n_heads, max_seqlen_kv, topk, softmax_scale, workspace,
                                                   static_cast<hipStream_t>(stream)));
}
