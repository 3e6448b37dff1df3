// decode.hip — one query token per sequence against a paged KV cache: split-KV partials, then a log-sum-exp
// combine.
//
// (Attention notes, makinaruto.github.io, posts/nlp/llm_learning/attention: "Page Attention" — fixed-size pages
//  plus a logical-to-physical map; "online-softmax" — partial results over disjoint key blocks merge exactly
//  through their maxima and exp-sums. "7 anti-patterns of DeepSeek attention optimisation", lpnh.cn, section
//  4.2 — the KV cache is [batch, seq, kv_heads, d] and each KV head serves a group of query heads.)
//
// Decode is HBM-bound (about 4 flop per byte of K/V), so the design goal is to read each K/V byte once, with
// wide loads and enough of them in flight:
//   * Split kernel: one wave per (logical 512-key chunk, KV head, sequence). The wave serves all query heads of
//     its KV group at once, so every K/V byte is read once. Chunks at or past the sequence length exit at once.
//   * Both products run on v_mfma_f32_16x16x32_bf16 with the group's query heads as the 16-wide N dimension
//     (heads beyond the group size are zero columns). K fragments are loaded straight from global memory into
//     the A-operand registers (S^T = K Q^T: lane = key, 8 contiguous dims). For O^T = V^T P^T each lane loads
//     full 16-byte V rows of 8 keys and an 8x8 register transpose (byte permutes) turns them into eight A
//     operands, one per dimension offset j = 0..7 (operand row m covers dimension 8m + j). The 8 keys of a lane
//     are exactly the keys of its S^T registers, so P^T feeds the second product from registers.
//   * Pages are looked up once per 16 keys (page size is a power of two >= 16, so 16 aligned keys share a page).
//   * Partial (O / l, lse) per chunk goes to the workspace; the combine kernel merges a sequence's chunks.
// Split boundaries are logical key positions, so the result does not depend on physical page placement.
#include "device.h"
#include "kernels.h"

namespace attn {
namespace {

constexpr int kD = 128;
static_assert(kDecodeChunk % 32 == 0 && kDecodeChunk / 16 <= 64, "a chunk's pages (>= 16 keys each) fit one wave");

// Grid order: 1 = the KV heads of one chunk are consecutive workgroups (they read interleaved 256-byte pieces
// of the same page slots at the same time); 0 = the chunks of one head are consecutive.
#ifndef ATTN_DECODE_HEAD_MAJOR
#define ATTN_DECODE_HEAD_MAJOR 0
#endif
// Build-time choice: software-prefetch the next 32 keys' K/V while computing on the current ones.
#ifndef ATTN_DECODE_PREFETCH
#define ATTN_DECODE_PREFETCH 0
#endif

struct DecodeArgs {
  const uint16_t* q;
  const uint16_t* kc;
  const uint16_t* vc;
  const int32_t* table;
  const int32_t* seq_lens;
  float* ws_o;      // [batch, hq, n_chunks, D]
  float* ws_lse;    // [batch, hq, n_chunks]
  int hq, hkv, page_shift, max_pages, max_len, n_chunks;
  int64_t num_pages;
  float scale;
};

__device__ __forceinline__ int clamp_len(int L, int max_len, int cap) { return max(0, min(L, min(max_len, cap))); }

// Element j (0..7) of each of the 8 loaded rows, packed in row order: the A operand for dimension offset j.
__device__ __forceinline__ bf16x8_t transpose_pick(const u32x4_t* vv, int j) {
  const uint32_t sel = (j & 1) ? 0x07060302u : 0x05040100u;
  u32x4_t w;
#pragma unroll
  for (int u = 0; u < 4; ++u) w[u] = __builtin_amdgcn_perm(vv[2 * u + 1][j >> 1], vv[2 * u][j >> 1], sel);
  return as_bf16x8(w);
}

__global__ __launch_bounds__(64) void decode_paged_split_kernel(DecodeArgs a) {
#if ATTN_DECODE_HEAD_MAJOR
  const int g = blockIdx.x, chunk = blockIdx.y, b = blockIdx.z;
#else
  const int chunk = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
#endif
  const int page_size = 1 << a.page_shift;
  const int L = clamp_len(a.seq_lens[b], a.max_len, a.max_pages * page_size);
  const int t_begin = chunk * kDecodeChunk;
  if (t_begin >= L) return;
  const int t_end = min(L, t_begin + kDecodeChunk);
  const int lane = threadIdx.x, n = lane & 15, grp4 = lane >> 4;
  const int G = a.hq / a.hkv;
  const int h = g * G + n;
  const bool hv = n < G;
  const float c = a.scale * kLog2e;

  // Q^T operand: lane holds head n, dims 8*(4*ks + grp4) .. +7 for k-step ks.
  bf16x8_t qop[4];
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) {
    u32x4_t w = {0u, 0u, 0u, 0u};
    if (hv) w = *reinterpret_cast<const u32x4_t*>(a.q + (int64_t(b) * a.hq + h) * kD + 8 * (4 * ks + grp4));
    qop[ks] = as_bf16x8(w);
  }
  f32x4_t oacc[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) oacc[j] = f32x4_t{};
  float m = -INFINITY, l = 0.f;
  const int32_t* trow = a.table + int64_t(b) * a.max_pages;
  // The chunk's page numbers, read once: lane i holds the entry of the chunk's i-th page (a chunk spans at most
  // 512/16 = 32 pages), fetched per 16 keys with a lane read instead of a dependent table load per iteration.
  const int first_page = t_begin >> a.page_shift;
  const int last_page = (t_end - 1) >> a.page_shift;
  const int pg_lane = (lane <= last_page - first_page) ? trow[first_page + lane] : -1;
  const int64_t row_stride = int64_t(a.hkv) * kD;           // elements between consecutive slots of a page
  const int64_t page_stride = int64_t(page_size) * row_stride;

  // K fragments (key t0 + 16*tb + n, dims 8*(4*ks + grp4) ..) and V rows (slot s: key t0 + 16*(s/4) + 4*grp4 + s%4,
  // dims 8n .. 8n+7) of the 32 keys at t0. Pages are looked up once per 16-key half (wave-uniform); keys at or past
  // t_end and pages outside [0, num_pages) are never dereferenced (zeros instead).
  auto load32 = [&](int t0, u32x4_t (&kv)[2][4], u32x4_t (&vv)[8]) {
    int pg[2];
    bool pv[2];
#pragma unroll
    for (int hf = 0; hf < 2; ++hf) {
      const int tt = min(t0 + 16 * hf, t_end - 1);
      pg[hf] = __builtin_amdgcn_readlane(pg_lane, (tt >> a.page_shift) - first_page);
      pv[hf] = pg[hf] >= 0 && pg[hf] < a.num_pages;
    }
#pragma unroll
    for (int tb = 0; tb < 2; ++tb) {
      const int key = t0 + 16 * tb + n;
      const bool ok = key < t_end && pv[tb];
      const uint16_t* kp = a.kc + int64_t(pg[tb]) * page_stride + int64_t(key & (page_size - 1)) * row_stride +
                           int64_t(g) * kD + 8 * grp4;
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        u32x4_t w = {0u, 0u, 0u, 0u};
        if (ok) w = *reinterpret_cast<const u32x4_t*>(kp + 32 * ks);
        kv[tb][ks] = w;
      }
    }
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      const int hf = s >> 2;
      const int key = t0 + 16 * hf + 4 * grp4 + (s & 3);
      const bool ok = key < t_end && pv[hf];
      u32x4_t w = {0u, 0u, 0u, 0u};
      if (ok)
        w = *reinterpret_cast<const u32x4_t*>(a.vc + int64_t(pg[hf]) * page_stride +
                                              int64_t(key & (page_size - 1)) * row_stride + int64_t(g) * kD + 8 * n);
      vv[s] = w;
    }
  };

  u32x4_t kv[2][4], vv[8];
  load32(t_begin, kv, vv);
  for (int t0 = t_begin; t0 < t_end; t0 += 32) {
#if ATTN_DECODE_PREFETCH
    // issue the next 32 keys' loads before computing on these (software pipelining, ~64 more registers)
    u32x4_t kvn[2][4], vvn[8];
    if (t0 + 32 < t_end) load32(t0 + 32, kvn, vvn);
#endif
    // S^T[key][head]: lane holds head n, keys t0 + 16*tb + 4*grp4 + r
    f32x4_t sacc[2] = {f32x4_t{}, f32x4_t{}};
#pragma unroll
    for (int tb = 0; tb < 2; ++tb)
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) sacc[tb] = mfma16x16x32(as_bf16x8(kv[tb][ks]), qop[ks], sacc[tb]);
    if (t0 + 32 > t_end) {
#pragma unroll
      for (int tb = 0; tb < 2; ++tb)
#pragma unroll
        for (int r = 0; r < 4; ++r)
          if (t0 + 16 * tb + 4 * grp4 + r >= t_end) sacc[tb][r] = -INFINITY;
    }
    // online softmax per head (column n): 8 values per lane, 4 lanes per head
    float mx = -INFINITY;
#pragma unroll
    for (int tb = 0; tb < 2; ++tb)
#pragma unroll
      for (int r = 0; r < 4; ++r) mx = fmaxf(mx, sacc[tb][r]);
    mx = fmaxf(mx, xor_lanes(mx, 16));
    mx = fmaxf(mx, xor_lanes(mx, 32));
    // Lazy rescale (see the prefill kernel): O and l move to a new reference max only when it grew by more
    // than 2^kRescaleLog2 for some lane.
    if (__any((mx - m) * c > kRescaleLog2)) {
      const float m_new = fmaxf(m, mx);
      const float alpha = fast_exp2((m - m_new) * c);
      l *= alpha;
#pragma unroll
      for (int j = 0; j < 8; ++j) oacc[j] *= alpha;
      m = m_new;
    }
    const float mc = m * c;
#pragma unroll
    for (int tb = 0; tb < 2; ++tb)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float p = fast_exp2(fmaf(sacc[tb][r], c, -mc));
        sacc[tb][r] = p;
        l += p;
      }
    const bf16x8_t pb = pack_bf16x8(sacc[0][0], sacc[0][1], sacc[0][2], sacc[0][3], sacc[1][0], sacc[1][1],
                                    sacc[1][2], sacc[1][3]);
#pragma unroll
    for (int j = 0; j < 8; ++j) oacc[j] = mfma16x16x32(transpose_pick(vv, j), pb, oacc[j]);
#if ATTN_DECODE_PREFETCH
    if (t0 + 32 < t_end) {
#pragma unroll
      for (int tb = 0; tb < 2; ++tb)
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) kv[tb][ks] = kvn[tb][ks];
#pragma unroll
      for (int s = 0; s < 8; ++s) vv[s] = vvn[s];
    }
#else
    if (t0 + 32 < t_end) load32(t0 + 32, kv, vv);
#endif
  }

  // partial result: O / l and lse for this chunk (lane holds head n, dims 8*(4*grp4 + r) + j)
  float lt = l + xor_lanes(l, 16);
  lt += xor_lanes(lt, 32);
  if (!hv) return;
  const int64_t slot = (int64_t(b) * a.hq + h) * a.n_chunks + chunk;
  const float inv = 1.f / lt;
  float* wo = a.ws_o + slot * kD;
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int d0 = 8 * (4 * grp4 + r);
    f32x4_t lo = {oacc[0][r] * inv, oacc[1][r] * inv, oacc[2][r] * inv, oacc[3][r] * inv};
    f32x4_t hi = {oacc[4][r] * inv, oacc[5][r] * inv, oacc[6][r] * inv, oacc[7][r] * inv};
    *reinterpret_cast<f32x4_t*>(wo + d0) = lo;
    *reinterpret_cast<f32x4_t*>(wo + d0 + 4) = hi;
  }
  if (grp4 == 0) a.ws_lse[slot] = m * a.scale + logf(lt);
}

// Merge the chunks of one (sequence, query head): M = max lse_c, w_c = exp(lse_c - M),
// O = sum_c w_c O_c / sum_c w_c, lse = M + ln sum_c w_c. A sequence of length 0 gets O = 0, lse = -inf.
__global__ __launch_bounds__(kD) void decode_combine_kernel(const float* __restrict__ ws_o,
    const float* __restrict__ ws_lse, const int32_t* __restrict__ seq_lens, uint16_t* __restrict__ o,
    float* __restrict__ lse, int hq, int n_chunks, int max_len, int cap) {
  const int h = blockIdx.x, b = blockIdx.y, d = threadIdx.x;
  const int L = clamp_len(seq_lens[b], max_len, cap);
  const int nc = (L + kDecodeChunk - 1) / kDecodeChunk;
  const int64_t base = (int64_t(b) * hq + h) * n_chunks;
  uint16_t* op = o + (int64_t(b) * hq + h) * kD;
  if (nc == 0) {
    op[d] = 0;
    if (lse && d == 0) lse[int64_t(b) * hq + h] = -INFINITY;
    return;
  }
  // Unrolled so that several independent partial loads are in flight (the loop is latency-bound otherwise).
  float mx = -INFINITY;
#pragma unroll 8
  for (int ci = 0; ci < nc; ++ci) mx = fmaxf(mx, ws_lse[base + ci]);
  float acc = 0.f, wsum = 0.f;
#pragma unroll 8
  for (int ci = 0; ci < nc; ++ci) {
    const float w = expf(ws_lse[base + ci] - mx);
    wsum += w;
    acc = fmaf(w, ws_o[(base + ci) * kD + d], acc);
  }
  op[d] = uint16_t(pack_bf16x2(acc / wsum, 0.f));
  if (lse && d == 0) lse[int64_t(b) * hq + h] = mx + logf(wsum);
}

}  // namespace

size_t decode_paged_workspace_bytes(int batch, int hq, int head_dim, int max_seqlen_kv) {
  if (batch <= 0 || hq <= 0 || head_dim <= 0 || max_seqlen_kv <= 0) return 0;
  const size_t n_chunks = (size_t(max_seqlen_kv) + kDecodeChunk - 1) / kDecodeChunk;
  const size_t slots = size_t(batch) * size_t(hq) * n_chunks;
  const size_t o_bytes = (slots * size_t(head_dim) * sizeof(float) + 255) & ~size_t(255);
  return o_bytes + slots * sizeof(float);
}

hipError_t launch_decode_paged(const void* q, const void* k_cache, const void* v_cache, const int32_t* block_table,
                               const int32_t* seq_lens, void* o, float* lse, int batch, int hq, int hkv,
                               int head_dim, int page_size, int max_pages_per_seq, int64_t num_pages,
                               int max_seqlen_kv, float scale, void* workspace, hipStream_t stream) {
  (void)head_dim;  // 128 (validated by the caller)
  const int n_chunks = max(1, (max_seqlen_kv + kDecodeChunk - 1) / kDecodeChunk);
  const size_t slots = size_t(batch) * size_t(hq) * size_t(n_chunks);
  const size_t o_bytes = (slots * kD * sizeof(float) + 255) & ~size_t(255);
  DecodeArgs a;
  a.q = static_cast<const uint16_t*>(q);
  a.kc = static_cast<const uint16_t*>(k_cache);
  a.vc = static_cast<const uint16_t*>(v_cache);
  a.table = block_table; a.seq_lens = seq_lens;
  a.ws_o = static_cast<float*>(workspace);
  a.ws_lse = reinterpret_cast<float*>(static_cast<char*>(workspace) + o_bytes);
  a.hq = hq; a.hkv = hkv;
  int shift = 0;
  while ((1 << shift) < page_size) ++shift;
  a.page_shift = shift; a.max_pages = max_pages_per_seq; a.max_len = max_seqlen_kv; a.n_chunks = n_chunks;
  a.num_pages = num_pages; a.scale = scale;
  if (max_seqlen_kv > 0)
    decode_paged_split_kernel<<<ATTN_DECODE_HEAD_MAJOR ? dim3(unsigned(hkv), unsigned(n_chunks), unsigned(batch))
                                                       : dim3(unsigned(n_chunks), unsigned(hkv), unsigned(batch)),
                                dim3(64), 0, stream>>>(a);
  decode_combine_kernel<<<dim3(unsigned(hq), unsigned(batch)), dim3(kD), 0, stream>>>(
      a.ws_o, a.ws_lse, seq_lens, static_cast<uint16_t*>(o), lse, hq, n_chunks, max_seqlen_kv,
      max_pages_per_seq * page_size);
  return hipGetLastError();
}

}  // namespace attn
