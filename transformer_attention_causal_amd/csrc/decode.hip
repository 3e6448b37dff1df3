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
//   * Split kernel: one wave per (logical 1024-key chunk, KV head, sequence). The wave serves all query heads of
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
// The default build stages K and V blocks through LDS with whole-row copies (the LDS-staged kernel below for bf16
// caches, the ATTN_DECODE_LDS8 path for 8-bit ones) and reads the same operand layouts from there; loading the
// operands straight into registers, as described above, is the measured-slower alternative kept for comparison.
//
// 8-bit caches ("7 anti-patterns of DeepSeek attention optimisation", lpnh.cn, section 3.3: FP8 E4M3, largest
// value 448; "DeepSeek 32K to 256K long context", tqpw.cn, section 2.5: int8 K/V with per-channel scales): the
// same kernel reads one byte per element. Every E4M3 and int8 value is exact in bf16, so codes become MFMA
// operands by exact conversion (v_cvt_scalef32_pk_bf16_fp8 with scale 1; int8 through float). The per-channel K
// scale is folded into the query (q_d * k_scale_d, rounded to bf16 once per query); the per-channel V scale
// multiplies the output channels at the end. For the K loads the contraction order over the 128 dims is
// permuted (k-steps 2i and 2i+1 of lane group g take dims 64i + 16g .. +15) so a lane loads 16 contiguous bytes.
#include <type_traits>

#include "device.h"
#include "kernels.h"

namespace attn {
namespace {

constexpr int kD = 128;
// Build-time choices (measured): bf16 and 8-bit caches staged through LDS (1) or loaded through registers (0).
#ifndef ATTN_DECODE_LDS
#define ATTN_DECODE_LDS 1
#endif
#ifndef ATTN_DECODE_LDS8
#define ATTN_DECODE_LDS8 1
#endif
#ifndef ATTN_DECODE_Q8_HEAD_MAJOR
#define ATTN_DECODE_Q8_HEAD_MAJOR 1
#endif
static_assert(kDecodeChunk % 32 == 0 && kDecodeChunk / 16 <= 64, "a chunk's pages (>= 16 keys each) fit one wave");

// Grid order: head-major = the KV heads of one chunk are consecutive workgroups (they read interleaved 256-byte
// pieces of the same page slots at the same time), chunk-major = the chunks of one head are consecutive. With
// 1024-key chunks head-major measured faster for every kernel here, so the launch uses it.


struct DecodeArgs {
  const uint16_t* q;
  const void* kc;
  const void* vc;
  const float* k_scale;    // 8-bit caches: [hkv, D]
  const float* v_scale;
  const int32_t* table;
  const int32_t* seq_lens;
  float* ws_o;      // [batch, hq, n_chunks, D]
  float* ws_lse;    // [batch, hq, n_chunks]
  int hq, hkv, page_shift, max_pages, max_len, n_chunks;
  int head_major;   // grid order: (hkv, n_chunks, batch) if set, else (n_chunks, hkv, batch)
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


template <int KV>
__global__ __launch_bounds__(64) void decode_paged_split_kernel(DecodeArgs a) {
  const int g = a.head_major ? blockIdx.x : blockIdx.y, chunk = a.head_major ? blockIdx.y : blockIdx.x;
  const int b = blockIdx.z;
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

  // Q^T operand: lane holds head n, dims kdim(ks) .. +7 for k-step ks (8-bit caches: times the K scale).
  auto kdim = [&](int ks) { return KV == kKvBf16 ? 8 * (4 * ks + grp4) : 64 * (ks >> 1) + 16 * grp4 + 8 * (ks & 1); };
  bf16x8_t qop[4];
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) {
    u32x4_t w = {0u, 0u, 0u, 0u};
    if (hv) w = *reinterpret_cast<const u32x4_t*>(a.q + (int64_t(b) * a.hq + h) * kD + kdim(ks));
    if constexpr (KV != kKvBf16) {
      const float* ks_p = a.k_scale + g * kD + kdim(ks);
      w = u32x4_t{pack_bf16x2(bf16lo_to_f32(w[0]) * ks_p[0], bf16hi_to_f32(w[0]) * ks_p[1]),
                  pack_bf16x2(bf16lo_to_f32(w[1]) * ks_p[2], bf16hi_to_f32(w[1]) * ks_p[3]),
                  pack_bf16x2(bf16lo_to_f32(w[2]) * ks_p[4], bf16hi_to_f32(w[2]) * ks_p[5]),
                  pack_bf16x2(bf16lo_to_f32(w[3]) * ks_p[6], bf16hi_to_f32(w[3]) * ks_p[7])};
    }
    qop[ks] = as_bf16x8(w);
  }
  f32x4_t oacc[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) oacc[j] = f32x4_t{};
  float m = -INFINITY, l = 0.f;
  const int32_t* trow = a.table + int64_t(b) * a.max_pages;
  // The chunk's page numbers, read once: lane i holds the entry of the chunk's i-th page (a chunk spans at most
  // 1024/16 = 64 pages), fetched per 16 keys with a lane read instead of a dependent table load per iteration.
  const int first_page = t_begin >> a.page_shift;
  const int last_page = (t_end - 1) >> a.page_shift;
  const int pg_lane = (lane <= last_page - first_page) ? trow[first_page + lane] : -1;
  const int64_t row_stride = int64_t(a.hkv) * kD;           // elements between consecutive slots of a page
  const int64_t page_stride = int64_t(page_size) * row_stride;

  // K fragments (key t0 + 16*tb + n, dims 8*(4*ks + grp4) ..) and V rows (slot s: key t0 + 16*(s/4) + 4*grp4 + s%4,
  // dims 8n .. 8n+7) of the 32 keys at t0. Pages are looked up once per 16-key half (wave-uniform); keys at or past
  // t_end and pages outside [0, num_pages) are never dereferenced (zeros instead).
  using E = std::conditional_t<KV == kKvBf16, uint16_t, uint8_t>;
  const E* kcache = static_cast<const E*>(a.kc);
  const E* vcache = static_cast<const E*>(a.vc);
  // 8-bit caches: K of key 16*tb + n as two 16-byte pieces (dims 16*grp4 .., 64 + 16*grp4 ..), V rows as 8 bytes.
  auto load32_q8 = [&](int t0, u32x4_t (&kv8)[2][2], u32x2_t (&vv8)[8]) {
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
      const E* kp = kcache + int64_t(pg[tb]) * page_stride + int64_t(key & (page_size - 1)) * row_stride +
                    int64_t(g) * kD + 16 * grp4;
#pragma unroll
      for (int hk = 0; hk < 2; ++hk) {
        u32x4_t w = {0u, 0u, 0u, 0u};
        if (ok) w = *reinterpret_cast<const u32x4_t*>(kp + 64 * hk);
        kv8[tb][hk] = w;
      }
    }
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      const int hf = s >> 2;
      const int key = t0 + 16 * hf + 4 * grp4 + (s & 3);
      const bool ok = key < t_end && pv[hf];
      u32x2_t w = {0u, 0u};
      if (ok)
        w = *reinterpret_cast<const u32x2_t*>(vcache + int64_t(pg[hf]) * page_stride +
                                              int64_t(key & (page_size - 1)) * row_stride + int64_t(g) * kD + 8 * n);
      vv8[s] = w;
    }
  };
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
      const E* kp = kcache + int64_t(pg[tb]) * page_stride + int64_t(key & (page_size - 1)) * row_stride +
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
        w = *reinterpret_cast<const u32x4_t*>(vcache + int64_t(pg[hf]) * page_stride +
                                              int64_t(key & (page_size - 1)) * row_stride + int64_t(g) * kD + 8 * n);
      vv[s] = w;
    }
  };
  // 8-bit codes -> the bf16 operands the loop uses (K in the permuted k-step order, V rows in order)
  auto widen = [&](const u32x4_t (&kv8)[2][2], const u32x2_t (&vv8)[8], u32x4_t (&kv)[2][4], u32x4_t (&vv)[8]) {
#pragma unroll
    for (int tb = 0; tb < 2; ++tb)
#pragma unroll
      for (int ks = 0; ks < 4; ++ks)
        kv[tb][ks] = codes_to_bf16x8<KV>(kv8[tb][ks >> 1][2 * (ks & 1)], kv8[tb][ks >> 1][2 * (ks & 1) + 1]);
#pragma unroll
    for (int s2 = 0; s2 < 8; ++s2) vv[s2] = codes_to_bf16x8<KV>(vv8[s2][0], vv8[s2][1]);
  };

  // One block of 32 keys: S^T = K Q^T, online softmax, O^T += V^T P^T (K and V as bf16 operands in kv, vv).
  auto block = [&](int t0, const u32x4_t (&kv)[2][4], const u32x4_t (&vv)[8]) {
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
  };

  u32x4_t kv[2][4], vv[8];
  if constexpr (KV == kKvBf16) {
    load32(t_begin, kv, vv);
    for (int t0 = t_begin; t0 < t_end; t0 += 32) {
      block(t0, kv, vv);
      if (t0 + 32 < t_end) load32(t0 + 32, kv, vv);
    }
  } else if (ATTN_DECODE_LDS8) {
    // 8-bit codes staged through LDS as in the bf16 kernel below: per 32-key block, 4 copy instructions per tensor
    // (8 keys x one 128-byte head slice each, non-temporal), read back into the register formats of load32_q8.
    // K chunk c of row r sits at c ^ ((r >> 1) & 3 | ((r >> 3) & 1) << 2) (conflict-free b128 reads); V rows are
    // unswizzled (their b64 reads pair two rows of equal parity: a 2-way conflict whatever the swizzle).
    __shared__ __attribute__((aligned(16))) uint8_t k8a[32 * kD], k8b[32 * kD], v8a[32 * kD], v8b[32 * kD];
    const int row_in = lane >> 3, pcs = lane & 7;
    const uint32_t row_bytes = uint32_t(row_stride);     // one byte per element
    auto swz8 = [](int r) { return ((r >> 1) & 3) | (((r >> 3) & 1) << 2); };
    auto copy8 = [&](uint8_t* kdst, uint8_t* vdst, int t0) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int key_first = t0 + 8 * i;
        const int pg = __builtin_amdgcn_readlane(pg_lane, (min(key_first, t_end - 1) >> a.page_shift) - first_page);
        const bool pv = pg >= 0 && pg < a.num_pages;
        const int rows = pv ? max(0, min(8, t_end - key_first)) : 0;
        const int64_t e0 = int64_t(max(pg, 0)) * page_stride + int64_t(key_first & (page_size - 1)) * row_stride +
                           int64_t(g) * kD;
        const buf_rsrc_t rk = make_buf_rsrc(kcache + e0, uint32_t(rows) * row_bytes);
        const buf_rsrc_t rv = make_buf_rsrc(vcache + e0, uint32_t(rows) * row_bytes);
        const int r = 8 * i + row_in;
        raw_buffer_load_lds(rk, (lds_void_t*)(kdst + i * 1024), 16, int(row_in * row_bytes + 16 * (pcs ^ swz8(r))),
                            0, 0, 2);
        raw_buffer_load_lds(rv, (lds_void_t*)(vdst + i * 1024), 16, int(row_in * row_bytes + 16 * pcs), 0, 0, 2);
      }
    };
    u32x4_t kv8[2][2];
    u32x2_t vv8[8];
    auto read8 = [&](const uint8_t* ks, const uint8_t* vs) {
#pragma unroll
      for (int tb = 0; tb < 2; ++tb)
#pragma unroll
        for (int hk = 0; hk < 2; ++hk) {
          const int r = 16 * tb + n;
          kv8[tb][hk] = *reinterpret_cast<const __attribute__((address_space(3))) u32x4_t*>(
              (const __attribute__((address_space(3))) uint8_t*)ks + r * 128 + 16 * ((4 * hk + grp4) ^ swz8(r)));
        }
#pragma unroll
      for (int s2 = 0; s2 < 8; ++s2) {
        const int r = 16 * (s2 >> 2) + 4 * grp4 + (s2 & 3);
        vv8[s2] = *reinterpret_cast<const __attribute__((address_space(3))) u32x2_t*>(
            (const __attribute__((address_space(3))) uint8_t*)vs + r * 128 + 8 * n);
      }
    };
    wait_vmem();              // q, scales and the page numbers are in: from here on only block copies are outstanding
    copy8(k8a, v8a, t_begin);
    for (int t0 = t_begin; t0 < t_end; t0 += 64) {
      wait_vmem();
      read8(k8a, v8a);                                   // block t0 into registers before the next copies
      if (t0 + 32 < t_end) copy8(k8b, v8b, t0 + 32);
      widen(kv8, vv8, kv, vv);
      block(t0, kv, vv);
      if (t0 + 32 >= t_end) break;
      wait_vmem();
      read8(k8b, v8b);
      if (t0 + 64 < t_end) copy8(k8a, v8a, t0 + 64);
      widen(kv8, vv8, kv, vv);
      block(t0 + 32, kv, vv);
    }
  } else {
    // 8-bit codes take half the registers: two blocks of codes in flight (ring of two), widened to bf16 operands
    // just before use.
    u32x4_t ka[2][2], kb[2][2];
    u32x2_t va[8], vb[8];
    load32_q8(t_begin, ka, va);
    if (t_begin + 32 < t_end) load32_q8(t_begin + 32, kb, vb);
    for (int t0 = t_begin; t0 < t_end; t0 += 64) {
      widen(ka, va, kv, vv);
      if (t0 + 64 < t_end) load32_q8(t0 + 64, ka, va);
      block(t0, kv, vv);
      if (t0 + 32 >= t_end) break;
      widen(kb, vb, kv, vv);
      if (t0 + 96 < t_end) load32_q8(t0 + 96, kb, vb);
      block(t0 + 32, kv, vv);
    }
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
    if constexpr (KV != kKvBf16) {                     // per-channel V scale
      const f32x4_t* vs = reinterpret_cast<const f32x4_t*>(a.v_scale + g * kD + d0);
      lo *= vs[0];
      hi *= vs[1];
    }
    *reinterpret_cast<f32x4_t*>(wo + d0) = lo;
    *reinterpret_cast<f32x4_t*>(wo + d0 + 4) = hi;
  }
  if (grp4 == 0) a.ws_lse[slot] = m * a.scale + logf(lt);
}

// ---- LDS-staged variant (bf16 caches). The register-loading kernel above reads, per load instruction, 64-byte
// halves of 16 different rows; here each 32-key block of K and of V is copied global -> LDS by buffer loads with
// the LDS bit, one instruction per 4 rows (1 KiB, whole 256-byte head slices), and the MFMA operands are read from
// LDS: K fragments with ds_read_b128, V^T fragments with the transposing ds_read_b64_tr_b16 (the O^T layout is then
// dims 16*db + 4*grp4 + r). 16-byte chunk c of tile row r is stored at c ^ swz(r) (the copy permutes its source
// chunks): K key r & 15 keeps each b128 lane set on 16 distinct slots; V key 2*(r & 7) keeps each 32-lane
// transposing read on 32 distinct 8-byte slots (measured bank model, see the prefill kernel).

#ifndef ATTN_DECODE_NBUF
#define ATTN_DECODE_NBUF 2
#endif
#ifndef ATTN_DECODE_COPY_AUX
#define ATTN_DECODE_COPY_AUX 2                           // non-temporal: each cache byte is read once
#endif
constexpr int kDecNbuf = ATTN_DECODE_NBUF;               // 32-key LDS blocks per wave (kDecNbuf - 1 in flight)

__device__ __forceinline__ int dec_swz_k(int row) { return row & 15; }
__device__ __forceinline__ int dec_swz_v(int row) { return 2 * (row & 7); }

template <int N>
__device__ __forceinline__ void wait_vmem_n() { asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory"); }

__global__ __launch_bounds__(64) void decode_paged_lds_kernel(DecodeArgs a) {
  // One LDS array per buffer and tensor: distinct objects, so the compiler can see that a block's copies in
  // flight do not alias the buffer being read, and keeps its waits at the block boundary.
  __shared__ __attribute__((aligned(16))) uint16_t kl0[32 * kD], kl1[32 * kD], kl2[kDecNbuf > 2 ? 32 * kD : 8];
  __shared__ __attribute__((aligned(16))) uint16_t vl0[32 * kD], vl1[32 * kD], vl2[kDecNbuf > 2 ? 32 * kD : 8];
  auto kbuf = [&](auto bufc) -> uint16_t* {
    constexpr int B = decltype(bufc)::value;
    if constexpr (B == 0) return kl0; else if constexpr (B == 1) return kl1; else return kl2;
  };
  auto vbuf = [&](auto bufc) -> uint16_t* {
    constexpr int B = decltype(bufc)::value;
    if constexpr (B == 0) return vl0; else if constexpr (B == 1) return vl1; else return vl2;
  };
  const int g = a.head_major ? blockIdx.x : blockIdx.y, chunk = a.head_major ? blockIdx.y : blockIdx.x;
  const int b = blockIdx.z;
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
  f32x4_t oacc[8];                                       // O^T: lane holds head n, dims 16*db + 4*grp4 + r
#pragma unroll
  for (int db = 0; db < 8; ++db) oacc[db] = f32x4_t{};
  float m = -INFINITY, l = 0.f;
  const int32_t* trow = a.table + int64_t(b) * a.max_pages;
  const int first_page = t_begin >> a.page_shift;
  const int last_page = (t_end - 1) >> a.page_shift;
  const int pg_lane = (lane <= last_page - first_page) ? trow[first_page + lane] : -1;
  const int64_t row_stride = int64_t(a.hkv) * kD;
  const int64_t page_stride = int64_t(page_size) * row_stride;
  const uint16_t* kcache = static_cast<const uint16_t*>(a.kc);
  const uint16_t* vcache = static_cast<const uint16_t*>(a.vc);

  // Copy instruction i of a block moves keys t0+4i .. t0+4i+3 (one page: pages hold >= 16 keys and t0 is a
  // multiple of 32); keys at or past t_end and pages outside [0, num_pages) read as zeros (empty resource).
  const int row_in = lane >> 4, pcs = lane & 15;
  const uint32_t row_bytes = uint32_t(row_stride * 2);
  auto copy_block = [&](auto bufc, int t0) {
    uint16_t* kdst = kbuf(bufc);
    uint16_t* vdst = vbuf(bufc);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int key_first = t0 + 4 * i;
      const int pg = __builtin_amdgcn_readlane(pg_lane, (min(key_first, t_end - 1) >> a.page_shift) - first_page);
      const bool pv = pg >= 0 && pg < a.num_pages;
      const int rows = pv ? max(0, min(4, t_end - key_first)) : 0;
      const int64_t e0 = int64_t(max(pg, 0)) * page_stride + int64_t(key_first & (page_size - 1)) * row_stride +
                         int64_t(g) * kD;
      const buf_rsrc_t rk = make_buf_rsrc(kcache + e0, uint32_t(rows) * row_bytes);
      const buf_rsrc_t rv = make_buf_rsrc(vcache + e0, uint32_t(rows) * row_bytes);
      const int r = 4 * i + row_in;
      raw_buffer_load_lds(rk, (lds_void_t*)(kdst + i * 512), 16, int(row_in * row_bytes + 16 * (pcs ^ dec_swz_k(r))),
                          0, 0, ATTN_DECODE_COPY_AUX);
      raw_buffer_load_lds(rv, (lds_void_t*)(vdst + i * 512), 16, int(row_in * row_bytes + 16 * (pcs ^ dec_swz_v(r))),
                          0, 0, ATTN_DECODE_COPY_AUX);
    }
  };
  // LDS read addresses (bytes): K row 16*tb + n, chunk 4*ks + grp4; V rows 4*grp4 + j (+16), dims 16*db + 4*(bl&3)
  uint32_t kaddr[4], vaddr[8];
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) kaddr[ks] = uint32_t(n * 256 + 16 * ((4 * ks + grp4) ^ dec_swz_k(n)));
  {
    const int vr = 4 * grp4 + (n >> 2), cq = n & 3;
#pragma unroll
    for (int db = 0; db < 8; ++db)
      vaddr[db] = uint32_t(vr * 256 + 16 * ((2 * db + (cq >> 1)) ^ dec_swz_v(vr)) + 8 * (cq & 1));
  }

  // A block's operand fragments are read from LDS into registers before the next block's copies are issued: the
  // compiler cannot tell the copies from these reads apart and would otherwise wait for the copies first.
  u32x4_t kf[2][4], vf[8];
  auto read_block = [&](auto bufc) {
    const uint16_t* Kt = kbuf(bufc);
    const uint16_t* Vt = vbuf(bufc);
#pragma unroll
    for (int tb = 0; tb < 2; ++tb)
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) kf[tb][ks] = lds_read16(Kt, kaddr[ks] + tb * 16 * 256);
#pragma unroll
    for (int db = 0; db < 8; ++db) {
      const u32x2_t lo = lds_read_tr16(Vt, vaddr[db]);
      const u32x2_t hi = lds_read_tr16(Vt, vaddr[db] + 16 * 256);
      vf[db] = u32x4_t{lo[0], lo[1], hi[0], hi[1]};
    }
  };
  auto block = [&](int t0) {
    f32x4_t sacc[2] = {f32x4_t{}, f32x4_t{}};
#pragma unroll
    for (int tb = 0; tb < 2; ++tb)
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) sacc[tb] = mfma16x16x32(as_bf16x8(kf[tb][ks]), qop[ks], sacc[tb]);
    if (t0 + 32 > t_end) {
#pragma unroll
      for (int tb = 0; tb < 2; ++tb)
#pragma unroll
        for (int r = 0; r < 4; ++r)
          if (t0 + 16 * tb + 4 * grp4 + r >= t_end) sacc[tb][r] = -INFINITY;
    }
    float mx = -INFINITY;
#pragma unroll
    for (int tb = 0; tb < 2; ++tb)
#pragma unroll
      for (int r = 0; r < 4; ++r) mx = fmaxf(mx, sacc[tb][r]);
    mx = fmaxf(mx, xor_lanes(mx, 16));
    mx = fmaxf(mx, xor_lanes(mx, 32));
    if (__any((mx - m) * c > kRescaleLog2)) {
      const float m_new = fmaxf(m, mx);
      const float alpha = fast_exp2((m - m_new) * c);
      l *= alpha;
#pragma unroll
      for (int db = 0; db < 8; ++db) oacc[db] *= alpha;
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
    for (int db = 0; db < 8; ++db) oacc[db] = mfma16x16x32(as_bf16x8(vf[db]), pb, oacc[db]);
  };

  // Ring of kDecNbuf blocks: at block u, wait for its copies, read its fragments, then issue the copies of block
  // u + kDecNbuf - 1 into the buffer block u - 1 used, and compute.
  constexpr int PRE = kDecNbuf - 1;
  const int nblk = (t_end - t_begin + 31) / 32;
  wait_vmem_n<0>();        // q and the page numbers are in: from here on only block copies are outstanding
  copy_block(std::integral_constant<int, 0>{}, t_begin);
  if (PRE >= 2 && 1 < nblk) copy_block(std::integral_constant<int, 1 % kDecNbuf>{}, t_begin + 32);
  for (int u = 0; u < nblk; u += kDecNbuf) {
#pragma unroll
    for (int k = 0; k < kDecNbuf; ++k) {
      const int uu = u + k;
      if (uu >= nblk) break;
      // copies of blocks uu+1 .. uu+PRE-1 may stay in flight (16 instructions per block)
      if (PRE >= 2 && uu + 1 < nblk) wait_vmem_n<16>();
      else wait_vmem_n<0>();
      if (k == 0) read_block(std::integral_constant<int, 0>{});
      else if (k == 1) read_block(std::integral_constant<int, 1 % kDecNbuf>{});
      else read_block(std::integral_constant<int, 2 % kDecNbuf>{});
      if (uu + PRE < nblk) {
        const int nb = (k + PRE) % kDecNbuf;
        if (nb == 0) copy_block(std::integral_constant<int, 0>{}, t_begin + 32 * (uu + PRE));
        else if (nb == 1) copy_block(std::integral_constant<int, 1 % kDecNbuf>{}, t_begin + 32 * (uu + PRE));
        else copy_block(std::integral_constant<int, 2 % kDecNbuf>{}, t_begin + 32 * (uu + PRE));
      }
      block(t_begin + 32 * uu);
    }
  }

  float lt = l + xor_lanes(l, 16);
  lt += xor_lanes(lt, 32);
  if (!hv) return;
  const int64_t slot = (int64_t(b) * a.hq + h) * a.n_chunks + chunk;
  const float inv = 1.f / lt;
  float* wo = a.ws_o + slot * kD + 4 * grp4;
#pragma unroll
  for (int db = 0; db < 8; ++db) *reinterpret_cast<f32x4_t*>(wo + 16 * db) = oacc[db] * inv;
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

namespace {
hipError_t launch_decode(int kind, const void* q, const void* k_cache, const void* v_cache, const float* k_scale,
                         const float* v_scale, const int32_t* block_table, const int32_t* seq_lens, void* o, float* lse,
                         int batch, int hq, int hkv, int page_size, int max_pages_per_seq, int64_t num_pages,
                         int max_seqlen_kv, float scale, void* workspace, hipStream_t stream) {
  const int n_chunks = max(1, (max_seqlen_kv + kDecodeChunk - 1) / kDecodeChunk);
  const size_t slots = size_t(batch) * size_t(hq) * size_t(n_chunks);
  const size_t o_bytes = (slots * kD * sizeof(float) + 255) & ~size_t(255);
  DecodeArgs a = {};
  a.q = static_cast<const uint16_t*>(q);
  a.kc = k_cache;
  a.vc = v_cache;
  a.k_scale = k_scale;
  a.v_scale = v_scale;
  a.table = block_table; a.seq_lens = seq_lens;
  a.ws_o = static_cast<float*>(workspace);
  a.ws_lse = reinterpret_cast<float*>(static_cast<char*>(workspace) + o_bytes);
  a.hq = hq; a.hkv = hkv;
  int shift = 0;
  while ((1 << shift) < page_size) ++shift;
  a.page_shift = shift; a.max_pages = max_pages_per_seq; a.max_len = max_seqlen_kv; a.n_chunks = n_chunks;
  a.num_pages = num_pages; a.scale = scale;
  a.head_major = kind == kKvBf16 ? 1 : ATTN_DECODE_Q8_HEAD_MAJOR;
  const dim3 grid = a.head_major ? dim3(unsigned(hkv), unsigned(n_chunks), unsigned(batch))
                                 : dim3(unsigned(n_chunks), unsigned(hkv), unsigned(batch));
  if (max_seqlen_kv > 0) {
    if (kind == kKvFp8) decode_paged_split_kernel<kKvFp8><<<grid, dim3(64), 0, stream>>>(a);
    else if (kind == kKvInt8) decode_paged_split_kernel<kKvInt8><<<grid, dim3(64), 0, stream>>>(a);
    else if (ATTN_DECODE_LDS) decode_paged_lds_kernel<<<grid, dim3(64), 0, stream>>>(a);
    else decode_paged_split_kernel<kKvBf16><<<grid, dim3(64), 0, stream>>>(a);
  }
  decode_combine_kernel<<<dim3(unsigned(hq), unsigned(batch)), dim3(kD), 0, stream>>>(
      a.ws_o, a.ws_lse, seq_lens, static_cast<uint16_t*>(o), lse, hq, n_chunks, max_seqlen_kv,
      max_pages_per_seq * page_size);
  return hipGetLastError();
}
}  // namespace

hipError_t launch_decode_paged(const void* q, const void* k_cache, const void* v_cache, const int32_t* block_table,
                               const int32_t* seq_lens, void* o, float* lse, int batch, int hq, int hkv,
                               int head_dim, int page_size, int max_pages_per_seq, int64_t num_pages,
                               int max_seqlen_kv, float scale, void* workspace, hipStream_t stream) {
  (void)head_dim;  // 128 (validated by the caller)
  return launch_decode(kKvBf16, q, k_cache, v_cache, nullptr, nullptr, block_table, seq_lens, o, lse, batch, hq, hkv,
                       page_size, max_pages_per_seq, num_pages, max_seqlen_kv, scale, workspace, stream);
}

hipError_t launch_decode_paged_q8(int fp8, const void* q, const void* k_cache, const void* v_cache,
                                  const float* k_scale, const float* v_scale, const int32_t* block_table,
                                  const int32_t* seq_lens, void* o, float* lse, int batch, int hq, int hkv,
                                  int page_size, int max_pages_per_seq, int64_t num_pages, int max_seqlen_kv,
                                  float scale, void* workspace, hipStream_t stream) {
  return launch_decode(fp8 ? kKvFp8 : kKvInt8, q, k_cache, v_cache, k_scale, v_scale, block_table, seq_lens, o, lse,
                       batch, hq, hkv, page_size, max_pages_per_seq, num_pages, max_seqlen_kv, scale, workspace,
                       stream);
}

}  // namespace attn
