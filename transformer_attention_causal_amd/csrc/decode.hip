// decode.hip — one query token per sequence against a paged KV cache: split-KV partials, then a log-sum-exp
// combine.
//
// (Attention notes, makinaruto.github.io, posts/nlp/llm_learning/attention: "Page Attention" — fixed-size pages
//  plus a logical-to-physical map; "online-softmax" — partial results over disjoint key blocks merge exactly
//  through their maxima and exp-sums. "7 anti-patterns of DeepSeek attention optimisation", lpnh.cn, section
//  4.2 — the KV cache is [batch, seq, kv_heads, d] and each KV head serves a group of query heads.)
//
// Decode is HBM-bound (about 4 flop per byte of K/V), so the design goal is to read each K/V byte once, with
// whole-line copies and enough of them in flight:
//   * Split kernels: one wave per (logical key chunk, KV head, sequence), launched head-major (the KV heads of one
//     chunk are consecutive workgroups: they read interleaved head slices of the same page slots at the same time).
//     The wave serves all query heads of its KV group at once, so every K/V byte is read once. Chunks at or past
//     the sequence length exit at once.
//   * K and V blocks are copied global -> LDS with buffer loads carrying the LDS bit (whole head slices,
//     non-temporal: every cache byte is read once), two blocks in a ring, and the MFMA operands are read from LDS.
//   * Both products run on v_mfma_f32_16x16x32_bf16 with the group's query heads as the 16-wide N dimension
//     (heads beyond the group size are zero columns). S^T = K Q^T gives each lane one head and 8 keys; those 8
//     keys are the contraction slots of its P^T operand, so P^T feeds O^T = V^T P^T from registers.
//   * The chunk's page numbers are read once per wave (lane i holds the chunk's i-th page) and taken per copy
//     with a lane read (pages hold >= 16 keys and a copy moves at most 16 aligned keys, so a copy never straddles
//     a page).
//   * Partial (O / l, lse) per chunk goes to the workspace; the combine kernel merges a sequence's chunks.
// Split boundaries are logical key positions, so the result does not depend on physical page placement.
//
// 8-bit caches ("7 anti-patterns of DeepSeek attention optimisation", lpnh.cn, section 3.3: FP8 E4M3, largest
// value 448; "DeepSeek 32K to 256K long context", tqpw.cn, section 2.5: int8 K/V with per-channel scales): the
// codes are staged the same way, one byte per element. Every E4M3 and int8 value is exact in bf16, so codes
// become MFMA operands by exact conversion (v_cvt_scalef32_pk_bf16_fp8 with scale 1; int8 through float). The
// per-channel K scale is folded into the query (q_d * k_scale_d, rounded to bf16 once per query); the per-channel
// V scale multiplies the output channels at the end. For the K reads the contraction order over the head dims is
// permuted (k-steps 2i and 2i+1 of lane group g take dims 64i + 16g .. +15) so a lane reads 16 contiguous bytes;
// V rows are read 8 bytes per lane and an 8x8 register transpose (byte permutes) turns them into eight A operands.
//
// Head dims 128 and 64 are template instances of the same kernels.
#include <type_traits>

#include "device.h"
#include "kernels.h"

namespace attn {
namespace {

static_assert(kDecodeChunk % 32 == 0 && kDecodeChunk / 16 <= 64, "a chunk's pages (>= 16 keys each) fit one wave");

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
  int64_t num_pages;
  float scale;
};

__device__ __forceinline__ int clamp_len(int L, int max_len, int cap) { return max(0, min(L, min(max_len, cap))); }

template <int N>
__device__ __forceinline__ void wait_vmem_n() { asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory"); }

// Element j (0..7) of each of the 8 rows in vv, packed in row order: the A operand for dimension offset j.
__device__ __forceinline__ bf16x8_t transpose_pick(const u32x4_t* vv, int j) {
  const uint32_t sel = (j & 1) ? 0x07060302u : 0x05040100u;
  u32x4_t w;
#pragma unroll
  for (int u = 0; u < 4; ++u) w[u] = __builtin_amdgcn_perm(vv[2 * u + 1][j >> 1], vv[2 * u][j >> 1], sel);
  return as_bf16x8(w);
}

// Per-wave chunk context shared by both kernels: sequence length, the chunk's key range and its page numbers.
struct Chunk {
  int t_begin, t_end, first_page;
  int pg_lane;        // lane i: block-table entry of the chunk's i-th page (-1 past the chunk)
};

__device__ __forceinline__ bool load_chunk(const DecodeArgs& a, int b, int chunk, Chunk& ck) {
  const int page_size = 1 << a.page_shift;
  const int L = clamp_len(a.seq_lens[b], a.max_len, a.max_pages * page_size);
  ck.t_begin = chunk * kDecodeChunk;
  if (ck.t_begin >= L) return false;
  ck.t_end = min(L, ck.t_begin + kDecodeChunk);
  ck.first_page = ck.t_begin >> a.page_shift;
  const int last_page = (ck.t_end - 1) >> a.page_shift;
  const int lane = threadIdx.x;
  const int32_t* trow = a.table + int64_t(b) * a.max_pages;
  ck.pg_lane = (lane <= last_page - ck.first_page) ? trow[ck.first_page + lane] : -1;
  return true;
}

// Online softmax over one 32-key block of S^T (lane: head n, keys t0 + 16*tb + 4*grp4 + r), lazily rescaling the
// NO output accumulators. Keys at or past t_end are masked. Leaves P (unnormalised, bf16) in the returned operand.
template <int NO>
__device__ __forceinline__ bf16x8_t softmax_block(f32x4_t (&sacc)[2], f32x4_t (&oacc)[NO], float& m, float& l,
                                                  int t0, int t_end, int grp4, float c) {
  if (t0 + 32 > t_end) {
#pragma unroll
    for (int tb = 0; tb < 2; ++tb)
#pragma unroll
      for (int r = 0; r < 4; ++r)
        if (t0 + 16 * tb + 4 * grp4 + r >= t_end) sacc[tb][r] = -INFINITY;
  }
  // row max per head (column n): 8 values per lane, 4 lanes per head
  float mx = -INFINITY;
#pragma unroll
  for (int tb = 0; tb < 2; ++tb)
#pragma unroll
    for (int r = 0; r < 4; ++r) mx = fmaxf(mx, sacc[tb][r]);
  mx = fmaxf(mx, xor_lanes(mx, 16));
  mx = fmaxf(mx, xor_lanes(mx, 32));
  // Lazy rescale (see the prefill kernel): O and l move to a new reference max only when it grew by more than
  // 2^kRescaleLog2 for some lane.
  if (__any((mx - m) * c > kRescaleLog2)) {
    const float m_new = fmaxf(m, mx);
    const float alpha = fast_exp2((m - m_new) * c);
    l *= alpha;
#pragma unroll
    for (int j = 0; j < NO; ++j) oacc[j] *= alpha;
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
  return pack_bf16x8(sacc[0][0], sacc[0][1], sacc[0][2], sacc[0][3], sacc[1][0], sacc[1][1], sacc[1][2],
                     sacc[1][3]);
}

// ---- bf16 caches. Each 32-key block of K and of V is copied global -> LDS, one buffer-load instruction per
// 1 KiB of whole head slices (4 rows at head dim 128, 8 at 64), and the operands are read from LDS: K fragments
// with ds_read_b128, V^T fragments with the transposing ds_read_b64_tr_b16 (the O^T layout is then dims
// 16*db + 4*grp4 + r). 16-byte chunk c of tile row r is stored at c ^ swz(r) (the copy permutes its source chunks);
// under the measured bank model (ds_read_b128 serves the lane sets {0-7, 24-31}, {8-15, 16-23}, {32-39, 56-63},
// {40-47, 48-55} one per cycle, ds_read_b64_tr_b16 32 consecutive lanes; a set is conflict-free when it hits
// distinct slots modulo 256 bytes) both read patterns are conflict-free:
//   head dim 128 (256-byte rows): K key r & 15, V key 2 (r & 7);
//   head dim 64 (128-byte rows, two rows per 256 bytes): K key (r >> 1) & 7, V key 2 ((r >> 1) & 3).
template <int D>
__device__ __forceinline__ int dec_swz_k(int r) { return D == 128 ? (r & 15) : ((r >> 1) & 7); }
template <int D>
__device__ __forceinline__ int dec_swz_v(int r) { return D == 128 ? 2 * (r & 7) : 2 * ((r >> 1) & 3); }

template <int D>
__global__ __launch_bounds__(64) void decode_paged_lds_kernel(DecodeArgs a) {
  static_assert(D == 128 || D == 64, "head dim");
  constexpr int kCh = D / 8;                 // 16-byte chunks per row
  constexpr int kRowsPerCopy = 64 / kCh;     // rows per 1 KiB copy instruction
  constexpr int kCopies = 32 / kRowsPerCopy; // copy instructions per tensor per block
  constexpr int kKs = D / 32;                // k-steps of S^T = K Q^T
  constexpr int kDb = D / 16;                // 16-dim row blocks of O^T
  // One LDS array per buffer and tensor: distinct objects, so the compiler can see that a block's copies in
  // flight do not alias the buffer being read, and keeps its waits at the block boundary.
  __shared__ __attribute__((aligned(16))) uint16_t kl0[32 * D], kl1[32 * D];
  __shared__ __attribute__((aligned(16))) uint16_t vl0[32 * D], vl1[32 * D];
  const int g = blockIdx.x, chunk = blockIdx.y, b = blockIdx.z;
  Chunk ck;
  if (!load_chunk(a, b, chunk, ck)) return;
  const int t_begin = ck.t_begin, t_end = ck.t_end;
  const int lane = threadIdx.x, n = lane & 15, grp4 = lane >> 4;
  const int G = a.hq / a.hkv;
  const int h = g * G + n;
  const bool hv = n < G;
  const float c = a.scale * kLog2e;
  const int page_size = 1 << a.page_shift;

  // Q^T operand: lane holds head n, dims 8*(4*ks + grp4) .. +7 for k-step ks.
  bf16x8_t qop[kKs];
#pragma unroll
  for (int ks = 0; ks < kKs; ++ks) {
    u32x4_t w = {0u, 0u, 0u, 0u};
    if (hv) w = *reinterpret_cast<const u32x4_t*>(a.q + (int64_t(b) * a.hq + h) * D + 8 * (4 * ks + grp4));
    qop[ks] = as_bf16x8(w);
  }
  f32x4_t oacc[kDb];                                     // O^T: lane holds head n, dims 16*db + 4*grp4 + r
#pragma unroll
  for (int db = 0; db < kDb; ++db) oacc[db] = f32x4_t{};
  float m = -INFINITY, l = 0.f;
  const int64_t row_stride = int64_t(a.hkv) * D;
  const int64_t page_stride = int64_t(page_size) * row_stride;
  const uint16_t* kcache = static_cast<const uint16_t*>(a.kc);
  const uint16_t* vcache = static_cast<const uint16_t*>(a.vc);

  // Copy instruction i of a block moves keys t0 + kRowsPerCopy*i ..; keys at or past t_end and pages outside
  // [0, num_pages) read as zeros (empty resource).
  const int row_in = lane / kCh, pcs = lane % kCh;
  const uint32_t row_bytes = uint32_t(row_stride * 2);
  auto copy_block = [&](uint16_t* kdst, uint16_t* vdst, int t0) {
#pragma unroll
    for (int i = 0; i < kCopies; ++i) {
      const int key_first = t0 + kRowsPerCopy * i;
      const int pg = __builtin_amdgcn_readlane(ck.pg_lane, (min(key_first, t_end - 1) >> a.page_shift) - ck.first_page);
      const bool pv = pg >= 0 && pg < a.num_pages;
      const int rows = pv ? max(0, min(kRowsPerCopy, t_end - key_first)) : 0;
      const int64_t e0 = int64_t(max(pg, 0)) * page_stride + int64_t(key_first & (page_size - 1)) * row_stride +
                         int64_t(g) * D;
      const buf_rsrc_t rk = make_buf_rsrc(kcache + e0, uint32_t(rows) * row_bytes);
      const buf_rsrc_t rv = make_buf_rsrc(vcache + e0, uint32_t(rows) * row_bytes);
      const int r = kRowsPerCopy * i + row_in;
      raw_buffer_load_lds(rk, (lds_void_t*)(kdst + i * 512), 16, int(row_in * row_bytes + 16 * (pcs ^ dec_swz_k<D>(r))),
                          0, 0, 2);
      raw_buffer_load_lds(rv, (lds_void_t*)(vdst + i * 512), 16, int(row_in * row_bytes + 16 * (pcs ^ dec_swz_v<D>(r))),
                          0, 0, 2);
    }
  };
  // LDS read addresses (bytes): K row 16*tb + n, chunk 4*ks + grp4; V rows 4*grp4 + j (+16), dims 16*db + 4*(n&3)
  uint32_t kaddr[kKs], vaddr[kDb];
#pragma unroll
  for (int ks = 0; ks < kKs; ++ks) kaddr[ks] = uint32_t(n * 2 * D + 16 * ((4 * ks + grp4) ^ dec_swz_k<D>(n)));
  {
    const int vr = 4 * grp4 + (n >> 2), cq = n & 3;
#pragma unroll
    for (int db = 0; db < kDb; ++db)
      vaddr[db] = uint32_t(vr * 2 * D + 16 * ((2 * db + (cq >> 1)) ^ dec_swz_v<D>(vr)) + 8 * (cq & 1));
  }

  // A block's operand fragments are read from LDS into registers before the next block's copies are issued: the
  // compiler cannot tell the copies from these reads apart and would otherwise wait for the copies first.
  u32x4_t kf[2][kKs], vf[kDb];
  auto read_block = [&](const uint16_t* Kt, const uint16_t* Vt) {
#pragma unroll
    for (int tb = 0; tb < 2; ++tb)
#pragma unroll
      for (int ks = 0; ks < kKs; ++ks) kf[tb][ks] = lds_read16(Kt, kaddr[ks] + tb * 16 * 2 * D);
#pragma unroll
    for (int db = 0; db < kDb; ++db) {
      const u32x2_t lo = lds_read_tr16(Vt, vaddr[db]);
      const u32x2_t hi = lds_read_tr16(Vt, vaddr[db] + 16 * 2 * D);
      vf[db] = u32x4_t{lo[0], lo[1], hi[0], hi[1]};
    }
  };
  auto block = [&](int t0) {
    f32x4_t sacc[2] = {f32x4_t{}, f32x4_t{}};
#pragma unroll
    for (int tb = 0; tb < 2; ++tb)
#pragma unroll
      for (int ks = 0; ks < kKs; ++ks) sacc[tb] = mfma16x16x32(as_bf16x8(kf[tb][ks]), qop[ks], sacc[tb]);
    const bf16x8_t pb = softmax_block<kDb>(sacc, oacc, m, l, t0, t_end, grp4, c);
#pragma unroll
    for (int db = 0; db < kDb; ++db) oacc[db] = mfma16x16x32(as_bf16x8(vf[db]), pb, oacc[db]);
  };

  // Ring of two blocks: at block u, wait for its copies, read its fragments, issue the copies of block u + 1 into
  // the other buffer, and compute.
  wait_vmem_n<0>();        // q and the page numbers are in: from here on only block copies are outstanding
  copy_block(kl0, vl0, t_begin);
  for (int t0 = t_begin; t0 < t_end; t0 += 64) {
    wait_vmem_n<0>();
    read_block(kl0, vl0);
    if (t0 + 32 < t_end) copy_block(kl1, vl1, t0 + 32);
    block(t0);
    if (t0 + 32 >= t_end) break;
    wait_vmem_n<0>();
    read_block(kl1, vl1);
    if (t0 + 64 < t_end) copy_block(kl0, vl0, t0 + 64);
    block(t0 + 32);
  }

  float lt = l + xor_lanes(l, 16);
  lt += xor_lanes(lt, 32);
  if (!hv) return;
  const int64_t slot = (int64_t(b) * a.hq + h) * a.n_chunks + chunk;
  const float inv = 1.f / lt;
  float* wo = a.ws_o + slot * D + 4 * grp4;
#pragma unroll
  for (int db = 0; db < kDb; ++db) *reinterpret_cast<f32x4_t*>(wo + 16 * db) = oacc[db] * inv;
  if (grp4 == 0) a.ws_lse[slot] = m * a.scale + logf(lt);
}

// ---- 8-bit caches. Per 32-key block, whole head slices of codes are copied global -> LDS (1 KiB per instruction:
// 8 rows at head dim 128, 16 at 64; non-temporal) and read back as 16-byte K pieces and 8-byte V rows. K chunk c of
// row r sits at c ^ swz8(r), conflict-free for the b128 reads (bank model above):
//   head dim 128 (128-byte rows): swz8(r) = ((r >> 1) & 3) | ((r >> 3) & 1) << 2;
//   head dim 64 (64-byte rows, four rows per 256 bytes): swz8(r) = (r >> 2) & 3.
// V rows are unswizzled (their b64 reads pair rows 256 bytes apart: a 2-way conflict whatever the swizzle). At head
// dim 64 the O^T operand rows 8 .. 15 (dims 64 .. 127) are unused: lanes 8 .. 15 of each row block re-read the
// rows of lanes 0 .. 7, and their results are not written.
template <int D>
__device__ __forceinline__ int dec_swz8(int r) {
  return D == 128 ? (((r >> 1) & 3) | (((r >> 3) & 1) << 2)) : ((r >> 2) & 3);
}

template <int KV, int D>
__global__ __launch_bounds__(64) void decode_paged_q8_kernel(DecodeArgs a) {
  static_assert(D == 128 || D == 64, "head dim");
  constexpr int kCh = D / 16;                // 16-byte chunks per row of codes
  constexpr int kRowsPerCopy = 64 / kCh;     // rows per 1 KiB copy instruction
  constexpr int kCopies = 32 / kRowsPerCopy; // copy instructions per tensor per block
  constexpr int kKs = D / 32;                // k-steps of S^T = K Q^T
  constexpr int kHk = D / 64;                // 16-byte K pieces per lane and key
  __shared__ __attribute__((aligned(16))) uint8_t k8a[32 * D], k8b[32 * D], v8a[32 * D], v8b[32 * D];
  const int g = blockIdx.x, chunk = blockIdx.y, b = blockIdx.z;
  Chunk ck;
  if (!load_chunk(a, b, chunk, ck)) return;
  const int t_begin = ck.t_begin, t_end = ck.t_end;
  const int lane = threadIdx.x, n = lane & 15, grp4 = lane >> 4;
  const int G = a.hq / a.hkv;
  const int h = g * G + n;
  const bool hv = n < G;
  const float c = a.scale * kLog2e;
  const int page_size = 1 << a.page_shift;

  // Q^T operand: lane holds head n, dims kdim(ks) .. +7 for k-step ks, times the K scale.
  auto kdim = [&](int ks) { return 64 * (ks >> 1) + 16 * grp4 + 8 * (ks & 1); };
  bf16x8_t qop[kKs];
#pragma unroll
  for (int ks = 0; ks < kKs; ++ks) {
    u32x4_t w = {0u, 0u, 0u, 0u};
    if (hv) w = *reinterpret_cast<const u32x4_t*>(a.q + (int64_t(b) * a.hq + h) * D + kdim(ks));
    const float* ks_p = a.k_scale + g * D + kdim(ks);
    w = u32x4_t{pack_bf16x2(bf16lo_to_f32(w[0]) * ks_p[0], bf16hi_to_f32(w[0]) * ks_p[1]),
                pack_bf16x2(bf16lo_to_f32(w[1]) * ks_p[2], bf16hi_to_f32(w[1]) * ks_p[3]),
                pack_bf16x2(bf16lo_to_f32(w[2]) * ks_p[4], bf16hi_to_f32(w[2]) * ks_p[5]),
                pack_bf16x2(bf16lo_to_f32(w[3]) * ks_p[6], bf16hi_to_f32(w[3]) * ks_p[7])};
    qop[ks] = as_bf16x8(w);
  }
  f32x4_t oacc[8];                                       // O^T: lane holds head n, dims 8*(4*grp4 + r) + j
#pragma unroll
  for (int j = 0; j < 8; ++j) oacc[j] = f32x4_t{};
  float m = -INFINITY, l = 0.f;
  const int64_t row_stride = int64_t(a.hkv) * D;       // bytes between consecutive slots of a page
  const int64_t page_stride = int64_t(page_size) * row_stride;
  const uint8_t* kcache = static_cast<const uint8_t*>(a.kc);
  const uint8_t* vcache = static_cast<const uint8_t*>(a.vc);

  const int row_in = lane / kCh, pcs = lane % kCh;
  const uint32_t row_bytes = uint32_t(row_stride);
  auto copy8 = [&](uint8_t* kdst, uint8_t* vdst, int t0) {
#pragma unroll
    for (int i = 0; i < kCopies; ++i) {
      const int key_first = t0 + kRowsPerCopy * i;
      const int pg = __builtin_amdgcn_readlane(ck.pg_lane, (min(key_first, t_end - 1) >> a.page_shift) - ck.first_page);
      const bool pv = pg >= 0 && pg < a.num_pages;
      const int rows = pv ? max(0, min(kRowsPerCopy, t_end - key_first)) : 0;
      const int64_t e0 = int64_t(max(pg, 0)) * page_stride + int64_t(key_first & (page_size - 1)) * row_stride +
                         int64_t(g) * D;
      const buf_rsrc_t rk = make_buf_rsrc(kcache + e0, uint32_t(rows) * row_bytes);
      const buf_rsrc_t rv = make_buf_rsrc(vcache + e0, uint32_t(rows) * row_bytes);
      const int r = kRowsPerCopy * i + row_in;
      raw_buffer_load_lds(rk, (lds_void_t*)(kdst + i * 1024), 16, int(row_in * row_bytes + 16 * (pcs ^ dec_swz8<D>(r))),
                          0, 0, 2);
      raw_buffer_load_lds(rv, (lds_void_t*)(vdst + i * 1024), 16, int(row_in * row_bytes + 16 * pcs), 0, 0, 2);
    }
  };
  // K of key 16*tb + n as 16-byte pieces (dims 64*hk + 16*grp4 ..), V rows of keys 16*(s/4) + 4*grp4 + s%4 as
  // 8 bytes (dims 8*n' .. 8*n' + 7, n' = n mod D/8).
  u32x4_t kv8[2][kHk];
  u32x2_t vv8[8];
  auto read8 = [&](const uint8_t* ks, const uint8_t* vs) {
#pragma unroll
    for (int tb = 0; tb < 2; ++tb)
#pragma unroll
      for (int hk = 0; hk < kHk; ++hk) {
        const int r = 16 * tb + n;
        kv8[tb][hk] = *reinterpret_cast<const __attribute__((address_space(3))) u32x4_t*>(
            (const __attribute__((address_space(3))) uint8_t*)ks + r * D + 16 * ((4 * hk + grp4) ^ dec_swz8<D>(r)));
      }
#pragma unroll
    for (int s2 = 0; s2 < 8; ++s2) {
      const int r = 16 * (s2 >> 2) + 4 * grp4 + (s2 & 3);
      vv8[s2] = *reinterpret_cast<const __attribute__((address_space(3))) u32x2_t*>(
          (const __attribute__((address_space(3))) uint8_t*)vs + r * D + 8 * (n % (D / 8)));
    }
  };
  auto block = [&](int t0) {
    u32x4_t kv[2][kKs], vv[8];
#pragma unroll
    for (int tb = 0; tb < 2; ++tb)
#pragma unroll
      for (int ks = 0; ks < kKs; ++ks)
        kv[tb][ks] = codes_to_bf16x8<KV>(kv8[tb][ks >> 1][2 * (ks & 1)], kv8[tb][ks >> 1][2 * (ks & 1) + 1]);
#pragma unroll
    for (int s2 = 0; s2 < 8; ++s2) vv[s2] = codes_to_bf16x8<KV>(vv8[s2][0], vv8[s2][1]);
    f32x4_t sacc[2] = {f32x4_t{}, f32x4_t{}};
#pragma unroll
    for (int tb = 0; tb < 2; ++tb)
#pragma unroll
      for (int ks = 0; ks < kKs; ++ks) sacc[tb] = mfma16x16x32(as_bf16x8(kv[tb][ks]), qop[ks], sacc[tb]);
    const bf16x8_t pb = softmax_block<8>(sacc, oacc, m, l, t0, t_end, grp4, c);
#pragma unroll
    for (int j = 0; j < 8; ++j) oacc[j] = mfma16x16x32(transpose_pick(vv, j), pb, oacc[j]);
  };

  wait_vmem_n<0>();        // q, scales and the page numbers are in: from here on only block copies are outstanding
  copy8(k8a, v8a, t_begin);
  for (int t0 = t_begin; t0 < t_end; t0 += 64) {
    wait_vmem_n<0>();
    read8(k8a, v8a);                                   // block t0 into registers before the next copies
    if (t0 + 32 < t_end) copy8(k8b, v8b, t0 + 32);
    block(t0);
    if (t0 + 32 >= t_end) break;
    wait_vmem_n<0>();
    read8(k8b, v8b);
    if (t0 + 64 < t_end) copy8(k8a, v8a, t0 + 64);
    block(t0 + 32);
  }

  // partial result: O / l and lse for this chunk (lane holds head n, dims 8*(4*grp4 + r) + j)
  float lt = l + xor_lanes(l, 16);
  lt += xor_lanes(lt, 32);
  if (!hv || 4 * grp4 >= D / 8) return;
  const int64_t slot = (int64_t(b) * a.hq + h) * a.n_chunks + chunk;
  const float inv = 1.f / lt;
  float* wo = a.ws_o + slot * D;
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int d0 = 8 * (4 * grp4 + r);
    const f32x4_t* vs = reinterpret_cast<const f32x4_t*>(a.v_scale + g * D + d0);     // per-channel V scale
    const f32x4_t lo = f32x4_t{oacc[0][r], oacc[1][r], oacc[2][r], oacc[3][r]} * inv * vs[0];
    const f32x4_t hi = f32x4_t{oacc[4][r], oacc[5][r], oacc[6][r], oacc[7][r]} * inv * vs[1];
    *reinterpret_cast<f32x4_t*>(wo + d0) = lo;
    *reinterpret_cast<f32x4_t*>(wo + d0 + 4) = hi;
  }
  if (grp4 == 0) a.ws_lse[slot] = m * a.scale + logf(lt);
}

// Merge the chunks of one (sequence, query head): M = max lse_c, w_c = exp(lse_c - M),
// O = sum_c w_c O_c / sum_c w_c, lse = M + ln sum_c w_c. A sequence of length 0 gets O = 0, lse = -inf.
// One thread per head dimension (blockDim.x = D).
__global__ __launch_bounds__(128) void decode_combine_kernel(const float* __restrict__ ws_o,
    const float* __restrict__ ws_lse, const int32_t* __restrict__ seq_lens, uint16_t* __restrict__ o,
    float* __restrict__ lse, int hq, int D, int n_chunks, int max_len, int cap) {
  const int h = blockIdx.x, b = blockIdx.y, d = threadIdx.x;
  const int L = clamp_len(seq_lens[b], max_len, cap);
  const int nc = (L + kDecodeChunk - 1) / kDecodeChunk;
  const int64_t base = (int64_t(b) * hq + h) * n_chunks;
  uint16_t* op = o + (int64_t(b) * hq + h) * D;
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
    acc = fmaf(w, ws_o[(base + ci) * D + d], acc);
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
template <int D>
void launch_split(int kind, const DecodeArgs& a, dim3 grid, hipStream_t stream) {
  if (kind == kKvFp8) decode_paged_q8_kernel<kKvFp8, D><<<grid, dim3(64), 0, stream>>>(a);
  else if (kind == kKvInt8) decode_paged_q8_kernel<kKvInt8, D><<<grid, dim3(64), 0, stream>>>(a);
  else decode_paged_lds_kernel<D><<<grid, dim3(64), 0, stream>>>(a);
}

hipError_t launch_decode(int kind, const void* q, const void* k_cache, const void* v_cache, const float* k_scale,
                         const float* v_scale, const int32_t* block_table, const int32_t* seq_lens, void* o, float* lse,
                         int batch, int hq, int hkv, int head_dim, int page_size, int max_pages_per_seq,
                         int64_t num_pages, int max_seqlen_kv, float scale, void* workspace, hipStream_t stream) {
  const int n_chunks = max(1, (max_seqlen_kv + kDecodeChunk - 1) / kDecodeChunk);
  const size_t slots = size_t(batch) * size_t(hq) * size_t(n_chunks);
  const size_t o_bytes = (slots * size_t(head_dim) * sizeof(float) + 255) & ~size_t(255);
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
  const dim3 grid{unsigned(hkv), unsigned(n_chunks), unsigned(batch)};     // head-major
  if (max_seqlen_kv > 0) {
    if (head_dim == 64) launch_split<64>(kind, a, grid, stream);
    else launch_split<128>(kind, a, grid, stream);
  }
  decode_combine_kernel<<<dim3(unsigned(hq), unsigned(batch)), dim3(unsigned(head_dim)), 0, stream>>>(
      a.ws_o, a.ws_lse, seq_lens, static_cast<uint16_t*>(o), lse, hq, head_dim, n_chunks, max_seqlen_kv,
      max_pages_per_seq * page_size);
  return hipGetLastError();
}
}  // namespace

hipError_t launch_decode_paged(const void* q, const void* k_cache, const void* v_cache, const int32_t* block_table,
                               const int32_t* seq_lens, void* o, float* lse, int batch, int hq, int hkv,
                               int head_dim, int page_size, int max_pages_per_seq, int64_t num_pages,
                               int max_seqlen_kv, float scale, void* workspace, hipStream_t stream) {
  return launch_decode(kKvBf16, q, k_cache, v_cache, nullptr, nullptr, block_table, seq_lens, o, lse, batch, hq, hkv,
                       head_dim, page_size, max_pages_per_seq, num_pages, max_seqlen_kv, scale, workspace, stream);
}

hipError_t launch_decode_paged_q8(int fp8, const void* q, const void* k_cache, const void* v_cache,
                                  const float* k_scale, const float* v_scale, const int32_t* block_table,
                                  const int32_t* seq_lens, void* o, float* lse, int batch, int hq, int hkv,
                                  int head_dim, int page_size, int max_pages_per_seq, int64_t num_pages,
                                  int max_seqlen_kv, float scale, void* workspace, hipStream_t stream) {
  return launch_decode(fp8 ? kKvFp8 : kKvInt8, q, k_cache, v_cache, k_scale, v_scale, block_table, seq_lens, o, lse,
                       batch, hq, hkv, head_dim, page_size, max_pages_per_seq, num_pages, max_seqlen_kv, scale,
                       workspace, stream);
}

}  // namespace attn
