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
//   * Split kernels: one wave per (logical key chunk, KV-head group, sequence), launched head-major (the head
//     groups of one chunk are consecutive workgroups: they read interleaved head slices of the same page slots at
//     the same time). The wave serves all query heads of its KV heads at once, so every K/V byte is read once.
//     Chunks at or past the sequence length exit at once. The chunk size is chosen per launch (2048 keys for bf16
//     caches when a chunk's pages fit one wave, else 1024).
//   * K and V blocks are copied global -> LDS with buffer loads carrying the LDS bit (whole head slices,
//     non-temporal: every cache byte is read once), in a ring of blocks (two by default), and the MFMA operands
//     are read from LDS by inline-assembly reads (see block_ring).
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
// With FP8 codes a wave takes two KV heads at head dim 128 (four at 64), so each copied row piece is 256 bytes.
//
// Head dims 128 and 64 are template instances of the same kernels.
#include <type_traits>

#include "device.h"
#include "kernels.h"

namespace attn {
namespace {

// Keys per split by cache kind (see launch_decode). Measured on the 64-sequence workload: bf16 2048 keys 3% faster
// than 1024 (fewer partials and wave starts); 8-bit 2% slower.
#ifndef ATTN_DECODE_CHUNK_BF16
#define ATTN_DECODE_CHUNK_BF16 2048
#endif
#ifndef ATTN_DECODE_CHUNK_Q8
#define ATTN_DECODE_CHUNK_Q8 1024
#endif
static_assert(kDecodeChunk % 32 == 0 && kDecodeChunk / 16 <= 64, "a chunk's pages (>= 16 keys each) fit one wave");
static_assert(ATTN_DECODE_CHUNK_BF16 % 32 == 0 && ATTN_DECODE_CHUNK_Q8 % 32 == 0, "chunks of whole 32-key blocks");

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
  int hq, hkv, page_shift, max_pages, max_len, n_chunks, batch;
  int n_hg;                // KV-head groups (one per wave): hkv / heads per wave
  int chunk;               // keys per split: a multiple of 32, at most 64 pages
  int64_t num_pages;
  float scale;
};

__device__ __forceinline__ int clamp_len(int L, int max_len, int cap) { return max(0, min(L, min(max_len, cap))); }

// Workgroup -> (KV-head group g, chunk, sequence b). The 1-D grid holds n_hg x n_chunks x batch workgroups (every
// sequence at the maximum length). The hardware hands workgroup i to XCD i mod 8 and shader engine i mod 32, and
// to a free slot within that engine; the order decides how the units' keys spread over the engines.
//   kOrderGrid: workgroup i is head group i mod n_hg of chunk (i / n_hg) mod n_chunks of sequence
//     i / (n_hg n_chunks); the head groups of one chunk are consecutive and read interleaved slices of the same
//     page slots; pairs past a sequence's length exit at once.
//   kOrderDense, kOrderDenseXcd: unit k counts only the (sequence, chunk) pairs that hold keys, sequence by
//     sequence, and workgroups past the last unit exit. Dense: head group i mod n_hg of unit i / n_hg. DenseXcd:
//     the head groups of one unit go to one XCD (workgroups i, i + 8, ...): head group (i / 8) mod n_hg of unit
//     8 (i / (8 n_hg)) + i mod 8.
// Measured on the 64-sequence workload (lengths 3.6k-32.6k): bf16 is fastest in grid order (dense 2.5% slower),
// the 8-bit caches with the dense orders (grid order left the engines' key shares up to 20% apart).
constexpr int kOrderGrid = 0, kOrderDense = 1, kOrderDenseXcd = 2;
#ifndef ATTN_DECODE_ORDER_BF16
#define ATTN_DECODE_ORDER_BF16 0
#endif
#ifndef ATTN_DECODE_ORDER_Q8
#define ATTN_DECODE_ORDER_Q8 2
#endif

template <int ORDER>
__device__ __forceinline__ bool decode_unit(const DecodeArgs& a, int& g, int& chunk, int& b) {
  const int id = blockIdx.x;
  if constexpr (ORDER == kOrderGrid) {
    g = id % a.n_hg;
    chunk = (id / a.n_hg) % a.n_chunks;
    b = id / (a.n_hg * a.n_chunks);
    return b < a.batch;
  } else {
    int k;
    if constexpr (ORDER == kOrderDense) {
      g = id % a.n_hg;
      k = id / a.n_hg;
    } else {
      g = (id >> 3) % a.n_hg;
      k = 8 * (id / (8 * a.n_hg)) + (id & 7);
    }
    const int lane = threadIdx.x;
    const int cap = a.max_pages << a.page_shift;
    for (int base = 0; base < a.batch; base += 64) {
      const int bb = base + lane;
      const int L = bb < a.batch ? clamp_len(a.seq_lens[bb], a.max_len, cap) : 0;
      const int nc = (L + a.chunk - 1) / a.chunk;
      int incl = nc;                                    // inclusive prefix sum of the chunk counts over the lanes
#pragma unroll
      for (int off = 1; off < 64; off <<= 1) {
        const int t = __shfl_up(incl, off);
        if (lane >= off) incl += t;
      }
      const int total = __builtin_amdgcn_readlane(incl, 63);
      if (k < total) {
        const int j = __builtin_ctzll(__ballot(incl > k));       // first sequence whose chunks reach past k
        b = base + j;
        chunk = k - (__builtin_amdgcn_readlane(incl, j) - __builtin_amdgcn_readlane(nc, j));
        return true;
      }
      k -= total;
    }
    return false;
  }
}

// Copy cache policy: non-temporal, every cache byte is read once (measured: cached copies 7% slower).
constexpr int kCopyAux = 2;

// LDS address `byte_off` bytes into a __shared__ buffer, formed in the LDS address space (a cast of the buffer
// itself, then the offset), so the copy's destination stays a known object the compiler can tell from the others.
template <class T>
__device__ __forceinline__ lds_void_t* lds_at(T* buf, int byte_off) {
  return (lds_void_t*)((__attribute__((address_space(3))) char*)buf + byte_off);
}

__device__ __forceinline__ uint32_t lds_addr(const void* buf) {
  return uint32_t(reinterpret_cast<uintptr_t>((const __attribute__((address_space(3))) char*)buf));
}

// Fragment reads of one block written out in inline assembly, each group ending with its own lgkmcnt(0) wait (the
// outputs are complete when the statement ends). The compiler's wait insertion cannot tell LDS reads at the head
// of the ring loop from the copies in flight there and would drain every copy before them; reads it does not
// see need no such wait, and the ring's own vmcnt wait orders them after their block's copies.
// bf16 block, K: kf[tb][ks] at ka[ks] + tb * 32 * D (16 rows of 2D bytes).
template <int D>
__device__ __forceinline__ void bf16_k_reads(const uint32_t (&ka)[D / 32], u32x4_t (&kf)[2][D / 32]) {
  if constexpr (D == 128) {
    asm volatile(
        "ds_read_b128 %0, %8\n\tds_read_b128 %1, %9\n\tds_read_b128 %2, %10\n\tds_read_b128 %3, %11\n\t"
        "ds_read_b128 %4, %8 offset:%12\n\tds_read_b128 %5, %9 offset:%12\n\t"
        "ds_read_b128 %6, %10 offset:%12\n\tds_read_b128 %7, %11 offset:%12\n\ts_waitcnt lgkmcnt(0)"
        : "=&v"(kf[0][0]), "=&v"(kf[0][1]), "=&v"(kf[0][2]), "=&v"(kf[0][3]), "=&v"(kf[1][0]), "=&v"(kf[1][1]),
          "=&v"(kf[1][2]), "=&v"(kf[1][3])
        : "v"(ka[0]), "v"(ka[1]), "v"(ka[2]), "v"(ka[3]), "n"(32 * D)
        : "memory");
  } else {
    asm volatile(
        "ds_read_b128 %0, %4\n\tds_read_b128 %1, %5\n\t"
        "ds_read_b128 %2, %4 offset:%6\n\tds_read_b128 %3, %5 offset:%6\n\ts_waitcnt lgkmcnt(0)"
        : "=&v"(kf[0][0]), "=&v"(kf[0][1]), "=&v"(kf[1][0]), "=&v"(kf[1][1])
        : "v"(ka[0]), "v"(ka[1]), "n"(32 * D)
        : "memory");
  }
}
// bf16 block, V^T: vf[db] = transposing reads at va[db] (keys 0-15) and va[db] + 32 * D (keys 16-31).
template <int D>
__device__ __forceinline__ void bf16_v_reads(const uint32_t (&va)[D / 16], u32x4_t (&vf)[D / 16]) {
  u32x2_t lo[D / 16], hi[D / 16];
  if constexpr (D == 128) {
    asm volatile(
        "ds_read_b64_tr_b16 %0, %16\n\tds_read_b64_tr_b16 %1, %17\n\tds_read_b64_tr_b16 %2, %18\n\t"
        "ds_read_b64_tr_b16 %3, %19\n\tds_read_b64_tr_b16 %4, %20\n\tds_read_b64_tr_b16 %5, %21\n\t"
        "ds_read_b64_tr_b16 %6, %22\n\tds_read_b64_tr_b16 %7, %23\n\t"
        "ds_read_b64_tr_b16 %8, %16 offset:%24\n\tds_read_b64_tr_b16 %9, %17 offset:%24\n\t"
        "ds_read_b64_tr_b16 %10, %18 offset:%24\n\tds_read_b64_tr_b16 %11, %19 offset:%24\n\t"
        "ds_read_b64_tr_b16 %12, %20 offset:%24\n\tds_read_b64_tr_b16 %13, %21 offset:%24\n\t"
        "ds_read_b64_tr_b16 %14, %22 offset:%24\n\tds_read_b64_tr_b16 %15, %23 offset:%24\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(lo[0]), "=&v"(lo[1]), "=&v"(lo[2]), "=&v"(lo[3]), "=&v"(lo[4]), "=&v"(lo[5]), "=&v"(lo[6]),
          "=&v"(lo[7]), "=&v"(hi[0]), "=&v"(hi[1]), "=&v"(hi[2]), "=&v"(hi[3]), "=&v"(hi[4]), "=&v"(hi[5]),
          "=&v"(hi[6]), "=&v"(hi[7])
        : "v"(va[0]), "v"(va[1]), "v"(va[2]), "v"(va[3]), "v"(va[4]), "v"(va[5]), "v"(va[6]), "v"(va[7]),
          "n"(32 * D)
        : "memory");
  } else {
    asm volatile(
        "ds_read_b64_tr_b16 %0, %8\n\tds_read_b64_tr_b16 %1, %9\n\tds_read_b64_tr_b16 %2, %10\n\t"
        "ds_read_b64_tr_b16 %3, %11\n\tds_read_b64_tr_b16 %4, %8 offset:%12\n\t"
        "ds_read_b64_tr_b16 %5, %9 offset:%12\n\tds_read_b64_tr_b16 %6, %10 offset:%12\n\t"
        "ds_read_b64_tr_b16 %7, %11 offset:%12\n\ts_waitcnt lgkmcnt(0)"
        : "=&v"(lo[0]), "=&v"(lo[1]), "=&v"(lo[2]), "=&v"(lo[3]), "=&v"(hi[0]), "=&v"(hi[1]), "=&v"(hi[2]),
          "=&v"(hi[3])
        : "v"(va[0]), "v"(va[1]), "v"(va[2]), "v"(va[3]), "n"(32 * D)
        : "memory");
  }
#pragma unroll
  for (int db = 0; db < D / 16; ++db) vf[db] = u32x4_t{lo[db][0], lo[db][1], hi[db][0], hi[db][1]};
}
// 8-bit block of one head (rows of RL bytes): K pieces kv8[tb][hk] at ka[hk] + tb * 16 * RL; V rows vv8[s] at
// va + (16 * (s / 4) + s % 4) * RL.
template <int D, int RL>
__device__ __forceinline__ void q8_reads(const uint32_t (&ka)[D / 64], uint32_t va, u32x4_t (&kv8)[2][D / 64],
                                         u32x2_t (&vv8)[8]) {
  if constexpr (D == 128) {
    asm volatile(
        "ds_read_b128 %0, %12\n\tds_read_b128 %1, %12 offset:%15\n\t"
        "ds_read_b128 %2, %13\n\tds_read_b128 %3, %13 offset:%15\n\t"
        "ds_read_b64 %4, %14\n\tds_read_b64 %5, %14 offset:%16\n\t"
        "ds_read_b64 %6, %14 offset:%17\n\tds_read_b64 %7, %14 offset:%18\n\t"
        "ds_read_b64 %8, %14 offset:%15\n\tds_read_b64 %9, %14 offset:%19\n\t"
        "ds_read_b64 %10, %14 offset:%20\n\tds_read_b64 %11, %14 offset:%21\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(kv8[0][0]), "=&v"(kv8[1][0]), "=&v"(kv8[0][1]), "=&v"(kv8[1][1]), "=&v"(vv8[0]), "=&v"(vv8[1]),
          "=&v"(vv8[2]), "=&v"(vv8[3]), "=&v"(vv8[4]), "=&v"(vv8[5]), "=&v"(vv8[6]), "=&v"(vv8[7])
        : "v"(ka[0]), "v"(ka[1]), "v"(va), "n"(16 * RL), "n"(RL), "n"(2 * RL), "n"(3 * RL), "n"(17 * RL),
          "n"(18 * RL), "n"(19 * RL)
        : "memory");
  } else {
    asm volatile(
        "ds_read_b128 %0, %10\n\tds_read_b128 %1, %10 offset:%12\n\t"
        "ds_read_b64 %2, %11\n\tds_read_b64 %3, %11 offset:%13\n\t"
        "ds_read_b64 %4, %11 offset:%14\n\tds_read_b64 %5, %11 offset:%15\n\t"
        "ds_read_b64 %6, %11 offset:%12\n\tds_read_b64 %7, %11 offset:%16\n\t"
        "ds_read_b64 %8, %11 offset:%17\n\tds_read_b64 %9, %11 offset:%18\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(kv8[0][0]), "=&v"(kv8[1][0]), "=&v"(vv8[0]), "=&v"(vv8[1]), "=&v"(vv8[2]), "=&v"(vv8[3]),
          "=&v"(vv8[4]), "=&v"(vv8[5]), "=&v"(vv8[6]), "=&v"(vv8[7])
        : "v"(ka[0]), "v"(va), "n"(16 * RL), "n"(RL), "n"(2 * RL), "n"(3 * RL), "n"(17 * RL), "n"(18 * RL), "n"(19 * RL)
        : "memory");
  }
}

template <int N>
__device__ __forceinline__ void wait_vmem_n() { asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory"); }

// Copy ring over the 32-key blocks of a chunk, NB buffers deep: while block u is read and computed, the copies of
// blocks u+1 .. u+NB-2 are in flight (NB-1 blocks are issued before the first is used). Every block index gets its
// copies, also past the chunk end (they have no rows: zeros, no memory access), so the number of copy
// instructions issued after block u is always (NB-2) * kPerBlock and one immediate vmcnt wait covers it.
// copy(buffer, t0) issues kPerBlock copies; read(buffer) takes the block's fragments from LDS into registers
// before the buffer of the previous block is refilled; compute(buffer, t0) does the block's products.
template <int NB, int kPerBlock, int I = 0, class Copy, class Read, class Compute>
__device__ __forceinline__ bool ring_stage(int t, int t_end, Copy& copy, Read& read, Compute& compute) {
  if constexpr (I == NB) {
    return true;
  } else {
    if (t >= t_end) return false;
    wait_vmem_n<(NB - 2) * kPerBlock>();
    read(std::integral_constant<int, I>{});
    __builtin_amdgcn_sched_barrier(0);                 // the reads are issued before the buffer refill
    copy(std::integral_constant<int, (I + NB - 1) % NB>{}, t + 32 * (NB - 1));
    compute(std::integral_constant<int, I>{}, t);
    return ring_stage<NB, kPerBlock, I + 1>(t + 32, t_end, copy, read, compute);
  }
}
template <int NB, int kPerBlock, int I = 0, class Copy>
__device__ __forceinline__ void ring_prologue(int t_begin, Copy& copy) {
  if constexpr (I < NB - 1) {
    copy(std::integral_constant<int, I>{}, t_begin + 32 * I);
    ring_prologue<NB, kPerBlock, I + 1>(t_begin, copy);
  }
}
template <int NB, int kPerBlock, class Copy, class Read, class Compute>
__device__ __forceinline__ void block_ring(int t_begin, int t_end, Copy& copy, Read& read, Compute& compute) {
  static_assert(NB >= 2 && (NB - 2) * kPerBlock <= 63, "ring depth within the vmcnt range");
  ring_prologue<NB, kPerBlock>(t_begin, copy);
  for (int t0 = t_begin; ring_stage<NB, kPerBlock>(t0, t_end, copy, read, compute); t0 += 32 * NB) {
  }
  wait_vmem_n<0>();        // the trailing empty copies have landed before the wave ends
}

// LDS buffer i of a ring (compile-time index): separate objects, so the compiler can tell a buffer being read
// from the ones with copies in flight. Unused buffers are not allocated.
#define ATTN_RING_BUFFERS(T, name, n)                                                                              \
  __shared__ __attribute__((aligned(16))) T name##0[n], name##1[n], name##2[n], name##3[n], name##4[n], name##5[n]; \
  auto name = [&](auto i) -> T* {                                                                                  \
    constexpr int k = decltype(i)::value;                                                                          \
    static_assert(k < 6, "at most six ring buffers");                                                              \
    if constexpr (k == 0) return name##0;                                                                          \
    else if constexpr (k == 1) return name##1;                                                                     \
    else if constexpr (k == 2) return name##2;                                                                     \
    else if constexpr (k == 3) return name##3;                                                                     \
    else if constexpr (k == 4) return name##4;                                                                     \
    else return name##5;                                                                                           \
  };

#ifndef ATTN_DECODE_RING_BF16
#define ATTN_DECODE_RING_BF16 2
#endif
// 8-bit caches: ring depth by kind and head dim (one KV head per wave, 8 KiB blocks). Measured: three buffers
// 0.8% faster for FP8 at head dim 128, 3.5% (FP8) and 2.5% (int8) at 64, 1.5% slower for int8 at 128.
#ifndef ATTN_DECODE_RING_Q8
#define ATTN_DECODE_RING_Q8 0
#endif
template <int KV, int D>
constexpr int q8_ring_depth() {
  return ATTN_DECODE_RING_Q8 > 0 ? ATTN_DECODE_RING_Q8 : (KV == kKvInt8 && D == 128) ? 2 : 3;
}

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
  ck.t_begin = chunk * a.chunk;
  if (ck.t_begin >= L) return false;
  ck.t_end = min(L, ck.t_begin + a.chunk);
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
  constexpr int NB = ATTN_DECODE_RING_BF16;
  ATTN_RING_BUFFERS(uint16_t, kl, 32 * D)
  ATTN_RING_BUFFERS(uint16_t, vl, 32 * D)
  int g, chunk, b;
  if (!decode_unit<ATTN_DECODE_ORDER_BF16>(a, g, chunk, b)) return;
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
      raw_buffer_load_lds(rk, lds_at(kdst, 1024 * i), 16, int(row_in * row_bytes + 16 * (pcs ^ dec_swz_k<D>(r))),
                          0, 0, kCopyAux);
      raw_buffer_load_lds(rv, lds_at(vdst, 1024 * i), 16, int(row_in * row_bytes + 16 * (pcs ^ dec_swz_v<D>(r))),
                          0, 0, kCopyAux);
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
    const uint32_t kb = lds_addr(Kt), vb = lds_addr(Vt);
    uint32_t ka[kKs], va[kDb];
#pragma unroll
    for (int ks = 0; ks < kKs; ++ks) ka[ks] = kb + kaddr[ks];
#pragma unroll
    for (int db = 0; db < kDb; ++db) va[db] = vb + vaddr[db];
    bf16_k_reads<D>(ka, kf);
    bf16_v_reads<D>(va, vf);
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

  wait_vmem_n<0>();        // q and the page numbers are in: from here on only block copies are outstanding
  auto copy_i = [&](auto i, int t0) { copy_block(kl(i), vl(i), t0); };
  auto read_i = [&](auto i) { read_block(kl(i), vl(i)); };
  auto compute_i = [&](auto, int t0) { block(t0); };
  block_ring<NB, 2 * kCopies>(t_begin, t_end, copy_i, read_i, compute_i);

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

// K chunk swizzle of the 8-bit rows: one head per wave keeps the 128- or 64-byte rows above; rows of 256 bytes or
// more (several heads) take chunk c of row r at c ^ (r & 15), conflict-free by the same count as the bf16 rows.
template <int D, int HPW>
__device__ __forceinline__ int q8_swz(int r) {
  if constexpr (HPW == 1) return dec_swz8<D>(r);
  else return r & 15;
}

template <int KV, int D, int HPW>
__global__ __launch_bounds__(64) void decode_paged_q8_kernel(DecodeArgs a) {
  static_assert(D == 128 || D == 64, "head dim");
  constexpr int RL = HPW * D;                // bytes of one key's codes for the wave's HPW heads (one LDS row)
  static_assert(HPW == 1 || RL >= 256, "several heads per wave take rows of at least 256 bytes");
  constexpr int kCh = RL / 16;               // 16-byte chunks per row
  constexpr int kRowsPerCopy = 64 / kCh;     // rows per 1 KiB copy instruction
  constexpr int kCopies = 32 / kRowsPerCopy; // copy instructions per tensor per block
  constexpr int kKs = D / 32;                // k-steps of S^T = K Q^T
  constexpr int kHk = D / 64;                // 16-byte K pieces per lane, key and head
  constexpr int NB = q8_ring_depth<KV, D>();
  ATTN_RING_BUFFERS(uint8_t, k8, 32 * RL)
  ATTN_RING_BUFFERS(uint8_t, v8, 32 * RL)
  int gw, chunk, b;
  if (!decode_unit<ATTN_DECODE_ORDER_Q8>(a, gw, chunk, b)) return;
  const int g0 = gw * HPW;                   // the wave's first KV head
  Chunk ck;
  if (!load_chunk(a, b, chunk, ck)) return;
  const int t_begin = ck.t_begin, t_end = ck.t_end;
  const int lane = threadIdx.x, n = lane & 15, grp4 = lane >> 4;
  const int G = a.hq / a.hkv;
  const bool hv = n < G;
  const float c = a.scale * kLog2e;
  const int page_size = 1 << a.page_shift;

  // Q^T operand per head: lane holds query head n of KV head g0 + e, dims kdim(ks) .. +7 for k-step ks, times the
  // K scale.
  auto kdim = [&](int ks) { return 64 * (ks >> 1) + 16 * grp4 + 8 * (ks & 1); };
  bf16x8_t qop[HPW][kKs];
#pragma unroll
  for (int e = 0; e < HPW; ++e)
#pragma unroll
    for (int ks = 0; ks < kKs; ++ks) {
      u32x4_t w = {0u, 0u, 0u, 0u};
      if (hv) w = *reinterpret_cast<const u32x4_t*>(a.q + (int64_t(b) * a.hq + (g0 + e) * G + n) * D + kdim(ks));
      const float* ks_p = a.k_scale + (g0 + e) * D + kdim(ks);
      w = u32x4_t{pack_bf16x2(bf16lo_to_f32(w[0]) * ks_p[0], bf16hi_to_f32(w[0]) * ks_p[1]),
                  pack_bf16x2(bf16lo_to_f32(w[1]) * ks_p[2], bf16hi_to_f32(w[1]) * ks_p[3]),
                  pack_bf16x2(bf16lo_to_f32(w[2]) * ks_p[4], bf16hi_to_f32(w[2]) * ks_p[5]),
                  pack_bf16x2(bf16lo_to_f32(w[3]) * ks_p[6], bf16hi_to_f32(w[3]) * ks_p[7])};
      qop[e][ks] = as_bf16x8(w);
    }
  f32x4_t oacc[HPW][8];                                  // O^T: lane holds head n, dims 8*(4*grp4 + r) + j
  float m[HPW], l[HPW];
#pragma unroll
  for (int e = 0; e < HPW; ++e) {
    m[e] = -INFINITY; l[e] = 0.f;
#pragma unroll
    for (int j = 0; j < 8; ++j) oacc[e][j] = f32x4_t{};
  }
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
                         int64_t(g0) * D;
      const buf_rsrc_t rk = make_buf_rsrc(kcache + e0, uint32_t(rows) * row_bytes);
      const buf_rsrc_t rv = make_buf_rsrc(vcache + e0, uint32_t(rows) * row_bytes);
      const int r = kRowsPerCopy * i + row_in;
      raw_buffer_load_lds(rk, lds_at(kdst, 1024 * i), 16, int(row_in * row_bytes + 16 * (pcs ^ q8_swz<D, HPW>(r))),
                          0, 0, kCopyAux);
      raw_buffer_load_lds(rv, lds_at(vdst, 1024 * i), 16, int(row_in * row_bytes + 16 * pcs), 0, 0, kCopyAux);
    }
  };
  // Head e's K of key 16*tb + n as 16-byte pieces (dims 64*hk + 16*grp4 ..), its V rows of keys
  // 16*(s/4) + 4*grp4 + s%4 as 8 bytes (dims 8*n' .. 8*n' + 7, n' = n mod D/8). The swizzle of row 16*tb + n is
  // that of row n, so tb is an immediate offset.
  uint32_t ko[HPW][kHk], vo[HPW];
#pragma unroll
  for (int e = 0; e < HPW; ++e) {
#pragma unroll
    for (int hk = 0; hk < kHk; ++hk)
      ko[e][hk] = uint32_t(n * RL + 16 * ((e * (D / 16) + 4 * hk + grp4) ^ q8_swz<D, HPW>(n)));
    vo[e] = uint32_t(4 * grp4 * RL + e * D + 8 * (n % (D / 8)));
  }
  // The fragments are read head by head inside the block step (inline-assembly reads, invisible to the compiler's
  // wait insertion): the copies issued just before target another buffer.
  auto block = [&](auto bufc, int t0) {
    const uint32_t kb = lds_addr(k8(bufc)), vb = lds_addr(v8(bufc));
#pragma unroll
    for (int e = 0; e < HPW; ++e) {
      u32x4_t kv8[2][kHk];
      u32x2_t vv8[8];
      uint32_t ka[kHk];
#pragma unroll
      for (int hk = 0; hk < kHk; ++hk) ka[hk] = kb + ko[e][hk];
      q8_reads<D, RL>(ka, vb + vo[e], kv8, vv8);
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
        for (int ks = 0; ks < kKs; ++ks) sacc[tb] = mfma16x16x32(as_bf16x8(kv[tb][ks]), qop[e][ks], sacc[tb]);
      const bf16x8_t pb = softmax_block<8>(sacc, oacc[e], m[e], l[e], t0, t_end, grp4, c);
#pragma unroll
      for (int j = 0; j < 8; ++j) oacc[e][j] = mfma16x16x32(transpose_pick(vv, j), pb, oacc[e][j]);
      __builtin_amdgcn_sched_barrier(0);             // one head's fragments live at a time
    }
  };

  wait_vmem_n<0>();        // q, scales and the page numbers are in: from here on only block copies are outstanding
  auto copy_i = [&](auto i, int t0) { copy8(k8(i), v8(i), t0); };
  auto read_i = [&](auto) {};
  block_ring<NB, 2 * kCopies>(t_begin, t_end, copy_i, read_i, block);

  // partial results: O / l and lse for this chunk (lane holds head n, dims 8*(4*grp4 + r) + j)
  float lt[HPW];
#pragma unroll
  for (int e = 0; e < HPW; ++e) {
    lt[e] = l[e] + xor_lanes(l[e], 16);
    lt[e] += xor_lanes(lt[e], 32);
  }
  if (!hv || 4 * grp4 >= D / 8) return;
#pragma unroll
  for (int e = 0; e < HPW; ++e) {
    const int64_t slot = (int64_t(b) * a.hq + (g0 + e) * G + n) * a.n_chunks + chunk;
    const float inv = 1.f / lt[e];
    float* wo = a.ws_o + slot * D;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int d0 = 8 * (4 * grp4 + r);
      const f32x4_t* vs = reinterpret_cast<const f32x4_t*>(a.v_scale + (g0 + e) * D + d0);   // per-channel V scale
      const f32x4_t lo = f32x4_t{oacc[e][0][r], oacc[e][1][r], oacc[e][2][r], oacc[e][3][r]} * inv * vs[0];
      const f32x4_t hi = f32x4_t{oacc[e][4][r], oacc[e][5][r], oacc[e][6][r], oacc[e][7][r]} * inv * vs[1];
      *reinterpret_cast<f32x4_t*>(wo + d0) = lo;
      *reinterpret_cast<f32x4_t*>(wo + d0 + 4) = hi;
    }
    if (grp4 == 0) a.ws_lse[slot] = m[e] * a.scale + logf(lt[e]);
  }
}

// Merge the chunks of one (sequence, query head): M = max lse_c, w_c = exp(lse_c - M),
// O = sum_c w_c O_c / sum_c w_c, lse = M + ln sum_c w_c. A sequence of length 0 gets O = 0, lse = -inf.
// One thread per head dimension (blockDim.x = D).
__global__ __launch_bounds__(128) void decode_combine_kernel(const float* __restrict__ ws_o,
    const float* __restrict__ ws_lse, const int32_t* __restrict__ seq_lens, uint16_t* __restrict__ o,
    float* __restrict__ lse, int hq, int D, int n_chunks, int chunk, int max_len, int cap) {
  const int h = blockIdx.x, b = blockIdx.y, d = threadIdx.x;
  const int L = clamp_len(seq_lens[b], max_len, cap);
  const int nc = (L + chunk - 1) / chunk;
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
template <class Kernel>
void launch_grid(Kernel kernel, DecodeArgs a, int hpw, hipStream_t stream) {
  a.n_hg = a.hkv / hpw;
  // every possible unit, rounded up to whole groups of 8 x n_hg workgroups (the XCD-grouped order maps those onto
  // units bijectively; the extra workgroups exit)
  const unsigned group = 8u * unsigned(a.n_hg);
  const unsigned units = unsigned(a.n_hg) * unsigned(a.n_chunks) * unsigned(a.batch);
  kernel<<<dim3((units + group - 1) / group * group), dim3(64), 0, stream>>>(a);
}

// One KV head per wave for both 8-bit kinds (128- or 64-byte rows), in the XCD-grouped dense order. Measured on the
// 64-sequence workload at head dim 128 (64): in grid order FP8 streamed 4.95 (2.94) TB/s with one head per wave and
// 5.10 (3.59) with two (four), which made rows of 256 bytes; with the head groups of a chunk on one XCD, one head
// per wave streams 5.62 (4.02) TB/s for FP8 and 5.25 (3.71) for int8. The multi-head instances
// (decode_paged_q8_kernel<KV, D, HPW > 1>) remain selectable for other layouts.
#ifndef ATTN_DECODE_Q8_HPW
#define ATTN_DECODE_Q8_HPW 1
#endif
template <int KV, int D>
void launch_q8(const DecodeArgs& a, hipStream_t stream) {
  constexpr int H = KV == kKvInt8 ? 1 : ATTN_DECODE_Q8_HPW;
  if constexpr (H > 1 && H * D >= 256) {
    if (a.hkv % H == 0) return launch_grid(decode_paged_q8_kernel<KV, D, H>, a, H, stream);
  }
  launch_grid(decode_paged_q8_kernel<KV, D, 1>, a, 1, stream);
}

template <int D>
void launch_split(int kind, const DecodeArgs& a, hipStream_t stream) {
  if (kind == kKvFp8) launch_q8<kKvFp8, D>(a, stream);
  else if (kind == kKvInt8) launch_q8<kKvInt8, D>(a, stream);
  else launch_grid(decode_paged_lds_kernel<D>, a, 1, stream);
}

hipError_t launch_decode(int kind, const void* q, const void* k_cache, const void* v_cache, const float* k_scale,
                         const float* v_scale, const int32_t* block_table, const int32_t* seq_lens, void* o, float* lse,
                         int batch, int hq, int hkv, int head_dim, int page_size, int max_pages_per_seq,
                         int64_t num_pages, int max_seqlen_kv, float scale, void* workspace, hipStream_t stream) {
  // Keys per split: a chunk's page numbers are held one per lane (at most 64 pages). The workspace is sized for
  // kDecodeChunk, the smallest chunk, so every choice fits it.
  const int want = kind == kKvBf16 ? ATTN_DECODE_CHUNK_BF16 : ATTN_DECODE_CHUNK_Q8;
  const int chunk = max(kDecodeChunk, min(want, 64 * page_size));
  const int n_chunks = max(1, (max_seqlen_kv + chunk - 1) / chunk);
  const size_t slots = size_t(batch) * size_t(hq) * size_t(n_chunks);
  if (size_t(hkv) * size_t(n_chunks) * size_t(batch) + 8 * size_t(hkv) > size_t(INT32_MAX)) return hipErrorInvalidValue;
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
  a.chunk = chunk;
  a.num_pages = num_pages; a.scale = scale;
  a.batch = batch;
  if (max_seqlen_kv > 0) {
    if (head_dim == 64) launch_split<64>(kind, a, stream);
    else launch_split<128>(kind, a, stream);
  }
  decode_combine_kernel<<<dim3(unsigned(hq), unsigned(batch)), dim3(unsigned(head_dim)), 0, stream>>>(
      a.ws_o, a.ws_lse, seq_lens, static_cast<uint16_t*>(o), lse, hq, head_dim, n_chunks, chunk, max_seqlen_kv,
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
