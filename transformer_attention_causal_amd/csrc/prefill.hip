// prefill.hip — exact causal (or full) grouped-query attention over whole sequences.
//
// (Attention notes, makinaruto.github.io, posts/nlp/llm_learning/attention: "FlashAttention" — all intermediate
//  work stays in fast on-chip memory and HBM is read and written once; "online-softmax" — per block, the block max
//  m_c and block exp-sum l_c update the running m and l, m_new = max(m_old, m_c), l_new = l_old e^(m_old - m_new)
//  + l_c e^(m_c - m_new); "Group-Query Attention" derivation table — consecutive query heads share a KV head.)
//
// bf16 path, one workgroup = 12 waves (one per CU, three per SIMD: registers capped at 168 per lane):
//   * Work unit: 3 blocks of 32 query positions x 4 query heads of one KV group ("heads mode", when the group
//     size is a multiple of 4: each K/V tile in LDS feeds 384 query rows), or 12 consecutive 32-position blocks of
//     one query head ("positions mode", any other group size). Each wave owns 32 queries of one head. The chunked
//     prefill from a paged cache uses 6 blocks x 2 heads in heads mode. Units are dealt heaviest first, in a snake
//     order over the shader engines (snake_id).
//   * K and V tiles of 64 keys x D are copied straight from global memory into LDS (buffer loads with the LDS
//     bit, 16 bytes per lane, no register staging), double-buffered, one barrier per tile. LDS rows are unpadded;
//     their 16-byte chunks are XOR-swizzled by a key of the row index (swz_key) that makes both LDS read patterns
//     below conflict-free on the 64-bank LDS. Three waves per SIMD let one wave's MFMAs overlap another's
//     softmax and LDS waits; sharing each tile over 12 waves keeps the L2-to-LDS copy rate well below its limit.
//   * Scores are formed transposed, S^T = K Q^T, on v_mfma_f32_32x32x16_bf16: K fragments come from LDS (16-byte
//     reads), Q^T stays in registers for the whole kernel. In the S^T accumulator each lane holds ONE query
//     (lane % 32) and 16 keys, so the row max and row sum need one cross-lane exchange (lanes l and l ^ 32), and
//     the output rescale by alpha = exp(m_old - m_new) is a per-lane scalar.
//   * P^T (bf16) is taken directly from the S^T registers as the B operand of O^T = V^T P^T: the 16 keys a lane
//     holds are used as its 8+8 contraction slots, and V^T fragments are read with the matching key order by
//     ds_read_b64_tr_b16 from the row-major V tile. P never leaves registers.
//   * exp is exp2 with scale*log2(e) folded into one FMA. Tiles fully above the diagonal are skipped; only tiles
//     that cross the diagonal or the ragged end are masked. Heaviest query blocks are launched first.
//   * Optionally Q is rotated as it is loaded (RoPE fused into the prefill, from a cos/sin table by position), so
//     the separate rotation pass over Q disappears; keys are rotated beforehand, since every workgroup of a KV
//     head reads them.
// fp32 path (correctness workload, head_dim 64/128): plain VALU, K/V tiles of 32 keys in LDS, fp32 throughout.
#include <type_traits>

#include "device.h"
#include "kernels.h"

namespace attn {
namespace {

// Waves per workgroup: in heads mode 4 heads x (kWaves/4) blocks of 32 positions share each K/V tile in LDS.
#ifndef ATTN_PREFILL_WAVES
#define ATTN_PREFILL_WAVES 12
#endif
constexpr int kWaves = ATTN_PREFILL_WAVES;
// Query heads per workgroup in heads mode (they share one KV head; the group size must be a multiple).
#ifndef ATTN_PREFILL_HEADS
#define ATTN_PREFILL_HEADS 4
#endif
constexpr int kHeads = ATTN_PREFILL_HEADS;
static_assert(kWaves % kHeads == 0, "waves split into heads x position blocks");
// The chunked prefill from a paged cache takes 2 heads x 6 position blocks: its units differ in cost by orders of
// magnitude, and the taller units balance better over the shader engines (measured 2% faster on four 2048-token
// chunks; the plain prefill is the same speed either way).
#ifndef ATTN_PREFILL_HEADS_PAGED
#define ATTN_PREFILL_HEADS_PAGED 2
#endif
constexpr int kHeadsPaged = ATTN_PREFILL_HEADS_PAGED;
static_assert(kWaves % kHeadsPaged == 0, "waves split into heads x position blocks");
constexpr int kThreads = 64 * kWaves;
// Keys per compute tile (32 or 64).
#ifndef ATTN_PREFILL_BN
#define ATTN_PREFILL_BN 64
#endif
constexpr int kBN = ATTN_PREFILL_BN;
constexpr int kKB2 = kBN / 32;   // 32-key blocks of S^T per tile
constexpr int kKB = kBN / 16;    // 16-key contraction blocks of P.V per tile
static_assert(kBN == 32 || kBN == 64, "tile of 32 or 64 keys");

// Build-time tuning: 32-query blocks per wave, and the minimum waves per SIMD the register allocation must
// allow (3 -> at most 168 registers per lane).
#ifndef ATTN_PREFILL_QB
#define ATTN_PREFILL_QB 1
#endif
// Software-pipelining depth of the LDS fragment reads in the tile products (fragments read ahead of the MFMA that
// uses them): K fragments for S^T, pairs of V^T fragment reads for O^T. Measured on the 8192-token GQA prefill:
// the compiler's own order keeps one K and one V^T fragment in flight (0.975 ms); 3 and 2 give 0.951 ms; deeper
// runs out of the 168 registers that three waves per SIMD allow.
#ifndef ATTN_PREFILL_VPRE
#define ATTN_PREFILL_VPRE 2
#endif
#ifndef ATTN_PREFILL_KPRE
#define ATTN_PREFILL_KPRE 3
#endif
// The chunked kernel keeps two K fragments in flight: its tile loop holds a few more registers (the next block-table
// entry), and with three the compiler fell back to one.
#ifndef ATTN_PREFILL_KPRE_PAGED
#define ATTN_PREFILL_KPRE_PAGED 2
#endif
#ifndef ATTN_PREFILL_MIN_WAVES_PER_SIMD
#define ATTN_PREFILL_MIN_WAVES_PER_SIMD 3
#endif

template <int D>
struct Tile {
  static constexpr int kChunks = D / 8;                  // 16-byte chunks per row
  static constexpr int kRowBytes = D * 2;
  static constexpr int kBytes = kBN * kRowBytes;         // one K or V tile
};

struct PrefillArgs {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  uint16_t* o;
  float* lse;
  int batch, seqlen, hq, hkv;
  float scale;
  int causal;
  int heads_mode;    // 1: H heads x (kWaves/H)*32 positions per workgroup (H = kHeads, or kHeadsPaged for the
                     // chunked kernel); 0: 1 head x kWaves*32 positions
  int n_pblk;        // position blocks per (batch, head group)
  int n_hgrp;        // head groups: hq/4 in heads mode, hq in positions mode
  // Chunked prefill from a paged cache (the PAGED kernel): the queries of sequence b are rows cu_new[b] ..
  // cu_new[b+1]-1 of q and o, query i sits at absolute position ctx_lens[b] + i, and the keys are the first
  // ctx_lens[b] + n_b tokens of the paged caches [num_pages, page_size, hkv, D]; lse is [hq, total rows].
  const int32_t* cu_new;
  const int32_t* ctx_lens;
  const int32_t* table;
  int page_shift, max_pages, total_new;
  int64_t num_pages;
  // Local + global mask (the WIN kernel): key j is visible to query i iff j <= i and (i - j < window, or
  // j < n_lead, or anchor_stride > 0 and j % anchor_stride == 0).
  int window, n_lead, anchor_stride;
  // RoPE of Q fused into its load: rope_cs is a [rope_len, D/2] table of (cos, sin) fp32 by integer position, and
  // the position of query row r is q_pos[r] (NULL: its position in the sequence, koff + i), clamped into
  // [0, rope_len). No rotation when rope_cs is NULL.
  const float2* rope_cs;
  const int32_t* q_pos;
  int rope_len, rope_inter;
};

// RoPE of the resident Q^T operands (DeepSeek 32K to 256K long context, tqpw.cn, section 2.1: pair i rotated by
// the angle position * theta^(-2i/d); section 2.5: cos and sin read from a table indexed by integer positions).
// The rope kernel's table values and arithmetic (fp32 FMA, bf16 rounding to nearest even), so a query rotated here
// is bit-identical to one rotated in place by the rope kernel first. A lane holds dims 16*ks + 8*lg + s: a
// half-split pair (i, i + D/2) lies in k-steps ks and ks + KS/2 of the same lane, an interleaved pair (2i, 2i+1)
// in slots s and s + 1 of one register. The table rows are loaded together with Q (load) and applied after the
// first tile copy is issued (apply), so their latency overlaps that copy.
template <int D, int QB>
struct RopeQ {
  static constexpr int KS = D / 16;
  f32x4_t t[QB][2 * KS];   // the lane's (cos, sin) pairs, in the order apply() consumes them
  int pos[QB];             // table row of each query

  // Positions first (an explicit position list is read before the Q loads are issued, so waiting for it does not
  // wait for them), then the table rows.
  __device__ __forceinline__ void positions(const PrefillArgs& a, int64_t qrow0, int qpos0, int koff, int S,
                                            int lq) {
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      const int qi = max(0, min(qpos0 + 32 * qb + lq, S - 1));
      pos[qb] = a.q_pos ? a.q_pos[qrow0 + qi] : koff + qi;
    }
  }

  __device__ __forceinline__ void load(const PrefillArgs& a, int lg) {
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      const int p = min(max(pos[qb], 0), a.rope_len - 1);
      const float* cs = reinterpret_cast<const float*>(a.rope_cs + int64_t(p) * (D / 2));
      if (a.rope_inter) {          // pairs 8*ks + 4*lg + j, j = 0..3
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
#pragma unroll
          for (int u = 0; u < 2; ++u) t[qb][2 * ks + u] = *reinterpret_cast<const f32x4_t*>(cs + 16 * ks + 8 * lg + 4 * u);
      } else {                     // pairs 16*ks + 8*lg + s, s = 0..7, ks < KS/2
#pragma unroll
        for (int ks = 0; ks < KS / 2; ++ks)
#pragma unroll
          for (int u = 0; u < 4; ++u) t[qb][4 * ks + u] = *reinterpret_cast<const f32x4_t*>(cs + 32 * ks + 16 * lg + 4 * u);
      }
    }
  }

  __device__ __forceinline__ void apply(bf16x8_t (&qop)[QB][KS], int inter) const {
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      if (inter) {
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
          u32x4_t w = __builtin_bit_cast(u32x4_t, qop[qb][ks]);
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const f32x4_t& tv = t[qb][2 * ks + (j >> 1)];
            const float c = tv[2 * (j & 1)], sn = tv[2 * (j & 1) + 1];
            const float x0 = bf16lo_to_f32(w[j]), x1 = bf16hi_to_f32(w[j]);
            w[j] = pack_bf16x2(fmaf(x0, c, -x1 * sn), fmaf(x0, sn, x1 * c));
          }
          qop[qb][ks] = as_bf16x8(w);
        }
      } else {
#pragma unroll
        for (int ks = 0; ks < KS / 2; ++ks) {
          u32x4_t wa = __builtin_bit_cast(u32x4_t, qop[qb][ks]);
          u32x4_t wb = __builtin_bit_cast(u32x4_t, qop[qb][ks + KS / 2]);
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const f32x4_t& tv = t[qb][4 * ks + j];              // pairs 2j and 2j + 1
            const float c0 = tv[0], s0 = tv[1], c1 = tv[2], s1 = tv[3];
            const float a0 = bf16lo_to_f32(wa[j]), a1 = bf16hi_to_f32(wa[j]);
            const float b0 = bf16lo_to_f32(wb[j]), b1 = bf16hi_to_f32(wb[j]);
            wa[j] = pack_bf16x2(fmaf(a0, c0, -b0 * s0), fmaf(a1, c1, -b1 * s1));
            wb[j] = pack_bf16x2(fmaf(a0, s0, b0 * c0), fmaf(a1, s1, b1 * c1));
          }
          qop[qb][ks] = as_bf16x8(wa);
          qop[qb][ks + KS / 2] = as_bf16x8(wb);
        }
      }
    }
  }
};

// LDS swizzle: 16-byte chunk c of tile row r is stored at chunk position c ^ swz_key(r). LDS has 64 four-byte
// banks (256 bytes per cycle). Measured on gfx950: ds_read_b128 serves 16 lanes per cycle, in the lane sets
// {0-7, 24-31}, {8-15, 16-23}, {32-39, 56-63}, {40-47, 48-55}; ds_read_b64(_tr_b16) serves 32 consecutive lanes
// per cycle. A set is conflict-free when its lanes hit distinct 16-byte (8-byte) slots modulo 256 bytes.
//   K reads (A operand of the 32x32x16 MFMA): lane l reads row l%32, so each b128 set holds rows {0-7, 24-31} or
//     {8-15, 16-23} at one logical chunk: the key must be distinct over each of those row sets.
//   V^T reads (ds_read_b64_tr_b16): 32 lanes read 4 consecutive rows (aligned to 4) x 4 consecutive chunks: the
//     key must send the 4 rows to 4 different groups of 4 chunk slots.
// 256-byte rows (head_dim 128): key = (r%4)*4 + (r/4)%4. 128-byte rows (head_dim 64; two rows per 256 bytes, so
// row parity already separates half the slots): key = ((r/2)%2)*4 + (r/4)%4. Both depend on r mod 16 only.
template <int D>
__device__ __forceinline__ int swz_key(int r) {
  if (D == 128) return ((r & 3) << 2) | ((r >> 2) & 3);
  return (((r >> 1) & 1) << 2) | ((r >> 2) & 3);
}

// Per-lane byte offsets of the direct-to-LDS copy of a ROWS-row tile by NW waves. Wave instruction i of wave w
// fills the 64 LDS slots of block i*NW + w; slot -> (row, physical chunk) -> logical chunk (physical ^
// swz_key(row)). The offsets are relative to row 0 of the tile and the same for K and V (same layout).
template <int D, int NW, int ROWS>
struct TileCopy {
  static constexpr int kBlocks = ROWS * Tile<D>::kChunks / 64;   // 64-slot blocks per tile
  static constexpr int kLoads = (kBlocks + NW - 1) / NW;         // per wave (the last round may be partial)
  static_assert(ROWS * Tile<D>::kChunks % 64 == 0, "tile must split into 64-slot blocks");
  uint32_t off[kLoads];

  // Tile row r is source row r * step (step > 1: a strided tile, e.g. every step-th key).
  __device__ __forceinline__ void init(int hkv, int g, int wave, int lane, int step = 1) {
#pragma unroll
    for (int i = 0; i < kLoads; ++i) {
      const int slot = (i * NW + wave) * 64 + lane;
      const int row = slot / Tile<D>::kChunks;
      const int lchunk = (slot % Tile<D>::kChunks) ^ swz_key<D>(row);
      off[i] = uint32_t(((row * step * hkv + g) * D + lchunk * 8) * 2);
    }
  }

  // Copy `rows` tile rows starting at `base` (row 0 of the tile, head 0) into `dst`. The buffer resource spans
  // exactly those rows; the others read as zeros (measured: an out-of-range lane of a buffer load-to-LDS writes 0),
  // which are finite, so their masked scores and P = 0 stay exact. Every wave issues kLoads instructions: when
  // the blocks do not split evenly, a wave's surplus instruction reads out of range into the 1 KiB `spare` LDS
  // block (zeros, no memory access), so the copies are never skipped by a branch and the compiler counts the
  // loads in flight exactly (with a skipped copy possible it waited for every load before the first use of
  // registers loaded ahead of the copy).
  __device__ __forceinline__ void issue(uint16_t* dst, const uint16_t* base, int rows, int hkv, int wave,
                                        uint16_t* spare, int step = 1) const {
    const int nr = max(0, min(ROWS, rows));
    const buf_rsrc_t rs = make_buf_rsrc(base, uint32_t(nr > 0 ? ((nr - 1) * step + 1) * hkv * D * 2 : 0));
#pragma unroll
    for (int i = 0; i < kLoads; ++i) {
      if (kBlocks % NW == 0) {
        load_lds16(rs, off[i], dst + (i * NW + wave) * 512);
      } else {
        const bool ok = i * NW + wave < kBlocks;       // wave-uniform
        load_lds16(rs, ok ? off[i] : 0x80000000u, ok ? dst + (i * NW + wave) * 512 : spare);
      }
    }
  }
};

// 64-key sub-tiles per LDS tile (one barrier and one copy round per tile).
#ifndef ATTN_PREFILL_SUB
#define ATTN_PREFILL_SUB 1
#endif
constexpr int kSub = ATTN_PREFILL_SUB;
constexpr int kTileKeys = kSub * kBN;

// ---- chunked prefill schedule. Work unit (b, p) of a sequence with S_b new tokens on ctx_b cached ones takes
// queries p*span .. min(S_b, (p+1)*span) - 1 and reads keys 0 .. kend - 1, kend = ctx_b + min(S_b, (p+1)*span):
// its cost is proportional to kend, and the contexts (device data) can differ by orders of magnitude between
// sequences. Rank r picks the unit with the r-th largest kend (ties: lower b first), so the heaviest units start
// first and the light ones fill the tail. Every wave computes the same answer from wave-wide reductions over the
// batch (64 sequences per step); no synchronisation, no workspace.
__device__ __forceinline__ int wave_max_i(int v) {
#pragma unroll
  for (int o = 32; o; o >>= 1) v = max(v, __shfl_xor(v, o, 64));
  return v;
}

__device__ bool pick_chunked_unit(const PrefillArgs& a, int span, int r, int& b_out, int& p_out) {
  const int lane = threadIdx.x & 63;
  // Up to 64 sequences: lane b reads sequence b's sizes once, and the search below runs on registers (reading
  // them again on every step put about 15 dependent memory round trips before each workgroup's first tile).
  const bool cached = a.batch <= 64;
  int S_l = 0, ctx_l = 0;
  if (cached && lane < a.batch) {
    S_l = min(a.cu_new[lane + 1] - a.cu_new[lane], a.seqlen);
    ctx_l = max(0, a.ctx_lens[lane]);
  }
  auto seq = [&](int b, int& S, int& ctx) {   // b = lane + 64 * k
    if (cached) {
      S = S_l; ctx = ctx_l;
    } else {
      S = min(a.cu_new[b + 1] - a.cu_new[b], a.seqlen);
      ctx = max(0, a.ctx_lens[b]);
    }
  };
  // Units are shifted back by sh = the excess of nb whole spans over S, rounded down to 32 queries (see the
  // kernel), so unit p ends at key ctx + (p+1)*span - sh, the last at ctx + S.
  auto shift = [&](int S) { return ((((S + span - 1) / span) * span - S) / 32) * 32; };
  // Wave-wide sum of per-lane counts below 2^nbits, bit by bit with ballots: scalar population counts instead of
  // a chain of cross-lane shuffles through LDS (the search below takes about 16 sums).
  const int nbits = 32 - __clz(max(1, ((a.batch + 63) / 64) * ((a.seqlen + span - 1) / span)));
  auto wave_count = [&](int c) {
    int total = 0;
    for (int j = 0; j < nbits; ++j) total += __popcll(__ballot((c >> j) & 1)) << j;
    return total;
  };
  // number of units with kend > X
  auto count_above = [&](int X) {
    int c = 0;
    for (int b = lane; b < a.batch; b += 64) {
      int S, ctx;
      seq(b, S, ctx);
      if (S > 0 && ctx + S > X) {
        const int nb = (S + span - 1) / span;
        const int y = X - ctx + shift(S);
        c += y < 0 ? nb : max(1, nb - y / span);
      }
    }
    return wave_count(c);
  };
  int hi = 0;
  for (int b = lane; b < a.batch; b += 64) {
    int S, ctx;
    seq(b, S, ctx);
    if (S > 0) hi = max(hi, ctx + S);
  }
  hi = wave_max_i(hi);
  if (r >= count_above(-1)) return false;
  int lo = 0;                                    // smallest X with count_above(X) <= r is the unit's kend
  while (lo < hi) {
    const int mid = lo + (hi - lo) / 2;
    if (count_above(mid) <= r) hi = mid; else lo = mid + 1;
  }
  const int K = lo;
  int m = r - count_above(K);                    // among the units with kend == K (one per sequence at most)
  for (int b0 = 0; b0 < a.batch; b0 += 64) {
    const int b = b0 + lane;
    bool has = false;
    int p = 0;
    if (b < a.batch) {
      int S, ctx;
      seq(b, S, ctx);
      const int y = K - ctx + shift(S);
      has = S > 0 && ctx < K && K <= ctx + S && (K == ctx + S || y % span == 0);
      p = K == ctx + S ? (S + span - 1) / span - 1 : y / span - 1;
    }
    uint64_t mask = __ballot(has);
    const int cnt = __popcll(mask);
    if (m < cnt) {
      for (int i = 0; i < m; ++i) mask &= mask - 1;
      const int src = __builtin_ctzll(mask);
      b_out = __builtin_amdgcn_readfirstlane(b0 + src);
      p_out = __builtin_amdgcn_readfirstlane(__shfl(p, src, 64));
      return true;
    }
    m -= cnt;
  }
  return false;                                  // unreachable for consistent inputs
}

// The WIN kernel (local + global mask, "DeepSeek 32K to 256K long context", tqpw.cn, section 4.1: a sliding window
// for the local neighbourhood plus a few global tokens such as a leading token and periodic anchors) visits, per
// workgroup, three disjoint kinds of key tiles, so the work is O(window + globals) per query instead of O(i):
//   lead   contiguous tiles over keys j < n_lead that fall outside some query's window;
//   anchor strided tiles over the anchors j = k * anchor_stride >= n_lead outside some query's window (each tile
//          row is every anchor_stride-th key, copied with the same direct-to-LDS copy and a strided offset);
//   window contiguous tiles over keys within window of the workgroup's queries.
// Per query the three sets are disjoint (lead and anchor keys count only when outside the query's window), and
// their union is exactly the visible set.
constexpr int kPhaseWin = 0, kPhaseLead = 1, kPhaseAnchor = 2;

// Work units go to workgroup ids heaviest first, with the n_hgrp head groups of a unit on consecutive ids. The
// hardware deals a launch's workgroups to its 32 shader engines (8 compute units each) round-robin, workgroup i to
// engine i mod 32 (measured), so an engine runs every 32nd unit of that order and the engines that take the first
// unit of each group of 32 would always hold its heaviest one. Odd groups of 32 ids take their units in reverse
// order (whole units; a head group stays on the same engine), which evens out the engines' totals: the chunked
// prefill's last engine finished 3% earlier in a replay of measured unit times. Outputs do not depend on the order.
__device__ __forceinline__ int snake_id(int id, int n, int n_hgrp) {
  const int g = id >> 5;
  if (n_hgrp <= 0 || 32 % n_hgrp != 0 || (g & 1) == 0 || 32 * g + 32 > n) return id;
  const int r = id & 31, per = 32 / n_hgrp;            // units per group of 32 ids
  return 32 * g + (per - 1 - r / n_hgrp) * n_hgrp + r % n_hgrp;
}

template <int D, int QB, bool PAGED, bool WIN = false>
__global__ __launch_bounds__(kThreads, ATTN_PREFILL_MIN_WAVES_PER_SIMD) void prefill_bf16_kernel(PrefillArgs a) {
  static_assert(!(WIN && (PAGED || kSub != 1)), "the local + global mask is for contiguous prefill, 64-key tiles");
  constexpr int kH = PAGED ? kHeadsPaged : kHeads;     // heads per workgroup in heads mode
  constexpr int kPB = kWaves / kH;                     // 32-position blocks per workgroup in heads mode
  constexpr int QW = 32 * QB;
  constexpr int KS = D / 16;   // k-steps of the QK^T contraction
  constexpr int DB = D / 32;   // 32-row blocks of O^T
  // [buffer][K, V]; buffers 0 and 1 hold the tiles, and after the last tile the whole array stages the output rows
  // (kWaves * QW rows of D, hence a third buffer when that is larger than two; the chunked kernel stores directly)
  constexpr int kStageBuf = (kWaves * QW + 2 * kTileKeys - 1) / (2 * kTileKeys);
  constexpr int kNBuf = !PAGED && kStageBuf > 2 ? kStageBuf : 2;
  __shared__ __attribute__((aligned(16))) uint16_t lds[kNBuf][2][kTileKeys * D];
  __shared__ __attribute__((aligned(16))) uint16_t lds_spare[512];             // target of surplus copies

  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // wave-uniform (scalar register)
  const int lane = threadIdx.x & 63;
  const int lq = lane & 31, lg = lane >> 5;
  // ---- work unit (heaviest position blocks first; consecutive ids share a position block)
  // (chunked prefill: heaviest units first by the device-side ranking above; head groups innermost, so the
  // blocks of one unit land on consecutive XCDs and each XCD keeps to a fixed set of KV heads)
  const int id = snake_id(blockIdx.x, gridDim.x, a.n_hgrp);
  int pblk, b, hgrp;
  if constexpr (PAGED) {
    hgrp = id % a.n_hgrp;
    const int span = a.heads_mode ? kPB * QW : kWaves * QW;
    int bb, pp;
    if (!pick_chunked_unit(a, span, id / a.n_hgrp, bb, pp)) return;
    // one scalar for both (measured: keeps the D=128 kernel within its register budget, no spills)
    const int code = __builtin_amdgcn_readfirstlane(bb * a.n_pblk + pp);
    b = code / a.n_pblk; pblk = code % a.n_pblk;
  } else {
    const int per_slice = a.batch * a.n_hgrp;
    pblk = a.n_pblk - 1 - id / per_slice;
    const int rest = id % per_slice;
    b = rest / a.n_hgrp; hgrp = rest % a.n_hgrp;
  }
  const int grp = a.hq / a.hkv;
  int h, qpos0, wg_pos0, wg_span;
  if (a.heads_mode) {
    h = hgrp * kH + wave % kH; wg_pos0 = pblk * kPB * QW; qpos0 = wg_pos0 + (wave / kH) * QW;
    wg_span = kPB * QW;
  } else {
    h = hgrp; wg_pos0 = pblk * kWaves * QW; qpos0 = wg_pos0 + wave * QW; wg_span = kWaves * QW;
  }
  const int g = h / grp;
  // S queries (positions 0 .. S-1 in this workgroup's numbering) at absolute positions koff .., T keys.
  int S, koff, T;
  int64_t qrow0;                                       // row of query 0 in q and o
  if constexpr (PAGED) {
    const int r0 = a.cu_new[b];
    S = min(a.cu_new[b + 1] - r0, a.seqlen); koff = max(0, a.ctx_lens[b]); T = koff + S; qrow0 = r0;
  } else {
    S = a.seqlen; koff = 0; T = S; qrow0 = int64_t(b) * S;
  }
  if constexpr (!WIN) {
    // The units of a sequence are shifted back so that the one that is partly outside the queries is its first,
    // the cheapest, rather than its last, the dearest (whole 32-query blocks: a wave's queries are either all at
    // positions >= 0 or all before 0). Each wave keeps its own key range, so the results are unchanged.
    const int sh = ((((S + wg_span - 1) / wg_span) * wg_span - S) / QW) * QW;
    wg_pos0 -= sh;
    qpos0 -= sh;
  }
  if (wg_pos0 >= S) return;                            // uniform: a block past this sequence's queries
  const int kend_wg = a.causal ? min(T, koff + wg_pos0 + wg_span) : T;
  // a wave whose queries all lie before position 0 has none and computes no tile
  const int kend_w = qpos0 + QW <= 0 ? 0 : a.causal ? min(T, koff + qpos0 + QW) : T;
  const int ntiles = (kend_wg + kTileKeys - 1) / kTileKeys;
  const float c = a.scale * kLog2e;

  // Paged: the block-table entry of a tile is read one tile ahead of its copy, by a vector load that the loop's
  // wait for the tile copies also covers, so no table-load latency sits between a barrier and the next copy
  // (measured: a scalar load there cost about 6% of the chunked prefill). Entries past max_pages read as 0 and
  // are replaced by -1 (no page) at use.
  buf_rsrc_t trs = {0, 0, 0, 0};
  if constexpr (PAGED) trs = make_buf_rsrc(a.table + int64_t(b) * a.max_pages, uint32_t(a.max_pages) * 4u);
  auto page_load = [&](int t) -> int {                 // raw table entry of tile t (in flight until the next wait)
    return PAGED ? raw_buffer_load_i32(trs, ((t * kTileKeys) >> a.page_shift) * 4, 0, 0) : 0;
  };
  // (the first entry is read before the Q loads, so no table-load latency sits before the first copy either)
  const int pg0 = page_load(0);
  RopeQ<D, QB> rq;
  const bool rope = !WIN && a.rope_cs != nullptr;     // uniform; the local + global kernel takes no table
  if (rope) rq.positions(a, qrow0, qpos0, koff, S, lq);

  // ---- Q^T operands, resident for the whole kernel: lane holds query (qpos0 + 32*qb + lq), dims 16*ks + 8*lg ..
  bf16x8_t qop[QB][KS];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    const int qpos = qpos0 + 32 * qb + lq;
    const uint16_t* qp = a.q + ((qrow0 + max(0, min(qpos, S - 1))) * a.hq + h) * D + 8 * lg;
    // Loaded unconditionally from the clamped row (loads under a lane mask made the compiler wait for the first of
    // them before issuing the rest). A lane past the last query then holds row S-1's query, sees the same keys
    // (all of them) and so takes the same online-softmax decisions as row S-1's lane in the same wave: the other
    // lanes' results are unchanged, and its own are never stored. Lanes before position 0 fill whole waves, which
    // compute no tile. The local + global mask depends on the position itself, so there such lanes hold zeros.
    const bool qin = qpos >= 0 && qpos < S;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const u32x4_t w = *reinterpret_cast<const u32x4_t*>(qp + 16 * ks);
      qop[qb][ks] = as_bf16x8(!WIN || qin ? w : u32x4_t{0u, 0u, 0u, 0u});
    }
  }
  if (rope) rq.load(a, lg);
  // paged: rotated at once, so the table rows are dead before the tile loop's registers come alive (rotating after
  // the first copy, as the plain kernel does, spills there)
  if (PAGED && rope) rq.apply(qop, a.rope_inter);

  f32x16_t oacc[QB][DB];
  float m[QB], l[QB];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    m[qb] = -INFINITY; l[qb] = 0.f;
#pragma unroll
    for (int db = 0; db < DB; ++db) oacc[qb][db] = f32x16_t{};
  }

  // Lane-fixed swizzled LDS addresses: the row parts that vary in the loops (32*kb2 for K, 16*kb for V) leave the
  // swizzle key unchanged, so every read is one of these bases plus a compile-time immediate.
  constexpr int RB = Tile<D>::kRowBytes;
  uint32_t kbase[KS];                                  // K: row lq (+32*kb2), chunk 2*ks + lg
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) kbase[ks] = uint32_t(lq * RB + 16 * ((2 * ks + lg) ^ swz_key<D>(lq)));
  const int bl = lane & 15, hh = (lane >> 4) & 1;
  const int vrow = 4 * lg + (bl >> 2);                 // V: rows vrow and vrow + 8 (+16*kb),
  uint32_t vlo[DB], vhi[DB];                           //    columns 32*db + 16*hh + 4*(bl&3)
#pragma unroll
  for (int db = 0; db < DB; ++db) {
    const int ch = 4 * db + 2 * hh + ((bl >> 1) & 1);
    vlo[db] = uint32_t(vrow * RB + 16 * (ch ^ swz_key<D>(vrow)) + 8 * (bl & 1));
    vhi[db] = uint32_t((vrow + 8) * RB + 16 * (ch ^ swz_key<D>(vrow + 8)) + 8 * (bl & 1));
  }

  TileCopy<D, kWaves, kTileKeys> cp;
  cp.init(a.hkv, g, wave, lane);
  // Row 0 of the K or V tile at key0 and its valid row count. Paged: tiles never straddle pages (page size a
  // multiple of the tile); a page number outside [0, num_pages), or a tile past the table's max_pages entries,
  // gives no rows (zeros, no memory access).
  auto tile_src = [&](const uint16_t* kv, int key0, int& rows, int page_raw) -> const uint16_t* {
    rows = max(0, min(kTileKeys, T - key0));
    if constexpr (PAGED) {
      const int pi = key0 >> a.page_shift;
      const int page = pi < a.max_pages ? __builtin_amdgcn_readfirstlane(page_raw) : -1;
      if (page < 0 || page >= a.num_pages) rows = 0;
      const int64_t slot0 = (int64_t(max(page, 0)) << a.page_shift) + (key0 & ((1 << a.page_shift) - 1));
      return kv + slot0 * a.hkv * D;
    } else {
      return kv + (int64_t(b) * S + min(key0, T - 1)) * a.hkv * D;
    }
  };
  auto copy_tile = [&](int buf, int t, int page_raw) {
    int rows;
    const uint16_t* kb = tile_src(a.k, t * kTileKeys, rows, page_raw);
    cp.issue(lds[buf][0], kb, rows, a.hkv, wave, lds_spare);
    const uint16_t* vb = tile_src(a.v, t * kTileKeys, rows, page_raw);
    cp.issue(lds[buf][1], vb, rows, a.hkv, wave, lds_spare);
  };

  // One kBN-key tile from LDS buffer BUF (a compile-time constant, so LDS addresses are base + immediate).
  auto tile = [&](auto bufc, auto subc, int key0, int kstep = 1, int phase = kPhaseWin, int nrows = kTileKeys) {
    constexpr int BUF = decltype(bufc)::value;
    constexpr int SUB = decltype(subc)::value;
    const uint16_t* Kt = lds[BUF][0] + SUB * kBN * D;
    const uint16_t* Vt = lds[BUF][1] + SUB * kBN * D;

    // ---- S^T = K Q^T for the tile's keys (32-key blocks kb2)
    f32x16_t sacc[QB][kKB2];
#pragma unroll
    for (int qb = 0; qb < QB; ++qb)
#pragma unroll
      for (int kb2 = 0; kb2 < kKB2; ++kb2) sacc[qb][kb2] = f32x16_t{};
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
#pragma unroll
      for (int kb2 = 0; kb2 < kKB2; ++kb2) {
        // row 32*kb2 + lq, 16-byte chunk 2*ks + lg
        const bf16x8_t ka = as_bf16x8(lds_read16(Kt, kbase[ks] + 32 * kb2 * RB));
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) sacc[qb][kb2] = mfma32x32x16(ka, qop[qb][ks], sacc[qb][kb2]);
      }
    }
    // K fragment reads run kKPre fragments ahead of the products that use them
    constexpr int kKPre = PAGED ? ATTN_PREFILL_KPRE_PAGED : ATTN_PREFILL_KPRE;
    if constexpr (kKPre > 0) {
#pragma unroll
      for (int i = 0; i < kKPre; ++i) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
#pragma unroll
      for (int i = 0; i < KS * kKB2; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, QB, 0);
        if (i + kKPre < KS * kKB2) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      }
    }

    // ---- mask. WIN: tiles not visible in full to every query of the wave, by the phase's rule; otherwise only
    // tiles crossing the diagonal or the ragged end
    bool win_full = false;
    if constexpr (WIN) {
      const int key_max = key0 + kstep * (kBN - 1), qw_max = min(S - 1, qpos0 + QW - 1);
      if (nrows == kBN && key_max <= qpos0 && key_max < T) {
        if (phase == kPhaseWin) win_full = key0 >= qw_max - a.window + 1;
        else if (phase == kPhaseLead) win_full = key_max < a.n_lead && key_max <= qpos0 - a.window;
        else win_full = key_max <= qpos0 - a.window;
      }
    }
    if constexpr (WIN) {
      if (!win_full) {
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) {
        const int qpos = qpos0 + 32 * qb + lq;
#pragma unroll
        for (int kb2 = 0; kb2 < kKB2; ++kb2)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int rel = 32 * kb2 + 8 * (r >> 2) + 4 * lg + (r & 3);
            const int key = key0 + kstep * rel;
            bool vis = key <= qpos && key < T && rel < nrows;
            if (phase == kPhaseWin) vis = vis && qpos - key < a.window;
            else if (phase == kPhaseLead) vis = vis && key < a.n_lead && qpos - key >= a.window;
            else vis = vis && qpos - key >= a.window;
            if (!vis) sacc[qb][kb2][r] = -INFINITY;
          }
      }
      }
    } else if ((a.causal && key0 + kBN - 1 > koff + qpos0) || key0 + kBN > T) {
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) {
        const int qpos = qpos0 + 32 * qb + lq;
#pragma unroll
        for (int kb2 = 0; kb2 < kKB2; ++kb2)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int key = key0 + 32 * kb2 + 8 * (r >> 2) + 4 * lg + (r & 3);
            if ((a.causal && key > koff + qpos) || key >= T) sacc[qb][kb2][r] = -INFINITY;
          }
      }
    }

    // ---- online softmax (one query per lane; partner lane l ^ 32 holds the other 16 keys)
    bf16x8_t pb[QB][kKB];
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      float mx = -INFINITY;
#pragma unroll
      for (int kb2 = 0; kb2 < kKB2; ++kb2)
#pragma unroll
        for (int r = 0; r < 16; ++r) mx = fmaxf(mx, sacc[qb][kb2][r]);
      mx = max_xor32(mx);
      // Lazy rescale: move the reference max (rescaling O and l) only when some lane's max grew by more than
      // 2^kRescaleLog2; otherwise unnormalised P stays below that factor. O / l is unchanged.
      if (__any((mx - m[qb]) * c > kRescaleLog2)) {
        const float m_new = fmaxf(m[qb], mx);
        // (WIN: a query may have seen no visible key yet, m = m_new = -inf; its O and l are still 0)
        const float alpha = (WIN && m_new == -INFINITY) ? 1.f : fast_exp2((m[qb] - m_new) * c);
        l[qb] *= alpha;
#pragma unroll
        for (int db = 0; db < DB; ++db) oacc[qb][db] *= alpha;
        m[qb] = m_new;
      }
      const float mc = (WIN && m[qb] == -INFINITY) ? 0.f : m[qb] * c;   // WIN: P = exp2(-inf) = 0 until then
#pragma unroll
      for (int kb2 = 0; kb2 < kKB2; ++kb2)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const float p = fast_exp2(fmaf(sacc[qb][kb2][r], c, -mc));
          sacc[qb][kb2][r] = p;
          l[qb] += p;
        }
#pragma unroll
      for (int kb = 0; kb < kKB; ++kb) {
        const f32x16_t& s = sacc[qb][kb >> 1];
        const int o8 = 8 * (kb & 1);
        pb[qb][kb] = pack_bf16x8(s[o8], s[o8 + 1], s[o8 + 2], s[o8 + 3], s[o8 + 4], s[o8 + 5], s[o8 + 6], s[o8 + 7]);
      }
    }

    // ---- O^T += V^T P^T: V^T fragments by transposing LDS reads, keys in the same order as the P^T slots
#pragma unroll
    for (int kb = 0; kb < kKB; ++kb) {
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        // rows 16*kb + vrow (+8), columns 32*db + vcol
        const u32x2_t lo = lds_read_tr16(Vt, vlo[db] + 16 * kb * RB);
        const u32x2_t hi = lds_read_tr16(Vt, vhi[db] + 16 * kb * RB);
        const u32x4_t w = {lo[0], lo[1], hi[0], hi[1]};
        const bf16x8_t va = as_bf16x8(w);
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) oacc[qb][db] = mfma32x32x16(va, pb[qb][kb], oacc[qb][db]);
      }
    }
#if ATTN_PREFILL_VPRE > 0
    // V^T fragment reads (two each) run ATTN_PREFILL_VPRE fragments ahead of the products that use them
#pragma unroll
    for (int i = 0; i < ATTN_PREFILL_VPRE; ++i) __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
#pragma unroll
    for (int i = 0; i < kKB * DB; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, QB, 0);
      if (i + ATTN_PREFILL_VPRE < kKB * DB) __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
    }
#endif
  };

  // All sub-tiles of one LDS tile (compile-time buffer and sub-tile indices, so LDS addresses are immediates);
  // sub-tiles entirely above this wave's diagonal are skipped.
  auto tiles = [&](auto bufc, int t) {
    tile(bufc, std::integral_constant<int, 0>{}, t * kTileKeys);
    if (kSub > 1 && t * kTileKeys + kBN < kend_w) tile(bufc, std::integral_constant<int, kSub - 1>{}, t * kTileKeys + kBN);
  };
  static_assert(kSub == 1 || kSub == 2, "one or two sub-tiles per LDS tile");

  if constexpr (WIN) {
    // Tile list of this workgroup (uniform): lead tiles, anchor tiles, window tiles.
    const int W = a.window, G = a.n_lead, P = a.anchor_stride;
    const int qmin = wg_pos0, qmax = min(S, wg_pos0 + wg_span) - 1;
    const int lead_end = min(G, qmax - W + 1);                      // keys [0, lead_end) may need the lead phase
    const int n_lead = lead_end > 0 ? (lead_end + kTileKeys - 1) / kTileKeys : 0;
    int k_lo = 0, n_anchor_keys = 0;
    if (P > 0 && qmax - W >= 0) {
      k_lo = (G + P - 1) / P;
      n_anchor_keys = max(0, (qmax - W) / P - k_lo + 1);
    }
    const int n_anch = (n_anchor_keys + kTileKeys - 1) / kTileKeys;
    const int w_first = max(0, qmin - W + 1) / kTileKeys, w_last = qmax / kTileKeys;
    const int nlist = n_lead + n_anch + (w_last - w_first + 1);
    TileCopy<D, kWaves, kTileKeys> cpa;                             // anchor tiles: every P-th key
    cpa.init(a.hkv, g, wave, lane, max(P, 1));
    // tile u -> (first key, key step, phase, rows)
    auto desc = [&](int u, int& key0, int& step, int& phase, int& rows) {
      if (u < n_lead) {
        key0 = u * kTileKeys; step = 1; phase = kPhaseLead; rows = min(kTileKeys, T - key0);
      } else if (u < n_lead + n_anch) {
        const int k0 = k_lo + (u - n_lead) * kTileKeys;
        key0 = k0 * P; step = P; phase = kPhaseAnchor; rows = min(kTileKeys, k_lo + n_anchor_keys - k0);
      } else {
        key0 = (w_first + u - n_lead - n_anch) * kTileKeys; step = 1; phase = kPhaseWin;
        rows = min(kTileKeys, T - key0);
      }
    };
    auto copy_u = [&](int buf, int u) {
      int key0, step, phase, rows;
      desc(u, key0, step, phase, rows);
      const int64_t row0 = int64_t(b) * S + key0;
      if (step == 1) {
        cp.issue(lds[buf][0], a.k + row0 * a.hkv * D, rows, a.hkv, wave, lds_spare);
        cp.issue(lds[buf][1], a.v + row0 * a.hkv * D, rows, a.hkv, wave, lds_spare);
      } else {
        cpa.issue(lds[buf][0], a.k + row0 * a.hkv * D, rows, a.hkv, wave, lds_spare, step);
        cpa.issue(lds[buf][1], a.v + row0 * a.hkv * D, rows, a.hkv, wave, lds_spare, step);
      }
    };
    // does this wave (queries qpos0 .. qw_max) see any key of tile u?
    const int qw_max = min(S - 1, qpos0 + QW - 1);
    auto run_u = [&](auto bufc, int u) {
      int key0, step, phase, rows;
      desc(u, key0, step, phase, rows);
      bool need;
      if (phase == kPhaseWin) need = key0 <= qw_max && key0 + kTileKeys - 1 >= qpos0 - W + 1;
      else need = key0 <= qw_max - W;                              // some key of the tile outside some window
      if (need && qpos0 < S) tile(bufc, std::integral_constant<int, 0>{}, key0, step, phase, rows);
    };
    copy_u(0, 0);
    if (rope) rq.apply(qop, a.rope_inter);
    for (int u = 0; u < nlist; u += 2) {
      wait_vmem();
      __syncthreads();                                 // tile u visible to all; buffer 1 free
      if (u + 1 < nlist) copy_u(1, u + 1);
      run_u(std::integral_constant<int, 0>{}, u);
      if (u + 1 >= nlist) break;
      wait_vmem();
      __syncthreads();                                 // tile u+1 visible to all; buffer 0 free
      if (u + 2 < nlist) copy_u(0, u + 2);
      run_u(std::integral_constant<int, 1>{}, u + 1);
    }
  } else {
  int pg = pg0;
  copy_tile(0, 0, pg);
  pg = page_load(1);                                   // table entry of the next tile to copy
  if (!PAGED && rope) rq.apply(qop, a.rope_inter);
  // Two tiles per trip so each tile's LDS buffer is a compile-time constant.
  for (int t = 0; t < ntiles; t += 2) {
    wait_vmem();
    __syncthreads();                                   // tile t visible to all; buffer 1 free
    if (t + 1 < ntiles) {
      const int cur = pg;
      pg = page_load(t + 2);
      copy_tile(1, t + 1, cur);
    }
    if (t * kTileKeys < kend_w) tiles(std::integral_constant<int, 0>{}, t);
    if (t + 1 >= ntiles) break;
    wait_vmem();
    __syncthreads();                                   // tile t+1 visible to all; buffer 0 free
    if (t + 2 < ntiles) {
      const int cur = pg;
      pg = page_load(t + 3);
      copy_tile(0, t + 2, cur);
    }
    if ((t + 1) * kTileKeys < kend_w) tiles(std::integral_constant<int, 1>{}, t + 1);
  }
  }

  // ---- epilogue: O = O^T / l (lane holds query lq, dims 32*db + 8*(r/4) + 4*lg + r%4), lse = scale*m + ln l.
  if constexpr (PAGED) {
    // (the chunked kernel stores straight from the accumulators: staging through LDS made it spill registers in
    // its tile loop, and its longer work units spend under 1% of their time here)
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      const int qpos = qpos0 + 32 * qb + lq;
      const float lt = sum_xor32(l[qb]);
      if (qpos < 0 || qpos >= S) continue;
      const float inv = 1.f / lt;
      uint16_t* op = a.o + ((qrow0 + qpos) * a.hq + h) * D + 4 * lg;
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int rq = 0; rq < 4; ++rq) {
          const f32x16_t& x = oacc[qb][db];
          const u32x2_t w = {pack_bf16x2(x[4 * rq] * inv, x[4 * rq + 1] * inv),
                             pack_bf16x2(x[4 * rq + 2] * inv, x[4 * rq + 3] * inv)};
          *reinterpret_cast<u32x2_t*>(op + 32 * db + 8 * rq) = w;
        }
      if (a.lse && lg == 0) a.lse[int64_t(h) * a.total_new + qrow0 + qpos] = m[qb] * a.scale + logf(lt);
    }
    return;
  }
  // O goes through LDS so that each store instruction writes whole rows (a row of D bf16 per query and head is
  // contiguous in o; written straight from the accumulator layout, every instruction writes 16-byte pieces of 32
  // rows, and that epilogue took about 2% of the S=8192 prefill). Staging row r of this wave holds query
  // qpos0 + r; its 16-byte chunk c sits at chunk c ^ key(r), and the two 8-byte halves swap when (r / 16) is odd,
  // so the accumulator-order writes (32 rows at one chunk per instruction half) and the row-order reads are
  // conflict-free.
  constexpr int RB2 = D * 2;                           // bytes per staging row
  constexpr int RPI = 1024 / RB2;                      // rows per 1 KiB store instruction
  auto stg_key = [](int r) { return D == 128 ? (r & 15) : ((r >> 1) & 7); };
  uint16_t* stg = &lds[0][0][0] + wave * QW * D;       // this wave's staging rows (the tile buffers are done)
  __syncthreads();                                     // every wave has finished reading the last tile
  // The lane index passes through an empty asm statement, so the staging addresses are formed here: shared with
  // the loop's lane-fixed addresses they kept registers alive across the tile loop, which then lost its read
  // pipelining.
  int ln = lane;
  asm volatile("" : "+v"(ln));
  const int slq = ln & 31, slg = ln >> 5;
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    const int qpos = qpos0 + 32 * qb + slq;
    const float lt = sum_xor32(l[qb]);
    const float inv = 1.f / lt;
    const int r = 32 * qb + slq;
    const int half = slg ^ ((r >> 4) & 1);
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int rq = 0; rq < 4; ++rq) {
        const f32x16_t& x = oacc[qb][db];
        const u32x2_t w = {pack_bf16x2(x[4 * rq] * inv, x[4 * rq + 1] * inv),
                           pack_bf16x2(x[4 * rq + 2] * inv, x[4 * rq + 3] * inv)};
        const int c = 4 * db + rq;                     // logical 16-byte chunk (dims 8c .. 8c+7)
        *reinterpret_cast<u32x2_t*>(stg + r * D + 8 * (c ^ stg_key(r)) + 4 * half) = w;
      }
    if (a.lse && slg == 0 && qpos >= 0 && qpos < S)
      a.lse[(int64_t(b) * a.hq + h) * S + qpos] = m[qb] * a.scale + logf(lt);
  }
  // (the wave reads back only its own rows: its LDS writes are complete at the reads' wait, no barrier needed)
#pragma unroll
  for (int it = 0; it < QW / RPI; ++it) {
    const int r = it * RPI + ln / (RB2 / 16), c = ln % (RB2 / 16);
    u32x4_t w = *reinterpret_cast<const u32x4_t*>(stg + r * D + 8 * (c ^ stg_key(r)));
    if ((r >> 4) & 1) w = u32x4_t{w[2], w[3], w[0], w[1]};
    const int qpos = qpos0 + r;
    if (qpos >= 0 && qpos < S)
      *reinterpret_cast<u32x4_t*>(a.o + ((qrow0 + qpos) * a.hq + h) * D + 8 * c) = w;
  }
}

// --------------------------------------------------------------------------------------------- fp32 path --
constexpr int kF32Keys = 32;     // keys per LDS tile
constexpr int kF32Queries = 64;  // queries per workgroup

// One workgroup: 64 queries of one head; TPQ = D/16 threads per query, each owning 16 dims of q and O.
template <int D>
__global__ __launch_bounds__(kF32Queries * (D / 16)) void prefill_fp32_kernel(const float* __restrict__ q,
    const float* __restrict__ k, const float* __restrict__ v, float* __restrict__ o, float* __restrict__ lse,
    int S, int hq, int hkv, int causal, float scale) {
  constexpr int TPQ = D / 16;
  constexpr int NT = kF32Queries * TPQ;
  __shared__ float ks[kF32Keys][D];
  __shared__ float vs[kF32Keys][D];
  const int qblk = gridDim.x - 1 - blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const int g = h / (hq / hkv);
  const int tid = threadIdx.x, part = tid % TPQ;
  const int qpos = qblk * kF32Queries + tid / TPQ;
  const float c = scale * kLog2e;
  float qr[16], acc[16];
  for (int i = 0; i < 16; ++i) {
    qr[i] = qpos < S ? q[((int64_t(b) * S + qpos) * hq + h) * D + 16 * part + i] : 0.f;
    acc[i] = 0.f;
  }
  float m = -INFINITY, l = 0.f;
  const int kend = causal ? min(S, (qblk + 1) * kF32Queries) : S;
  for (int key0 = 0; key0 < kend; key0 += kF32Keys) {
    __syncthreads();
    for (int e = tid; e < kF32Keys * D; e += NT) {
      const int r = e / D, d = e % D;
      const int key = min(key0 + r, S - 1);
      const int64_t off = ((int64_t(b) * S + key) * hkv + g) * D + d;
      ks[r][d] = k[off];
      vs[r][d] = v[off];
    }
    __syncthreads();
    float s[kF32Keys];
    float mx = -INFINITY;
    for (int j = 0; j < kF32Keys; ++j) {
      float part_dot = 0.f;
      for (int i = 0; i < 16; ++i) part_dot = fmaf(qr[i], ks[j][16 * part + i], part_dot);
      for (int w = 1; w < TPQ; w <<= 1) part_dot += xor_lanes(part_dot, w);
      const int key = key0 + j;
      s[j] = ((causal && key > qpos) || key >= S) ? -INFINITY : part_dot;
      mx = fmaxf(mx, s[j]);
    }
    const float m_new = fmaxf(m, mx);
    if (m_new == -INFINITY) continue;                 // every key of this tile is masked for this query
    const float alpha = exp2f((m - m_new) * c);
    const float mc = m_new * c;
    l *= alpha;
    for (int i = 0; i < 16; ++i) acc[i] *= alpha;
    for (int j = 0; j < kF32Keys; ++j) {
      const float p = exp2f(fmaf(s[j], c, -mc));
      l += p;
      for (int i = 0; i < 16; ++i) acc[i] = fmaf(p, vs[j][16 * part + i], acc[i]);
    }
    m = m_new;
  }
  if (qpos < S) {
    const float inv = 1.f / l;
    for (int i = 0; i < 16; ++i) o[((int64_t(b) * S + qpos) * hq + h) * D + 16 * part + i] = acc[i] * inv;
    if (lse && part == 0) lse[(int64_t(b) * hq + h) * S + qpos] = m * scale + logf(l);
  }
}

}  // namespace

namespace {
// Shared launch geometry: n_pblk position blocks (heaviest first) x batch x head groups.
PrefillArgs prefill_args(const void* q, const void* k, const void* v, void* o, float* lse, int batch, int max_q,
                         int hq, int hkv, int causal, float scale, int heads = kHeads) {
  PrefillArgs a = {};
  a.q = static_cast<const uint16_t*>(q); a.k = static_cast<const uint16_t*>(k);
  a.v = static_cast<const uint16_t*>(v); a.o = static_cast<uint16_t*>(o); a.lse = lse;
  a.batch = batch; a.seqlen = max_q; a.hq = hq; a.hkv = hkv; a.scale = scale; a.causal = causal;
  const int grp = hq / hkv;
  a.heads_mode = (grp % heads == 0) ? 1 : 0;
  const int span = a.heads_mode ? (kWaves / heads) * 32 : kWaves * 32;
  a.n_pblk = (max_q + span - 1) / span;
  a.n_hgrp = a.heads_mode ? hq / heads : hq;
  return a;
}
}  // namespace

hipError_t launch_prefill_bf16(const void* q, const void* k, const void* v, void* o, float* lse, int batch,
                               int seqlen, int hq, int hkv, int head_dim, int causal, float scale,
                               hipStream_t stream, const void* rope_table, int rope_len, const int32_t* q_positions,
                               int rope_interleaved) {
  PrefillArgs a = prefill_args(q, k, v, o, lse, batch, seqlen, hq, hkv, causal, scale);
  a.rope_cs = static_cast<const float2*>(rope_table); a.rope_len = rope_len; a.q_pos = q_positions;
  a.rope_inter = rope_interleaved;
  const dim3 grid(static_cast<unsigned>(int64_t(a.n_pblk) * batch * a.n_hgrp));
  if (head_dim == 128) prefill_bf16_kernel<128, 1, false><<<grid, dim3(kThreads), 0, stream>>>(a);
  else prefill_bf16_kernel<64, 1, false><<<grid, dim3(kThreads), 0, stream>>>(a);
  return hipGetLastError();
}

hipError_t launch_prefill_window(const void* q, const void* k, const void* v, void* o, float* lse, int batch,
                                 int seqlen, int hq, int hkv, int head_dim, int window, int n_lead, int anchor_stride,
                                 float scale, hipStream_t stream) {
  PrefillArgs a = prefill_args(q, k, v, o, lse, batch, seqlen, hq, hkv, 1, scale);
  a.window = window; a.n_lead = n_lead; a.anchor_stride = anchor_stride;
  const dim3 grid(static_cast<unsigned>(int64_t(a.n_pblk) * batch * a.n_hgrp));
  if (head_dim == 128) prefill_bf16_kernel<128, 1, false, true><<<grid, dim3(kThreads), 0, stream>>>(a);
  else prefill_bf16_kernel<64, 1, false, true><<<grid, dim3(kThreads), 0, stream>>>(a);
  return hipGetLastError();
}

hipError_t launch_prefill_paged(const void* q, const void* k_cache, const void* v_cache, const int32_t* block_table,
                                const int32_t* cu_new, const int32_t* ctx_lens, void* o, float* lse, int batch,
                                int total_new, int max_new, int hq, int hkv, int head_dim, int page_size,
                                int max_pages_per_seq, int64_t num_pages, float scale, hipStream_t stream,
                                const void* rope_table, int rope_len, const int32_t* q_positions,
                                int rope_interleaved) {
  if (max_new <= 0 || total_new <= 0) return hipSuccess;
  PrefillArgs a = prefill_args(q, k_cache, v_cache, o, lse, batch, max_new, hq, hkv, 1, scale, kHeadsPaged);
  a.rope_cs = static_cast<const float2*>(rope_table); a.rope_len = rope_len; a.q_pos = q_positions;
  a.rope_inter = rope_interleaved;
  a.cu_new = cu_new; a.ctx_lens = ctx_lens; a.table = block_table;
  int shift = 0;
  while ((1 << shift) < page_size) ++shift;
  a.page_shift = shift; a.max_pages = max_pages_per_seq; a.total_new = total_new; a.num_pages = num_pages;
  const dim3 grid(static_cast<unsigned>(int64_t(a.n_pblk) * batch * a.n_hgrp));
  if (head_dim == 128) prefill_bf16_kernel<128, 1, true><<<grid, dim3(kThreads), 0, stream>>>(a);
  else prefill_bf16_kernel<64, 1, true><<<grid, dim3(kThreads), 0, stream>>>(a);
  return hipGetLastError();
}

hipError_t launch_prefill_fp32(const void* q, const void* k, const void* v, void* o, float* lse, int batch,
                               int seqlen, int hq, int hkv, int head_dim, int causal, float scale,
                               hipStream_t stream) {
  const dim3 grid(unsigned((seqlen + kF32Queries - 1) / kF32Queries), unsigned(hq), unsigned(batch));
  const float* qf = static_cast<const float*>(q);
  const float* kf = static_cast<const float*>(k);
  const float* vf = static_cast<const float*>(v);
  float* of = static_cast<float*>(o);
  if (head_dim == 128)
    prefill_fp32_kernel<128><<<grid, dim3(kF32Queries * 8), 0, stream>>>(qf, kf, vf, of, lse, seqlen, hq, hkv, causal, scale);
  else
    prefill_fp32_kernel<64><<<grid, dim3(kF32Queries * 4), 0, stream>>>(qf, kf, vf, of, lse, seqlen, hq, hkv, causal, scale);
  return hipGetLastError();
}

}  // namespace attn
