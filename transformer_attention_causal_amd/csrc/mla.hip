// mla.hip — multi-head latent attention decode in the absorbed form.
//
// (DeepSeek-V3 attention guide: einsum vs manual optimisation, dksg.cn: absorb-mode scores are
//  scale * (q_nope . kv_cache + q_pe . pe_cache), two contractions over the latent cache and the shared rope
//  cache; Attention notes, makinaruto.github.io, "Multi-Head Latent Attention": W^K_up folds into the query and
//  W^V_up into W^O, so attention runs in the latent space with O_latent = P . C^KV; "RoPE" compatibility section:
//  the rotated key part is one vector per token shared by every head.)
//
// Every head reads the same 576-wide key row [c_kv ; k_pe] and the same 512-wide value row c_kv, so MLA decode is
// a single-KV-head attention with 128 query rows: the same structure as the prefill kernel with heads in place
// of query positions.
//   * One workgroup = (token split, sequence), 8 waves x 16 heads. Token tiles of 64 rows x 576 are copied
//     straight into LDS (buffer loads with the LDS bit, non-temporal, one latent row or eight rope rows per
//     instruction, spread over the score MFMAs), double-buffered, one barrier per tile. Latent rows are padded
//     to 1056 bytes and rope rows XOR-swizzled (layout below), so both read patterns are conflict-free.
//   * S^T = Kc Q^T on v_mfma_f32_16x16x32_bf16 (K fragments from LDS, the 576-wide query of the wave's 16 heads
//     resident in registers). Each lane then holds one head, so the online-softmax statistics and the output
//     rescale are per-lane scalars plus two exchanges across the four 16-lane groups.
//   * O^T = c_kv^T P^T: the value operand is the SAME LDS tile read through ds_read_b64_tr_b16 (no second copy),
//     P^T comes straight from the S^T registers. O^T for 16 heads x 512 stays in registers (128 per lane).
//   * Splits over tokens write (O / l, lse) partials; the combine kernel merges them by log-sum-exp.
//   * Sparse form (DeepSeek Sparse Attention, Attention notes "Lighting Indexer": only the selected tokens take
//     part): the same kernel over a list of token indices per sequence. The splits cut the list; each copy
//     instruction of a latent row takes its token from the list (a lane read of the tile's index vector into the
//     scalar offset), the rope rows take theirs per lane; list entries outside [0, L) are masked like the tail.
//   * 8-bit latent cache (FP8 E4M3 or int8 codes with per-channel scales; DeepSeek 32K to 256K long context,
//     tqpw.cn, section 2.5; 7 anti-patterns of DeepSeek attention optimisation, lpnh.cn, section 3.3); key scales
//     fold into the query, value scales multiply the output channels. FP8 codes go straight to the FP8 matrix
//     cores (mla_split_fp8mma_kernel, below). int8 codes are staged in LDS, widened exactly into the bf16 tile by
//     all waves between two barriers, and the product code above runs unchanged.
// HBM-bound in principle (about 240 flop per byte) but close to the MFMA ridge, so both matter; measured, the
// LDS fragment reads (three in flight per wave) are what bound it.
#include <type_traits>

#include "device.h"
#include "kernels.h"

namespace attn {
namespace {

constexpr int kC = 512;             // kv_lora_rank
constexpr int kR = 64;              // rope dim
constexpr int kDK = kC + kR;        // key width
constexpr int kTargetBlocks = 256;  // one workgroup per compute unit on MI355X
// FP8 latent caches on the FP8 matrix cores (1), or widened into bf16 tiles like int8 (0).
#ifndef ATTN_MLA_FP8_MMA
#define ATTN_MLA_FP8_MMA 1
#endif
#ifndef ATTN_MLA_COPY_AUX
#define ATTN_MLA_COPY_AUX 2         // tile copies non-temporal: every cache row is read once (measured 3-7% faster)
#endif

// Tokens per LDS tile = 32 * ATTN_MLA_TILE_HALVES.
#ifndef ATTN_MLA_TILE_HALVES
#define ATTN_MLA_TILE_HALVES 2
#endif
constexpr int kHalves = ATTN_MLA_TILE_HALVES;
constexpr int kRows = 32 * kHalves;                 // tokens per tile
// LDS tile: the latent rows first, each padded to 1056 bytes (1024 + 32), then the rope rows, 128 bytes each.
// LDS has 64 four-byte banks; measured on gfx950, ds_read_b128 serves the lane sets {0-7, 24-31}, {8-15, 16-23},
// {32-39, 56-63}, {40-47, 48-55} one per cycle and ds_read_b64_tr_b16 32 consecutive lanes per cycle; a set is
// conflict-free when its lanes hit distinct slots modulo 256 bytes.
//   latent: unswizzled. The 32-byte pad shifts row r by 2r 16-byte slots: the transposing value reads (rows
//           r0..r0+7 x 32 bytes per 32 lanes) fill all 64 banks, and each K-read set (8 rows at one chunk, the
//           other 8 of the 16 rows at the next chunk) lands on the even and the odd slots.
//   rope:   chunk c of row r sits at c ^ ((r >> 1) & 7), which spreads the 16-row K reads over all banks.
constexpr int kCkvStride = 2 * kC + 32;             // bytes per latent row in LDS
constexpr int kPeOff = kRows * kCkvStride;          // byte offset of the rope rows
constexpr int kTileBytes = kPeOff + kRows * kR * 2;
constexpr int kCopies = kRows + kRows / 8;          // wave instructions per tile copy (one per latent row, 8 rope rows)

struct MlaArgs {
  const uint16_t* q_lat;
  const uint16_t* q_pe;
  const uint16_t* c_kv;
  const uint16_t* k_pe;
  const int32_t* seq_lens;
  float* ws_o;     // [batch, heads, n_split, 512]
  float* ws_lse;   // [batch, heads, n_split]
  int heads, max_len, n_split, split_len;
  float scale;
  const int32_t* idx;   // sparse form: [batch, topk] token indices (entries outside [0, L) are ignored)
  int topk;
  const float* c_scale;   // 8-bit latent cache: [kC] and [kR] per-channel scales
  const float* pe_scale;
};

// 8-bit latent cache (the KV template argument): a tile's codes (64 latent rows of 512 bytes, then 64 rope rows of
// 64 bytes, in token order) are copied into a staging buffer, then widened by all waves into the bf16 tile above,
// which the unchanged product code reads. Each copy instruction moves 1 KiB of contiguous codes.
constexpr int kStageBytes = kRows * (kC + kR);
constexpr int kStagePeOff = kRows * kC;
constexpr int kCopies8 = kStageBytes / 1024;        // 36 at 64-token tiles

// The per-lane offset is formed at the copy (opaque to the compiler): precomputed for every copy of a tile it would
// hold one register per instruction across the loop. Offsets stay in the range-checked voffset, so rows past the
// resource read zeros.
__device__ __forceinline__ void mla_copy_one8(uint8_t* stage, const buf_rsrc_t& rc, const buf_rsrc_t& rp, int i,
                                              int lane) {
  uint32_t vo = uint32_t(16 * lane);
  asm volatile("" : "+v"(vo));
  if (i < kStagePeOff / 1024)
    load_lds16<ATTN_MLA_COPY_AUX>(rc, vo + uint32_t(1024 * i), stage + 1024 * i);
  else
    load_lds16<ATTN_MLA_COPY_AUX>(rp, vo + uint32_t(1024 * (i - kStagePeOff / 1024)), stage + 1024 * i);
}

// One tile copy: tokens t_tile .. t_tile + kRows - 1 of sequence b. Copy instruction i < kRows moves latent row
// i (1024 contiguous bytes), the others 8 rope rows each (1024 contiguous bytes). Tokens at or past t_end come from
// token t_end - 1 (finite data; their scores are masked and P is exactly 0). The buffer resources span exactly the
// valid rows; a tile past the end gets none, so its copy instructions read nothing (out of range: zeros).
struct MlaCopy {
  buf_rsrc_t rc, rp;
  int rows;
};

__device__ __forceinline__ MlaCopy mla_copy_setup(const MlaArgs& a, int b, int t_tile, int t_end) {
  MlaCopy cp;
  cp.rows = max(0, min(kRows, t_end - t_tile));
  const int64_t tok0 = int64_t(b) * a.max_len + min(t_tile, t_end - 1);
  cp.rc = make_buf_rsrc(a.c_kv + tok0 * kC, uint32_t(cp.rows * kC * 2));
  cp.rp = make_buf_rsrc(a.k_pe + tok0 * kR, uint32_t(cp.rows * kR * 2));
  return cp;
}

// 8-bit resources over the codes of tokens t_tile .. min(t_tile + kRows, t_end) - 1 of sequence b (a tile past the
// end gets empty resources: its copies read zeros).
__device__ __forceinline__ void mla_rsrc8(const MlaArgs& a, int b, int t_tile, int t_end, buf_rsrc_t& rc,
                                          buf_rsrc_t& rp) {
  const int rows = max(0, min(kRows, t_end - t_tile));
  const int64_t tok0 = int64_t(b) * a.max_len + min(t_tile, max(t_end - 1, 0));
  rc = make_buf_rsrc(reinterpret_cast<const uint8_t*>(a.c_kv) + tok0 * kC, uint32_t(rows * kC));
  rp = make_buf_rsrc(reinterpret_cast<const uint8_t*>(a.k_pe) + tok0 * kR, uint32_t(rows * kR));
}

// Sparse form. The token list of a tile (64 entries) is staged in LDS by one 4-byte-per-lane load-to-LDS; slot
// position q holds the entry of tile row (q % 8) * 8 + q / 8 (an 8 x 8 transpose: the map is its own inverse).
// The resources span the whole sequence. A row whose entry is outside [0, L), or past the end of the list, is
// copied from an out-of-range offset, so it reads as zeros (finite, masked, P = 0) and no unselected token is
// ever read.
__device__ __forceinline__ int idx_pos(int row) { return (row & 7) * 8 + (row >> 3); }

__device__ __forceinline__ MlaCopy mla_copy_setup_sparse(const MlaArgs& a, int b) {
  MlaCopy cp;
  cp.rows = kRows;
  cp.rc = make_buf_rsrc(a.c_kv + int64_t(b) * a.max_len * kC, uint32_t(a.max_len * kC * 2));
  cp.rp = make_buf_rsrc(a.k_pe + int64_t(b) * a.max_len * kR, uint32_t(a.max_len * kR * 2));
  return cp;
}

// `nrows` = list entries in this tile; `oob` = a byte offset at or past both resources' ends.
__device__ __forceinline__ void mla_copy_one_sparse(char* dst, const MlaCopy& cp, int i, int lane,
                                                    const int32_t* slot, int L, int nrows, uint32_t oob) {
  if (i < kRows) {
    const int id = __builtin_amdgcn_readfirstlane(slot[idx_pos(i)]);   // uniform: scalar offset
    const bool ok = i < nrows && id >= 0 && id < L;
    load_lds16<ATTN_MLA_COPY_AUX>(cp.rc, uint32_t(16 * lane) + (ok ? 0u : oob), dst + i * kCkvStride,
                                  ok ? uint32_t(id * kC * 2) : 0u);
  } else {
    const int r = 8 * (i - kRows) + (lane >> 3);
    const int id = slot[idx_pos(r)];
    const bool ok = r < nrows && id >= 0 && id < L;
    load_lds16<ATTN_MLA_COPY_AUX>(cp.rp,
                                  (ok ? uint32_t(id * kR * 2) : oob) + uint32_t(16 * ((lane & 7) ^ ((r >> 1) & 7))),
               dst + kPeOff + (i - kRows) * 1024);
  }
}

// Copy instruction i (wave-uniform) of a tile copy into the LDS tile at `dst`.
__device__ __forceinline__ void mla_copy_one(char* dst, const MlaCopy& cp, int i, int lane) {
  if (i < kRows) {
    const int row = max(0, min(i, cp.rows - 1));       // uniform: goes in the scalar offset
    load_lds16<ATTN_MLA_COPY_AUX>(cp.rc, uint32_t(16 * lane), dst + i * kCkvStride, uint32_t(row * kC * 2));
  } else {
    const int r = 8 * (i - kRows) + (lane >> 3);
    const int row = max(0, min(r, cp.rows - 1));
    load_lds16<ATTN_MLA_COPY_AUX>(cp.rp, uint32_t(row * kR * 2 + 16 * ((lane & 7) ^ ((r >> 1) & 7))),
                                  dst + kPeOff + (i - kRows) * 1024);
  }
}

// Heads per wave: 16 (the N dimension of v_mfma_f32_16x16x32_bf16), so a wave keeps its 576-wide query
// (72 registers) and its O^T = 512 x 16 fp32 (128 registers) resident without spilling; 8 waves cover 128 heads.
constexpr int kHeadsPerWave = 16;

// LDS fragments in flight ahead of the MFMA that consumes them (4 registers each).
#ifndef ATTN_MLA_PIPE
#define ATTN_MLA_PIPE 3
#endif
constexpr int kPipe = ATTN_MLA_PIPE;
// 1: pin the read/MFMA interleave with scheduling groups; 0: leave the order to the compiler.
#ifndef ATTN_MLA_SGB
#define ATTN_MLA_SGB 1
#endif
#define MLA_SGB(mask, n) do { if (ATTN_MLA_SGB) __builtin_amdgcn_sched_group_barrier(mask, n, 0); } while (0)

// NW waves per workgroup (16 heads each). Each wave issues kCopies / NW copy instructions per tile, spread over
// its score MFMAs (one every NW), so the copy of tile t+1 overlaps tile t's work instead of stalling every wave
// on a burst of vector-memory issues right after the barrier.
template <int NW, bool SPARSE, int KV = kKvBf16>
__global__ __launch_bounds__(64 * NW) void mla_split_kernel(MlaArgs a) {
  static_assert(!(SPARSE && KV != kKvBf16), "the sparse form reads a bf16 cache");
  // LDS fragments in flight (the sparse form keeps two: its token-list handling needs the registers)
  constexpr int kP = SPARSE ? 2 : kPipe;
  static_assert(kCopies % NW == 0, "copy instructions must split evenly over the waves");
  constexpr int NC = kCopies / NW;
  // bf16 tiles: two (double-buffered copies) for a bf16 cache; one for an 8-bit cache, whose copies go to the two
  // staging buffers instead
  __shared__ __attribute__((aligned(16))) char lds[KV ? 1 : 2][kTileBytes];
  __shared__ __attribute__((aligned(16))) uint8_t stage[KV ? 2 : 1][KV ? kStageBytes : 16];
  constexpr int NC8 = (kCopies8 + NW - 1) / NW;      // 8-bit copy instructions per wave per tile
  __shared__ int32_t lds_idx[SPARSE ? 4 : 1][64];     // sparse: token lists of tiles t .. t+3 (slot t & 3)
  const int split = blockIdx.x, b = blockIdx.y;
  // Wave index in a scalar register, with its range [0, NW) visible to the compiler (resolves at compile time
  // whether each copy instruction moves a latent or a rope block).
  const int wave = int(unsigned(__builtin_amdgcn_readfirstlane(threadIdx.x >> 6)) % unsigned(NW));
  const int lane = threadIdx.x & 63;
  const int n = lane & 15, g4 = lane >> 4;
  const int L = max(0, min(a.seq_lens[b], a.max_len));
  const int t_begin = split * a.split_len;
  // dense: tokens t_begin .. t_end-1; sparse: list positions t_begin .. t_end-1 (every split writes a partial)
  if (!SPARSE && t_begin >= L) return;                // uniform over the workgroup
  const int t_end = min(SPARSE ? a.topk : L, t_begin + a.split_len);
  const int ntiles = (t_end - t_begin + kRows - 1) / kRows;
  const int h = wave * kHeadsPerWave + n;
  const float c = a.scale * kLog2e;

  // query [q_lat ; q_pe] of head h: B operands of the 18 k-steps, dims 32*ks + 8*g4 ..
  bf16x8_t qop[kDK / 32];
#pragma unroll
  for (int ks = 0; ks < kDK / 32; ++ks) {
    const int d = 32 * ks + 8 * g4;
    const uint16_t* p = d < kC ? a.q_lat + (int64_t(b) * a.heads + h) * kC + d
                               : a.q_pe + (int64_t(b) * a.heads + h) * kR + (d - kC);
    qop[ks] = as_bf16x8(*reinterpret_cast<const u32x4_t*>(p));
    if constexpr (KV != kKvBf16) {
      // a key channel's scale folds into the query: q . (code * s) = (q * s) . code (one bf16 rounding)
      const float* sc = d < kC ? a.c_scale + d : a.pe_scale + (d - kC);
      const u32x4_t w = __builtin_bit_cast(u32x4_t, qop[ks]);
      const f32x4_t s0 = *reinterpret_cast<const f32x4_t*>(sc), s1 = *reinterpret_cast<const f32x4_t*>(sc + 4);
      qop[ks] = pack_bf16x8(bf16lo_to_f32(w[0]) * s0[0], bf16hi_to_f32(w[0]) * s0[1], bf16lo_to_f32(w[1]) * s0[2],
                            bf16hi_to_f32(w[1]) * s0[3], bf16lo_to_f32(w[2]) * s1[0], bf16hi_to_f32(w[2]) * s1[1],
                            bf16lo_to_f32(w[3]) * s1[2], bf16hi_to_f32(w[3]) * s1[3]);
    }
  }
  // O^T: 32 blocks of 16 latent dims; lane holds head n, dims 16*db + 4*g4 + r
  f32x4_t oacc[kC / 16];
#pragma unroll
  for (int db = 0; db < kC / 16; ++db) oacc[db] = f32x4_t{};
  float m = -INFINITY, l = 0.f;

  // Lane-fixed parts of the LDS addresses (layout above); the loops add only compile-time immediates.
  //   K reads (A operand): token row n (+16*tb), chunk 4*ks + g4.
  const uint32_t abase = uint32_t(n * kCkvStride + 16 * g4);
  uint32_t pbase[2];
#pragma unroll
  for (int j = 0; j < 2; ++j) pbase[j] = uint32_t(kPeOff + n * kR * 2 + 16 * ((4 * j + g4) ^ ((n >> 1) & 7)));
  //   value reads (transposing): rows vrow (+16), latent columns 16*db + 4*(bl&3) .. +3.
  const int bl = lane & 15;
  const int vrow = 4 * g4 + (bl >> 2);
  const uint32_t vbase = uint32_t(vrow * kCkvStride + 8 * (bl & 3));

  // Sparse form: wave 0 stages the token list of tile u into lds_idx[u & 3] (entries past the split read 0;
  // validity also checks the list position).
  MlaCopy cps;
  buf_rsrc_t ri;
  const uint32_t oob = uint32_t(a.max_len) * kC * 2;  // past the end of both sparse resources
  auto stage_idx = [&](int u) {
    if (wave == 0 && u < ntiles)
      load_lds4(ri, uint32_t(4 * (u * kRows + idx_pos(lane))), lds_idx[u & 3]);
  };
  if constexpr (SPARSE) {
    cps = mla_copy_setup_sparse(a, b);
    ri = make_buf_rsrc(a.idx + int64_t(b) * a.topk + t_begin, uint32_t(max(0, t_end - t_begin) * 4));
    stage_idx(0);
    stage_idx(1);
    wait_vmem();
    __syncthreads();
    if (ntiles > 0) {
#pragma unroll
      for (int k = 0; k < NC; ++k)
        mla_copy_one_sparse(lds[0], cps, wave + k * NW, lane, lds_idx[0], L, t_end - t_begin, oob);
    }
  } else if constexpr (KV != kKvBf16) {
    buf_rsrc_t rc, rp;
    mla_rsrc8(a, b, t_begin, t_end, rc, rp);
#pragma unroll
    for (int k = 0; k < NC8; ++k)
      if (wave + k * NW < kCopies8) mla_copy_one8(stage[0], rc, rp, wave + k * NW, lane);
  } else {
    const MlaCopy cp0 = mla_copy_setup(a, b, t_begin, t_end);
#pragma unroll
    for (int k = 0; k < NC; ++k) mla_copy_one(lds[0], cp0, wave + k * NW, lane);
  }

  for (int t = 0; t < ntiles; ++t) {
    wait_vmem();
    __syncthreads();                                   // tile t visible to all; buffer (t+1)&1 free
    uint64_t valid = ~0ull;                            // sparse: rows of tile t holding a token of the sequence
    if constexpr (SPARSE) {
      const int id = lds_idx[t & 3][idx_pos(lane)];    // tile row `lane`
      valid = __ballot(t * kRows + lane < t_end - t_begin && id >= 0 && id < L);
      stage_idx(t + 2);                                // lands with this iteration's copies
    }
    const MlaCopy cpn = SPARSE ? cps : mla_copy_setup(a, b, t_begin + (t + 1) * kRows, t_end);
    char* nbuf = lds[(t + 1) & 1 & (KV ? 0 : 1)];
    const uint16_t* T = reinterpret_cast<const uint16_t*>(lds[t & 1 & (KV ? 0 : 1)]);
    buf_rsrc_t rc8, rp8;                               // 8-bit: resources of tile t+1
    if constexpr (KV != kKvBf16) {
      mla_rsrc8(a, b, t_begin + (t + 1) * kRows, t_end, rc8, rp8);
      // widen staged tile t into the bf16 tile, 8 codes (one 8-byte chunk) at a time. Thread tid takes latent
      // chunks tid + 64*NW*u: row tid/64 + NW*u, chunk tid%64 (the padded row stride), and rope chunks likewise
      // (row tid/8 + 8*NW*u, chunk tid%8, whose XOR key ((row >> 1) & 7) does not depend on u), so every address
      // is a per-thread base plus an immediate.
      const uint8_t* st = stage[t & 1];
      char* tile = lds[0];
      const int tid = threadIdx.x;
      auto widen8 = [&](uint32_t rd, uint32_t wr) {
        const u32x2_t w = *reinterpret_cast<const __attribute__((address_space(3))) u32x2_t*>(
            (const __attribute__((address_space(3))) uint8_t*)st + rd);
        *reinterpret_cast<__attribute__((address_space(3))) u32x4_t*>((__attribute__((address_space(3))) char*)tile +
                                                                      wr) = codes_to_bf16x8<KV>(w[0], w[1]);
      };
      const uint32_t rd_c = uint32_t(8 * tid), wr_c = uint32_t((tid / 64) * kCkvStride + 16 * (tid % 64));
#pragma unroll 4
      for (int u = 0; u < (kStagePeOff / 8 + 64 * NW - 1) / (64 * NW); ++u)
        if (tid + 64 * NW * u < kStagePeOff / 8) widen8(rd_c + 512 * NW * u, wr_c + NW * kCkvStride * u);
      const uint32_t rd_p = uint32_t(kStagePeOff + 8 * tid);
      const uint32_t wr_p = uint32_t(kPeOff + (tid / 8) * kR * 2 + 16 * ((tid % 8) ^ ((tid / 16) & 7)));
#pragma unroll
      for (int u = 0; u < (kRows * kR / 8 + 64 * NW - 1) / (64 * NW); ++u)
        if (tid + 64 * NW * u < kRows * kR / 8) widen8(rd_p + 512 * NW * u, wr_p + 8 * NW * kR * 2 * u);
      __syncthreads();                                 // bf16 tile t ready; stage (t+1)&1 free for the next copy
    }
    const int tok0 = t_begin + t * kRows;

    // S^T = Kc Q^T: 16-token blocks tb; lane holds head n, tokens 16*tb + 4*g4 + r. The K fragments are
    // software-pipelined kP MFMAs ahead (one wave-uniform order pinned by scheduling groups), so LDS latency
    // overlaps the MFMAs instead of stalling each one.
    constexpr int TB = 2 * kHalves;
    constexpr int NQ = (kDK / 32) * TB;                // MFMAs of the score contraction
    f32x4_t sacc[TB];
#pragma unroll
    for (int tb = 0; tb < TB; ++tb) sacc[tb] = f32x4_t{};
    auto kfrag = [&](int j) {                           // j = ks * TB + tb
      const int ks = j / TB, tb = j % TB;
      return as_bf16x8(ks < kC / 32 ? lds_read16(T, abase + 64 * ks + 16 * tb * kCkvStride)
                                    : lds_read16(T, pbase[ks - kC / 32] + 16 * tb * kR * 2));
    };
    bf16x8_t kf[kP];
#pragma unroll
    for (int j = 0; j < kP; ++j) kf[j] = kfrag(j);
    MLA_SGB(0x100, kP);
#pragma unroll
    for (int j = 0; j < NQ; ++j) {
      const bf16x8_t cur = kf[j % kP];
      if (j + kP < NQ) kf[j % kP] = kfrag(j + kP);
      sacc[j % TB] = mfma16x16x32(cur, qop[j / TB], sacc[j % TB]);
      MLA_SGB(0x008, 1);
      if (j + kP < NQ) MLA_SGB(0x100, 1);
      if (j % NW == 0 && j / NW < (KV ? NC8 : NC)) {   // next tile's copy, one instruction every NW MFMAs
        if constexpr (SPARSE) {
          if (t + 1 < ntiles)
            mla_copy_one_sparse(nbuf, cpn, wave + (j / NW) * NW, lane, lds_idx[(t + 1) & 3], L,
                                t_end - t_begin - (t + 1) * kRows, oob);
        } else if constexpr (KV != kKvBf16) {
          if (t + 1 < ntiles && wave + (j / NW) * NW < kCopies8)
            mla_copy_one8(stage[(t + 1) & 1], rc8, rp8, wave + (j / NW) * NW, lane);
        } else {
          mla_copy_one(nbuf, cpn, wave + (j / NW) * NW, lane);
        }
        MLA_SGB(0x020, 1);
      }
    }
    if constexpr (SPARSE) {
      if (valid != ~0ull) {
#pragma unroll
        for (int tb = 0; tb < TB; ++tb)
#pragma unroll
          for (int r = 0; r < 4; ++r)
            sacc[tb][r] = (uint32_t(valid >> (16 * tb + r)) >> (4 * g4)) & 1 ? sacc[tb][r] : -INFINITY;
      }
    } else if (tok0 + kRows > t_end) {
#pragma unroll
      for (int tb = 0; tb < TB; ++tb)
#pragma unroll
        for (int r = 0; r < 4; ++r)
          sacc[tb][r] = tok0 + 16 * tb + 4 * g4 + r >= t_end ? -INFINITY : sacc[tb][r];
    }
    float mx = -INFINITY;
#pragma unroll
    for (int tb = 0; tb < TB; ++tb)
#pragma unroll
      for (int r = 0; r < 4; ++r) mx = fmaxf(mx, sacc[tb][r]);
    mx = fmaxf(mx, xor_lanes(mx, 16));
    mx = fmaxf(mx, xor_lanes(mx, 32));
    // Lazy rescale: the reference max moves (and O, l are rescaled) only when it grows by more than
    // 2^kRescaleLog2 for some lane of the wave; otherwise P may exceed 1 by at most that factor. O / l is unchanged.
    if (__any((mx - m) * c > kRescaleLog2)) {
      const float m_new = fmaxf(m, mx);
      const float alpha = fast_exp2((m - m_new) * c);
      l *= alpha;
#pragma unroll
      for (int db = 0; db < kC / 16; ++db) oacc[db] *= alpha;
      m = m_new;
    }
    // (sparse: until a selected token is seen m is -inf and every P is 0)
    const float mc = (SPARSE && m == -INFINITY) ? 0.f : m * c;
#pragma unroll
    for (int tb = 0; tb < TB; ++tb)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float p = fast_exp2(fmaf(sacc[tb][r], c, -mc));
        sacc[tb][r] = p;
        l += p;
      }
    // P^T operand of each 32-token half: slots 0..3 are tokens 4*g4 + s, slots 4..7 tokens 16 + 4*g4 + s
    bf16x8_t pb[kHalves];
#pragma unroll
    for (int kh = 0; kh < kHalves; ++kh)
      pb[kh] = pack_bf16x8(sacc[2 * kh][0], sacc[2 * kh][1], sacc[2 * kh][2], sacc[2 * kh][3], sacc[2 * kh + 1][0],
                           sacc[2 * kh + 1][1], sacc[2 * kh + 1][2], sacc[2 * kh + 1][3]);
    // O^T += c_kv^T P^T: the value operand is the same tile read through the transposing LDS read; 32-token
    // halves outer so consecutive MFMAs use independent accumulators; value fragments pipelined like K.
    constexpr int NV = kHalves * (kC / 16);
    auto vfrag = [&](int j) {                           // j = kh * 32 + db
      const int kh = j / (kC / 16), db = j % (kC / 16);
      const uint32_t off = vbase + 32 * db + 32 * kh * kCkvStride;
      const u32x2_t lo = lds_read_tr16(T, off);
      const u32x2_t hi = lds_read_tr16(T, off + 16 * kCkvStride);
      const u32x4_t w = {lo[0], lo[1], hi[0], hi[1]};
      return as_bf16x8(w);
    };
    bf16x8_t vf[kP];
#pragma unroll
    for (int j = 0; j < kP; ++j) vf[j] = vfrag(j);
    MLA_SGB(0x100, 2 * kP);
#pragma unroll
    for (int j = 0; j < NV; ++j) {
      const bf16x8_t cur = vf[j % kP];
      if (j + kP < NV) vf[j % kP] = vfrag(j + kP);
      oacc[j % (kC / 16)] = mfma16x16x32(cur, pb[j / (kC / 16)], oacc[j % (kC / 16)]);
      MLA_SGB(0x008, 1);
      if (j + kP < NV) MLA_SGB(0x100, 2);
    }
  }

  float lt = l + xor_lanes(l, 16);
  lt += xor_lanes(lt, 32);
  const float inv = (SPARSE && lt == 0.f) ? 0.f : 1.f / lt;   // sparse: a split may select nothing
  const int64_t slot = (int64_t(b) * a.heads + h) * a.n_split + split;
  float* wo = a.ws_o + slot * kC + 4 * g4;
#pragma unroll
  for (int db = 0; db < kC / 16; ++db) {
    f32x4_t v = {oacc[db][0] * inv, oacc[db][1] * inv, oacc[db][2] * inv, oacc[db][3] * inv};
    if constexpr (KV != kKvBf16) v *= *reinterpret_cast<const f32x4_t*>(a.c_scale + 16 * db + 4 * g4);   // code * s
    *reinterpret_cast<f32x4_t*>(wo + 16 * db) = v;
  }
  if (g4 == 0) a.ws_lse[slot] = (SPARSE && lt == 0.f) ? -INFINITY : m * a.scale + logf(lt);
}

// ---- FP8 latent cache on the FP8 matrix cores.
// The codes stay 8-bit all the way: tiles of 64 tokens are copied into LDS as codes, and both products run on
// v_mfma_scale_f32_16x16x128_f8f6f4 (E4M3 x E4M3, unit scales). The bf16 query and the probabilities are carried
// as two E4M3 terms each (hi = e4m3(x), lo = e4m3(x - hi): about 8 significant bits, like bf16), so the matrix-core
// time equals the bf16 kernel's (FP8 runs at twice the bf16 rate), while the LDS fragment bytes and the HBM bytes
// halve and the widening pass disappears.
//   * Query: q' = q * c_scale (a key channel's scale folds into the query) times a power of two per head, 2^k,
//     that brings the head's largest |q'| into [128, 256), then split; scores come out multiplied by 2^k, and that
//     head's softmax constant is scale * log2(e) / 2^k.
//   * Scores S^T (16 tokens x 16 heads per MFMA) take the query's hi and lo terms in two MFMAs over the same key
//     fragment. K positions: K-step ks (128 of the 512 latent channels) gives lane group g the 16-channel chunks
//     4ks + 2(g>>1) + 16(g&1) + e, e = 0, 1; the rope K-step holds the 64 rope channels twice (A: the codes twice;
//     B: the hi term in groups 0-1, the lo term in groups 2-3). Lane holds head n = l%16, tokens 16tb + 4g + r.
//   * O^T = V^T P^T in one MFMA per 16 latent channels and tile: lane group g's 32 K positions are its own 16
//     tokens twice, 4tb + r for the hi term of token 16tb + 4g + r and 16 + 4tb + r for its lo term, so P^T is
//     packed straight from the score registers and V^T needs two ds_read_b64_tr_b8 reads, used twice.
//   * LDS: latent rows of 512 codes at a 528-byte pitch, 16-byte chunk c of row r stored at chunk c ^ 8*((r>>4)&1);
//     rope rows of 64 codes, chunk c at c ^ ((r>>2)&1). Both read patterns are conflict-free under the measured
//     bank model (checked exhaustively on the CPU), and each read is a per-lane base plus an immediate.
//   * Probabilities are carried as 2^7 * exp(s - m) with the reference max m moved whenever the max grows by more
//     than a factor of 2, so they stay below 256 (E4M3 reaches 448) and the subnormal range of the lo term starts
//     2^13 below the largest probability; the factor cancels in O = sum p v / sum p.
//   * The tile loop's LDS reads are inline assembly, each block with its own wait: compiled reads got a vmcnt wait
//     for every next-tile copy in flight (the compiler cannot tell the copies fill the other buffer). A block reads
//     the fragments of two K-steps (four products) or four 16-channel value blocks (four products) and is issued
//     right after the previous block's products, so its latency overlaps them. The register file is full (256 at
//     two waves per SIMD: the 512 x 16 output and the split query take 192), which bounds the blocks. Measured
//     0.281-0.285 ms against 0.304 ms for the widening kernel on the same box (one read per product: 0.295).
constexpr int kRowsF8 = 64;                            // tokens per tile
constexpr float kRescaleLog2F8 = 1.0f;                 // lazy-rescale threshold (log2 units)
constexpr float kPExpF8 = 7.0f;                        // probabilities carried times 2^7
constexpr int kLatPitch = 528;                         // LDS bytes per latent row (512 codes + 16)
constexpr int kLatBytes = kRowsF8 * kLatPitch;
constexpr int kPeBytesF8 = kRowsF8 * kR;
constexpr int kLatCopies = kLatBytes / 1024;          // 33 copy instructions of 1 KiB
constexpr int kCopiesF8 = kLatCopies + kPeBytesF8 / 1024;   // + 4 for the rope rows
static_assert(kLatBytes % 1024 == 0 && kPeBytesF8 % 1024 == 0, "tiles split into 1 KiB copy instructions");

// Copy instruction ci (wave-uniform) of a tile: latent instructions fill LDS bytes [1024 ci, 1024 ci + 1024) of the
// padded latent tile (pad bytes read out of range: zeros), rope instructions 16 rope rows each. Rows past the
// resources (the end of the split) read zeros.
__device__ __forceinline__ void mla_f8_copy(uint8_t* lat, uint8_t* pe, const buf_rsrc_t& rc, const buf_rsrc_t& rp,
                                            int ci, int lane) {
  if (ci < kLatCopies) {
    const uint32_t at = uint32_t(1024 * ci + 16 * lane);
    const uint32_t row = at / kLatPitch, col = at - row * kLatPitch;
    const uint32_t chunk = (col >> 4) ^ (((row >> 4) & 1u) << 3);
    load_lds16<ATTN_MLA_COPY_AUX>(rc, col < 512u ? row * 512u + 16u * chunk : 0x80000000u, lat + 1024 * ci);
  } else {
    const int i = ci - kLatCopies;
    const uint32_t row = uint32_t(16 * i + (lane >> 2));
    const uint32_t chunk = uint32_t(lane & 3) ^ ((row >> 2) & 1u);
    load_lds16<ATTN_MLA_COPY_AUX>(rp, row * 64u + 16u * chunk, pe + 1024 * i);
  }
}

// Resources over the codes of tokens t_tile .. min(t_tile + 64, t_end) - 1 of sequence b.
__device__ __forceinline__ void mla_rsrc_f8(const MlaArgs& a, int b, int t_tile, int t_end, buf_rsrc_t& rc,
                                            buf_rsrc_t& rp) {
  const int rows = max(0, min(kRowsF8, t_end - t_tile));
  const int64_t tok0 = int64_t(b) * a.max_len + min(t_tile, max(t_end - 1, 0));
  rc = make_buf_rsrc(reinterpret_cast<const uint8_t*>(a.c_kv) + tok0 * kC, uint32_t(rows * kC));
  rp = make_buf_rsrc(reinterpret_cast<const uint8_t*>(a.k_pe) + tok0 * kR, uint32_t(rows * kR));
}

// LDS reads of the FP8 kernel, written out in inline assembly with their own lgkmcnt(0) wait: compiled reads
// after an in-flight direct-to-LDS copy get a vmcnt(0) wait for that copy (the compiler cannot tell that the copy
// fills the other tile buffer), which serialised every next-tile copy behind the reads.
__device__ __forceinline__ uint32_t lds_u32(const void* p) {
  return uint32_t(reinterpret_cast<uintptr_t>((const __attribute__((address_space(3))) char*)p));
}
template <int N, int I = 0, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (I < N) {
    f(std::integral_constant<int, I>{});
    static_for<N, I + 1>(f);
  }
}
// Two 32-byte key fragments (K-steps at OFF0 and OFF1: 16 bytes there and 16 bytes after).
template <int OFF0, int OFF1>
__device__ __forceinline__ void lds_read_k2_asm(uint32_t addr, i32x8_t& f0, i32x8_t& f1) {
  u32x4_t a, b, c, d;
  asm volatile("ds_read_b128 %0, %4 offset:%5\n\tds_read_b128 %1, %4 offset:%6\n\t"
               "ds_read_b128 %2, %4 offset:%7\n\tds_read_b128 %3, %4 offset:%8\n\ts_waitcnt lgkmcnt(0)"
               : "=&v"(a), "=&v"(b), "=&v"(c), "=&v"(d)
               : "v"(addr), "n"(OFF0), "n"(OFF0 + 16), "n"(OFF1), "n"(OFF1 + 16)
               : "memory");
  f0 = __builtin_bit_cast(i32x8_t, __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7));
  f1 = __builtin_bit_cast(i32x8_t, __builtin_shufflevector(c, d, 0, 1, 2, 3, 4, 5, 6, 7));
}
// The rope key fragment (16 bytes at r0 + OFF and r1 + OFF) and the rope query operand (q and q + 1024).
template <int OFF>
__device__ __forceinline__ void lds_read_rq_asm(uint32_t r0, uint32_t r1, uint32_t q, i32x8_t& rf, i32x8_t& qf) {
  u32x4_t a, b, c, d;
  asm volatile("ds_read_b128 %0, %4 offset:%7\n\tds_read_b128 %1, %5 offset:%7\n\t"
               "ds_read_b128 %2, %6\n\tds_read_b128 %3, %6 offset:1024\n\ts_waitcnt lgkmcnt(0)"
               : "=&v"(a), "=&v"(b), "=&v"(c), "=&v"(d)
               : "v"(r0), "v"(r1), "v"(q), "n"(OFF)
               : "memory");
  rf = __builtin_bit_cast(i32x8_t, __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7));
  qf = __builtin_bit_cast(i32x8_t, __builtin_shufflevector(c, d, 0, 1, 2, 3, 4, 5, 6, 7));
}
// Four V^T operands (latent chunks at a + OFF + 16 i, i = 0..3, all on one side of the swizzle's 128-byte shift).
// Each operand is two transposing reads (tokens 0-31 and 32-63 of the tile, STEP apart); its second half, the lo
// K positions, repeats the first (register copies, not a second pair of reads).
template <int OFF, int STEP>
__device__ __forceinline__ void lds_read_v4_asm(uint32_t a, i32x8_t (&v)[4]) {
  u32x2_t w[8];
  asm volatile("ds_read_b64_tr_b8 %0, %8 offset:%9\n\tds_read_b64_tr_b8 %1, %8 offset:%10\n\t"
               "ds_read_b64_tr_b8 %2, %8 offset:%11\n\tds_read_b64_tr_b8 %3, %8 offset:%12\n\t"
               "ds_read_b64_tr_b8 %4, %8 offset:%13\n\tds_read_b64_tr_b8 %5, %8 offset:%14\n\t"
               "ds_read_b64_tr_b8 %6, %8 offset:%15\n\tds_read_b64_tr_b8 %7, %8 offset:%16\n\t"
               "s_waitcnt lgkmcnt(0)"
               : "=&v"(w[0]), "=&v"(w[1]), "=&v"(w[2]), "=&v"(w[3]), "=&v"(w[4]), "=&v"(w[5]), "=&v"(w[6]),
                 "=&v"(w[7])
               : "v"(a), "n"(OFF), "n"(OFF + STEP), "n"(OFF + 16), "n"(OFF + 16 + STEP), "n"(OFF + 32),
                 "n"(OFF + 32 + STEP), "n"(OFF + 48), "n"(OFF + 48 + STEP)
               : "memory");
#pragma unroll
  for (int i = 0; i < 4; ++i)
    v[i] = i32x8_t{int(w[2 * i][0]), int(w[2 * i][1]), int(w[2 * i + 1][0]), int(w[2 * i + 1][1]),
                   int(w[2 * i][0]), int(w[2 * i][1]), int(w[2 * i + 1][0]), int(w[2 * i + 1][1])};
}

// 16 fp32 values (scaled) -> their hi and lo E4M3 terms, four dwords each, in order.
__device__ __forceinline__ void split_e4m3_16(const float (&v)[16], uint32_t* hi, uint32_t* lo) {
#pragma unroll
  for (int d = 0; d < 4; ++d) {
    uint32_t hw = f32x2_to_fp8(0u, v[4 * d], v[4 * d + 1], false);
    hw = f32x2_to_fp8(hw, v[4 * d + 2], v[4 * d + 3], true);
    const f32x2_t d0 = fp8x2_to_f32(hw, false), d1 = fp8x2_to_f32(hw, true);
    uint32_t lw = f32x2_to_fp8(0u, v[4 * d] - d0[0], v[4 * d + 1] - d0[1], false);
    lw = f32x2_to_fp8(lw, v[4 * d + 2] - d1[0], v[4 * d + 3] - d1[1], true);
    hi[d] = hw;
    lo[d] = lw;
  }
}

template <int NW>
__global__ __launch_bounds__(64 * NW) void mla_split_fp8mma_kernel(MlaArgs a) {
  constexpr int NC = (kCopiesF8 + NW - 1) / NW;       // copy instructions per wave per tile
  __shared__ __attribute__((aligned(16))) uint8_t lat[2][kLatBytes];
  __shared__ __attribute__((aligned(16))) uint8_t pe[2][kPeBytesF8];
  // the rope K-step's query operand (32 bytes per lane) waits in LDS, two 16-byte planes per wave: registers are
  // the limit of this kernel
  __shared__ __attribute__((aligned(16))) uint8_t qrl[NW][2][64 * 16];
  const int split = blockIdx.x, b = blockIdx.y;
  const int wave = int(unsigned(__builtin_amdgcn_readfirstlane(threadIdx.x >> 6)) % unsigned(NW));
  const int lane = threadIdx.x & 63;
  const int n = lane & 15, g = lane >> 4;
  const int L = max(0, min(a.seq_lens[b], a.max_len));
  const int t_begin = split * a.split_len;
  if (t_begin >= L) return;                            // uniform over the workgroup
  const int t_end = min(L, t_begin + a.split_len);
  const int ntiles = (t_end - t_begin + kRowsF8 - 1) / kRowsF8;
  const int h = wave * kHeadsPerWave + n;
  {
    buf_rsrc_t rc, rp;
    mla_rsrc_f8(a, b, t_begin, t_end, rc, rp);
#pragma unroll
    for (int k = 0; k < NC; ++k)
      if (wave + k * NW < kCopiesF8) mla_f8_copy(lat[0], pe[0], rc, rp, wave + k * NW, lane);
  }

  // ---- query: hi and lo E4M3 terms of q * scale * 2^k
  const uint16_t* qlat = a.q_lat + (int64_t(b) * a.heads + h) * kC;
  const uint16_t* qpe = a.q_pe + (int64_t(b) * a.heads + h) * kR;
  auto lat_chunk = [&](int ks, int e) { return 4 * ks + 2 * (g >> 1) + 16 * (g & 1) + e; };
  auto qvals = [&](const uint16_t* q, const float* sc, int c, float mul, float (&v)[16]) {
    const u32x4_t w0 = *reinterpret_cast<const u32x4_t*>(q + c), w1 = *reinterpret_cast<const u32x4_t*>(q + c + 8);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const f32x4_t sv = *reinterpret_cast<const f32x4_t*>(sc + c + 4 * i);
      const uint32_t wa = i < 2 ? w0[2 * i] : w1[2 * i - 4], wb = i < 2 ? w0[2 * i + 1] : w1[2 * i - 3];
      v[4 * i] = bf16lo_to_f32(wa) * sv[0] * mul;
      v[4 * i + 1] = bf16hi_to_f32(wa) * sv[1] * mul;
      v[4 * i + 2] = bf16lo_to_f32(wb) * sv[2] * mul;
      v[4 * i + 3] = bf16hi_to_f32(wb) * sv[3] * mul;
    }
  };
  float mx = 0.f;
  {
    float v[16];
#pragma unroll
    for (int ks = 0; ks < 4; ++ks)
#pragma unroll
      for (int e = 0; e < 2; ++e) {
        qvals(qlat, a.c_scale, 16 * lat_chunk(ks, e), 1.f, v);
#pragma unroll
        for (int i = 0; i < 16; ++i) mx = fmaxf(mx, fabsf(v[i]));
      }
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      qvals(qpe, a.pe_scale, 32 * (g & 1) + 16 * e, 1.f, v);
#pragma unroll
      for (int i = 0; i < 16; ++i) mx = fmaxf(mx, fabsf(v[i]));
    }
  }
  mx = fmaxf(mx, xor_lanes(mx, 16));
  mx = fmaxf(mx, xor_lanes(mx, 32));
  int ex = 0;
  (void)frexpf(mx, &ex);
  const int kexp = mx > 0.f ? max(-64, min(64, 8 - ex)) : 0;
  const float up = ldexpf(1.f, kexp);
  const float c = ldexpf(a.scale * kLog2e, -kexp);      // softmax constant in the scaled score units
  i32x8_t qh[4], qlo[4];
  {
    float v[16];
    uint32_t hw[8], lw[8];
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
#pragma unroll
      for (int e = 0; e < 2; ++e) {
        qvals(qlat, a.c_scale, 16 * lat_chunk(ks, e), up, v);
        split_e4m3_16(v, hw + 4 * e, lw + 4 * e);
      }
      qh[ks] = i32x8_t{int(hw[0]), int(hw[1]), int(hw[2]), int(hw[3]), int(hw[4]), int(hw[5]), int(hw[6]), int(hw[7])};
      qlo[ks] = i32x8_t{int(lw[0]), int(lw[1]), int(lw[2]), int(lw[3]), int(lw[4]), int(lw[5]), int(lw[6]), int(lw[7])};
    }
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      qvals(qpe, a.pe_scale, 32 * (g & 1) + 16 * e, up, v);
      split_e4m3_16(v, hw + 4 * e, lw + 4 * e);
    }
    const uint32_t* t = g < 2 ? hw : lw;
    *reinterpret_cast<u32x4_t*>(&qrl[wave][0][16 * lane]) = u32x4_t{t[0], t[1], t[2], t[3]};
    *reinterpret_cast<u32x4_t*>(&qrl[wave][1][16 * lane]) = u32x4_t{t[4], t[5], t[6], t[7]};
  }

  f32x4_t oacc[kC / 16];
#pragma unroll
  for (int db = 0; db < kC / 16; ++db) oacc[db] = f32x4_t{};
  float m = -INFINITY, l = 0.f;

  // lane-fixed LDS read bases (layout above)
  const uint32_t kb = uint32_t(kLatPitch * n + 32 * (g >> 1) + 256 * (g & 1));     // latent K reads
  const uint32_t q2 = uint32_t((n >> 2) & 1);
  const uint32_t rb0 = uint32_t(64 * n + 32 * (g & 1)) + 16u * q2;                   // rope K reads, e = 0
  const uint32_t rb1 = uint32_t(64 * n + 32 * (g & 1)) + 16u * (1u - q2);            // e = 1
  const int jp = (lane & 15) >> 1, vs = jp >> 2;                                     // V^T reads
  const uint32_t vrow = uint32_t((16 * vs + 4 * g + (jp & 3)) * kLatPitch + 8 * (lane & 1));
  const uint32_t va = vrow + 128u * uint32_t(vs), vb = vrow - 128u * uint32_t(vs);
  const uint32_t qa = lds_u32(&qrl[0][0][0]) + uint32_t(2048 * wave + 16 * lane);    // this lane's rope query

  for (int t = 0; t < ntiles; ++t) {
    wait_vmem();
    __syncthreads();                                   // tile t visible to all; buffer (t+1)&1 free
    const int tok0 = t_begin + t * kRowsF8;
    buf_rsrc_t rcn, rpn;
    mla_rsrc_f8(a, b, tok0 + kRowsF8, t_end, rcn, rpn);
    const uint8_t* Lt = lat[t & 1];
    const uint8_t* Pt = pe[t & 1];
    uint8_t* Ln = lat[(t + 1) & 1];
    uint8_t* Pn = pe[(t + 1) & 1];
    f32x4_t sacc[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) sacc[i] = f32x4_t{};
    const uint32_t lk = lds_u32(Lt) + kb, lr0 = lds_u32(Pt) + rb0, lr1 = lds_u32(Pt) + rb1;
    static_for<4>([&](auto tbc) {
      constexpr int tb = decltype(tbc)::value;
      // key fragment of K-step ks: row 16tb + n, chunk (4ks + ...) ^ 8 * (tb & 1) (see the layout); two K-steps per
      // read block, so a block's wait overlaps the four products of the previous one
      constexpr int kt = 16 * kLatPitch * tb, kodd = (tb & 1) ? 128 : 0;
      i32x8_t f0, f1;
      lds_read_k2_asm<kt + kodd, kt + 64 + kodd>(lk, f0, f1);
      sacc[tb] = mfma16x16x128_fp8(f0, qh[0], sacc[tb]);
      sacc[tb] = mfma16x16x128_fp8(f0, qlo[0], sacc[tb]);
      sacc[tb] = mfma16x16x128_fp8(f1, qh[1], sacc[tb]);
      sacc[tb] = mfma16x16x128_fp8(f1, qlo[1], sacc[tb]);
      __builtin_amdgcn_sched_barrier(0);
      lds_read_k2_asm<kt + 128 - kodd, kt + 192 - kodd>(lk, f0, f1);
      sacc[tb] = mfma16x16x128_fp8(f0, qh[2], sacc[tb]);
      sacc[tb] = mfma16x16x128_fp8(f0, qlo[2], sacc[tb]);
      sacc[tb] = mfma16x16x128_fp8(f1, qh[3], sacc[tb]);
      sacc[tb] = mfma16x16x128_fp8(f1, qlo[3], sacc[tb]);
      __builtin_amdgcn_sched_barrier(0);
      i32x8_t rf, qr;
      lds_read_rq_asm<1024 * tb>(lr0, lr1, qa, rf, qr);
      sacc[tb] = mfma16x16x128_fp8(rf, qr, sacc[tb]);
      __builtin_amdgcn_sched_barrier(0);
      // next tile's copies, spread over the score products
      if (t + 1 < ntiles) {
#pragma unroll
        for (int k = 0; k < NC; ++k)
          if (k % 4 == tb && wave + k * NW < kCopiesF8) mla_f8_copy(Ln, Pn, rcn, rpn, wave + k * NW, lane);
      }
    });
    if (tok0 + kRowsF8 > t_end) {
#pragma unroll
      for (int tb = 0; tb < 4; ++tb)
#pragma unroll
        for (int r = 0; r < 4; ++r) sacc[tb][r] = tok0 + 16 * tb + 4 * g + r >= t_end ? -INFINITY : sacc[tb][r];
    }
    float hm = -INFINITY;
#pragma unroll
    for (int tb = 0; tb < 4; ++tb)
#pragma unroll
      for (int r = 0; r < 4; ++r) hm = fmaxf(hm, sacc[tb][r]);
    hm = fmaxf(hm, xor_lanes(hm, 16));
    hm = fmaxf(hm, xor_lanes(hm, 32));
    if (__any((hm - m) * c > kRescaleLog2F8)) {
      const float m_new = fmaxf(m, hm);
      const float alpha = fast_exp2((m - m_new) * c);
      l *= alpha;
#pragma unroll
      for (int db = 0; db < kC / 16; ++db) oacc[db] *= alpha;
      m = m_new;
    }
    const float mc = m * c - kPExpF8;
    uint32_t ph[4], pl[4];                             // P^T: hi and lo codes, one dword per 16-token block
#pragma unroll
    for (int tb = 0; tb < 4; ++tb) {
      float p[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        p[r] = fast_exp2(fmaf(sacc[tb][r], c, -mc));
        l += p[r];
      }
      uint32_t hw = f32x2_to_fp8(0u, p[0], p[1], false);
      hw = f32x2_to_fp8(hw, p[2], p[3], true);
      const f32x2_t d0 = fp8x2_to_f32(hw, false), d1 = fp8x2_to_f32(hw, true);
      const uint32_t lw = f32x2_to_fp8(0u, p[0] - d0[0], p[1] - d0[1], false);
      ph[tb] = hw;
      pl[tb] = f32x2_to_fp8(lw, p[2] - d1[0], p[3] - d1[1], true);
    }
    const i32x8_t bp = i32x8_t{int(ph[0]), int(ph[1]), int(ph[2]), int(ph[3]), int(pl[0]), int(pl[1]), int(pl[2]),
                               int(pl[3])};
    // O^T += V^T P^T: 16 latent channels per MFMA; the two V^T reads (16 tokens) serve the hi and lo positions
    const uint32_t lva = lds_u32(Lt) + va, lvb = lds_u32(Lt) + vb;
    static_for<kC / 64>([&](auto dqc) {
      constexpr int d0 = 4 * decltype(dqc)::value;     // four 16-channel blocks per read block
      i32x8_t v[4];
      lds_read_v4_asm<16 * d0, 32 * kLatPitch>((d0 & 8) ? lvb : lva, v);
#pragma unroll
      for (int i = 0; i < 4; ++i) oacc[d0 + i] = mfma16x16x128_fp8(v[i], bp, oacc[d0 + i]);
      __builtin_amdgcn_sched_barrier(0);
    });
  }

  float lt = l + xor_lanes(l, 16);
  lt += xor_lanes(lt, 32);
  const float inv = 1.f / lt;
  const int64_t slot = (int64_t(b) * a.heads + h) * a.n_split + split;
  float* wo = a.ws_o + slot * kC + 4 * g;
#pragma unroll
  for (int db = 0; db < kC / 16; ++db) {
    f32x4_t v = {oacc[db][0] * inv, oacc[db][1] * inv, oacc[db][2] * inv, oacc[db][3] * inv};
    v *= *reinterpret_cast<const f32x4_t*>(a.c_scale + 16 * db + 4 * g);   // code * s
    *reinterpret_cast<f32x4_t*>(wo + 16 * db) = v;
  }
  if (g == 0) a.ws_lse[slot] = m * ldexpf(a.scale, -kexp) + logf(lt) - kPExpF8 * 0.6931471805599453f;
}

// Merge splits: M = max lse_s, w_s = exp(lse_s - M), O = sum w_s O_s / sum w_s; length 0 -> O = 0, lse = -inf.
__global__ __launch_bounds__(256) void mla_combine_kernel(const float* __restrict__ ws_o,
    const float* __restrict__ ws_lse, const int32_t* __restrict__ seq_lens, uint16_t* __restrict__ o,
    float* __restrict__ lse, int heads, int n_split, int split_len, int max_len, int sparse) {
  const int h = blockIdx.x, b = blockIdx.y;
  const int L = max(0, min(seq_lens[b], max_len));
  // dense: the splits that cover tokens below L; sparse: every split (an empty one has lse = -inf, O = 0)
  const int ns = sparse ? n_split : (L + split_len - 1) / split_len;
  const int64_t base = (int64_t(b) * heads + h) * n_split;
  uint16_t* op = o + (int64_t(b) * heads + h) * kC;
  const int d0 = 2 * threadIdx.x;
  if (ns == 0) {
    *reinterpret_cast<uint32_t*>(op + d0) = 0u;
    if (lse && threadIdx.x == 0) lse[int64_t(b) * heads + h] = -INFINITY;
    return;
  }
  // Unrolled so that several independent partial loads are in flight (the loop is latency-bound otherwise).
  float mx = -INFINITY;
#pragma unroll 8
  for (int s = 0; s < ns; ++s) mx = fmaxf(mx, ws_lse[base + s]);
  if (mx == -INFINITY) {                               // sparse: nothing selected at all
    *reinterpret_cast<uint32_t*>(op + d0) = 0u;
    if (lse && threadIdx.x == 0) lse[int64_t(b) * heads + h] = -INFINITY;
    return;
  }
  float a0 = 0.f, a1 = 0.f, wsum = 0.f;
#pragma unroll 8
  for (int s = 0; s < ns; ++s) {
    const float w = expf(ws_lse[base + s] - mx);
    wsum += w;
    const f32x2_t v = *reinterpret_cast<const f32x2_t*>(ws_o + (base + s) * kC + d0);
    a0 = fmaf(w, v[0], a0);
    a1 = fmaf(w, v[1], a1);
  }
  *reinterpret_cast<uint32_t*>(op + d0) = pack_bf16x2(a0 / wsum, a1 / wsum);
  if (lse && threadIdx.x == 0) lse[int64_t(b) * heads + h] = mx + logf(wsum);
}

}  // namespace

// Workgroups the sparse form aims for: its splits are short (top-k tokens), so each split's partial output
// (heads x 512 fp32) is a large share of its traffic.
#ifndef ATTN_MLA_SPARSE_TARGET
#define ATTN_MLA_SPARSE_TARGET 256
#endif

int mla_num_splits(int batch, int n_heads, int max_seqlen_kv, int target) {
  (void)n_heads;
  if (batch <= 0 || max_seqlen_kv <= 0) return 1;
  const int by_cu = (target + batch - 1) / batch;
  const int by_len = (max_seqlen_kv + kRows - 1) / kRows;
  return max(1, min(by_cu, by_len));
}

int mla_split_len(int batch, int n_heads, int max_seqlen_kv, int target) {
  const int ns = mla_num_splits(batch, n_heads, max_seqlen_kv, target);
  const int per = (max(1, max_seqlen_kv) + ns - 1) / ns;
  return (per + kRows - 1) / kRows * kRows;
}

namespace {
size_t workspace_bytes(int batch, int n_heads, int kv_lora_rank, int len, int target) {
  if (batch <= 0 || n_heads <= 0 || kv_lora_rank <= 0 || len <= 0) return 0;
  const size_t slots = size_t(batch) * size_t(n_heads) * size_t(mla_num_splits(batch, n_heads, len, target));
  const size_t o_bytes = (slots * size_t(kv_lora_rank) * sizeof(float) + 255) & ~size_t(255);
  return o_bytes + slots * sizeof(float);
}
}  // namespace

size_t mla_decode_workspace_bytes(int batch, int n_heads, int kv_lora_rank, int max_seqlen_kv) {
  return workspace_bytes(batch, n_heads, kv_lora_rank, max_seqlen_kv, kTargetBlocks);
}

size_t mla_sparse_workspace_bytes(int batch, int n_heads, int kv_lora_rank, int topk) {
  return workspace_bytes(batch, n_heads, kv_lora_rank, topk, ATTN_MLA_SPARSE_TARGET);
}

hipError_t launch_mla_decode(const void* q_latent, const void* q_pe, const void* c_kv, const void* k_pe,
                             const int32_t* seq_lens, void* o_latent, float* lse, int batch, int n_heads,
                             int max_seqlen_kv, float scale, void* workspace, hipStream_t stream) {
  MlaArgs a = {};
  a.q_lat = static_cast<const uint16_t*>(q_latent);
  a.q_pe = static_cast<const uint16_t*>(q_pe);
  a.c_kv = static_cast<const uint16_t*>(c_kv);
  a.k_pe = static_cast<const uint16_t*>(k_pe);
  a.seq_lens = seq_lens;
  a.heads = n_heads; a.max_len = max_seqlen_kv; a.scale = scale;
  a.n_split = mla_num_splits(batch, n_heads, max_seqlen_kv, kTargetBlocks);
  a.split_len = mla_split_len(batch, n_heads, max_seqlen_kv, kTargetBlocks);
  const size_t slots = size_t(batch) * size_t(n_heads) * size_t(a.n_split);
  const size_t o_bytes = (slots * kC * sizeof(float) + 255) & ~size_t(255);
  a.ws_o = static_cast<float*>(workspace);
  a.ws_lse = reinterpret_cast<float*>(static_cast<char*>(workspace) + o_bytes);
  if (max_seqlen_kv > 0) {
    const dim3 grid(unsigned(a.n_split), unsigned(batch)), block(64 * (n_heads / kHeadsPerWave));
    switch (n_heads / kHeadsPerWave) {
      case 2: mla_split_kernel<2, false><<<grid, block, 0, stream>>>(a); break;
      case 4: mla_split_kernel<4, false><<<grid, block, 0, stream>>>(a); break;
      case 6: mla_split_kernel<6, false><<<grid, block, 0, stream>>>(a); break;
      default: mla_split_kernel<8, false><<<grid, block, 0, stream>>>(a); break;
    }
  }
  mla_combine_kernel<<<dim3(unsigned(n_heads), unsigned(batch)), dim3(kC / 2), 0, stream>>>(
      a.ws_o, a.ws_lse, seq_lens, static_cast<uint16_t*>(o_latent), lse, n_heads, a.n_split, a.split_len,
      max_seqlen_kv, 0);
  return hipGetLastError();
}

hipError_t launch_mla_decode_q8(const void* q_latent, const void* q_pe, const void* c_kv, const void* k_pe,
                                const float* c_scale, const float* pe_scale, int kind, const int32_t* seq_lens,
                                void* o_latent, float* lse, int batch, int n_heads, int max_seqlen_kv, float scale,
                                void* workspace, hipStream_t stream) {
  MlaArgs a = {};
  a.q_lat = static_cast<const uint16_t*>(q_latent);
  a.q_pe = static_cast<const uint16_t*>(q_pe);
  a.c_kv = static_cast<const uint16_t*>(c_kv);        // 8-bit codes, read as bytes
  a.k_pe = static_cast<const uint16_t*>(k_pe);
  a.c_scale = c_scale; a.pe_scale = pe_scale;
  a.seq_lens = seq_lens;
  a.heads = n_heads; a.max_len = max_seqlen_kv; a.scale = scale;
  a.n_split = mla_num_splits(batch, n_heads, max_seqlen_kv, kTargetBlocks);
  a.split_len = mla_split_len(batch, n_heads, max_seqlen_kv, kTargetBlocks);
  const size_t slots = size_t(batch) * size_t(n_heads) * size_t(a.n_split);
  const size_t o_bytes = (slots * kC * sizeof(float) + 255) & ~size_t(255);
  a.ws_o = static_cast<float*>(workspace);
  a.ws_lse = reinterpret_cast<float*>(static_cast<char*>(workspace) + o_bytes);
  if (max_seqlen_kv > 0) {
    const dim3 grid(unsigned(a.n_split), unsigned(batch)), block(64 * (n_heads / kHeadsPerWave));
    const bool fp8 = kind == kKvFp8;
    if (fp8 && ATTN_MLA_FP8_MMA) {
      switch (n_heads / kHeadsPerWave) {
        case 2: mla_split_fp8mma_kernel<2><<<grid, block, 0, stream>>>(a); break;
        case 4: mla_split_fp8mma_kernel<4><<<grid, block, 0, stream>>>(a); break;
        case 6: mla_split_fp8mma_kernel<6><<<grid, block, 0, stream>>>(a); break;
        default: mla_split_fp8mma_kernel<8><<<grid, block, 0, stream>>>(a); break;
      }
    } else {
      switch (n_heads / kHeadsPerWave) {
        case 2: fp8 ? mla_split_kernel<2, false, kKvFp8><<<grid, block, 0, stream>>>(a)
                    : mla_split_kernel<2, false, kKvInt8><<<grid, block, 0, stream>>>(a); break;
        case 4: fp8 ? mla_split_kernel<4, false, kKvFp8><<<grid, block, 0, stream>>>(a)
                    : mla_split_kernel<4, false, kKvInt8><<<grid, block, 0, stream>>>(a); break;
        case 6: fp8 ? mla_split_kernel<6, false, kKvFp8><<<grid, block, 0, stream>>>(a)
                    : mla_split_kernel<6, false, kKvInt8><<<grid, block, 0, stream>>>(a); break;
        default: fp8 ? mla_split_kernel<8, false, kKvFp8><<<grid, block, 0, stream>>>(a)
                     : mla_split_kernel<8, false, kKvInt8><<<grid, block, 0, stream>>>(a); break;
      }
    }
  }
  mla_combine_kernel<<<dim3(unsigned(n_heads), unsigned(batch)), dim3(kC / 2), 0, stream>>>(
      a.ws_o, a.ws_lse, seq_lens, static_cast<uint16_t*>(o_latent), lse, n_heads, a.n_split, a.split_len,
      max_seqlen_kv, 0);
  return hipGetLastError();
}

hipError_t launch_mla_sparse_decode(const void* q_latent, const void* q_pe, const void* c_kv, const void* k_pe,
                                    const int32_t* seq_lens, const int32_t* indices, void* o_latent, float* lse,
                                    int batch, int n_heads, int max_seqlen_kv, int topk, float scale, void* workspace,
                                    hipStream_t stream) {
  MlaArgs a = {};
  a.q_lat = static_cast<const uint16_t*>(q_latent);
  a.q_pe = static_cast<const uint16_t*>(q_pe);
  a.c_kv = static_cast<const uint16_t*>(c_kv);
  a.k_pe = static_cast<const uint16_t*>(k_pe);
  a.seq_lens = seq_lens;
  a.idx = indices;
  a.topk = topk;
  a.heads = n_heads; a.max_len = max_seqlen_kv; a.scale = scale;
  a.n_split = mla_num_splits(batch, n_heads, topk, ATTN_MLA_SPARSE_TARGET);
  a.split_len = mla_split_len(batch, n_heads, topk, ATTN_MLA_SPARSE_TARGET);
  const size_t slots = size_t(batch) * size_t(n_heads) * size_t(a.n_split);
  const size_t o_bytes = (slots * kC * sizeof(float) + 255) & ~size_t(255);
  a.ws_o = static_cast<float*>(workspace);
  a.ws_lse = reinterpret_cast<float*>(static_cast<char*>(workspace) + o_bytes);
  const dim3 grid(unsigned(a.n_split), unsigned(batch)), block(64 * (n_heads / kHeadsPerWave));
  switch (n_heads / kHeadsPerWave) {
    case 2: mla_split_kernel<2, true><<<grid, block, 0, stream>>>(a); break;
    case 4: mla_split_kernel<4, true><<<grid, block, 0, stream>>>(a); break;
    case 6: mla_split_kernel<6, true><<<grid, block, 0, stream>>>(a); break;
    default: mla_split_kernel<8, true><<<grid, block, 0, stream>>>(a); break;
  }
  mla_combine_kernel<<<dim3(unsigned(n_heads), unsigned(batch)), dim3(kC / 2), 0, stream>>>(
      a.ws_o, a.ws_lse, seq_lens, static_cast<uint16_t*>(o_latent), lse, n_heads, a.n_split, a.split_len,
      max_seqlen_kv, 1);
  return hipGetLastError();
}

}  // namespace attn
