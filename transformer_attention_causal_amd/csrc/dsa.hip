// dsa.hip — DeepSeek Sparse Attention selection for decode: the lightning indexer and the top-k selection.
//
// (Attention notes, makinaruto.github.io, "Lighting Indexer": every earlier token s is scored for the current
//  query token by the sum over indexer heads j of w_j * ReLU(q_j . k_s), with one indexer key per token shared by
//  all indexer heads; only the most relevant tokens then take part in the attention.)
//
// Indexer. One query token per sequence, so per 32 cached tokens the scores of all H_I indexer heads are one
// (H_I x D_I) x (D_I x 32) product: v_mfma_f32_32x32x16_bf16 with the heads as rows (A, resident in registers for
// the whole kernel) and the tokens as columns (B). A lane's B operand is 8 consecutive values of ONE token's key;
// the contraction order over the D_I dims is permuted (k-step ks, lane half hh takes dims (D_I/2)*hh + 8*ks ..)
// identically on both operands, so a lane's fragments of a key row are contiguous. Key rows reach the fragments
// through LDS: each wave copies blocks of 32 whole rows global -> LDS (non-temporal buffer loads with the LDS bit,
// 1 KiB of contiguous rows per instruction), double-buffered, and reads its fragments with swizzled 16-byte LDS
// reads (measured with cold caches: 77.8 -> 53.0 us against loading the fragments straight from HBM, whose 16-byte
// pieces of 32 rows per instruction the memory pipeline serves poorly). After the product a lane holds 16 head
// rows of one token: ReLU, times the head weight, summed in registers, then one exchange with lane l^32.
// HBM-bound: every key row is read once (256 bytes per token at D_I = 128) and one fp32 score written.
//
// Top-k. One workgroup per sequence holds the sequence's scores in registers (32 per lane for up to 32768 tokens;
// longer sequences are taken in rounds of 32768) as order-preserving 32-bit keys, finds the k-th largest key by
// radix selection (four 8-bit digits from the top; LDS histograms in 16 lane-interleaved copies so that the
// heavily shared leading digits do not serialise the atomics), then writes the indices above the threshold and the
// lowest-index ties at it, in ascending order, from wave-wide ballot counts. Deterministic; no workspace.
#include "device.h"
#include "kernels.h"

namespace attn {
namespace {

constexpr int kIdxWaves = 4;            // waves per indexer workgroup
#ifndef ATTN_IDX_KPW
#define ATTN_IDX_KPW 1024
#endif
// LDS buffers per wave in the staged path (2: one block's copy in flight while one is scored; 3: two).
#ifndef ATTN_IDX_NBUF
#define ATTN_IDX_NBUF 2
#endif
#ifndef ATTN_IDX_PIPE
#define ATTN_IDX_PIPE 2
#endif
#ifndef ATTN_IDX_NT
#define ATTN_IDX_NT 0
#endif
// 1: key rows staged through LDS by whole-row copies (each wave its own two 32-row buffers); 0: loaded straight
// into operand registers.
#ifndef ATTN_IDX_LDS
#define ATTN_IDX_LDS 1
#endif
constexpr int kIdxKeysPerWave = ATTN_IDX_KPW;   // tokens per wave (blocks of 32)
constexpr int kIdxPipe = ATTN_IDX_PIPE;         // 32-token blocks of key rows in registers (kIdxPipe - 1 in flight)

template <int HI, int DI>
__global__ __launch_bounds__(64 * kIdxWaves, 2) void dsa_indexer_kernel(const uint16_t* __restrict__ q_idx,
    const float* __restrict__ w_idx, const uint16_t* __restrict__ k_idx, const int32_t* __restrict__ seq_lens,
    float* __restrict__ scores, int max_len) {
  constexpr int MB = HI / 32;          // 32-head row blocks
  constexpr int KS = DI / 16;          // k-steps
  const int b = blockIdx.y;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int col = lane & 31, hh = lane >> 5;
  const int key_begin = (blockIdx.x * kIdxWaves + wave) * kIdxKeysPerWave;
  if (key_begin >= max_len) return;
  const int key_end = min(max_len, key_begin + kIdxKeysPerWave);
  const int L = max(0, min(seq_lens[b], max_len));
  float* srow = scores + int64_t(b) * max_len;
  if (key_begin >= L) {                                // nothing to score: the slots past the length are -inf
    for (int t = key_begin + lane; t < key_end; t += 64) srow[t] = -INFINITY;
    return;
  }

  // A operands: head 32*mb + col, dims (DI/2)*hh + 8*ks ..; head weights of the 16 rows a lane holds after the
  // product (row 8*(r/4) + 4*hh + r%4 of each 32-head block).
  bf16x8_t qa[MB][KS];
  float wr[MB][16];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) {
    const uint16_t* qp = q_idx + (int64_t(b) * HI + 32 * mb + col) * DI + (DI / 2) * hh;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) qa[mb][ks] = as_bf16x8(*reinterpret_cast<const u32x4_t*>(qp + 8 * ks));
#pragma unroll
    for (int r = 0; r < 16; ++r) wr[mb][r] = w_idx[int64_t(b) * HI + 32 * mb + 8 * (r / 4) + 4 * hh + (r % 4)];
  }

  const uint16_t* kbase = k_idx + int64_t(b) * max_len * DI + (DI / 2) * hh;
  // Key row of this lane's token in block key0 (clamped into the sequence: finite data, result discarded).
  auto load_block = [&](u32x4_t (&kb)[KS], int key0) {
    const uint16_t* kp = kbase + int64_t(min(key0 + col, L - 1)) * DI;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const u32x4_t* src = reinterpret_cast<const u32x4_t*>(kp + 8 * ks);
      kb[ks] = ATTN_IDX_NT ? __builtin_nontemporal_load(src) : *src;   // read once: non-temporal
    }
  };
  auto score_block = [&](const u32x4_t (&kb)[KS], int key0) {
    float part = 0.f;
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
      f32x16_t acc = {};
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) acc = mfma32x32x16(qa[mb][ks], as_bf16x8(kb[ks]), acc);
#pragma unroll
      for (int r = 0; r < 16; ++r) part = fmaf(wr[mb][r], fmaxf(acc[r], 0.f), part);
    }
    part += xor_lanes(part, 32);
    const int t = key0 + col;
    if (hh == 0 && t < key_end) srow[t] = t < L ? part : -INFINITY;
  };

  const int nblk = (key_end - key_begin + 31) / 32;
  if constexpr (ATTN_IDX_LDS) {
    // Blocks of 32 key rows copied global -> LDS with the LDS bit (1 KiB of contiguous rows per instruction, the
    // copy of block i+1 in flight while block i is scored), then read as operand fragments. Chunk c of row r is
    // stored at c ^ swz(r), which makes the 16-byte fragment reads (32 rows at one chunk) conflict-free on the
    // 64-bank LDS. Rows at or past L are outside the block's buffer resource and read as zeros (scores discarded).
    constexpr int RB = 2 * DI;                 // bytes per key row
    constexpr int NCH = DI / 8;                // 16-byte chunks per row
    constexpr int RPI = 1024 / RB;             // rows per copy instruction
    constexpr int NI = 32 / RPI;               // copy instructions per block
    constexpr int NB = ATTN_IDX_NBUF;
    static_assert(NB == 2 || NB == 3, "two or three buffers");
    __shared__ __attribute__((aligned(16))) uint16_t kl0[kIdxWaves][32 * DI], kl1[kIdxWaves][32 * DI],
        kl2[kIdxWaves][NB > 2 ? 32 * DI : 8];
    auto buf = [&](auto bc) -> uint16_t* {
      constexpr int B = decltype(bc)::value;
      if constexpr (B == 0) return kl0[wave]; else if constexpr (B == 1) return kl1[wave]; else return kl2[wave];
    };
    auto swz = [](int r) { return (NCH == 16 ? r : r >> 1) & (NCH - 1); };
    const uint16_t* kseq = k_idx + int64_t(b) * max_len * DI;
    const int crow = lane / NCH, cslot = lane % NCH;
    auto copy_block = [&](uint16_t* dst, int key0) {
      const buf_rsrc_t rs = make_buf_rsrc(kseq + int64_t(key0) * DI, uint32_t(max(0, min(32, L - key0))) * RB);
#pragma unroll
      for (int j = 0; j < NI; ++j) {
        const int r = RPI * j + crow;
        load_lds16<2>(rs, uint32_t(r * RB + 16 * (cslot ^ swz(r))), dst + j * 512);
      }
    };
    uint32_t koff[KS];                         // lane (col, hh): row col, chunk (NCH/2)*hh + ks
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) koff[ks] = uint32_t(col * RB + 16 * (((NCH / 2) * hh + ks) ^ swz(col)));
    auto read_block = [&](const uint16_t* src, u32x4_t (&kb)[KS]) {
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) kb[ks] = lds_read16(src, koff[ks]);
    };
    wait_vmem();                               // query and weights are in: only block copies are outstanding now
    constexpr int PRE = NB - 1;                // blocks in flight while one is scored
    copy_block(buf(std::integral_constant<int, 0>{}), key_begin);
    if (PRE >= 2 && 1 < nblk) copy_block(buf(std::integral_constant<int, 1>{}), key_begin + 32);
    u32x4_t kb[KS];
    for (int u = 0; u < nblk; u += NB) {
#pragma unroll
      for (int k = 0; k < NB; ++k) {
        const int i = u + k;
        if (i >= nblk) break;
        // issue block i + PRE into the buffer read at step i - 1, then wait for block i (the PRE blocks after it
        // may stay in flight)
        const int nfly = min(PRE, nblk - 1 - i);
        if (nfly == PRE) {
          const int nb = (k + PRE) % NB;         // resolves at compile time once the loop is unrolled
          uint16_t* dst = nb == 0 ? buf(std::integral_constant<int, 0>{})
                        : nb == 1 ? buf(std::integral_constant<int, 1>{}) : buf(std::integral_constant<int, 2>{});
          copy_block(dst, key_begin + 32 * (i + PRE));
        }
        if (nfly >= 2) asm volatile("s_waitcnt vmcnt(%0)" ::"n"(2 * NI) : "memory");
        else if (nfly == 1) asm volatile("s_waitcnt vmcnt(%0)" ::"n"(NI) : "memory");
        else wait_vmem();
        const uint16_t* src = k == 0 ? buf(std::integral_constant<int, 0>{})
                            : k == 1 ? buf(std::integral_constant<int, 1>{}) : buf(std::integral_constant<int, 2>{});
        read_block(src, kb);
        score_block(kb, key_begin + 32 * i);
      }
    }
    return;
  }
  // Blocks of 32 tokens in a ring of kIdxPipe register buffers: the next kIdxPipe - 1 blocks' key rows are in
  // flight while one is scored.
  u32x4_t kb[kIdxPipe][KS];
#pragma unroll
  for (int p = 0; p + 1 < kIdxPipe; ++p)
    if (p < nblk) load_block(kb[p], key_begin + 32 * p);
  for (int i = 0; i < nblk; i += kIdxPipe) {
#pragma unroll
    for (int u = 0; u < kIdxPipe; ++u) {
      const int blk = i + u;
      if (blk >= nblk) break;
      if (blk + kIdxPipe - 1 < nblk) load_block(kb[(u + kIdxPipe - 1) % kIdxPipe], key_begin + 32 * (blk + kIdxPipe - 1));
      score_block(kb[u], key_begin + 32 * blk);
    }
  }
}

// ---------------------------------------------------------------------------------------------------- top-k --
constexpr int kTopkThreads = 1024;
constexpr int kTopkWaves = kTopkThreads / 64;
constexpr int kTopkPer = 32;                          // scores per lane held in registers per round
constexpr int kTopkRound = kTopkThreads * kTopkPer;   // 32768 scores per round (one round for <= 32768 tokens)
// The digit histogram is kept in kHistCopies copies, lane l counting into copy l % kHistCopies: the leading
// digits are shared by most keys, and same-address LDS atomics serialise. Copy stride 257 words puts the copies of
// one bin in distinct banks.
constexpr int kHistCopies = 16;
constexpr int kHistStride = 257;

// Order-preserving key: a larger float gives a larger unsigned key (-0 is taken as +0). Every NaN maps to key 0,
// below -inf's key 0x007fffff: a NaN score is the least relevant, and NaNs tie (the lower index wins).
__device__ __forceinline__ uint32_t order_key(float f) {
  const uint32_t u = __float_as_uint(f == 0.f ? 0.f : f);
  const uint32_t k = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
  return f != f ? 0u : k;
}

// Number of set bits of `m` below this lane.
__device__ __forceinline__ int lanes_below(uint64_t m) {
  return int(__builtin_amdgcn_mbcnt_hi(uint32_t(m >> 32), __builtin_amdgcn_mbcnt_lo(uint32_t(m), 0u)));
}

// Round r covers scores [r*kTopkRound, (r+1)*kTopkRound); in it wave w owns the contiguous segment of 64*kTopkPer
// scores starting at w*64*kTopkPer, and lane i holds its scores 64*j + i (j < kTopkPer) as keys in registers, so
// every pass over a resident round reads registers only and the ordered write-out needs only wave-wide counts.
__global__ __launch_bounds__(kTopkThreads) void topk_kernel(const float* __restrict__ scores,
    const int32_t* __restrict__ seq_lens, int32_t* __restrict__ out, int max_len, int k) {
  __shared__ uint32_t hist[kHistCopies * kHistStride];
  __shared__ int wtot[2][kTopkWaves];
  __shared__ uint32_t sel_digit, sel_above;
  const int b = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int n = max(0, min(seq_lens[b], max_len));
  const int kk = min(k, n);
  const float* s = scores + int64_t(b) * max_len;
  int32_t* o = out + int64_t(b) * k;
  if (kk == n) {                                       // every token is kept
    for (int i = tid; i < k; i += kTopkThreads) o[i] = i < n ? i : -1;
    return;
  }
  const int rounds = (n + kTopkRound - 1) / kTopkRound;
  uint32_t x[kTopkPer];
  auto first = [&](int r) { return r * kTopkRound + wave * (64 * kTopkPer) + lane; };   // index of x[0]
  auto load_round = [&](int r) {
    const int i0 = first(r);
#pragma unroll
    for (int j = 0; j < kTopkPer; ++j) x[j] = order_key(s[min(i0 + 64 * j, n - 1)]);   // unconditional: all in flight
  };
  if (rounds == 1) load_round(0);

  // ---- radix selection of the kk-th largest key: after digit pass p the top 8(p+1) bits of the threshold are
  // known (prefix under mask) and krem more keys with that prefix must be taken.
  uint32_t prefix = 0, mask = 0;
  int krem = kk;
  for (int pass = 0; pass < 4; ++pass) {
    const int shift = 24 - 8 * pass;
    for (int i = tid; i < kHistCopies * kHistStride; i += kTopkThreads) hist[i] = 0;
    __syncthreads();
    uint32_t* my_hist = hist + (lane % kHistCopies) * kHistStride;
    for (int r = 0; r < rounds; ++r) {
      if (rounds > 1) load_round(r);
      const int i0 = first(r);
#pragma unroll
      for (int j = 0; j < kTopkPer; ++j) {
        if (i0 + 64 * j < n && (x[j] & mask) == prefix) atomicAdd(&my_hist[(x[j] >> shift) & 255u], 1u);
      }
    }
    __syncthreads();
    if (wave == 0) {
      // bins in descending order: lane j takes bins 255-4j .. 252-4j
      uint32_t c[4], t = 0;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        c[q] = 0;
        for (int cp = 0; cp < kHistCopies; ++cp) c[q] += hist[cp * kHistStride + 255 - 4 * lane - q];
        t += c[q];
      }
      uint32_t incl = t;
#pragma unroll
      for (int off = 1; off < 64; off <<= 1) {
        const uint32_t y = __shfl_up(incl, off, 64);
        if (lane >= off) incl += y;
      }
      uint32_t cum = incl - t;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        if (cum < uint32_t(krem) && cum + c[q] >= uint32_t(krem)) { sel_digit = 255 - 4 * lane - q; sel_above = cum; }
        cum += c[q];
      }
    }
    __syncthreads();
    prefix |= sel_digit << shift;
    mask |= 255u << shift;
    krem -= int(sel_above);
    __syncthreads();                                   // sel_* are rewritten by the next pass
  }
  const uint32_t thr = prefix;                          // the kk-th largest key; krem ties at thr are taken

  // ---- ordered write-out, round by round: keys above thr, and the first krem keys equal to thr (by index).
  int eq_carry = 0, sel_carry = 0;                      // ties and selections in earlier rounds
  for (int r = 0; r < rounds; ++r) {
    if (rounds > 1) load_round(r);
    const int i0 = first(r);
    int gtc = 0, eqc = 0;
#pragma unroll
    for (int j = 0; j < kTopkPer; ++j) {
      const bool v = i0 + 64 * j < n;
      gtc += __popcll(__ballot(v && x[j] > thr));
      eqc += __popcll(__ballot(v && x[j] == thr));
    }
    if (lane == 0) { wtot[0][wave] = gtc; wtot[1][wave] = eqc; }
    __syncthreads();
    int eq_seen = eq_carry, pos = sel_carry, eq_run = eq_carry, sel_run = sel_carry;
    for (int v = 0; v < kTopkWaves; ++v) {              // segments in index order
      const int g = wtot[0][v], e = wtot[1][v];
      if (v == wave) { eq_seen = eq_run; pos = sel_run; }
      sel_run += g + max(0, min(e, krem - eq_run));
      eq_run += e;
    }
    __syncthreads();                                   // wtot is rewritten by the next round
    eq_carry = eq_run;
    sel_carry = sel_run;
#pragma unroll
    for (int j = 0; j < kTopkPer; ++j) {
      const int i = i0 + 64 * j;
      const bool v = i < n;
      const bool above = v && x[j] > thr, tie = v && x[j] == thr;
      const uint64_t em = __ballot(tie);
      const bool sel = above || (tie && eq_seen + lanes_below(em) < krem);
      const uint64_t sm = __ballot(sel);
      const int p = pos + lanes_below(sm);
      if (sel && p < kk) o[p] = i;                     // p < kk always holds for a consistent selection
      pos += __popcll(sm);
      eq_seen += __popcll(em);
    }
  }
  for (int i = kk + tid; i < k; i += kTopkThreads) o[i] = -1;
}

}  // namespace

hipError_t launch_dsa_indexer(const void* q_idx, const float* w_idx, const void* k_idx, const int32_t* seq_lens,
                              float* scores, int batch, int n_heads_idx, int idx_dim, int max_seqlen_kv,
                              hipStream_t stream) {
  if (batch <= 0 || max_seqlen_kv <= 0) return hipSuccess;
  const int per_wg = kIdxWaves * kIdxKeysPerWave;
  const dim3 grid(unsigned((max_seqlen_kv + per_wg - 1) / per_wg), unsigned(batch)), block(64 * kIdxWaves);
  const uint16_t* q = static_cast<const uint16_t*>(q_idx);
  const uint16_t* kk = static_cast<const uint16_t*>(k_idx);
  if (n_heads_idx == 64 && idx_dim == 128)
    dsa_indexer_kernel<64, 128><<<grid, block, 0, stream>>>(q, w_idx, kk, seq_lens, scores, max_seqlen_kv);
  else if (n_heads_idx == 64)
    dsa_indexer_kernel<64, 64><<<grid, block, 0, stream>>>(q, w_idx, kk, seq_lens, scores, max_seqlen_kv);
  else if (idx_dim == 128)
    dsa_indexer_kernel<32, 128><<<grid, block, 0, stream>>>(q, w_idx, kk, seq_lens, scores, max_seqlen_kv);
  else
    dsa_indexer_kernel<32, 64><<<grid, block, 0, stream>>>(q, w_idx, kk, seq_lens, scores, max_seqlen_kv);
  return hipGetLastError();
}

hipError_t launch_topk(const float* scores, const int32_t* seq_lens, int32_t* indices, int batch, int max_seqlen_kv,
                       int k, hipStream_t stream) {
  if (batch <= 0 || k <= 0) return hipSuccess;
  topk_kernel<<<dim3(unsigned(batch)), dim3(kTopkThreads), 0, stream>>>(scores, seq_lens, indices, max_seqlen_kv, k);
  return hipGetLastError();
}

}  // namespace attn
