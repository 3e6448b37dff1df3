// dsa.hip — DeepSeek Sparse Attention selection for decode: the lightning indexer and the top-k selection.
//
// (Attention notes, makinaruto.github.io, "Lighting Indexer": every earlier token s is scored for the current
//  query token by the sum over indexer heads j of w_j * ReLU(q_j . k_s), with one indexer key per token shared by
//  all indexer heads; only the most relevant tokens then take part in the attention.)
//
// Indexer. One query token per sequence, so per 32 cached tokens the scores of all H_I indexer heads are one
// (H_I x D_I) x (D_I x 32) product: v_mfma_f32_32x32x16_bf16 with the heads as rows (A, resident in registers for
// the whole kernel) and the tokens as columns (B). A lane's B operand is 8 consecutive values of ONE token's key,
// so the key rows load straight from HBM into operand registers with 16-byte loads; the contraction order over
// the D_I dims is permuted (k-step ks, lane half hh takes dims (D_I/2)*hh + 8*ks ..) identically on both operands,
// which makes each lane's loads of a key row contiguous. After the product a lane holds 16 head rows of one
// token: ReLU, times the head weight, summed in registers, then one exchange with lane l^32. HBM-bound: every key
// row is read once (256 bytes per token at D_I = 128) and one fp32 score written.
//
// Top-k. One workgroup per sequence finds the k-th largest score by radix selection on an order-preserving 32-bit
// key (four 8-bit digits from the top; LDS histograms with wave-aggregated atomics for the heavily shared leading
// digits), then writes the indices above the threshold and the lowest-index ties at it, in ascending order, with
// two block-wide prefix sums. Deterministic; no workspace.
#include "device.h"
#include "kernels.h"

namespace attn {
namespace {

constexpr int kIdxWaves = 4;            // waves per indexer workgroup
constexpr int kIdxKeysPerWave = 256;    // tokens per wave (8 blocks of 32)

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
    for (int ks = 0; ks < KS; ++ks) kb[ks] = *reinterpret_cast<const u32x4_t*>(kp + 8 * ks);
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

  // Blocks of 32 tokens, the next block's key rows in flight while the current one is scored.
  const int nblk = (key_end - key_begin + 31) / 32;
  u32x4_t k0[KS], k1[KS];
  load_block(k0, key_begin);
  for (int i = 0; i < nblk; i += 2) {
    if (i + 1 < nblk) load_block(k1, key_begin + 32 * (i + 1));
    score_block(k0, key_begin + 32 * i);
    if (i + 1 >= nblk) break;
    if (i + 2 < nblk) load_block(k0, key_begin + 32 * (i + 2));
    score_block(k1, key_begin + 32 * (i + 1));
  }
}

// ---------------------------------------------------------------------------------------------------- top-k --
constexpr int kTopkThreads = 1024;
constexpr int kTopkWaves = kTopkThreads / 64;

// Order-preserving key: a larger float gives a larger unsigned key (-0 is taken as +0).
__device__ __forceinline__ uint32_t order_key(float f) {
  const uint32_t u = __float_as_uint(f == 0.f ? 0.f : f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Exclusive prefix sum over the workgroup (threads in order); `total` gets the sum. Uses red[0..kTopkWaves).
__device__ int block_exclusive_scan(int v, int* red, int& total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int x = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int y = __shfl_up(x, o, 64);
    if (lane >= o) x += y;
  }
  if (lane == 63) red[wave] = x;
  __syncthreads();
  int before = 0, sum = 0;
  for (int i = 0; i < kTopkWaves; ++i) {
    const int t = red[i];
    if (i < wave) before += t;
    sum += t;
  }
  __syncthreads();                                     // red is free again
  total = sum;
  return before + x - v;
}

__global__ __launch_bounds__(kTopkThreads) void topk_kernel(const float* __restrict__ scores,
    const int32_t* __restrict__ seq_lens, int32_t* __restrict__ out, int max_len, int k) {
  __shared__ uint32_t hist[256];
  __shared__ int red[kTopkWaves];
  __shared__ uint32_t sel_digit, sel_above;
  const int b = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int n = max(0, min(seq_lens[b], max_len));
  const int kk = min(k, n);
  const float* s = scores + int64_t(b) * max_len;
  int32_t* o = out + int64_t(b) * k;
  if (kk == n) {                                       // every token is kept
    for (int i = tid; i < k; i += kTopkThreads) o[i] = i < n ? i : -1;
    return;
  }

  // ---- radix selection of the kk-th largest key: after digit pass p the top 8(p+1) bits of the threshold are
  // known (prefix under mask) and krem more elements with that prefix must be taken.
  uint32_t prefix = 0, mask = 0;
  int krem = kk;
  for (int pass = 0; pass < 4; ++pass) {
    const int shift = 24 - 8 * pass;
    if (tid < 256) hist[tid] = 0;
    __syncthreads();
    for (int i0 = 0; i0 < n; i0 += kTopkThreads) {     // uniform trip count: every lane takes part in the ballots
      const int i = i0 + tid;
      uint32_t key = 0;
      bool act = false;
      if (i < n) {
        key = order_key(s[i]);
        act = (key & mask) == prefix;
      }
      const uint32_t d = (key >> shift) & 255u;
      const uint64_t am = __ballot(act);
      if (am) {
        // the digit of the first active lane is counted with one atomic (leading digits are shared by most
        // keys, and same-address LDS atomics serialise); the others individually
        const int leader = __builtin_ctzll(am);
        const uint32_t d0 = __shfl(d, leader, 64);
        const uint64_t same = __ballot(act && d == d0);
        if (lane == leader) atomicAdd(&hist[d0], uint32_t(__popcll(same)));
        if (act && d != d0) atomicAdd(&hist[d], 1u);
      }
    }
    __syncthreads();
    if (wave == 0) {
      // bins in descending order: lane j takes bins 255-4j .. 252-4j
      uint32_t c[4], t = 0;
#pragma unroll
      for (int q = 0; q < 4; ++q) { c[q] = hist[255 - 4 * lane - q]; t += c[q]; }
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

  // ---- ordered compaction: thread t owns elements [t*E, (t+1)*E)
  const int E = (n + kTopkThreads - 1) / kTopkThreads;
  const int lo = min(n, tid * E), hi = min(n, lo + E);
  int gt = 0, eq = 0;
  for (int i = lo; i < hi; ++i) {
    const uint32_t key = order_key(s[i]);
    gt += key > thr;
    eq += key == thr;
  }
  int tot;
  const int eq_before = block_exclusive_scan(eq, red, tot);
  const int take_eq = max(0, min(eq, krem - eq_before));
  int pos = block_exclusive_scan(gt + take_eq, red, tot);
  int taken = 0;
  for (int i = lo; i < hi; ++i) {
    const uint32_t key = order_key(s[i]);
    if (key > thr || (key == thr && taken < take_eq)) {
      taken += key == thr;
      if (pos < kk) o[pos] = i;                        // always true for a consistent selection; keeps writes in the row
      ++pos;
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
