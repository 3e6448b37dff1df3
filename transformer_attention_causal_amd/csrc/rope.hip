// rope.hip — rotary position embedding, in place, for bf16 or fp32 rows [n_tokens, n_heads, head_dim].
//
// (DeepSeek 32K to 256K long context, tqpw.cn, section 2.1: pair i of the head dimension is rotated by the
//  matrix [cos -sin; sin cos] of angle position * theta^(-2i/d); section 2.5: a cos/sin table indexed by integer
//  positions, so the angle is never accumulated.)
//
// One workgroup takes kTokens consecutive token rows. It first builds, in LDS, the frequency table
// theta^(-2i/d) (fp64) and then the cos/sin table of its tokens: angle = position * frequency in fp64, sin and
// cos in fp64 (full range reduction), rounded to fp32. Every head of a token reuses the same table row, so the
// fp64 work is d/2 angles per token, not per element. The rotation itself is fp32 FMA on 16-byte vectors,
// rounded back to the storage type (bf16: nearest even). HBM-bound: one read and one write of x.
// rope_table_kernel writes the same cos/sin values for every position of a range, for the prefill kernel's fused
// rotation of Q.
#include "device.h"
#include "kernels.h"

namespace attn {
namespace {

constexpr int kRopeThreads = 256;
constexpr int kTokens = 4;          // token rows per workgroup
constexpr int kMaxPairs = 512;      // head_dim <= 1024

template <typename T> struct Elem;
template <> struct Elem<uint16_t> {   // bf16 storage
  static __device__ __forceinline__ float load(const uint16_t* p) { return __uint_as_float(uint32_t(*p) << 16); }
  static __device__ __forceinline__ void store(uint16_t* p, float v) { *p = uint16_t(pack_bf16x2(v, 0.f)); }
};
template <> struct Elem<float> {
  static __device__ __forceinline__ float load(const float* p) { return *p; }
  static __device__ __forceinline__ void store(float* p, float v) { *p = v; }
};

// Unpack / pack 16 bytes of storage type T into fp32 lanes.
template <typename T> struct Vec16;
template <> struct Vec16<uint16_t> {
  static constexpr int N = 8;
  static __device__ __forceinline__ void unpack(u32x4_t w, float* f) {
    for (int i = 0; i < 4; ++i) { f[2 * i] = bf16lo_to_f32(w[i]); f[2 * i + 1] = bf16hi_to_f32(w[i]); }
  }
  static __device__ __forceinline__ u32x4_t pack(const float* f) {
    u32x4_t w;
    for (int i = 0; i < 4; ++i) w[i] = pack_bf16x2(f[2 * i], f[2 * i + 1]);
    return w;
  }
};
template <> struct Vec16<float> {
  static constexpr int N = 4;
  static __device__ __forceinline__ void unpack(u32x4_t w, float* f) {
    for (int i = 0; i < 4; ++i) f[i] = __uint_as_float(w[i]);
  }
  static __device__ __forceinline__ u32x4_t pack(const float* f) {
    u32x4_t w;
    for (int i = 0; i < 4; ++i) w[i] = __float_as_uint(f[i]);
    return w;
  }
};

// Fill cs[tok][i] = (cos, sin) of positions[t0 + tok] * theta^(-2i/d).
__device__ __forceinline__ void build_table(float2 (*cs)[kMaxPairs], double* inv_freq, const int32_t* positions,
                                            int64_t t0, int64_t n_tokens, int head_dim, double theta) {
  const int half = head_dim / 2;
  for (int i = threadIdx.x; i < half; i += kRopeThreads)
    inv_freq[i] = pow(theta, -2.0 * double(i) / double(head_dim));
  __syncthreads();
  for (int e = threadIdx.x; e < kTokens * half; e += kRopeThreads) {
    const int tok = e / half, i = e % half;
    if (t0 + tok < n_tokens) {
      const double ang = double(positions[t0 + tok]) * inv_freq[i];
      double s, c;
      sincos(ang, &s, &c);
      cs[tok][i] = make_float2(float(c), float(s));
    }
  }
  __syncthreads();
}

// 16-byte vectors (x 16-byte aligned; interleaved: head_dim % N == 0, half-split: (head_dim/2) % N == 0,
// N = elements per 16 bytes). Interleaved: one vector holds N/2 whole pairs.
// Half-split: a vector at dims [d0, d0 + N) pairs with the vector at [d0 + d/2, d0 + d/2 + N).
template <typename T, bool kInterleaved>
__global__ __launch_bounds__(kRopeThreads) void rope_vec_kernel(T* __restrict__ x, const int32_t* __restrict__ positions,
                                                               int64_t n_tokens, int n_heads, int head_dim, double theta) {
  __shared__ float2 cs[kTokens][kMaxPairs];
  __shared__ double inv_freq[kMaxPairs];
  const int64_t t0 = int64_t(blockIdx.x) * kTokens;
  build_table(cs, inv_freq, positions, t0, n_tokens, head_dim, theta);
  constexpr int N = Vec16<T>::N;
  const int row = n_heads * head_dim;                                  // elements per token row
  const int units_per_tok = kInterleaved ? row / N : row / (2 * N);    // 16-byte units (half-split: unit pairs)
  for (int u = threadIdx.x; u < kTokens * units_per_tok; u += kRopeThreads) {
    const int tok = u / units_per_tok, w = u % units_per_tok;
    if (t0 + tok >= n_tokens) break;
    T* xrow = x + (t0 + tok) * int64_t(row);
    float a[N], b[N];
    if (kInterleaved) {
      const int e0 = w * N, d0 = e0 % head_dim;
      u32x4_t* p = reinterpret_cast<u32x4_t*>(xrow + e0);
      Vec16<T>::unpack(*p, a);
      for (int k = 0; k < N / 2; ++k) {
        const float2 t = cs[tok][d0 / 2 + k];
        const float x0 = a[2 * k], x1 = a[2 * k + 1];
        b[2 * k] = fmaf(x0, t.x, -x1 * t.y);
        b[2 * k + 1] = fmaf(x0, t.y, x1 * t.x);
      }
      *p = Vec16<T>::pack(b);
    } else {
      const int per_head = head_dim / (2 * N);
      const int h = w / per_head, d0 = (w % per_head) * N;
      u32x4_t* p0 = reinterpret_cast<u32x4_t*>(xrow + h * head_dim + d0);
      u32x4_t* p1 = reinterpret_cast<u32x4_t*>(xrow + h * head_dim + d0 + head_dim / 2);
      Vec16<T>::unpack(*p0, a);
      Vec16<T>::unpack(*p1, b);
      float ra[N], rb[N];
      for (int k = 0; k < N; ++k) {
        const float2 t = cs[tok][d0 + k];
        ra[k] = fmaf(a[k], t.x, -b[k] * t.y);
        rb[k] = fmaf(a[k], t.y, b[k] * t.x);
      }
      *p0 = Vec16<T>::pack(ra);
      *p1 = Vec16<T>::pack(rb);
    }
  }
}

// Any even head_dim: one pair per thread iteration.
template <typename T, bool kInterleaved>
__global__ __launch_bounds__(kRopeThreads) void rope_pair_kernel(T* __restrict__ x, const int32_t* __restrict__ positions,
                                                                int64_t n_tokens, int n_heads, int head_dim, double theta) {
  __shared__ float2 cs[kTokens][kMaxPairs];
  __shared__ double inv_freq[kMaxPairs];
  const int64_t t0 = int64_t(blockIdx.x) * kTokens;
  build_table(cs, inv_freq, positions, t0, n_tokens, head_dim, theta);
  const int half = head_dim / 2;
  const int pairs_per_tok = n_heads * half;
  for (int u = threadIdx.x; u < kTokens * pairs_per_tok; u += kRopeThreads) {
    const int tok = u / pairs_per_tok, w = u % pairs_per_tok;
    if (t0 + tok >= n_tokens) break;
    const int h = w / half, i = w % half;
    T* xh = x + (t0 + tok) * int64_t(n_heads) * head_dim + int64_t(h) * head_dim;
    T* p0 = kInterleaved ? xh + 2 * i : xh + i;
    T* p1 = kInterleaved ? xh + 2 * i + 1 : xh + i + half;
    const float x0 = Elem<T>::load(p0), x1 = Elem<T>::load(p1);
    const float2 t = cs[tok][i];
    Elem<T>::store(p0, fmaf(x0, t.x, -x1 * t.y));
    Elem<T>::store(p1, fmaf(x0, t.y, x1 * t.x));
  }
}

// Table of (cos, sin) by integer position for every pair: the same fp64 expressions as build_table.
__global__ __launch_bounds__(kRopeThreads) void rope_table_kernel(float2* __restrict__ table, int n_positions,
                                                                 int head_dim, double theta) {
  const int half = head_dim / 2;
  const int64_t e = int64_t(blockIdx.x) * kRopeThreads + threadIdx.x;
  if (e >= int64_t(n_positions) * half) return;
  const int p = int(e / half), i = int(e % half);
  const double inv_freq = pow(theta, -2.0 * double(i) / double(head_dim));
  const double ang = double(p) * inv_freq;
  double sn, cs;
  sincos(ang, &sn, &cs);
  table[e] = make_float2(float(cs), float(sn));
}

template <typename T>
hipError_t launch_typed(T* x, int64_t n_tokens, int n_heads, int head_dim, const int32_t* positions, double theta,
                        int interleaved, hipStream_t stream) {
  const int64_t blocks = (n_tokens + kTokens - 1) / kTokens;
  const dim3 grid(static_cast<unsigned>(blocks)), block(kRopeThreads);
  constexpr int N = Vec16<T>::N;
  const bool aligned = (reinterpret_cast<uintptr_t>(x) % 16) == 0;
  if (aligned && (interleaved ? head_dim % N : (head_dim / 2) % N) == 0) {
    if (interleaved) rope_vec_kernel<T, true><<<grid, block, 0, stream>>>(x, positions, n_tokens, n_heads, head_dim, theta);
    else rope_vec_kernel<T, false><<<grid, block, 0, stream>>>(x, positions, n_tokens, n_heads, head_dim, theta);
  } else {
    if (interleaved) rope_pair_kernel<T, true><<<grid, block, 0, stream>>>(x, positions, n_tokens, n_heads, head_dim, theta);
    else rope_pair_kernel<T, false><<<grid, block, 0, stream>>>(x, positions, n_tokens, n_heads, head_dim, theta);
  }
  return hipGetLastError();
}

// ------------------------------------------------------------------------------------ paged KV append --
// (Attention notes, makinaruto.github.io, "Page Attention": logical token t of a sequence lives in page
//  block_table[t / page_size], slot t % page_size.) New row r of k_new / v_new belongs to the sequence b with
// cu_new[b] <= r < cu_new[b+1] and has absolute position ctx_lens[b] + r - cu_new[b]. Its key is rotated at that
// position (same fp64 table as above) and written with its value to the page slot. Rows whose page number is
// outside [0, num_pages) or past the table are not written.

// The sequence of row r: the last b with cu_new[b] <= r (binary search over the batch offsets).
__device__ __forceinline__ int seq_of_row(const int32_t* cu_new, int batch, int64_t r) {
  int lo = 0, hi = batch - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (cu_new[mid] <= r) lo = mid; else hi = mid - 1;
  }
  return lo;
}

template <bool kInterleaved>
__global__ __launch_bounds__(kRopeThreads) void kv_append_kernel(const uint16_t* __restrict__ k_new,
    const uint16_t* __restrict__ v_new, const int32_t* __restrict__ cu_new, const int32_t* __restrict__ ctx_lens,
    uint16_t* __restrict__ kc, uint16_t* __restrict__ vc, const int32_t* __restrict__ table, int batch,
    int64_t total_new, int hkv, int head_dim, int page_shift, int max_pages, int64_t num_pages, double theta) {
  __shared__ float2 cs[kTokens][kMaxPairs];
  __shared__ double inv_freq[kMaxPairs];
  __shared__ int32_t pos[kTokens];
  __shared__ int64_t dst_row[kTokens];                  // destination slot row (page * page_size + slot), or -1
  const int64_t t0 = int64_t(blockIdx.x) * kTokens;
  if (threadIdx.x < kTokens) {
    const int64_t r = t0 + threadIdx.x;
    int32_t p = 0;
    int64_t dst = -1;
    if (r < total_new) {
      const int b = seq_of_row(cu_new, batch, r);
      p = ctx_lens[b] + int32_t(r - cu_new[b]);
      const int pi = p >> page_shift;
      if (p >= 0 && pi < max_pages) {
        const int page = table[int64_t(b) * max_pages + pi];
        if (page >= 0 && page < num_pages) dst = (int64_t(page) << page_shift) + (p & ((1 << page_shift) - 1));
      }
    }
    pos[threadIdx.x] = p;
    dst_row[threadIdx.x] = dst;
  }
  __syncthreads();
  build_table(cs, inv_freq, pos, 0, kTokens, head_dim, theta);
  constexpr int N = 8;                                   // bf16 per 16 bytes
  const int row = hkv * head_dim;
  const int units = kInterleaved ? row / N : row / (2 * N);
  for (int u = threadIdx.x; u < kTokens * units; u += kRopeThreads) {
    const int tok = u / units, w = u % units;
    if (t0 + tok >= total_new || dst_row[tok] < 0) continue;
    const uint16_t* src = k_new + (t0 + tok) * int64_t(row);
    uint16_t* dst = kc + dst_row[tok] * row;
    float a[N], b[N];
    if (kInterleaved) {
      const int e0 = w * N, d0 = e0 % head_dim;
      Vec16<uint16_t>::unpack(*reinterpret_cast<const u32x4_t*>(src + e0), a);
      for (int k = 0; k < N / 2; ++k) {
        const float2 t = cs[tok][d0 / 2 + k];
        b[2 * k] = fmaf(a[2 * k], t.x, -a[2 * k + 1] * t.y);
        b[2 * k + 1] = fmaf(a[2 * k], t.y, a[2 * k + 1] * t.x);
      }
      *reinterpret_cast<u32x4_t*>(dst + e0) = Vec16<uint16_t>::pack(b);
    } else {
      const int per_head = head_dim / (2 * N);
      const int h = w / per_head, d0 = (w % per_head) * N;
      const int e0 = h * head_dim + d0, e1 = e0 + head_dim / 2;
      Vec16<uint16_t>::unpack(*reinterpret_cast<const u32x4_t*>(src + e0), a);
      Vec16<uint16_t>::unpack(*reinterpret_cast<const u32x4_t*>(src + e1), b);
      float ra[N], rb[N];
      for (int k = 0; k < N; ++k) {
        const float2 t = cs[tok][d0 + k];
        ra[k] = fmaf(a[k], t.x, -b[k] * t.y);
        rb[k] = fmaf(a[k], t.y, b[k] * t.x);
      }
      *reinterpret_cast<u32x4_t*>(dst + e0) = Vec16<uint16_t>::pack(ra);
      *reinterpret_cast<u32x4_t*>(dst + e1) = Vec16<uint16_t>::pack(rb);
    }
  }
  // values: plain 16-byte copies
  const int vunits = row / N;
  for (int u = threadIdx.x; u < kTokens * vunits; u += kRopeThreads) {
    const int tok = u / vunits, w = u % vunits;
    if (t0 + tok >= total_new || dst_row[tok] < 0) continue;
    *reinterpret_cast<u32x4_t*>(vc + dst_row[tok] * row + w * N) =
        *reinterpret_cast<const u32x4_t*>(v_new + (t0 + tok) * int64_t(row) + w * N);
  }
}

}  // namespace

hipError_t launch_kv_append_paged(const void* k_new, const void* v_new, const int32_t* cu_new,
                                  const int32_t* ctx_lens, void* k_cache, void* v_cache, const int32_t* block_table,
                                  int batch, int total_new, int hkv, int head_dim, int page_size, int max_pages_per_seq,
                                  int64_t num_pages, double theta, int interleaved, hipStream_t stream) {
  if (total_new <= 0) return hipSuccess;
  int shift = 0;
  while ((1 << shift) < page_size) ++shift;
  const dim3 grid(static_cast<unsigned>((int64_t(total_new) + kTokens - 1) / kTokens)), block(kRopeThreads);
  const uint16_t* kn = static_cast<const uint16_t*>(k_new);
  const uint16_t* vn = static_cast<const uint16_t*>(v_new);
  uint16_t* kc = static_cast<uint16_t*>(k_cache);
  uint16_t* vc = static_cast<uint16_t*>(v_cache);
  if (interleaved)
    kv_append_kernel<true><<<grid, block, 0, stream>>>(kn, vn, cu_new, ctx_lens, kc, vc, block_table, batch, total_new,
                                                        hkv, head_dim, shift, max_pages_per_seq, num_pages, theta);
  else
    kv_append_kernel<false><<<grid, block, 0, stream>>>(kn, vn, cu_new, ctx_lens, kc, vc, block_table, batch, total_new,
                                                         hkv, head_dim, shift, max_pages_per_seq, num_pages, theta);
  return hipGetLastError();
}

hipError_t launch_rope(void* x, int dtype, int64_t n_tokens, int n_heads, int head_dim, const int32_t* positions,
                       double theta, int interleaved, hipStream_t stream) {
  if (dtype == 0)
    return launch_typed(static_cast<uint16_t*>(x), n_tokens, n_heads, head_dim, positions, theta, interleaved, stream);
  return launch_typed(static_cast<float*>(x), n_tokens, n_heads, head_dim, positions, theta, interleaved, stream);
}

hipError_t launch_rope_table(void* table, int n_positions, int head_dim, double theta, hipStream_t stream) {
  const int64_t n = int64_t(n_positions) * (head_dim / 2);
  if (n == 0) return hipSuccess;
  const dim3 grid(static_cast<unsigned>((n + kRopeThreads - 1) / kRopeThreads)), block(kRopeThreads);
  rope_table_kernel<<<grid, block, 0, stream>>>(static_cast<float2*>(table), n_positions, head_dim, theta);
  return hipGetLastError();
}

}  // namespace attn
