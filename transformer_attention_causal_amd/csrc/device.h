// device.h — gfx950 device helpers shared by the attention kernels (vector types, bf16 packing, MFMA
// wrappers, LDS transpose reads, direct-to-LDS loads, wave64 cross-lane reductions).
//
// MFMA operand layouts used throughout (gfx950, wave64; verified on hardware):
//   v_mfma_f32_32x32x16_bf16  D[32x32] += A[32x16] * B[16x32]
//     A: lane l holds A[l%32][8*(l/32) + s], s = 0..7        B: lane l holds B[8*(l/32) + s][l%32]
//     D: lane l, register r holds D[8*(r/4) + 4*(l/32) + r%4][l%32]
//   v_mfma_f32_16x16x32_bf16  D[16x16] += A[16x32] * B[32x16]
//     A: lane l holds A[l%16][8*(l/16) + s]                   B: lane l holds B[8*(l/16) + s][l%16]
//     D: lane l, register r holds D[4*(l/16) + r][l%16]
//   ds_read_b64_tr_b16: within each block of 16 lanes, result lane i, element j is element i%4 of the 8 bytes
//     addressed by lane 4*j + i/4 of the block. So if block lane 4*j + c addresses row (k0 + j), columns
//     (n0 + 4c .. n0 + 4c + 3) of a row-major 16-bit matrix, lane i receives column n0 + i, rows k0 .. k0 + 3.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace attn {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4_t __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef short i16x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

typedef __attribute__((address_space(3))) void lds_void_t;

// ------------------------------------------------------------------------------------------ bf16 packing --
__device__ __forceinline__ float bf16lo_to_f32(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16hi_to_f32(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// Two fp32 -> two bf16 (round to nearest even), packed lo | hi << 16 (one v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  f32x2_t v = {lo, hi};
  bf16x2_t b = __builtin_convertvector(v, bf16x2_t);
  return __builtin_bit_cast(uint32_t, b);
}

__device__ __forceinline__ bf16x8_t as_bf16x8(u32x4_t v) { return __builtin_bit_cast(bf16x8_t, v); }

// Eight fp32 values -> an 8 x bf16 MFMA operand.
__device__ __forceinline__ bf16x8_t pack_bf16x8(float a0, float a1, float a2, float a3, float a4, float a5,
                                                float a6, float a7) {
  u32x4_t w = {pack_bf16x2(a0, a1), pack_bf16x2(a2, a3), pack_bf16x2(a4, a5), pack_bf16x2(a6, a7)};
  return as_bf16x8(w);
}

// ------------------------------------------------------------------------------------------------ MFMA --
__device__ __forceinline__ f32x16_t mfma32x32x16(bf16x8_t a, bf16x8_t b, f32x16_t c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4_t mfma16x16x32(bf16x8_t a, bf16x8_t b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// v_mfma_scale_f32_16x16x128_f8f6f4 with both operands FP8 E4M3 (OCP: 0x38 is 1.0) and unit scales:
// D[16x16] += A[16x128] * B[128x16]. Lane l holds row l%16 of A (32 codes) and column l%16 of B (32 codes), and
// the K index of each of those 32 bytes is the same function of (l / 16, byte) for A and B, so a kernel may assign
// K positions to (lane group, byte) as it likes as long as both operands follow it. D as for the 16x16x32 form.
// (Measured on gfx950 with small integers, which the products and sums keep exact.)
typedef int i32x8_t __attribute__((ext_vector_type(8)));
__device__ __forceinline__ f32x4_t mfma16x16x128_fp8(i32x8_t a, i32x8_t b, f32x4_t c) {
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 0, 0, 0, 0, 0, 0);
}

// FP8 E4M3 (OCP) conversions, round to nearest even: two fp32 into word `hi` of `old`, and the two codes of word
// `hi` of `w` back to fp32 (exact).
__device__ __forceinline__ uint32_t f32x2_to_fp8(uint32_t old, float a, float b, bool hi) {
  typedef short s16x2_t __attribute__((ext_vector_type(2)));
  const s16x2_t o = __builtin_bit_cast(s16x2_t, old);
  return __builtin_bit_cast(uint32_t, hi ? __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(o, a, b, 1.0f, true)
                                         : __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(o, a, b, 1.0f, false));
}
__device__ __forceinline__ f32x2_t fp8x2_to_f32(uint32_t w, bool hi) {
  return hi ? __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(w, 1.0f, true)
            : __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(w, 1.0f, false);
}

// ------------------------------------------------------------------------------------- 8-bit cache codes --
// Cache element kinds: 0 bf16, 1 FP8 E4M3 codes, 2 int8 codes (the 8-bit kinds carry per-channel scales). Every
// E4M3 and int8 value is exact in bf16, so codes become bf16 MFMA operands by exact conversion.
constexpr int kKvBf16 = 0, kKvFp8 = 1, kKvInt8 = 2;

// Two 8-bit codes (bytes 0-1, or 2-3 when hi) of `w` as two bf16 (exact).
template <int KV>
__device__ __forceinline__ uint32_t codes_to_bf16x2(uint32_t w, bool hi) {
  if constexpr (KV == kKvFp8) {
    return __builtin_bit_cast(uint32_t, hi ? __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, true)
                                           : __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, false));
  } else {
    // Each byte sign-extended and converted in one instruction (a byte-select of the convert's source), then
    // packed: 1.5 instructions per code, against 3 for converting the biased byte and subtracting 128.
    const int sh = hi ? 16 : 0;
    return pack_bf16x2(float(int8_t(w >> sh)), float(int8_t(w >> (sh + 8))));
  }
}

// Eight 8-bit codes (two dwords) as eight bf16 (four dwords), in order.
template <int KV>
__device__ __forceinline__ u32x4_t codes_to_bf16x8(uint32_t w0, uint32_t w1) {
  return u32x4_t{codes_to_bf16x2<KV>(w0, false), codes_to_bf16x2<KV>(w0, true), codes_to_bf16x2<KV>(w1, false),
                 codes_to_bf16x2<KV>(w1, true)};
}

// ------------------------------------------------------------------------------------------------- LDS --
// LDS reads. The base pointer is __restrict__ so that, once inlined, each read carries alias-scope
// metadata; without it the compiler treats every LDS read as possibly aliasing an in-flight direct-to-LDS
// copy and inserts a full vmcnt(0) wait before it, which would stall the copy of the next tile behind the
// current tile's reads. The kernels order tile copies and reads themselves (vmcnt wait + workgroup barrier
// before a tile is read; the copy in flight always targets the other buffer).
//
// 16-byte LDS read.
__device__ __forceinline__ u32x4_t lds_read16(const uint16_t* __restrict__ lds_base, uint32_t byte_off) {
  return *(const __attribute__((address_space(3))) u32x4_t*)((const __attribute__((address_space(3))) char*)lds_base +
                                                                byte_off);
}
__device__ __forceinline__ u32x4_t lds_read16(const uint8_t* __restrict__ lds_base, uint32_t byte_off) {
  return *(const __attribute__((address_space(3))) u32x4_t*)((const __attribute__((address_space(3))) char*)lds_base +
                                                                byte_off);
}

// 8-byte LDS read.
__device__ __forceinline__ u32x2_t lds_read8(const uint8_t* __restrict__ lds_base, uint32_t byte_off) {
  return *(const __attribute__((address_space(3))) u32x2_t*)((const __attribute__((address_space(3))) char*)lds_base +
                                                                byte_off);
}

// Transposing 8-byte read of 8-bit elements: within each block of 16 lanes, result lane i, byte j is byte i%8 of
// the 8 bytes addressed by lane 2*j + i/8 of the block (measured on gfx950).
__device__ __forceinline__ u32x2_t lds_read_tr8(const uint8_t* __restrict__ lds_base, uint32_t byte_off) {
  typedef int i32x2_t __attribute__((ext_vector_type(2)));
  i32x2_t t = __builtin_amdgcn_ds_read_tr8_b64_v2i32(
      (__attribute__((address_space(3))) i32x2_t*)((__attribute__((address_space(3))) const char*)lds_base + byte_off));
  return __builtin_bit_cast(u32x2_t, t);
}

// Transposing 8-byte LDS read (see the layout note at the top of this file).
__device__ __forceinline__ u32x2_t lds_read_tr16(const uint16_t* __restrict__ lds_base, uint32_t byte_off) {
  i16x4_t t = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) i16x4_t*)((__attribute__((address_space(3))) char*)lds_base + byte_off));
  return __builtin_bit_cast(u32x2_t, t);
}

// Direct global -> LDS copies go through buffer loads (MUBUF with the LDS bit), addressed by a buffer
// resource plus a 32-bit per-lane byte offset. The FLAT-encoded global_load_lds would do the same copy, but
// while one is in flight the compiler's wait insertion cannot count LDS reads in order and turns every LDS
// wait into lgkmcnt(0), which serialises software-pipelined LDS reads behind their MFMAs.
// Buffer resource (V#) as four dwords. The resource is built from wave-uniform words so it lives in scalar
// registers; the opaque __amdgpu_buffer_rsrc_t form is assembled in vector registers and makes the compiler wrap
// every load in a per-lane waterfall loop.
typedef int buf_rsrc_t __attribute__((ext_vector_type(4)));

// The LLVM raw buffer load-to-LDS intrinsic, taking the resource as 4 x i32.
__device__ void raw_buffer_load_lds(buf_rsrc_t rsrc, lds_void_t* lds, int size, int voffset, int soffset, int offset,
                                    int aux) __asm("llvm.amdgcn.raw.buffer.load.lds");

// Raw buffer resource over `bytes` bytes at `base` (stride 0, 32-bit dword data format); loads at offsets
// >= bytes return zero. `base` and `bytes` must be wave-uniform.
__device__ __forceinline__ buf_rsrc_t make_buf_rsrc(const void* base, uint32_t bytes) {
  const uint64_t p = reinterpret_cast<uint64_t>(base);
  buf_rsrc_t r = {__builtin_amdgcn_readfirstlane(static_cast<int>(uint32_t(p))),
                  __builtin_amdgcn_readfirstlane(static_cast<int>(uint32_t(p >> 32) & 0xffffu)),
                  __builtin_amdgcn_readfirstlane(static_cast<int>(bytes)), 0x00020000};
  return r;
}

// 16 bytes per lane from `rsrc` at byte offset voff + soff into LDS: lane i's bytes land at lds_wave_base + 16*i,
// where lds_wave_base and soff must be the same for the whole wave. Only voff is range-checked against the
// resource size, so soff must keep the access inside the resource whenever voff is in range.
// aux = 2: non-temporal (for data read once).
template <int AUX = 0>
__device__ __forceinline__ void load_lds16(buf_rsrc_t rsrc, uint32_t voff, void* lds_wave_base, uint32_t soff = 0) {
  raw_buffer_load_lds(rsrc, (lds_void_t*)lds_wave_base, 16, static_cast<int>(voff), static_cast<int>(soff), 0, AUX);
}

// 4 bytes per lane: lane i's dword lands at lds_wave_base + 4*i (same addressing rules as load_lds16).
__device__ __forceinline__ void load_lds4(buf_rsrc_t rsrc, uint32_t voff, void* lds_wave_base, uint32_t soff = 0) {
  raw_buffer_load_lds(rsrc, (lds_void_t*)lds_wave_base, 4, static_cast<int>(voff), static_cast<int>(soff), 0, 0);
}

// One dword per lane from `rsrc` at byte offset voffset + soffset into a VGPR (counted by vmcnt like the copies;
// offsets past the resource read 0).
__device__ int raw_buffer_load_i32(buf_rsrc_t rsrc, int voffset, int soffset, int aux)
    __asm("llvm.amdgcn.raw.buffer.load.i32");

__device__ __forceinline__ void wait_vmem() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// ---------------------------------------------------------------------------------------- cross-lane --
__device__ __forceinline__ float xor_lanes(float v, int mask) { return __shfl_xor(v, mask, 64); }

// Reductions across lane halves / 16-lane rows with the gfx950 permlane swaps (one VALU op each, no LDS):
// with both operands = v, the two results hold, on every lane, the values of the lane pair {l, l ^ 32}
// (permlane32) or {l, l ^ 16} (permlane16); both lanes of a pair get bitwise the same combination.
__device__ __forceinline__ float max_xor32(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float sum_xor32(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float max_xor16(float v) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float sum_xor16(float v) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
// Online-softmax lazy rescale threshold (log2 units): the running reference max is only moved when the new block
// max exceeds it by more than this, so unnormalised probabilities stay below 2^kRescaleLog2.
constexpr float kRescaleLog2 = 8.0f;

}  // namespace attn
