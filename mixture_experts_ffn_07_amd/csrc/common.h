// Device helpers shared by the gfx950 kernels of this library.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4;
typedef float f32x2 __attribute__((ext_vector_type(2)));   // hardware FP8 pair conversions
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16;
typedef __attribute__((__vector_size__(8 * sizeof(int)))) int i32x8;
typedef __attribute__((__vector_size__(4 * sizeof(int)))) int i32x4;

constexpr int kWave = 64;

__device__ __forceinline__ int lane_id() { return threadIdx.x & (kWave - 1); }
__device__ __forceinline__ int wave_id() { return threadIdx.x / kWave; }

// 16-byte global load / store through plain vector memory instructions.
__device__ __forceinline__ i32x4 ld16(const void* p) {
  return *reinterpret_cast<const i32x4*>(p);
}
__device__ __forceinline__ void st16(void* p, i32x4 v) { *reinterpret_cast<i32x4*>(p) = v; }
// Streaming 16-byte load (non-temporal hint) for data read once per call, such
// as expert weights in decode: it keeps them from displacing reused data in the
// caches, and it sustains a higher HBM read rate than plain loads.
__device__ __forceinline__ i32x4 ld16_stream(const void* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const i32x4*>(p));
}

__device__ __forceinline__ bf16x8 as_bf16x8(i32x4 v) { return __builtin_bit_cast(bf16x8, v); }

// Streaming (non-temporal) stores of results written once while a kernel streams
// its weights: a projection epilogue's plain stores, mixed into the weight read
// stream, cost the Kimi-shaped batched gate_up 6% for 0.3% of its bytes (67 MB of
// h), the streaming form about half of that; the BF16 down projection's FP32 slot
// slices (read back by the combine right after) 3-7% faster, the backward's dh
// epilogue and dx slices 2-3%, the MXFP8 kernel's FP32 outputs (slot slices,
// pre-activations, dh) 4-8% (its 4-byte code stores measured 2% slower that way,
// and keep plain stores).
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ void st8_stream(void* p, uint2 v) {
  __builtin_nontemporal_store(u32x2{v.x, v.y}, reinterpret_cast<u32x2*>(p));
}
__device__ __forceinline__ void st16_stream(void* p, f32x4 v) {
  __builtin_nontemporal_store(v, reinterpret_cast<f32x4*>(p));
}
// The same for the write-bound kernels' whole-line stores (weight gradients, the
// MXFP8 weight re-encoding): ~1-2% on those segments, and the caches they would
// have filled stay with the next kernel's operands.
__device__ __forceinline__ void st16_stream(void* p, i32x4 v) {
  __builtin_nontemporal_store(v, reinterpret_cast<i32x4*>(p));
}

// FP32 -> BF16, round to nearest, ties to even, on gfx950's conversion
// instruction (v_cvt_pk_bf16_f32, two values per instruction): pack_bf16x2
// returns a's bits in the low half and b's in the high half; f32_to_bf16_rne
// one value's bits.
typedef __bf16 bf16x2_cvt __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{a, b}, bf16x2_cvt));
}
__device__ __forceinline__ uint32_t f32_to_bf16_rne(float f) { return pack_bf16x2(f, 0.f) & 0xFFFFu; }
__device__ __forceinline__ float bf16_to_f32(uint32_t b) { return __uint_as_float(b << 16); }

// silu(z) * u in FP32.  For z -> -inf, exp(-z) overflows to +inf and
// z / inf gives -0, the correct limit.
__device__ __forceinline__ float swiglu(float g, float u) {
  return g / (1.0f + __expf(-g)) * u;
}

// Wave-wide sum with a fixed butterfly order (deterministic).
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v += __shfl_xor(v, m, kWave);
  return v;
}

__device__ __forceinline__ f32x4 mfma16x16x32(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// Block-scaled FP8 (E4M3 x E4M3) MFMA, 16x16x128.  Operand lane layout: lane
// (r, g) = (lane % 16, lane / 16) holds row r, K elements [16g, 16g+16) in
// bytes 0..15 and [64+16g, 64+16g+16) in bytes 16..31; the E8M0 scale in the
// low byte of lane (r, g)'s scale operand applies to K block [32g, 32g+32).
__device__ __forceinline__ f32x4 mfma_mx16x16x128(i32x8 a, i32x8 b, int sa, int sb, f32x4 c) {
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 0, 0, 0, sa, 0, sb);
}

__device__ __forceinline__ i32x8 cat8(i32x4 lo, i32x4 hi) {
  return i32x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
}

// MX scale exponent of a block (OCP Microscaling v1.0 rule for E4M3):
// s = floor(log2(amax)) - 8, clamped to [-127, 127]; amax = 0 gives -127.
__device__ __forceinline__ int mx_scale_exp(float amax) {
  const uint32_t u = __float_as_uint(amax) & 0x7FFFFFFFu;
  int fl;
  if (u == 0) return -127;
  if ((u >> 23) == 0) fl = (31 - __clz(u)) - 149;      // subnormal amax
  else fl = static_cast<int>(u >> 23) - 127;
  int s = fl - 8;
  return s < -127 ? -127 : (s > 127 ? 127 : s);
}

// 2^-s as an exact FP32 value, s in [-127, 127].
__device__ __forceinline__ float exp2_neg(int s) {
  const int e = -s;                                      // in [-127, 127]
  return e >= -126 ? __uint_as_float(static_cast<uint32_t>(e + 127) << 23)
                   : __uint_as_float(0x00400000u);       // 2^-127, subnormal
}

// FP32 -> E4M3 code: round to nearest even, saturate to +-448, sign copied.
__device__ __forceinline__ uint32_t f32_to_e4m3(float y) {
  const uint32_t u = __float_as_uint(y);
  const uint32_t sign = (u >> 24) & 0x80u;
  const float a = __uint_as_float(u & 0x7FFFFFFFu);
  uint32_t mag;
  if (a >= 448.0f) {
    mag = 0x7Eu;
  } else if (a < 0.015625f) {                           // below 2^-6: step 2^-9
    mag = static_cast<uint32_t>(rintf(a * 512.0f));     // 0..8, 8 = smallest normal
  } else {
    const uint32_t ab = __float_as_uint(a);
    const uint32_t r = ab + 0x7FFFFu + ((ab >> 20) & 1u);   // RNE at the 3rd mantissa bit
    mag = (r >> 20) - (120u << 3);                      // rebias 127 -> 7
  }
  return sign | mag;
}

// Four FP32 -> four E4M3 codes, code t in byte t: the hardware conversion
// (round to nearest even) on inputs clamped to +-448 (exactly representable),
// which yields the codes of f32_to_e4m3 - checked on every E4M3 value, every
// midpoint between neighbours and its 1-ulp neighbours, and 2e6 random inputs.
__device__ __forceinline__ uint32_t f32x4_to_e4m3x4(float a, float b, float c, float d) {
  const float lo = -448.0f, hi = 448.0f;
  int w = __builtin_amdgcn_cvt_pk_fp8_f32(__builtin_amdgcn_fmed3f(a, lo, hi),
                                          __builtin_amdgcn_fmed3f(b, lo, hi), 0, false);
  w = __builtin_amdgcn_cvt_pk_fp8_f32(__builtin_amdgcn_fmed3f(c, lo, hi),
                                      __builtin_amdgcn_fmed3f(d, lo, hi), w, true);
  return static_cast<uint32_t>(w);
}

}  // namespace moe
