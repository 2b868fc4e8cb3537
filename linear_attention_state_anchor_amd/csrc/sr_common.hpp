// Device-side helpers shared by the gfx950 kernels of the replay library.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace sr {

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint16_t u16x8 __attribute__((ext_vector_type(8)));
typedef uint16_t u16x4 __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;
constexpr int kGfx950Cus = 256;  // compute units of the gfx950 parts (MI350X, MI355X)

// Element-type tags used as template parameters.
struct BF16 {};
struct F16 {};
struct F32 {};

__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
  return __uint_as_float(static_cast<uint32_t>(b) << 16);
}

// fp32 -> bf16 bits, round to nearest even (the gfx950 conversion
// instruction, which pairs up neighbouring conversions).
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  return __builtin_bit_cast(uint16_t, static_cast<__bf16>(f));
}

__device__ __forceinline__ uint16_t f16_bits(_Float16 h) {
  return __builtin_bit_cast(uint16_t, h);
}

// Load 8 consecutive elements of a 16-byte aligned row as fp16.
template <typename T>
struct Ld8;
template <>
struct Ld8<BF16> {
  __device__ __forceinline__ static f16x8 load(const void* p) {
    u16x8 raw = *reinterpret_cast<const u16x8*>(p);
    f16x8 r;
#pragma unroll
    for (int e = 0; e < 8; ++e) r[e] = static_cast<_Float16>(bf16_to_f32(raw[e]));
    return r;
  }
  static constexpr int kBytes = 2;
};
template <>
struct Ld8<F16> {
  __device__ __forceinline__ static f16x8 load(const void* p) {
    return *reinterpret_cast<const f16x8*>(p);
  }
  static constexpr int kBytes = 2;
};

// Load 4 consecutive elements (8-byte aligned) as fp16.
template <typename T>
__device__ __forceinline__ f16x4 ld4_f16(const void* p);
template <>
__device__ __forceinline__ f16x4 ld4_f16<BF16>(const void* p) {
  u16x4 raw = *reinterpret_cast<const u16x4*>(p);
  f16x4 r;
#pragma unroll
  for (int e = 0; e < 4; ++e) r[e] = static_cast<_Float16>(bf16_to_f32(raw[e]));
  return r;
}
template <>
__device__ __forceinline__ f16x4 ld4_f16<F16>(const void* p) {
  return *reinterpret_cast<const f16x4*>(p);
}

// Store one value of the output type.
template <typename T>
__device__ __forceinline__ void store1(void* base, size_t idx, float v);
template <>
__device__ __forceinline__ void store1<BF16>(void* base, size_t idx, float v) {
  reinterpret_cast<uint16_t*>(base)[idx] = f32_to_bf16(v);
}
template <>
__device__ __forceinline__ void store1<F16>(void* base, size_t idx, float v) {
  reinterpret_cast<_Float16*>(base)[idx] = static_cast<_Float16>(v);
}
template <>
__device__ __forceinline__ void store1<F32>(void* base, size_t idx, float v) {
  reinterpret_cast<float*>(base)[idx] = v;
}

// Store 4 consecutive values of the output type (8- or 16-byte aligned).
template <typename T>
__device__ __forceinline__ void store4(void* base, size_t idx, f32x4 v);
template <>
__device__ __forceinline__ void store4<BF16>(void* base, size_t idx, f32x4 v) {
  typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
  bf16x4 r;
#pragma unroll
  for (int e = 0; e < 4; ++e) r[e] = static_cast<__bf16>(v[e]);
  *reinterpret_cast<bf16x4*>(reinterpret_cast<uint16_t*>(base) + idx) = r;
}
template <>
__device__ __forceinline__ void store4<F16>(void* base, size_t idx, f32x4 v) {
  f16x4 r;
#pragma unroll
  for (int e = 0; e < 4; ++e) r[e] = static_cast<_Float16>(v[e]);
  *reinterpret_cast<f16x4*>(reinterpret_cast<_Float16*>(base) + idx) = r;
}
template <>
__device__ __forceinline__ void store4<F32>(void* base, size_t idx, f32x4 v) {
  *reinterpret_cast<f32x4*>(reinterpret_cast<float*>(base) + idx) = v;
}

// Read one element as fp32.
template <typename T>
__device__ __forceinline__ float load1(const void* base, size_t idx);
template <>
__device__ __forceinline__ float load1<BF16>(const void* base, size_t idx) {
  return bf16_to_f32(reinterpret_cast<const uint16_t*>(base)[idx]);
}
template <>
__device__ __forceinline__ float load1<F16>(const void* base, size_t idx) {
  return static_cast<float>(reinterpret_cast<const _Float16*>(base)[idx]);
}
template <>
__device__ __forceinline__ float load1<F32>(const void* base, size_t idx) {
  return reinterpret_cast<const float*>(base)[idx];
}

// D = A*B + C on the matrix cores, 16x16 output, K = 32, fp16 operands.
// Lane l holds A row (l % 16) and B column (l % 16), k-slots 8*(l/16)..+7;
// D column (l % 16), rows 4*(l/16)..+3.
__device__ __forceinline__ f32x4 mfma16x16x32(f16x8 a, f16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}

// Same shape with bf16 operands.
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
__device__ __forceinline__ f32x4 mfma16x16x32_bf16(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// 32x32 output, K = 16, fp16 operands.  Lane l holds A row (l % 32) and B
// column (l % 32), k-slots 8*(l/32)..+7; D column (l % 32), register r holds
// row 8*(r/4) + 4*(l/32) + (r % 4).
__device__ __forceinline__ f32x16 mfma32x32x16(f16x8 a, f16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ f16x8 cat44(f16x4 lo, f16x4 hi) {
  f16x8 r;
  r[0] = lo[0]; r[1] = lo[1]; r[2] = lo[2]; r[3] = lo[3];
  r[4] = hi[0]; r[5] = hi[1]; r[6] = hi[2]; r[7] = hi[3];
  return r;
}

__device__ __forceinline__ f16x4 to_f16x4(f32x4 v) {
  f16x4 r;
  r[0] = static_cast<_Float16>(v[0]);
  r[1] = static_cast<_Float16>(v[1]);
  r[2] = static_cast<_Float16>(v[2]);
  r[3] = static_cast<_Float16>(v[3]);
  return r;
}

__device__ __forceinline__ f16x8 to_f16x8(f32x4 lo, f32x4 hi) {
  return cat44(to_f16x4(lo), to_f16x4(hi));
}

// Inclusive prefix sum over the 64 lanes of a wave with DPP row shifts and
// row broadcasts (no LDS round trips).
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ float dpp_f32(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, ROW_MASK, 0xf, false));
}
__device__ __forceinline__ float wave_inclusive_sum(float x) {
  x += dpp_f32<0x111, 0xf>(x);  // row_shr:1
  x += dpp_f32<0x112, 0xf>(x);  // row_shr:2
  x += dpp_f32<0x114, 0xf>(x);  // row_shr:4
  x += dpp_f32<0x118, 0xf>(x);  // row_shr:8
  x += dpp_f32<0x142, 0xa>(x);  // row_bcast:15 into rows 1 and 3
  x += dpp_f32<0x143, 0xc>(x);  // row_bcast:31 into rows 2 and 3
  return x;
}
// Sum over the 64 lanes of a wave, returned to every lane.
__device__ __forceinline__ float wave_sum(float x) {
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(wave_inclusive_sum(x)), kWave - 1));
}
// Maximum of non-negative values over the 64 lanes of a wave, returned to
// every lane as a wave-uniform value (lanes that receive nothing from a DPP
// step see 0, the identity for non-negative inputs).
__device__ __forceinline__ float wave_max_nonneg(float x) {
  x = fmaxf(x, dpp_f32<0x111, 0xf>(x));  // row_shr:1
  x = fmaxf(x, dpp_f32<0x112, 0xf>(x));  // row_shr:2
  x = fmaxf(x, dpp_f32<0x114, 0xf>(x));  // row_shr:4
  x = fmaxf(x, dpp_f32<0x118, 0xf>(x));  // row_shr:8
  x = fmaxf(x, dpp_f32<0x142, 0xa>(x));  // row_bcast:15
  x = fmaxf(x, dpp_f32<0x143, 0xc>(x));  // row_bcast:31
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), kWave - 1));
}

__device__ __forceinline__ float silu(float x) { return x / (1.0f + __expf(-x)); }

__device__ __forceinline__ float softplus(float x) {
  // log(1 + e^x), without overflow for large x
  return x > 20.0f ? x + log1pf(__expf(-x)) : log1pf(__expf(x));
}

__device__ __forceinline__ float sigmoid(float x) { return 1.0f / (1.0f + __expf(-x)); }

}  // namespace sr
