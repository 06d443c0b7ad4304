// Device-side helpers shared by the HIP kernels of libmoe (gfx950 only).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

typedef uint16_t bf16_t;
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef int i32x8 __attribute__((ext_vector_type(8)));

#define MOE_DEV __device__ __forceinline__

MOE_DEV float bf16_to_f32(bf16_t v) { return __uint_as_float((uint32_t)v << 16); }

// round to nearest, ties to even (inputs are finite)
MOE_DEV bf16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (bf16_t)(u >> 16);
}

MOE_DEV uint32_t pack_bf16x2(float a, float b) {
  return (uint32_t)f32_to_bf16(a) | ((uint32_t)f32_to_bf16(b) << 16);
}

MOE_DEV i32x4 ld16(const void* p) { return *reinterpret_cast<const i32x4*>(p); }
MOE_DEV i32x8 ld32(const void* p) {
  const i32x4* q = reinterpret_cast<const i32x4*>(p);
  i32x4 a = q[0], b = q[1];
  i32x8 r = {a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
  return r;
}

// D(16x16, fp32) += A(16x32, bf16) * B(32x16, bf16).
// Lane l holds A row (l % 16) and B column (l % 16), eight consecutive k values of
// chunk (l / 16); the accumulator holds column (l % 16), rows 4 * (l / 16) + i.
MOE_DEV f32x4 mfma_bf16_16x16x32(i32x4 a, i32x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                 __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}

// D(16x16, fp32) += A(16x128, e4m3) * B(128x16, e4m3), unit block scales (E8M0 127 = 1.0).
// Lane l holds row / column (l % 16) and 32 consecutive k values of chunk (l / 16).
MOE_DEV f32x4 mfma_fp8_16x16x128(i32x8 a, i32x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 0, 0, 0, 127, 0, 127);
}

MOE_DEV float silu_mul(float g, float u) { return g / (1.0f + expf(-g)) * u; }

// Two fp32 values -> two OCP e4m3fn codes in the low 16 bits (round to nearest even;
// inputs are clamped to +-448 first so the conversion saturates).
MOE_DEV uint32_t f32x2_to_e4m3(float a, float b) {
  a = fminf(fmaxf(a, -448.0f), 448.0f);
  b = fminf(fmaxf(b, -448.0f), 448.0f);
  return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false) & 0xFFFFu;
}

MOE_DEV float wave_max(float v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v = fmaxf(v, __shfl_xor(v, off));
  return v;
}

// Tile of rows handled by one GEMM work item: `expert` (E = the shared expert),
// first row (routed: dispatch row; shared: token), number of rows, and the index of
// the expert's first tile in the list.
struct Tile {
  int expert, row0, nrows, first;
};
