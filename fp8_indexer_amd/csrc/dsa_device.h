// dsa_device.h -- small device-side helpers shared by the libdsa kernels
// (gfx950 / CDNA4 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dsa {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef short i16x8 __attribute__((ext_vector_type(8)));

constexpr int kWave = 64;

// D = A*B + C on a 16x16 fp32 tile, A/B 16x128 OCP e4m3fn (32 bytes per lane).
// Lane l holds A row (l%16), k-chunk [32*(l/16), +32); B likewise by column;
// C lane l holds column l%16, rows 4*(l/16)+i.
__device__ __forceinline__ f32x4 mfma_f8_16x16x128(const i32x8& a, const i32x8& b, f32x4 c) {
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 0, 0, 0, 0, 0, 0);
}

// D = A*B + C on a 16x16 fp32 tile, A/B 16x32 bf16 (8 values per lane).
// Lane l holds A row (l%16), k-chunk [8*(l/16), +8); C as above.
__device__ __forceinline__ f32x4 mfma_bf16_16x16x32(const bf16x8& a, const bf16x8& b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ float wave_xor(float v, int mask) {
  return __shfl_xor(v, mask, kWave);
}

typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// Two fp32 -> packed bf16 (lo in bits 0..15), round to nearest even
// (one v_cvt_pk_bf16_f32 on gfx950).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{lo, hi}, bf16x2));
}

// 2^x on the transcendental unit (v_exp_f32); -inf -> 0.
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

__device__ __forceinline__ int clampi(int v, int lo, int hi) {
  return v < lo ? lo : (v > hi ? hi : v);
}

// Split launches (S workgroups per row, row = blockIdx / S, split =
// blockIdx % S): when the row count is a multiple of the 8 XCDs, remap so
// that the S splits of a row run on one XCD.  Workgroups are dealt to the
// XCDs in turn (workgroup g on XCD g % 8), so the row's q, which every split
// reads, comes from HBM once and from that XCD's L2 for the others.  The map
// is a bijection of (row, split) pairs whatever the placement.
__device__ __forceinline__ void split_to_xcd(int& row, int& split, int S) {
  constexpr int kXcd = 8;
  const int g = (int)blockIdx.x, rows = (int)gridDim.x / S;
  if (S > 1 && rows % kXcd == 0) {
    const int j = g / kXcd;  // position among the workgroups of XCD g % 8
    row = (j / S) * kXcd + g % kXcd;
    split = j % S;
  }
}

}  // namespace dsa
