// Device helpers shared by the gfx950 attention kernels: bf16 packing,
// the 32x32x16 / 16x16x32 bf16 matrix-core products, and the rotary angle.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace g4a {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// bf16 halves of a packed dword -> fp32 (exact)
__device__ __forceinline__ float bf_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// two fp32 -> packed bf16 pair, round to nearest even (v_cvt_pk_bf16_f32)
__device__ __forceinline__ uint32_t pack_bf16(float a, float b) {
  f32x2 f = {a, b};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f, bf16x2_t));
}

// D(32x32, fp32) += A(32x16) * B(16x32), bf16 operands.
// Lane l holds A[l % 32][8*(l/32) .. +7], B[8*(l/32) .. +7][l % 32] and
// D[8*(r/4) + 4*(l/32) + r%4][l % 32] in register r.
__device__ __forceinline__ f32x16 mfma32x32x16(u32x4 a, u32x4 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                  __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}

// D(16x16, fp32) += A(16x32) * B(32x16), bf16 operands.
// Lane l holds A[l % 16][8*(l/16) .. +7], B[8*(l/16) .. +7][l % 16] and
// D[4*(l/16) + r][l % 16] in register r.
__device__ __forceinline__ f32x4 mfma16x16x32(u32x4 a, u32x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                  __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}

// Revolutions per unit of position for rotary pair t of a head of dim d:
// theta^(-2t/d) / (2 pi), in fp64.
__device__ __forceinline__ double rope_rev_per_pos(int t, int d, double log2_theta) {
  return exp2(-(2.0 * (double)t / (double)d) * log2_theta) * 0.15915494309189533577;
}

// cos/sin of the angle pos * theta^(-2t/d), from g = rope_rev_per_pos(t).
// The product and the reduction to [-1/2, 1/2] revolution are done in fp64, so
// the angle stays accurate at positions near 2^18 and beyond; the hardware
// sine/cosine (argument in revolutions) then sees a small argument.
__device__ __forceinline__ void rope_cs_fast(int pos, double g, float& c, float& s) {
  double r = (double)pos * g;
  r -= __builtin_rint(r);
  const float x = (float)r;
  s = __builtin_amdgcn_sinf(x);
  c = __builtin_amdgcn_cosf(x);
}

// Same angle with the accurate library sin(pi*y)/cos(pi*y) (fp32 path).
__device__ __forceinline__ void rope_cs_accurate(int pos, double g, float& c, float& s) {
  double r = (double)pos * g;
  r -= __builtin_rint(r);
  sincospif((float)(2.0 * r), &s, &c);
}

// Rotate the 4 pairs packed in a 16-byte chunk of bf16 (dims 8c .. 8c+7, pairs
// 4c .. 4c+3) at position pos; pairs >= n_rot keep their bits.  gtab holds
// rope_rev_per_pos for every pair.  Branch-free: callers skip whole chunks
// with a wave-uniform test.
__device__ __forceinline__ u32x4 rotate_chunk_bf16(u32x4 x, int c, int pos, int n_rot,
                                                   const double* gtab) {
  u32x4 y;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int t = 4 * c + i;
    float cs, sn;
    rope_cs_fast(pos, gtab[t], cs, sn);
    const float x0 = bf_lo(x[i]), x1 = bf_hi(x[i]);
    const uint32_t r = pack_bf16(x0 * cs - x1 * sn, x0 * sn + x1 * cs);
    y[i] = t < n_rot ? r : x[i];
  }
  return y;
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
  return v;
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
  return v;
}

}  // namespace g4a
