// Key/value rows of a prefill written into the decode cache layout, so that
// decoding continues where the prefill ended (the KV cache grows with the
// prompt and the generated tokens: "Visao geral do modelo Gemma 4", section
// "Principais Consideracoes para o planejamento de memoria").
//
// Bound by HBM: one thread per 16-byte chunk, consecutive threads along a row,
// so reads and writes are coalesced row by row.  A cache with separate values
// stores its keys already turned at their positions (RoPE / p-RoPE, section
// "p-RoPE" of "Guia visual do Gemma 4"), once, so that no decode step turns
// them again; a K=V cache stores the raw tensor, which the decode reads raw
// as the values.  The fp8 variant quantizes on the way (16 elements per
// thread).
#include "common.hpp"
#include "kernels.hpp"

namespace g4a {

namespace {

// Revolutions per position of every pair of the head (a bf16 chunk turn reads
// all four pairs of its chunk before selecting), for one block.  Returns true
// when this launch turns keys at all (separate values, n_rot > 0).
__device__ __forceinline__ bool build_turn_table(const FillArgs& a, double* gtab) {
  if (!a.v || a.n_rot == 0) return false;
  for (int t = threadIdx.x; t < a.d / 2; t += 256) gtab[t] = rope_rev_per_pos(t, a.d, a.log2_theta);
  __syncthreads();
  return true;
}

// Tokens first .. first+nw-1 of every sequence: token i goes to slot
// pos mod capacity of a ring, or to row pos of a linear cache when
// 0 <= pos < capacity.  Negative positions are not written.
// Keys of a cache with separate values are turned (bf16: fp32 arithmetic with
// the hardware sine and cosine after an fp64 angle reduction, rounded to
// nearest even, the arithmetic the decode used to apply per step; f32: the
// accurate library sine and cosine).
__global__ void __launch_bounds__(256) fill_cache_kernel(FillArgs a, int first, int nw,
                                                         int total) {
  __shared__ double gtab[256];
  const bool turn = build_turn_table(a, gtab);
  for (int idx = blockIdx.x * 256 + threadIdx.x; idx < total; idx += gridDim.x * 256) {
    const int c = idx % a.row_chunks;
    int r = idx / a.row_chunks;
    const int g = r % a.Hkv;
    r /= a.Hkv;
    const int i = first + r % nw;
    const int b = r / nw;
    const int P = a.pos[(size_t)b * a.S + i];
    if (P < 0 || (a.window == 0 && P >= a.capacity)) continue;
    const int slot = a.window > 0 ? P % a.capacity : P;
    const size_t src = (((size_t)b * a.S + i) * a.Hkv + g) * a.row_chunks + c;
    const size_t dst = (((size_t)b * a.Hkv + g) * a.capacity + slot) * a.row_chunks + c;
    // streaming copy: each chunk is read and written once (non-temporal)
    u32x4 kx = __builtin_nontemporal_load(static_cast<const u32x4*>(a.k) + src);
    if (turn) {
      if (a.in_f32) {  // dims 4c .. 4c+3: pairs 2c, 2c+1
#pragma unroll
        for (int e = 0; e < 2; ++e) {
          const int t = 2 * c + e;
          if (t < a.n_rot) {
            float cs, sn;
            rope_cs_accurate(P, gtab[t], cs, sn);
            const float x0 = __uint_as_float(kx[2 * e]), x1 = __uint_as_float(kx[2 * e + 1]);
            kx[2 * e] = __float_as_uint(x0 * cs - x1 * sn);
            kx[2 * e + 1] = __float_as_uint(x0 * sn + x1 * cs);
          }
        }
      } else if (8 * c < 2 * a.n_rot) {  // dims 8c .. 8c+7: pairs 4c .. 4c+3
        kx = rotate_chunk_bf16(kx, c, P, a.n_rot, gtab);
      }
    }
    __builtin_nontemporal_store(kx, static_cast<u32x4*>(a.k_cache) + dst);
    if (a.v)
      __builtin_nontemporal_store(__builtin_nontemporal_load(static_cast<const u32x4*>(a.v) + src),
                                  static_cast<u32x4*>(a.v_cache) + dst);
  }
}

// E4M3 code of y, round to nearest even (the hardware conversion), after
// saturating |y| >= 448 (infinities too) to +-448; NaN stays NaN.
__device__ __forceinline__ float sat448(float y) {
  return __builtin_fabsf(y) > 448.f ? __builtin_copysignf(448.f, y) : y;
}

// 4 values divided by the scale (IEEE division, rounded once to fp32) -> 4 codes
__device__ __forceinline__ uint32_t quantize4(f32x4 x, float s) {
  int pk = __builtin_amdgcn_cvt_pk_fp8_f32(sat448(x[0] / s), sat448(x[1] / s), 0, false);
  pk = __builtin_amdgcn_cvt_pk_fp8_f32(sat448(x[2] / s), sat448(x[3] / s), pk, true);
  return (uint32_t)pk;
}

// Pairs (x[2i], x[2i+1]) of 4 values, pair t0 + i, turned at position pos
// when t0 + i < n_rot (fp32 arithmetic; F32: accurate sine and cosine).
template <bool F32>
__device__ __forceinline__ f32x4 turn4(f32x4 x, int t0, int pos, int n_rot, const double* gtab) {
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    if (t0 + i < n_rot) {
      float cs, sn;
      if constexpr (F32) rope_cs_accurate(pos, gtab[t0 + i], cs, sn);
      else rope_cs_fast(pos, gtab[t0 + i], cs, sn);
      const float x0 = x[2 * i], x1 = x[2 * i + 1];
      x[2 * i] = x0 * cs - x1 * sn;
      x[2 * i + 1] = x0 * sn + x1 * cs;
    }
  }
  return x;
}

// 16 input elements (bf16 or fp32) of row element offset e -> 16 codes; with
// gtab, the 8 pairs t0 .. t0+7 they hold are first turned at position pos.
template <bool F32>
__device__ __forceinline__ u32x4 quantize16(const void* src, size_t e, float s,
                                            const double* gtab = nullptr, int t0 = 0,
                                            int pos = 0, int n_rot = 0) {
  f32x4 x[4];
  if constexpr (F32) {
    const f32x4* p = reinterpret_cast<const f32x4*>(static_cast<const float*>(src) + e);
#pragma unroll
    for (int j = 0; j < 4; ++j) x[j] = __builtin_nontemporal_load(p + j);
  } else {
    const u32x4* p = reinterpret_cast<const u32x4*>(static_cast<const uint16_t*>(src) + e);
    const u32x4 w0 = __builtin_nontemporal_load(p), w1 = __builtin_nontemporal_load(p + 1);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const uint32_t lo = j < 2 ? w0[2 * j] : w1[2 * j - 4];
      const uint32_t hi = j < 2 ? w0[2 * j + 1] : w1[2 * j - 3];
      x[j] = f32x4{bf_lo(lo), bf_hi(lo), bf_lo(hi), bf_hi(hi)};
    }
  }
  if (gtab && t0 < n_rot) {
#pragma unroll
    for (int j = 0; j < 4; ++j) x[j] = turn4<F32>(x[j], t0 + 2 * j, pos, n_rot, gtab);
  }
  u32x4 out;
#pragma unroll
  for (int j = 0; j < 4; ++j) out[j] = quantize4(x[j], s);
  return out;
}

// The same placement as fill_cache_kernel into a cache of OCP FP8 E4M3 codes
// (cached value = code value * scale of the KV head; the pages leave the
// format of their optimized KV caches open): each 16-byte chunk of codes is
// quantized from 16 input elements, code = E4M3(x / scale).
template <bool F32>
__global__ void __launch_bounds__(256) fill_cache_fp8_kernel(FillArgs a, int first, int nw,
                                                             int total) {
  __shared__ double gtab[256];
  const bool turn = build_turn_table(a, gtab);
  for (int idx = blockIdx.x * 256 + threadIdx.x; idx < total; idx += gridDim.x * 256) {
    const int c = idx % a.row_chunks;
    int r = idx / a.row_chunks;
    const int g = r % a.Hkv;
    r /= a.Hkv;
    const int i = first + r % nw;
    const int b = r / nw;
    const int P = a.pos[(size_t)b * a.S + i];
    if (P < 0 || (a.window == 0 && P >= a.capacity)) continue;
    const int slot = a.window > 0 ? P % a.capacity : P;
    const size_t src = ((((size_t)b * a.S + i) * a.Hkv + g) * a.row_chunks + c) * 16;  // element
    const size_t dst = (((size_t)b * a.Hkv + g) * a.capacity + slot) * a.row_chunks + c;
    __builtin_nontemporal_store(
        quantize16<F32>(a.k, src, a.k_scale[g], turn ? gtab : nullptr, 8 * c, P, a.n_rot),
        static_cast<u32x4*>(a.k_cache) + dst);
    if (a.v)
      __builtin_nontemporal_store(quantize16<F32>(a.v, src, a.v_scale[g]),
                                  static_cast<u32x4*>(a.v_cache) + dst);
  }
}

}  // namespace

hipError_t launch_fill_cache_fp8(const FillArgs& a, hipStream_t st) {
  const int nw = a.window > 0 ? (a.S < a.capacity ? a.S : a.capacity) : a.S;
  const long long total = (long long)a.B * nw * a.Hkv * a.row_chunks;
  if (total == 0) return hipSuccess;
  if (total > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  const long long blocks = (total + 255) / 256;
  const dim3 grid((unsigned)(blocks < 65536 ? blocks : 65536));
  if (a.in_f32)
    hipLaunchKernelGGL(fill_cache_fp8_kernel<true>, grid, dim3(256), 0, st, a, a.S - nw, nw,
                       (int)total);
  else
    hipLaunchKernelGGL(fill_cache_fp8_kernel<false>, grid, dim3(256), 0, st, a, a.S - nw, nw,
                       (int)total);
  return hipGetLastError();
}

hipError_t launch_fill_cache(const FillArgs& a, hipStream_t st) {
  // a ring keeps only the last `capacity` tokens of a sequence
  const int nw = a.window > 0 ? (a.S < a.capacity ? a.S : a.capacity) : a.S;
  const long long total = (long long)a.B * nw * a.Hkv * a.row_chunks;
  if (total == 0) return hipSuccess;
  if (total > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  const long long blocks = (total + 255) / 256;
  hipLaunchKernelGGL(fill_cache_kernel, dim3((unsigned)(blocks < 65536 ? blocks : 65536)),
                     dim3(256), 0, st, a, a.S - nw, nw, (int)total);
  return hipGetLastError();
}

}  // namespace g4a
