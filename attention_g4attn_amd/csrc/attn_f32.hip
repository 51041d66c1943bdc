// float32-input attention (prefill and decode) on the fp32 vector units.
//
// Computes the same function as the bf16 matrix-core kernels (prefill.hpp,
// decode_bf16.hip) for f32 inputs, keeping every product in fp32 so that the
// result tracks the exact one to ~1e-6.  One wave per (query token, KV head)
// handles the G query heads of that KV head: keys stream in blocks of 64 (one
// per lane) for the scores, the block softmax is merged online, and the value
// product runs with lanes over head dims.  Rotation angles are reduced in fp64
// and evaluated with the accurate sin/cos of pi*x.
#include "common.hpp"
#include "kernels.hpp"

namespace g4a {

namespace {

// Prefill keys: row j of the sequence at its own position.
struct SeqKeys {
  const float* k;
  const float* v;
  const int32_t* pos;
  size_t base;     // (b * S) * Hkv + hkv, in rows
  size_t stride;   // Hkv * D
  size_t pbase;    // b * S + first key
  int D;
  __device__ const float* krow(int j) const { return k + (base + (size_t)j * (stride / D)) * D; }
  __device__ const float* vrow(int j) const { return v + (base + (size_t)j * (stride / D)) * D; }
  __device__ int kpos(int j) const { return pos[pbase + j]; }
};

// Decode keys: index j -> position t0 + j, cache slot t mod capacity (ring) or t.
struct CacheKeys {
  const float* k;
  const float* v;
  size_t base;  // ((b * Hkv) + hkv) * capacity, in rows
  int D, window, capacity, t0;
  __device__ int slot(int j) const { return window > 0 ? (t0 + j) % capacity : t0 + j; }
  __device__ const float* krow(int j) const { return k + (base + slot(j)) * D; }
  __device__ const float* vrow(int j) const { return v + (base + slot(j)) * D; }
  __device__ int kpos(int j) const { return t0 + j; }
};

// Attention of the G query heads in qs (already rotated) over keys 0..n-1 of
// src, each key turned at its position (pairs t < n_rot; 0 for keys cached
// already turned); writes acc/l to out rows out_h[h].
template <int D, int G, class Src>
__device__ void attend_f32(const Src& src, int n, const float (*qs)[D], float (*ps)[64],
                           const double* gt, int n_rot, float scale, float* const* out_h) {
  const int lane = threadIdx.x;
  float m[G], l[G], acc[G][D / 64];
#pragma unroll
  for (int h = 0; h < G; ++h) {
    m[h] = -INFINITY;
    l[h] = 0.f;
#pragma unroll
    for (int e = 0; e < D / 64; ++e) acc[h][e] = 0.f;
  }
  for (int jb = 0; jb < n; jb += 64) {
    const int j = jb + lane;
    const bool valid = j < n;
    const int jc = valid ? j : n - 1;
    const float* kr = src.krow(jc);
    const int kp = src.kpos(jc);
    float s[G];
#pragma unroll
    for (int h = 0; h < G; ++h) s[h] = 0.f;
    for (int t = 0; t < D / 2; ++t) {
      float y0 = kr[2 * t], y1 = kr[2 * t + 1];
      if (t < n_rot) {
        float c, sn;
        rope_cs_accurate(kp, gt[t], c, sn);
        const float x0 = y0, x1 = y1;
        y0 = x0 * c - x1 * sn;
        y1 = x0 * sn + x1 * c;
      }
#pragma unroll
      for (int h = 0; h < G; ++h) s[h] += qs[h][2 * t] * y0 + qs[h][2 * t + 1] * y1;
    }
#pragma unroll
    for (int h = 0; h < G; ++h) {
      const float sv = valid ? s[h] * scale : -INFINITY;
      const float mn = fmaxf(m[h], wave_max(sv));
      const float alpha = m[h] == -INFINITY ? 0.f : expf(m[h] - mn);
      const float p = valid ? expf(sv - mn) : 0.f;
      ps[h][lane] = p;
      l[h] = l[h] * alpha + wave_sum(p);
#pragma unroll
      for (int e = 0; e < D / 64; ++e) acc[h][e] *= alpha;
      m[h] = mn;
    }
    __syncthreads();
    const int nj = min(64, n - jb);
    for (int jj = 0; jj < nj; ++jj) {
      const float* vr = src.vrow(jb + jj);
#pragma unroll
      for (int e = 0; e < D / 64; ++e) {
        const float vv = vr[lane + 64 * e];
#pragma unroll
        for (int h = 0; h < G; ++h) acc[h][e] += ps[h][jj] * vv;
      }
    }
    __syncthreads();
  }
#pragma unroll
  for (int h = 0; h < G; ++h)
#pragma unroll
    for (int e = 0; e < D / 64; ++e) out_h[h][lane + 64 * e] = acc[h][e] / l[h];
}

// Load the G query rows q[qrow + h*D] into qs and rotate them to position qpos.
template <int D, int G>
__device__ void load_queries(const float* q, float (*qs)[D], const double* gt, int n_rot,
                             int qpos) {
  const int lane = threadIdx.x;
  for (int idx = lane; idx < G * D; idx += 64) qs[idx / D][idx % D] = q[idx];
  __syncthreads();
  for (int idx = lane; idx < G * (D / 2); idx += 64) {
    const int h = idx / (D / 2), t = idx % (D / 2);
    if (t < n_rot) {
      float c, sn;
      rope_cs_accurate(qpos, gt[t], c, sn);
      const float x0 = qs[h][2 * t], x1 = qs[h][2 * t + 1];
      qs[h][2 * t] = x0 * c - x1 * sn;
      qs[h][2 * t + 1] = x0 * sn + x1 * c;
    }
  }
  __syncthreads();
}

template <int D, int G>
__global__ void __launch_bounds__(64) prefill_f32_kernel(PrefillArgs a) {
  __shared__ float qs[G][D];
  __shared__ float ps[G][64];
  __shared__ double gt[D / 2];
  const int lane = threadIdx.x;
  const int nh = a.B * a.Hkv;
  const int hb = blockIdx.x % nh;
  const int i = a.S - 1 - blockIdx.x / nh;  // longest rows first
  const int b = hb / a.Hkv, hkv = hb % a.Hkv;
  for (int t = lane; t < D / 2; t += 64) gt[t] = rope_rev_per_pos(t, D, a.log2_theta);
  __syncthreads();
  const size_t qrow = (((size_t)b * a.S + i) * a.Hq + hkv * G) * D;
  load_queries<D, G>(static_cast<const float*>(a.q) + qrow, qs, gt, a.n_rot,
                     a.pos[(size_t)b * a.S + i]);
  const int lo = a.window > 0 ? max(0, i - a.window + 1) : 0;
  SeqKeys src;
  src.k = static_cast<const float*>(a.k);
  src.v = static_cast<const float*>(a.v);
  src.pos = a.pos;
  src.D = D;
  src.stride = (size_t)a.Hkv * D;
  src.base = ((size_t)b * a.S + lo) * a.Hkv + hkv;
  src.pbase = (size_t)b * a.S + lo;
  float* outp[G];
#pragma unroll
  for (int h = 0; h < G; ++h) outp[h] = static_cast<float*>(a.out) + qrow + (size_t)h * D;
  attend_f32<D, G>(src, i - lo + 1, qs, ps, gt, a.n_rot, a.scale, outp);
}

// One wave per (b, kv head, query token j); token j sits at P - q_len + 1 + j.
template <int D, int G>
__global__ void __launch_bounds__(64) decode_f32_kernel(DecodeArgs a) {
  __shared__ float qs[G][D];
  __shared__ float ps[G][64];
  __shared__ double gt[D / 2];
  const int lane = threadIdx.x;
  const int j = blockIdx.x % a.q_len;
  const int bh = blockIdx.x / a.q_len;
  const int b = bh / a.Hkv, hkv = bh % a.Hkv;
  const int P = a.pos[b], Pj = P - a.q_len + 1 + j;
  const size_t qrow = (((size_t)b * a.q_len + j) * a.Hq + hkv * G) * D;
  float* outp[G];
#pragma unroll
  for (int h = 0; h < G; ++h) outp[h] = static_cast<float*>(a.out) + qrow + (size_t)h * D;
  if (P < 0 || Pj < 0 || (a.window == 0 && P >= a.capacity)) {
    for (int idx = lane; idx < G * D; idx += 64) outp[idx / D][idx % D] = __builtin_nanf("");
    return;
  }
  for (int t = lane; t < D / 2; t += 64) gt[t] = rope_rev_per_pos(t, D, a.log2_theta);
  __syncthreads();
  load_queries<D, G>(static_cast<const float*>(a.q) + qrow, qs, gt, a.n_rot, Pj);
  const int t0 = a.window > 0 ? max(0, Pj - a.window + 1) : 0;
  CacheKeys src;
  src.k = static_cast<const float*>(a.k);
  src.v = static_cast<const float*>(a.v);
  src.base = ((size_t)b * a.Hkv + hkv) * a.capacity;
  src.D = D;
  src.window = a.window;
  src.capacity = a.capacity;
  src.t0 = t0;
  // a cache with separate values holds its keys turned; K=V keys are raw
  attend_f32<D, G>(src, Pj - t0 + 1, qs, ps, gt, a.v == a.k ? a.n_rot : 0, a.scale, outp);
}

template <int D>
hipError_t prefill_g(const PrefillArgs& a, hipStream_t st) {
  const long long n = (long long)a.B * a.Hkv * a.S;
  if (n == 0) return hipSuccess;
  if (n > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  switch (a.Hq / a.Hkv) {
    case 1: hipLaunchKernelGGL((prefill_f32_kernel<D, 1>), dim3(n), dim3(64), 0, st, a); break;
    case 2: hipLaunchKernelGGL((prefill_f32_kernel<D, 2>), dim3(n), dim3(64), 0, st, a); break;
    case 4: hipLaunchKernelGGL((prefill_f32_kernel<D, 4>), dim3(n), dim3(64), 0, st, a); break;
    case 8: hipLaunchKernelGGL((prefill_f32_kernel<D, 8>), dim3(n), dim3(64), 0, st, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <int D>
hipError_t decode_g(const DecodeArgs& a, hipStream_t st) {
  const long long n = (long long)a.B * a.Hkv * a.q_len;
  if (n == 0) return hipSuccess;
  if (n > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  switch (a.Hq / a.Hkv) {
    case 1: hipLaunchKernelGGL((decode_f32_kernel<D, 1>), dim3(n), dim3(64), 0, st, a); break;
    case 2: hipLaunchKernelGGL((decode_f32_kernel<D, 2>), dim3(n), dim3(64), 0, st, a); break;
    case 4: hipLaunchKernelGGL((decode_f32_kernel<D, 4>), dim3(n), dim3(64), 0, st, a); break;
    case 8: hipLaunchKernelGGL((decode_f32_kernel<D, 8>), dim3(n), dim3(64), 0, st, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_prefill_f32(const PrefillArgs& a, hipStream_t st) {
  switch (a.D) {
    case 64: return prefill_g<64>(a, st);
    case 128: return prefill_g<128>(a, st);
    case 256: return prefill_g<256>(a, st);
    case 512: return prefill_g<512>(a, st);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_decode_f32(const DecodeArgs& a, hipStream_t st) {
  switch (a.D) {
    case 64: return decode_g<64>(a, st);
    case 128: return decode_g<128>(a, st);
    case 256: return decode_g<256>(a, st);
    case 512: return decode_g<512>(a, st);
  }
  return hipErrorInvalidValue;
}

}  // namespace g4a
