// Raw key/value rows of a prefill written into the decode cache layout, so
// that decoding continues where the prefill ended (the KV cache grows with the
// prompt and the generated tokens: "Visao geral do modelo Gemma 4", section
// "Principais Consideracoes para o planejamento de memoria").
//
// A plain copy, bound by HBM: one thread per 16-byte chunk, consecutive
// threads along a row, so reads and writes are coalesced row by row.
#include "common.hpp"
#include "kernels.hpp"

namespace g4a {

namespace {

// Tokens first .. first+nw-1 of every sequence: token i goes to slot
// pos mod capacity of a ring, or to row pos of a linear cache when
// 0 <= pos < capacity.  Negative positions are not written.
__global__ void __launch_bounds__(256) fill_cache_kernel(FillArgs a, int first, int nw,
                                                         int total) {
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
    static_cast<u32x4*>(a.k_cache)[dst] = static_cast<const u32x4*>(a.k)[src];
    if (a.v) static_cast<u32x4*>(a.v_cache)[dst] = static_cast<const u32x4*>(a.v)[src];
  }
}

}  // namespace

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
