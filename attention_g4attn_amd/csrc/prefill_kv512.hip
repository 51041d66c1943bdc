// Instances of the bf16 prefill kernel for K=V with head dim 512 (global
// layers): a quarter-width rotated slab with a 3-deep tile ring when at most
// 64 pairs turn (p <= 0.25), otherwise a full-width slab with 2 stages.
#include "prefill.hpp"

namespace g4a {

template <int G, bool OBF>
static hipError_t kv512(const PrefillArgs& a, hipStream_t st) {
  // without a window, 4 or 8 query heads per KV head put a workgroup's tokens
  // in one key tile: every wave computes every tile, so the loop can be
  // software-pipelined (3-deep ring, loads spread over the products, pairs
  // of waves sharing their rows' value products)
  if constexpr (G >= 4)
    if (a.n_rot <= 64 && a.window == 0) return pf::launch<512, G, true, OBF, 128, 3, 1, true>(a, st);
  if (a.n_rot <= 64) return pf::launch<512, G, true, OBF, 128, 3, 1>(a, st);
  return pf::launch<512, G, true, OBF, 512, 2, 1>(a, st);
}

template <bool OBF>
static hipError_t kv512_g(const PrefillArgs& a, hipStream_t st) {
  switch (a.Hq / a.Hkv) {
    case 1: return kv512<1, OBF>(a, st);
    case 2: return kv512<2, OBF>(a, st);
    case 4: return kv512<4, OBF>(a, st);
    case 8: return kv512<8, OBF>(a, st);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_prefill_kv512(const PrefillArgs& a, bool out_bf16, hipStream_t st) {
  return out_bf16 ? kv512_g<true>(a, st) : kv512_g<false>(a, st);
}

}  // namespace g4a
