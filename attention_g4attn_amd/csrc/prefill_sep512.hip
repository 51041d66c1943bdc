// Instances of the bf16 prefill kernel for separate K and V with head dim 512:
// quarter-width rotated slab (at most 64 turning pairs), 2 stages (two raw
// 32 KB tiles per stage fill the LDS).
#include "prefill.hpp"

namespace g4a {

template <int G, bool OBF>
static hipError_t sep512(const PrefillArgs& a, hipStream_t st) {
  if (a.n_rot <= 64) return pf::launch<512, G, false, OBF, 128, 2, 1>(a, st);
  return pf::launch<512, G, false, OBF, 512, 2, 1>(a, st);
}

template <bool OBF>
static hipError_t sep512_g(const PrefillArgs& a, hipStream_t st) {
  switch (a.Hq / a.Hkv) {
    case 1: return sep512<1, OBF>(a, st);
    case 2: return sep512<2, OBF>(a, st);
    case 4: return sep512<4, OBF>(a, st);
    case 8: return sep512<8, OBF>(a, st);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_prefill_sep512(const PrefillArgs& a, bool out_bf16, hipStream_t st) {
  return out_bf16 ? sep512_g<true>(a, st) : sep512_g<false>(a, st);
}

bool prefill_supported(int D) { return D == 256 || D == 512; }

int prefill_slab_dims(int D, int n_rot) { return (D == 512 && n_rot <= 64) ? 128 : D; }

hipError_t launch_prefill_bf16(const PrefillArgs& a, bool kv_shared, bool out_bf16,
                               hipStream_t st) {
  if (!prefill_supported(a.D)) return hipErrorInvalidValue;
  if (a.D == 256) return launch_prefill_d256(a, kv_shared, out_bf16, st);
  if (kv_shared) return launch_prefill_kv512(a, out_bf16, st);
  return launch_prefill_sep512(a, out_bf16, st);
}

}  // namespace g4a
