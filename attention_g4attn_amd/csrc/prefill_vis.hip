// Instances of the bf16 prefill kernel for the vision encoder's attention:
// 2D RoPE (half c of the head dims turns by component c of the patch
// position (w, h)) and no causal mask, over the valid patches of each image
// ("Guia visual do Gemma 4", sections "Encoder de visao" and "Suporte a
// proporcao variavel").  Head dim 256 with separate K and V, at the local
// layers' tiling: full-width rotated slab, 2-stage tile ring, 32 query rows
// per wave, two workgroups per CU.  128-row workgroups also keep the small
// grids of a few images from ending in a mostly empty round.
#include "prefill.hpp"

namespace g4a {

template <int G, bool OBF>
static hipError_t vis(const PrefillArgs& a, hipStream_t st) {
  return pf::launch<256, G, false, OBF, 256, 2, 1, false, true>(a, st);
}

template <bool OBF>
static hipError_t vis_g(const PrefillArgs& a, hipStream_t st) {
  switch (a.Hq / a.Hkv) {
    case 1: return vis<1, OBF>(a, st);
    case 2: return vis<2, OBF>(a, st);
    case 4: return vis<4, OBF>(a, st);
    case 8: return vis<8, OBF>(a, st);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_vision_prefill(const PrefillArgs& a, bool out_bf16, hipStream_t st) {
  if (a.D != 256) return hipErrorInvalidValue;
  return out_bf16 ? vis_g<true>(a, st) : vis_g<false>(a, st);
}

}  // namespace g4a
