// Instances of the bf16 prefill kernel for the vision encoder's attention:
// 2D RoPE (half c of the head dims turns by component c of the patch
// position (w, h)) and no causal mask, over the valid patches of each image
// ("Guia visual do Gemma 4", sections "Encoder de visao" and "Suporte a
// proporcao variavel").  Head dim 256 with separate K and V: the local
// layers' tiling (full-width rotated slab, 3-deep tile ring).
#include "prefill.hpp"

namespace g4a {

// Workgroups of 256 query rows (two 32-row blocks per wave, every K/V
// fragment read feeding both) or of 128 rows.  An image holds at most a few
// thousand patches, so the grid is often only a round or two of workgroups
// across the CUs, and a last round that is mostly empty costs more than the
// second block's sharing saves: the launcher takes the row count whose grid
// fills its rounds better, counting a 128-row workgroup as 0.9 of the work
// rate of a 256-row one (about what the shared fragment reads are worth).
static int cu_count() {
  int dev = 0, n = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
    return 256;
  return n;
}

static double fill_rate(long long blocks, int cus) {
  const long long rounds = (blocks + cus - 1) / cus;
  return rounds > 0 ? (double)blocks / ((double)rounds * cus) : 1.0;
}

template <int G, bool OBF>
static hipError_t vis(const PrefillArgs& a, hipStream_t st) {
  const int cus = cu_count();
  const long long heads = (long long)a.B * a.Hkv;
  const long long blk2 = (a.S + 256 / G - 1) / (256 / G) * heads;
  const long long blk1 = (a.S + 128 / G - 1) / (128 / G) * heads;
  if (0.9 * fill_rate(blk1, cus) > fill_rate(blk2, cus))
    return pf::launch<256, G, false, OBF, 256, 3, 1, false, true>(a, st);
  return pf::launch<256, G, false, OBF, 256, 3, 2, false, true>(a, st);
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
