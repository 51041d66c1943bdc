// Instances of the bf16 prefill kernel for head dim 256 (local layers, and K=V
// at d = 256): full-width rotated slab, 2-stage tile ring, 32 query rows per
// wave, two workgroups per CU.  Measured against 64 rows per wave (two
// 32-row blocks sharing every K/V fragment) with a 3-stage ring at one
// workgroup per CU: 6.7 -> 6.4 ms at S = 262144 and 0.95 -> 0.85 ms at
// S = 32768 (window 1024, 16 query and 8 KV heads).
#include "prefill.hpp"

namespace g4a {

template <int G, bool KVS, bool OBF>
static hipError_t d256(const PrefillArgs& a, hipStream_t st) {
  return pf::launch<256, G, KVS, OBF, 256, 2, 1>(a, st);
}

template <bool KVS, bool OBF>
static hipError_t d256_g(const PrefillArgs& a, hipStream_t st) {
  switch (a.Hq / a.Hkv) {
    case 1: return d256<1, KVS, OBF>(a, st);
    case 2: return d256<2, KVS, OBF>(a, st);
    case 4: return d256<4, KVS, OBF>(a, st);
    case 8: return d256<8, KVS, OBF>(a, st);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_prefill_d256(const PrefillArgs& a, bool kv_shared, bool out_bf16,
                               hipStream_t st) {
  if (kv_shared) return out_bf16 ? d256_g<true, true>(a, st) : d256_g<true, false>(a, st);
  return out_bf16 ? d256_g<false, true>(a, st) : d256_g<false, false>(a, st);
}

}  // namespace g4a
