// C ABI of libg4attn: argument validation and dispatch to the gfx950 kernels.
// Every check runs on the host before anything is launched; the library keeps
// no state between calls apart from a per-thread copy of the last launch
// error.  See include/g4attn.h for the contract of each call.
#include "../../include/g4attn.h"

#include <math.h>

#include "kernels.hpp"

#define G4A_API extern "C" __attribute__((visibility("default")))

namespace {

thread_local int g_last_hip_error = 0;

bool misaligned(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) != 0; }

bool valid_group(int G) { return G == 1 || G == 2 || G == 4 || G == 8; }

// n_rot = floor(p * d / 2), the number of rotated pairs
int rotated_pairs(int d, float p) {
  int n = (int)floor((double)p * (double)d / 2.0);
  if (n < 0) n = 0;
  if (n > d / 2) n = d / 2;
  return n;
}

// Shared checks of head layout, rotary parameters and dtypes.
int check_common(int Hq, int Hkv, int d, int window, float theta, float p, int in_dtype,
                 int out_dtype) {
  if (Hq <= 0 || Hkv <= 0 || d <= 0 || (d & 1) || window < 0) return G4A_EINVAL;
  if (Hq % Hkv) return G4A_EINVAL;
  if (!(theta > 0.f) || isinf(theta)) return G4A_EINVAL;
  if (!(p >= 0.f && p <= 1.f)) return G4A_EINVAL;
  if ((in_dtype != G4A_F32 && in_dtype != G4A_BF16) ||
      (out_dtype != G4A_F32 && out_dtype != G4A_BF16))
    return G4A_EINVAL;
  if (in_dtype == G4A_F32 && out_dtype != G4A_F32) return G4A_EUNSUPPORTED;
  if (!valid_group(Hq / Hkv)) return G4A_EUNSUPPORTED;
  if (in_dtype == G4A_BF16 && d != 256 && d != 512) return G4A_EUNSUPPORTED;
  if (in_dtype == G4A_F32 && d != 64 && d != 128 && d != 256 && d != 512) return G4A_EUNSUPPORTED;
  return G4A_OK;
}

// The bf16 prefill kernels address a key row inside a tile as row * (Hkv * d
// * 2 bytes) with a 24-bit multiply, so one token's keys of all KV heads must
// span fewer than 2^24 bytes (Hkv < 16384 at d = 512, < 32768 at d = 256).
bool prefill_rows_addressable(int Hkv, int d) { return (long long)Hkv * d * 2 < (1LL << 24); }

int finish(hipError_t e) {
  if (e == hipSuccess) return G4A_OK;
  g_last_hip_error = (int)e;
  return G4A_EHIP;
}

// bytes of the rotated key slab a bf16 prefill needs (0 for f32 inputs)
size_t prefill_ws_bytes(int B, int S, int Hkv, int d, int n_rot, int in_dtype) {
  if (in_dtype != G4A_BF16) return 0;
  return (size_t)B * S * Hkv * g4a::prefill_slab_dims(d, n_rot) * 2;
}

// Fields of a prefill launch shared by the causal and the vision calls.
g4a::PrefillArgs prefill_args(const void* q, const void* k, const void* v, void* out,
                              const int32_t* pos, int B, int S, int Hq, int Hkv, int d, int window,
                              float theta, int n_rot) {
  g4a::PrefillArgs a{};
  a.q = q;
  a.k = k;
  a.v = v;
  a.out = out;
  a.pos = pos;
  a.B = B;
  a.S = S;
  a.Hq = Hq;
  a.Hkv = Hkv;
  a.D = d;
  a.window = window;
  a.n_rot = n_rot;
  a.log2_theta = log2((double)theta);
  a.scale = (float)(1.0 / sqrt((double)d));
  a.scale_log2e = (float)(1.4426950408889634 / sqrt((double)d));
  return a;
}

int prefill(const void* q, const void* k, const void* v, void* out, const int32_t* pos, int B,
            int S, int Hq, int Hkv, int d, int window, float theta, float p, int in_dtype,
            int out_dtype, void* workspace, size_t workspace_bytes, void* stream,
            bool kv_shared) {
  if (B < 0 || S < 0) return G4A_EINVAL;
  int rc = check_common(Hq, Hkv, d, window, theta, p, in_dtype, out_dtype);
  if (rc) return rc;
  if (B == 0 || S == 0) return G4A_OK;
  if (!q || !k || !v || !out || !pos) return G4A_EINVAL;
  if (misaligned(q) || misaligned(k) || misaligned(v) || misaligned(out) || misaligned(pos))
    return G4A_EALIGN;
  // element counts must stay addressable; the grid must fit in 2^31 workgroups
  if ((double)B * S * Hq * d > 9.0e18 || (double)B * S * Hkv > 2.0e9) return G4A_EINVAL;
  g4a::PrefillArgs a =
      prefill_args(q, k, v, out, pos, B, S, Hq, Hkv, d, window, theta, rotated_pairs(d, p));
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (in_dtype == G4A_F32) return finish(g4a::launch_prefill_f32(a, st));
  if (!g4a::prefill_supported(d) || !prefill_rows_addressable(Hkv, d)) return G4A_EUNSUPPORTED;
  const size_t need = prefill_ws_bytes(B, S, Hkv, d, a.n_rot, in_dtype);
  if (!workspace || workspace_bytes < need) return G4A_EWORKSPACE;
  if (misaligned(workspace)) return G4A_EALIGN;
  a.ws = workspace;
  return finish(g4a::launch_prefill_bf16(a, kv_shared, out_dtype == G4A_BF16, st));
}

}  // namespace

G4A_API size_t g4attn_prefill_workspace_bytes(int B, int S, int Hkv, int d, float p,
                                              int in_dtype) {
  if (B < 0 || S < 0 || Hkv <= 0 || d <= 0 || !(p >= 0.f && p <= 1.f)) return 0;
  return prefill_ws_bytes(B, S, Hkv, d, rotated_pairs(d, p), in_dtype);
}

G4A_API int g4attn_local_prefill(const void* q, const void* k, const void* v, void* out,
                                 const int32_t* pos, int B, int S, int Hq, int Hkv, int d,
                                 int window, float theta, float p, int in_dtype, int out_dtype,
                                 void* workspace, size_t workspace_bytes, void* stream) {
  return prefill(q, k, v, out, pos, B, S, Hq, Hkv, d, window, theta, p, in_dtype, out_dtype,
                 workspace, workspace_bytes, stream, k == v);
}

G4A_API int g4attn_global_prefill(const void* q, const void* kv, void* out, const int32_t* pos,
                                  int B, int S, int Hq, int Hkv, int d, int window, float theta,
                                  float p, int in_dtype, int out_dtype, void* workspace,
                                  size_t workspace_bytes, void* stream) {
  return prefill(q, kv, kv, out, pos, B, S, Hq, Hkv, d, window, theta, p, in_dtype, out_dtype,
                 workspace, workspace_bytes, stream, true);
}

G4A_API int g4attn_vision_prefill(const void* q, const void* k, const void* v, void* out,
                                  const int32_t* pos2, const int32_t* lengths, int B, int S,
                                  int Hq, int Hkv, int d, float theta, int in_dtype,
                                  int out_dtype, void* workspace, size_t workspace_bytes,
                                  void* stream) {
  if (B < 0 || S < 0) return G4A_EINVAL;
  int rc = check_common(Hq, Hkv, d, 0, theta, 1.f, in_dtype, out_dtype);
  if (rc) return rc;
  if (in_dtype != G4A_BF16 || d != 256 || !prefill_rows_addressable(Hkv, d))
    return G4A_EUNSUPPORTED;
  if (B == 0 || S == 0) return G4A_OK;
  if (!q || !k || !v || !out || !pos2) return G4A_EINVAL;
  if (misaligned(q) || misaligned(k) || misaligned(v) || misaligned(out) || misaligned(pos2) ||
      (lengths && misaligned(lengths)))
    return G4A_EALIGN;
  if ((double)B * S * Hq * d > 9.0e18 || (double)B * S * Hkv > 2.0e9) return G4A_EINVAL;
  // every pair of both halves turns
  g4a::PrefillArgs a = prefill_args(q, k, v, out, pos2, B, S, Hq, Hkv, d, 0, theta, d / 2);
  a.lengths = lengths;
  const size_t need = prefill_ws_bytes(B, S, Hkv, d, a.n_rot, in_dtype);
  if (!workspace || workspace_bytes < need) return G4A_EWORKSPACE;
  if (misaligned(workspace)) return G4A_EALIGN;
  a.ws = workspace;
  return finish(g4a::launch_vision_prefill(a, out_dtype == G4A_BF16,
                                           static_cast<hipStream_t>(stream)));
}

namespace {

// Ring rule: plain decode keeps capacity == window; several query tokens need
// capacity >= window + q_len - 1 (the first token's window must still be held).
bool ring_ok(int capacity, int window, int q_len, bool multi) {
  if (window == 0) return true;
  return multi ? capacity >= window + q_len - 1 : capacity == window;
}

// Fields of a decode launch shared by every cache type; chunking, workspace
// and scales are set by the caller.
g4a::DecodeArgs decode_args(const void* q, const void* k_cache, const void* v_cache, void* out,
                            const int32_t* pos, int B, int q_len, int Hq, int Hkv, int d,
                            int capacity, int window, float theta, float p) {
  g4a::DecodeArgs a{};
  a.q = q;
  a.k = k_cache;
  a.v = v_cache ? v_cache : k_cache;
  a.out = out;
  a.pos = pos;
  a.B = B;
  a.Hq = Hq;
  a.Hkv = Hkv;
  a.D = d;
  a.capacity = capacity;
  a.window = window;
  a.n_rot = rotated_pairs(d, p);
  a.q_len = q_len;
  a.ncb = ((Hq / Hkv) * q_len + 15) / 16;
  a.log2_theta = log2((double)theta);
  a.scale = (float)(1.0 / sqrt((double)d));
  a.scale_log2e = (float)(1.4426950408889634 / sqrt((double)d));
  return a;
}

size_t decode_ws_bytes(int B, int q_len, int Hq, int Hkv, int d, int capacity, int window,
                       bool multi) {
  if (B < 0 || q_len < 1 || q_len > 8 || Hq <= 0 || Hkv <= 0 || d <= 0 || capacity <= 0 ||
      window < 0)
    return 0;
  if (!ring_ok(capacity, window, q_len, multi)) return 0;
  const size_t nch = (size_t)g4a::decode_num_chunks(d, capacity, window, false);
  const size_t bytes = (size_t)B * q_len * Hq * nch * ((size_t)d + 2) * sizeof(float);
  return bytes > 0 ? bytes : 16;
}

int decode(const void* q, const void* k_cache, const void* v_cache, void* out,
           const int32_t* pos, int B, int q_len, int Hq, int Hkv, int d, int capacity,
           int window, float theta, float p, int in_dtype, int out_dtype, void* workspace,
           size_t workspace_bytes, void* stream, bool multi) {
  if (B < 0 || capacity <= 0 || q_len < 1 || q_len > 8) return G4A_EINVAL;
  if (!ring_ok(capacity, window, q_len, multi)) return G4A_EINVAL;
  int rc = check_common(Hq, Hkv, d, window, theta, p, in_dtype, out_dtype);
  if (rc) return rc;
  if (B == 0) return G4A_OK;
  if (!q || !k_cache || !out || !pos) return G4A_EINVAL;
  if (misaligned(q) || misaligned(k_cache) || (v_cache && misaligned(v_cache)) ||
      misaligned(out) || misaligned(pos))
    return G4A_EALIGN;
  if ((double)B * Hkv * capacity * d > 9.0e18) return G4A_EINVAL;
  const bool f32 = in_dtype == G4A_F32;
  g4a::DecodeArgs a = decode_args(q, k_cache, v_cache, out, pos, B, q_len, Hq, Hkv, d, capacity,
                                  window, theta, p);
  a.chunk = g4a::decode_chunk_rows(d, capacity, window, f32);
  a.nchunk = g4a::decode_num_chunks(d, capacity, window, f32);
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (f32) return finish(g4a::launch_decode_f32(a, st));
  const size_t need = decode_ws_bytes(B, q_len, Hq, Hkv, d, capacity, window, multi);
  if (!workspace || workspace_bytes < need) return G4A_EWORKSPACE;
  if (misaligned(workspace)) return G4A_EALIGN;
  if ((double)B * Hkv * a.ncb * a.nchunk > 2.0e9) return G4A_EINVAL;
  a.part_o = static_cast<float*>(workspace);
  a.part_ml = a.part_o + (size_t)B * q_len * Hq * a.nchunk * d;
  return finish(g4a::launch_decode_bf16(a, v_cache == nullptr || v_cache == k_cache,
                                        out_dtype == G4A_BF16, st));
}

}  // namespace

G4A_API int g4attn_decode_noalloc(const void* q, const void* k_cache, const void* v_cache,
                                  void* out, const int32_t* pos, int B, int Hq, int Hkv, int d,
                                  int capacity, int window, float theta, float p, int in_dtype,
                                  int out_dtype, void* stream) {
  // Sizes are checked against the fixed buffer before any HIP call; the rest
  // of the validation is g4attn_decode's.
  const bool bf16 = in_dtype == G4A_BF16;
  size_t need = 0;
  if (bf16) {
    need = decode_ws_bytes(B, 1, Hq, Hkv, d, capacity, window, false);
    if (need > g4a::kDecodeScratchBytes) return G4A_ESCRATCH;
  }
  if (B <= 0 || !bf16) {  // nothing launched, or the fp32 path (no partials)
    return decode(q, k_cache, v_cache, out, pos, B, 1, Hq, Hkv, d, capacity, window, theta, p,
                  in_dtype, out_dtype, nullptr, 0, stream, false);
  }
  if (need == 0) return G4A_EINVAL;  // sizes the workspace query rejects
  int rc = check_common(Hq, Hkv, d, window, theta, p, in_dtype, out_dtype);
  if (rc) return rc;
  if (!q || !k_cache || !out || !pos) return G4A_EINVAL;
  void* ws = nullptr;
  const hipError_t e = g4a::decode_scratch(&ws);
  if (e != hipSuccess) return finish(e);
  return decode(q, k_cache, v_cache, out, pos, B, 1, Hq, Hkv, d, capacity, window, theta, p,
                in_dtype, out_dtype, ws, g4a::kDecodeScratchBytes, stream, false);
}

G4A_API size_t g4attn_decode_workspace_bytes(int B, int Hq, int Hkv, int d, int capacity,
                                             int window) {
  return decode_ws_bytes(B, 1, Hq, Hkv, d, capacity, window, false);
}

G4A_API size_t g4attn_decode_multi_workspace_bytes(int B, int q_len, int Hq, int Hkv, int d,
                                                   int capacity, int window) {
  return decode_ws_bytes(B, q_len, Hq, Hkv, d, capacity, window, true);
}

G4A_API int g4attn_decode(const void* q, const void* k_cache, const void* v_cache, void* out,
                          const int32_t* pos, int B, int Hq, int Hkv, int d, int capacity,
                          int window, float theta, float p, int in_dtype, int out_dtype,
                          void* workspace, size_t workspace_bytes, void* stream) {
  return decode(q, k_cache, v_cache, out, pos, B, 1, Hq, Hkv, d, capacity, window, theta, p,
                in_dtype, out_dtype, workspace, workspace_bytes, stream, false);
}

G4A_API int g4attn_decode_multi(const void* q, const void* k_cache, const void* v_cache,
                                void* out, const int32_t* pos, int B, int q_len, int Hq, int Hkv,
                                int d, int capacity, int window, float theta, float p,
                                int in_dtype, int out_dtype, void* workspace,
                                size_t workspace_bytes, void* stream) {
  return decode(q, k_cache, v_cache, out, pos, B, q_len, Hq, Hkv, d, capacity, window, theta, p,
                in_dtype, out_dtype, workspace, workspace_bytes, stream, true);
}

namespace {

// Fields of a cache fill shared by the byte copy and the quantizing fill; a
// false return means the grid would not fit (G4A_EINVAL).
bool fill_args(g4a::FillArgs& a, const void* k, const void* v, const int32_t* pos, int B, int S,
               int Hkv, void* k_cache, void* v_cache, int capacity, int window, int row_chunks) {
  a = g4a::FillArgs{};
  a.k = k;
  a.v = v;
  a.pos = pos;
  a.k_cache = k_cache;
  a.v_cache = v ? v_cache : nullptr;
  a.B = B;
  a.S = S;
  a.Hkv = Hkv;
  a.capacity = capacity;
  a.window = window;
  a.row_chunks = row_chunks;
  const int nw = window > 0 ? (S < capacity ? S : capacity) : S;  // tokens a ring keeps
  return (double)B * nw * Hkv * row_chunks <= 2.0e9;
}

}  // namespace

namespace {

// Rotary parameters of a fill: the keys of a cache with separate values are
// turned (pairs t < n_rot), so theta and p must be valid there, and the head
// dim at most 512 (the per-block table of pair frequencies).
int fill_turn_check(const void* v, int d, float theta, float p) {
  if (!(theta > 0.f) || isinf(theta)) return G4A_EINVAL;
  if (!(p >= 0.f && p <= 1.f)) return G4A_EINVAL;
  if (v && rotated_pairs(d, p) > 0 && d > 512) return G4A_EUNSUPPORTED;
  return G4A_OK;
}

}  // namespace

G4A_API int g4attn_fill_cache(const void* k, const void* v, const int32_t* pos, int B, int S,
                              int Hkv, int d, void* k_cache, void* v_cache, int capacity,
                              int window, float theta, float p, int dtype, void* stream) {
  if (B < 0 || S < 0 || Hkv <= 0 || d <= 0 || capacity <= 0 || window < 0) return G4A_EINVAL;
  if (dtype != G4A_F32 && dtype != G4A_BF16) return G4A_EUNSUPPORTED;
  const int esize = dtype == G4A_F32 ? 4 : 2;
  if (((long long)d * esize) % 16) return G4A_EUNSUPPORTED;
  if (int rc = fill_turn_check(v, d, theta, p)) return rc;
  if (B == 0 || S == 0) return G4A_OK;
  if (!k || !pos || !k_cache || (v && !v_cache)) return G4A_EINVAL;
  if (misaligned(k) || (v && misaligned(v)) || misaligned(pos) || misaligned(k_cache) ||
      (v && misaligned(v_cache)))
    return G4A_EALIGN;
  g4a::FillArgs a;
  if (!fill_args(a, k, v, pos, B, S, Hkv, k_cache, v_cache, capacity, window,
                 (int)((long long)d * esize / 16)))
    return G4A_EINVAL;
  a.in_f32 = dtype == G4A_F32;
  a.d = d;
  a.n_rot = rotated_pairs(d, p);
  a.log2_theta = log2((double)theta);
  return finish(g4a::launch_fill_cache(a, static_cast<hipStream_t>(stream)));
}

namespace {

size_t decode_fp8_ws_bytes(int B, int q_len, int Hq, int Hkv, int d, int capacity, int window) {
  if (B < 0 || q_len < 1 || q_len > 8 || Hq <= 0 || Hkv <= 0 || d <= 0 || capacity <= 0 ||
      window < 0)
    return 0;
  if (!ring_ok(capacity, window, q_len, true)) return 0;
  const size_t nch = (size_t)g4a::decode_fp8_num_chunks(capacity, window);
  const size_t bytes = (size_t)B * q_len * Hq * nch * ((size_t)d + 2) * sizeof(float);
  return bytes > 0 ? bytes : 16;
}

}  // namespace

G4A_API size_t g4attn_decode_fp8_workspace_bytes(int B, int q_len, int Hq, int Hkv, int d,
                                                 int capacity, int window) {
  return decode_fp8_ws_bytes(B, q_len, Hq, Hkv, d, capacity, window);
}

G4A_API int g4attn_decode_fp8(const void* q, const void* k_cache, const void* v_cache,
                              const float* k_scale, const float* v_scale, void* out,
                              const int32_t* pos, int B, int q_len, int Hq, int Hkv, int d,
                              int capacity, int window, float theta, float p, int out_dtype,
                              void* workspace, size_t workspace_bytes, void* stream) {
  if (B < 0 || capacity <= 0 || q_len < 1 || q_len > 8) return G4A_EINVAL;
  if (!ring_ok(capacity, window, q_len, true)) return G4A_EINVAL;
  int rc = check_common(Hq, Hkv, d, window, theta, p, G4A_BF16, out_dtype);
  if (rc) return rc;
  if (B == 0) return G4A_OK;
  const bool kv_shared = v_cache == nullptr || v_cache == k_cache;
  if (!q || !k_cache || !out || !pos || !k_scale || (!kv_shared && !v_scale)) return G4A_EINVAL;
  if (misaligned(q) || misaligned(k_cache) || (v_cache && misaligned(v_cache)) ||
      misaligned(out) || misaligned(pos) || misaligned(k_scale) ||
      (!kv_shared && misaligned(v_scale)))
    return G4A_EALIGN;
  if ((double)B * Hkv * capacity * d > 9.0e18) return G4A_EINVAL;
  g4a::DecodeArgs a = decode_args(q, k_cache, kv_shared ? nullptr : v_cache, out, pos, B, q_len,
                                  Hq, Hkv, d, capacity, window, theta, p);
  a.chunk = g4a::decode_fp8_chunk_rows(capacity, window);
  a.nchunk = g4a::decode_fp8_num_chunks(capacity, window);
  a.k_scale = k_scale;
  a.v_scale = kv_shared ? k_scale : v_scale;
  const size_t need = decode_fp8_ws_bytes(B, q_len, Hq, Hkv, d, capacity, window);
  if (!workspace || workspace_bytes < need) return G4A_EWORKSPACE;
  if (misaligned(workspace)) return G4A_EALIGN;
  if ((double)B * Hkv * a.ncb * a.nchunk > 2.0e9) return G4A_EINVAL;
  a.part_o = static_cast<float*>(workspace);
  a.part_ml = a.part_o + (size_t)B * q_len * Hq * a.nchunk * d;
  return finish(g4a::launch_decode_fp8(a, kv_shared, out_dtype == G4A_BF16,
                                       static_cast<hipStream_t>(stream)));
}

G4A_API int g4attn_fill_cache_fp8(const void* k, const void* v, const float* k_scale,
                                  const float* v_scale, const int32_t* pos, int B, int S, int Hkv,
                                  int d, void* k_cache, void* v_cache, int capacity, int window,
                                  float theta, float p, int in_dtype, void* stream) {
  if (B < 0 || S < 0 || Hkv <= 0 || d <= 0 || capacity <= 0 || window < 0) return G4A_EINVAL;
  if (in_dtype != G4A_F32 && in_dtype != G4A_BF16) return G4A_EUNSUPPORTED;
  if (d % 16) return G4A_EUNSUPPORTED;
  if (int rc = fill_turn_check(v, d, theta, p)) return rc;
  if (B == 0 || S == 0) return G4A_OK;
  if (!k || !pos || !k_cache || !k_scale || (v && (!v_cache || !v_scale))) return G4A_EINVAL;
  if (misaligned(k) || (v && misaligned(v)) || misaligned(pos) || misaligned(k_cache) ||
      misaligned(k_scale) || (v && (misaligned(v_cache) || misaligned(v_scale))))
    return G4A_EALIGN;
  g4a::FillArgs a;
  if (!fill_args(a, k, v, pos, B, S, Hkv, k_cache, v_cache, capacity, window, d / 16))
    return G4A_EINVAL;
  a.in_f32 = in_dtype == G4A_F32;
  a.d = d;
  a.n_rot = rotated_pairs(d, p);
  a.log2_theta = log2((double)theta);
  a.k_scale = k_scale;
  a.v_scale = v ? v_scale : nullptr;
  return finish(g4a::launch_fill_cache_fp8(a, static_cast<hipStream_t>(stream)));
}

G4A_API const char* g4attn_strerror(int status) {
  switch (status) {
    case G4A_OK: return "ok";
    case G4A_EINVAL: return "invalid argument";
    case G4A_EUNSUPPORTED: return "unsupported head dim, group size or dtype pair";
    case G4A_EALIGN: return "tensor pointer not 16-byte aligned";
    case G4A_EWORKSPACE: return "workspace missing or too small";
    case G4A_EHIP: return "HIP launch failed (see g4attn_last_hip_error)";
    case G4A_ESCRATCH:
      return "decode partials exceed the library's fixed 64 MiB scratch; use g4attn_decode "
             "with a workspace";
  }
  return "unknown status";
}

G4A_API int g4attn_last_hip_error(void) { return g_last_hip_error; }
