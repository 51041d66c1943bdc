// Launch entry points of the gfx950 kernels, called by the C ABI layer (api.cpp)
// after it has validated every argument.
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace g4a {

struct PrefillArgs {
  const void* q;
  const void* k;
  const void* v;  // equals k for the K=V layer
  void* out;
  const int32_t* pos;
  void* ws;       // rotated key slab [B, S, Hkv, prefill_slab_dims(D, n_rot)] bf16
  int B, S, Hq, Hkv, D, window, n_rot;
  double log2_theta;
  float scale_log2e;  // log2(e) / sqrt(D)
  float scale;        // 1 / sqrt(D)
  int nq, nheads;     // filled in by the launcher
  // vision attention only: pos is [B, S, 2] (w, h) and lengths [B] the valid
  // patches of each image (null: all S)
  const int32_t* lengths;
};

// Decode of q_len query tokens per sequence: q, out [B, q_len, Hq, D]; pos[b]
// is the position P of the last token, token j sits at P - q_len + 1 + j.  A
// ring (window > 0) keeps position t in slot t mod capacity.
struct DecodeArgs {
  const void* q;
  const void* k;
  const void* v;  // equals k for K=V
  void* out;
  const int32_t* pos;
  int B, Hq, Hkv, D, capacity, window, n_rot;
  int q_len;    // query tokens per sequence (1 = ordinary decode)
  int ncb;      // 16-column blocks over the q_len * G (token, head) columns
  double log2_theta;
  float scale_log2e;
  float scale;
  int chunk;    // cache rows per workgroup
  int nchunk;   // chunks per (b, kv head)
  float* part_o;   // [B, q_len, Hq, nchunk, D]
  float* part_ml;  // [B, q_len, Hq, nchunk, 2]
  // fp8 caches only: value = code value * scale[kv head] (v_scale is k_scale for K=V)
  const float* k_scale;
  const float* v_scale;
};

// Raw key/value rows of a prefill into the decode cache layout.
struct FillArgs {
  const void* k;
  const void* v;   // null for K=V (only k_cache is written)
  const int32_t* pos;
  void* k_cache;
  void* v_cache;
  int B, S, Hkv, capacity, window;
  int row_chunks;  // 16-byte chunks per cache row (d * element size / 16)
  // input dtype (0 f32, 1 bf16), head dim; the fp8 fill's per-KV-head scales
  int in_f32, d;
  const float* k_scale;
  const float* v_scale;
  // caches with separate values hold their keys turned at their positions:
  // pairs t < n_rot, angle pos * theta^(-2t/d)
  int n_rot;
  double log2_theta;
};

// bf16 inputs, matrix-core path; D in {256, 512}, G in {1, 2, 4, 8}.
bool prefill_supported(int D);
// key dims kept in the rotated slab (workspace) for this head dim and n_rot
int prefill_slab_dims(int D, int n_rot);
hipError_t launch_prefill_bf16(const PrefillArgs& a, bool kv_shared, bool out_bf16,
                               hipStream_t st);
// per-family launchers (one translation unit each)
hipError_t launch_prefill_kv512(const PrefillArgs& a, bool out_bf16, hipStream_t st);
hipError_t launch_prefill_d256(const PrefillArgs& a, bool kv_shared, bool out_bf16,
                               hipStream_t st);
hipError_t launch_prefill_sep512(const PrefillArgs& a, bool out_bf16, hipStream_t st);
// vision-encoder attention (2D RoPE, no causal mask): bf16, D = 256, separate K/V
hipError_t launch_vision_prefill(const PrefillArgs& a, bool out_bf16, hipStream_t st);
// f32 inputs, fp32 vector path; D in {64, 128, 256, 512}, G in {1, 2, 4, 8}
hipError_t launch_prefill_f32(const PrefillArgs& a, hipStream_t st);

// split + merge decode
hipError_t launch_decode_bf16(const DecodeArgs& a, bool kv_shared, bool out_bf16,
                              hipStream_t st);
hipError_t launch_decode_f32(const DecodeArgs& a, hipStream_t st);
// K=V decode of more than 16 (query token, head) columns per KV head: one
// workgroup per chunk reads each cache tile once, one wave per 16-column block
hipError_t launch_decode_mc(const DecodeArgs& a, bool out_bf16, hipStream_t st);
// merge of the split partials (the chunks of every (token, query head))
hipError_t launch_decode_merge(const DecodeArgs& a, bool out_bf16, hipStream_t st);
// bf16 query over fp8 E4M3 caches; D in {256, 512}, G in {1, 2, 4, 8} (K=V
// caches take a kernel of their own, with two 16-row tile slots per wave)
hipError_t launch_decode_fp8(const DecodeArgs& a, bool kv_shared, bool out_bf16, hipStream_t st);
hipError_t launch_fill_cache(const FillArgs& a, hipStream_t st);
hipError_t launch_fill_cache_fp8(const FillArgs& a, hipStream_t st);

// Fixed per-device scratch of the decode that allocates nothing (64 MiB):
// decode_scratch returns its device address on the current device, looked up
// once per device.
constexpr size_t kDecodeScratchBytes = size_t(64) << 20;
hipError_t decode_scratch(void** ptr);

// rows of the cache one decode workgroup covers, and chunks per (b, kv head)
int decode_chunk_rows(int D, int capacity, int window, bool f32);
int decode_num_chunks(int D, int capacity, int window, bool f32);
int decode_fp8_chunk_rows(int capacity, int window);
int decode_fp8_num_chunks(int capacity, int window);

}  // namespace g4a
