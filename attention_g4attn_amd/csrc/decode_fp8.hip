// Decode attention over a low-precision KV cache: one byte per cached element
// in the OCP FP8 E4M3 format, the cached value being code value x scale of its
// KV head, on the gfx950 matrix cores.
//
// What is computed is decode (or decode of q_len query tokens) over the
// dequantized cache: the pages list optimized KV caches among the memory
// savings of the mobile checkpoints and note that the cache dominates memory
// at long context ("Visao geral do modelo Gemma 4", sections "Treinamento com
// reconhecimento de quantizacao (QAT)" and "Principais Consideracoes para o
// planejamento de memoria"); the format is not given there, E4M3 with a scale
// per KV head is the reading taken.  The attention itself is the one of the
// bf16 decode: "Guia visual do Gemma 4", sections "GQA", "Tecnica K=V",
// "p-RoPE" and "Intercalacao de camadas de atencao".
//
// Every E4M3 value is exact in bf16, so the codes are widened to bf16 in
// registers (one conversion instruction per two codes) and multiplied on the
// bf16 matrix cores exactly as the bf16 cache would be; the scales leave the
// sums: score = scale_k * <q~, code_k~>, out = scale_v * sum p code_v / l.  A
// cache with separate values holds the codes of keys already turned at their
// positions (the quantizing fill turns each key once, before quantizing); a
// K=V cache holds the codes of the raw tensor, whose keys are turned here:
// the turn is linear, so turning the code is turning the value.
//
// Separate K and V caches (decode_fp8_kernel): one 4-wave workgroup per
// (column block, b, kv head, chunk of cache rows), each wave streaming 32-row
// tiles (a 16 KB tile at d = 512, the bytes of a 16-row bf16 tile) of K and V
// straight into its own LDS slots with 16-byte direct loads, tiles claimed
// from a workgroup counter.  Per tile the wave
//   - forms S^T = K~ Q~^T in two 16-key halves with the 16x16x32 product: key
//     row operands are 16-byte LDS reads (16 codes = two k-steps of 8 dims)
//     of turned keys, widened in registers; the head dims are taken in the
//     order that makes those 16 codes contiguous (the query operand uses the
//     same order);
//   - updates the softmax of its columns over the 32 keys; lane (g, column)
//     ends up with keys 8g .. 8g+7, i.e. P^T as the B operand of a 32-key
//     product;
//   - forms O^T += V^T P^T with the 16x16x32 product, the value operand read
//     by 8-bit LDS transpose reads (8 consecutive rows of one dim per lane)
//     and widened.
// K=V caches take the kernel further down (decode_fp8_kv_kernel).  The merge
// of chunks is the bf16 decode's.
#include "common.hpp"
#include "decode_common.hpp"
#include "kernels.hpp"

namespace g4a {

namespace {

using namespace dec;

constexpr int TR8 = 32;  // cache rows per tile
constexpr int NW8 = 4;   // waves per workgroup

typedef int i32x2 __attribute__((ext_vector_type(2)));

// 16-byte chunk swizzle of tile row r (chunk c stored at slot c ^ fswz(r)).
// With r = 8a + 4h + j (j < 4): fswz = j + 4 * ((a + 2h) mod 4).  A score read
// (16 lanes: rows 8a + 4h + j for all a, j at one h) and a transpose read (32
// lanes: rows 8a + 4h + j for two consecutive a, all h, j) each hit 16
// distinct slots of a 256-byte bank window.
__device__ __forceinline__ int fswz(int r) {
  return (r & 3) | ((((r >> 3) + 2 * ((r >> 2) & 1)) & 3) << 2);
}

// 8 E4M3 codes (bytes of w0 then w1) -> 8 bf16 in the same order, exact
__device__ __forceinline__ u32x4 widen8(uint32_t w0, uint32_t w1) {
  u32x4 r;
  r[0] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w0, 1.0f, false));
  r[1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w0, 1.0f, true));
  r[2] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w1, 1.0f, false));
  r[3] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w1, 1.0f, true));
  return r;
}

// 8-bit transpose read: within each 16-lane group, the lanes' 8-byte segments
// form an 8 x 16 byte matrix (lane n holds row n/2, bytes 8*(n%2) .. +7), and
// lane n receives column n (byte k from row k).
__device__ __forceinline__ u32x2 lds_read_tr8(const unsigned char* p) {
  const i32x2 v = __builtin_amdgcn_ds_read_tr8_b64_v2i32((__attribute__((address_space(3))) i32x2*)(p));
  return __builtin_bit_cast(u32x2, v);
}

// 8-dim chunk of the head taken by lane group gq at k-step s: k-steps 2u and
// 2u + 1 share the 16 dims 64u + 16gq .. +15, low half first
__device__ __forceinline__ int kchunk(int s, int gq) { return 8 * (s >> 1) + 2 * gq + (s & 1); }

// RK = query k-steps that may hold turning pairs (4 when n_rot <= 64).
template <int D, int G, int RK, bool OBF>
__global__ void __launch_bounds__(64 * NW8) __attribute__((amdgpu_waves_per_eu(2, 2)))
decode_fp8_kernel(DecodeArgs a) {
  constexpr int NW = NW8;
  constexpr int NS = D / 32;       // 32-dim k-steps of the score product
  constexpr int NB = D / 16;       // 16-dim blocks of the output
  constexpr int KB = TR8 * D;      // one tensor's tile, bytes
  constexpr int NLD = KB / 1024;   // direct loads per lane per tensor tile
  static_assert(G <= 8 && RK <= NS && RK % 2 == 0 && NS % 2 == 0, "shape");
  static_assert(KB >= 8 * D * 4, "a wave's tile slot holds 8 columns of D floats for the merge");
  __shared__ __attribute__((aligned(16))) unsigned char tk[NW * KB];            // K (or K=V) tiles
  __shared__ __attribute__((aligned(16))) unsigned char tv[NW * KB];            // V tiles
  __shared__ double gtab[D / 2];
  __shared__ float mls[NW][16][2];
  __shared__ int tnext;  // next unclaimed tile of the chunk

  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int l16 = lane & 15, g4 = lane >> 4;
  const Unit u = unit_of_block(a);  // XCD-aware grid order
  if (u.b < 0) return;
  const int cb = u.cb, ch = u.ch, b = u.b, hkv = u.hkv;
  const int P = a.pos[b];
  const int W = a.window, C = a.capacity, QL = a.q_len;
  // Column n of the block is (token, head) pair c = 16*cb + n: query token
  // c / G at position P - QL + 1 + c / G, query head hkv*G + c % G.
  const int ncol = min(16, G * QL - 16 * cb);
  auto col_out = [&](int n) -> size_t {
    const int c = 16 * cb + n;
    return (((size_t)b * QL + c / G) * a.Hq + hkv * G + c % G) * D;
  };
  auto col_pos = [&](int n) { return P - QL + 1 + (16 * cb + n) / G; };
  const bool col_ok = l16 < ncol;
  const int Pq = col_pos(col_ok ? l16 : 0);
  const bool direct = a.nchunk == 1;  // this workgroup writes the output
  if (P < 0 || (W == 0 && P >= C)) {
    if (direct) nan_columns<D, NW, OBF>(a, ncol, col_out);
    return;
  }
  const int last = W > 0 ? min(P, C - 1) : P;  // highest row index that may be visible
  const int r0 = ch * a.chunk;
  if (r0 > last) return;
  const int r1 = min(r0 + a.chunk, last + 1);  // exclusive
  const int nt = (r1 - r0 + TR8 - 1) / TR8;
  const int n_rot = a.n_rot;
  unsigned char* kt = tk + w * KB;
  unsigned char* vt = tv + w * KB;

  // query heads as B operands of the score product, dims in kchunk order
  u32x4 qf[NS];
  {
    const uint16_t* qrow = static_cast<const uint16_t*>(a.q) + col_out(col_ok ? l16 : 0);
#pragma unroll
    for (int s = 0; s < NS; ++s) qf[s] = *reinterpret_cast<const u32x4*>(qrow + 8 * kchunk(s, g4));
  }
  const float cs = a.scale_log2e * a.k_scale[hkv];            // score scale, base 2
  const float vsc = a.v_scale[hkv];                           // value scale

  const size_t hoff = ((size_t)b * a.Hkv + hkv) * C * D;
  const uint8_t* kbase = static_cast<const uint8_t*>(a.k) + hoff;
  const uint8_t* vbase = static_cast<const uint8_t*>(a.v) + hoff;

  const bool stream_loads = a.ncb == 1;  // cache rows read once: non-temporal
  // 32 rows of tile i of one tensor into an LDS tile; rows past r1 read as zeros
  auto issue = [&](const uint8_t* base, int i, unsigned char* dst) {
    const int rr0 = r0 + i * TR8;
    const uint32_t bytes = (uint32_t)min(TR8, r1 - rr0) * D;
    const __amdgpu_buffer_rsrc_t rs = make_rsrc(base + (size_t)rr0 * D, bytes);
    constexpr int CPR = D / 16;   // chunks per row
    constexpr int RPI = 64 / CPR; // rows per direct load
    int ln = lane;
    asm volatile("" : "+v"(ln));
#pragma unroll
    for (int n = 0; n < NLD; ++n) {
      const int row = n * RPI + ln / CPR;
      const uint32_t voff = (uint32_t)row * D + ((uint32_t)((ln % CPR) ^ fswz(row)) << 4);
      lds_dma16(rs, voff, dst + n * 1024, stream_loads);
    }
  };

  for (int t = threadIdx.x; t < D / 2; t += 64 * NW) gtab[t] = rope_rev_per_pos(t, D, a.log2_theta);
  if (threadIdx.x == 0) tnext = NW;
  __syncthreads();
  auto claim = [&]() -> int {
    int t = 0;
    if (lane == 0) t = atomicAdd(&tnext, 1);
    return __builtin_amdgcn_readfirstlane(t);
  };
  const int tA = w;
  if (tA < nt) {
    issue(kbase, tA, kt);
    issue(vbase, tA, vt);
  }
#pragma unroll
  for (int s = 0; s < NS; ++s) {
    qf[s] = col_ok ? qf[s] : u32x4{0, 0, 0, 0};
    if (s < RK) qf[s] = rotate_chunk_bf16(qf[s], kchunk(s, g4), Pq, n_rot, gtab);
  }

  f32x4 oacc[NB];
#pragma unroll
  for (int i = 0; i < NB; ++i) oacc[i] = f32x4{};
  float m_run = -INFINITY, l_run = 0.f;  // per column, base 2

  // scores of tile i: half h holds keys 8*gq + 4h + j in register j of lane
  // (gq, column); the two halves are two independent accumulation chains
  auto scores = [&](f32x4& s0, f32x4& s1) {
    int ln = lane;
    asm volatile("" : "+v"(ln));
    const int row = ln & 15, gq = ln >> 4;
    int base[2], sw[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int kr = 8 * (row >> 2) + 4 * h + (row & 3);  // tile row of operand row `row`
      base[h] = kr * D;
      sw[h] = fswz(kr);
    }
    f32x4 acc[2] = {};
#pragma unroll
    for (int u2 = 0; u2 < NS / 2; ++u2) {
      u32x4 raw[2];
#pragma unroll
      for (int h = 0; h < 2; ++h) raw[h] = lds_at<u32x4>(kt, base[h] + (((4 * u2 + gq) ^ sw[h]) << 4));
#pragma unroll
      for (int e = 0; e < 2; ++e) {  // k-step 2*u2 + e: codes 8e .. 8e+7 of the read
        const u32x4 k0 = widen8(raw[0][2 * e], raw[0][2 * e + 1]);
        const u32x4 k1 = widen8(raw[1][2 * e], raw[1][2 * e + 1]);
        acc[0] = mfma16x16x32(k0, qf[2 * u2 + e], acc[0]);
        acc[1] = mfma16x16x32(k1, qf[2 * u2 + e], acc[1]);
      }
    }
    s0 = acc[0];
    s1 = acc[1];
  };
  // softmax update over the tile's 32 keys; returns P^T (keys 8*g4 .. +7 of
  // column l16) as the B operand of the value product
  auto softmax = [&](int i, f32x4 s0, f32x4 s1) -> u32x4 {
    const int nrows = min(TR8, r1 - (r0 + i * TR8));
    float sv[8];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      sv[j] = s0[j];
      sv[4 + j] = s1[j];
    }
#pragma unroll
    for (int k = 0; k < 8; ++k) sv[k] = 8 * g4 + k < nrows ? sv[k] : -INFINITY;
    // wave-uniform: each column sees keys up to its own position, and a ring
    // larger than the window holds keys before every column's window
    if (QL > 1 || (W > 0 && C > W)) {
      const int rk = r0 + i * TR8 + 8 * g4;     // this lane's first key row
      const int m0 = W > 0 ? (P - rk) % C : 0;  // (P - row) mod C of that row
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        const int mj = m0 - k;
        const int tp = W > 0 ? P - (mj >= 0 ? mj : mj + C) : rk + k;  // key position
        const bool vis = tp <= Pq && (W == 0 || tp > Pq - W);
        sv[k] = vis ? sv[k] : -INFINITY;
      }
    }
    float mx = sv[0];
#pragma unroll
    for (int k = 1; k < 8; ++k) mx = fmaxf(mx, sv[k]);
    mx = fmaxf(mx, __shfl_xor(mx, 16));
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    const float mt = mx * cs;
    if (__any(mt > m_run + 8.f)) {  // wave-uniform; rare after the first tile
      const float mn = fmaxf(m_run, mt);
      const float al = m_run == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m_run - mn);
#pragma unroll
      for (int db = 0; db < NB; ++db) oacc[db] *= al;
      l_run *= al;
      m_run = mn;
    }
    const float mr = m_run == -INFINITY ? 0.f : m_run;  // no key seen: every p is 0
    float p[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      p[k] = __builtin_amdgcn_exp2f(__builtin_fmaf(sv[k], cs, -mr));
      l_run += p[k];
    }
    return u32x4{pack_bf16(p[0], p[1]), pack_bf16(p[2], p[3]), pack_bf16(p[4], p[5]),
                 pack_bf16(p[6], p[7])};
  };
  // O^T += V^T P^T: source lane (gq, n) addresses tile row 8*gq + n/2, bytes
  // 8*(n%2) .. +7 of chunk db; it receives dim 16*db + n of rows 8*gq .. +7
  auto values = [&](const unsigned char* vtile, u32x4 pf) {
    int ln = lane;
    asm volatile("" : "+v"(ln));
    const int n = ln & 15, gq = ln >> 4;
    const int kk = 8 * gq + (n >> 1);
    const int base = kk * D + (n & 1) * 8;
    const int sw = fswz(kk);
#pragma unroll
    for (int db = 0; db < NB; ++db) {
      const u32x2 raw = lds_read_tr8(vtile + base + ((db ^ sw) << 4));
      oacc[db] = mfma16x16x32(widen8(raw[0], raw[1]), pf, oacc[db]);
    }
  };

  // the next keys are requested once the scores have read the key slot, the
  // next values once the value product has read theirs
  for (int t = tA; t < nt;) {
    const int tn = claim();
    wait_vmcnt<NLD>();  // keys of t (its values may still be in flight)
    f32x4 s0, s1;
    scores(s0, s1);
    if (tn < nt) issue(kbase, tn, kt);
    const u32x4 pf = softmax(t, s0, s1);
    if (tn < nt) wait_vmcnt<NLD>();  // values of t (the next keys may be in flight)
    else wait_vmcnt<0>();
    values(vt, pf);
    if (tn < nt) issue(vbase, tn, vt);
    t = tn;
  }

#pragma unroll
  for (int db = 0; db < NB; ++db) oacc[db] *= vsc;
  l_run += __shfl_xor(l_run, 16);
  l_run += __shfl_xor(l_run, 32);
  finish_chunk<D, NW, OBF>(a, oacc, m_run, l_run, ch, ncol, direct,
                           reinterpret_cast<float*>(tk), mls, col_out, col_pos);
}

// ---- K=V caches: 16-row tiles, two LDS slots per wave ----
//
// The kernel above keeps one 16 KB slot per wave, so a wave's loads and its
// compute alternate: load, wait, compute, load.  With fp8 the compute of a
// tile (widening, key rotation, softmax) is as long as the load's latency,
// and the wave's slot sits idle for one or the other.  Here a wave holds two
// 8 KB slots of 16 rows and requests its next tile before computing the
// current one, so every wave keeps a load in flight while it computes, at
// the same 16 KB of LDS per wave (8 waves per CU).
//
// Per 16-row tile the wave
//   - forms S^T = K~ Q~^T with the 16x16x32 product, one key row per lane
//     and 16 codes per 16-byte LDS read (two k-steps, the dims in the kchunk
//     order of the query operand), rotating the turning pairs of its row;
//   - updates the softmax of its columns over the 16 keys; lane (g, column)
//     holds keys 4g .. 4g+3, the B operand of a 16-key value product;
//   - forms O^T += V^T P^T with the 16x16x16 product, V^T from 8-bit
//     transpose reads whose eight source rows are keys 4g .. 4g+3 twice (the
//     first four bytes are used).
// Loads are issued from inline assembly (lds_dma16_nt_asm): with the builtin,
// the compiler would wait for the next tile before reading the current one.

constexpr int TRK = 16;  // cache rows per tile of the K=V kernel

// chunk c of row r of a 16-row tile sits at c ^ r: a score read (16 rows,
// one chunk) and a transpose read (4 rows) hit distinct 16-byte slots
__device__ __forceinline__ int kswz(int r) { return r & 15; }

// 8 codes (bytes of w0 then w1) of dims 8c .. 8c+7 of one key: widened to
// fp32 (exact), pairs t < n_rot (ALL: all four) turned at position pos,
// packed to bf16 (round to nearest even)
template <bool ALL>
__device__ __forceinline__ u32x4 widen_rotate8(uint32_t w0, uint32_t w1, int c, int pos,
                                               int n_rot, const double* gtab) {
  const f32x2 x[4] = {__builtin_amdgcn_cvt_pk_f32_fp8(w0, false),
                      __builtin_amdgcn_cvt_pk_f32_fp8(w0, true),
                      __builtin_amdgcn_cvt_pk_f32_fp8(w1, false),
                      __builtin_amdgcn_cvt_pk_f32_fp8(w1, true)};
  u32x4 y;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int t = 4 * c + i;
    float cs, sn;
    rope_cs_fast(pos, gtab[t], cs, sn);
    const uint32_t r = pack_bf16(x[i][0] * cs - x[i][1] * sn, x[i][0] * sn + x[i][1] * cs);
    y[i] = (ALL || t < n_rot) ? r : pack_bf16(x[i][0], x[i][1]);
  }
  return y;
}

typedef short s16x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ f32x4 mfma16x16x16(u32x2 a, u32x2 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(s16x4, a),
                                                   __builtin_bit_cast(s16x4, b), c, 0, 0, 0);
}

template <int D, int G, int RK, bool ALL, bool OBF>
__global__ void __launch_bounds__(64 * NW8) __attribute__((amdgpu_waves_per_eu(2, 2)))
decode_fp8_kv_kernel(DecodeArgs a) {
  constexpr int NW = NW8;
  constexpr int NS = D / 32;       // 32-dim k-steps of the score product
  constexpr int NB = D / 16;       // 16-dim blocks of the output
  constexpr int KB = TRK * D;      // one tile, bytes
  constexpr int NLD = KB / 1024;   // direct loads per tile
  static_assert(G <= 8 && RK <= NS && RK % 2 == 0 && NS % 2 == 0, "shape");
  static_assert(2 * KB >= 8 * D * 4, "a wave's two slots hold 8 columns of D floats for the merge");
  __shared__ __attribute__((aligned(16))) unsigned char tk[NW * 2 * KB];  // two slots per wave
  __shared__ double gtab[RK * 16];  // pairs of the k-steps that may turn
  __shared__ float mls[NW][16][2];
  __shared__ int tnext;  // next unclaimed tile of the chunk

  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int l16 = lane & 15, g4 = lane >> 4;
  const Unit u = unit_of_block(a);  // XCD-aware grid order
  if (u.b < 0) return;
  const int cb = u.cb, ch = u.ch, b = u.b, hkv = u.hkv;
  const int P = a.pos[b];
  const int W = a.window, C = a.capacity, QL = a.q_len;
  // Column n of the block is (token, head) pair c = 16*cb + n: query token
  // c / G at position P - QL + 1 + c / G, query head hkv*G + c % G.
  const int ncol = min(16, G * QL - 16 * cb);
  auto col_out = [&](int n) -> size_t {
    const int c = 16 * cb + n;
    return (((size_t)b * QL + c / G) * a.Hq + hkv * G + c % G) * D;
  };
  auto col_pos = [&](int n) { return P - QL + 1 + (16 * cb + n) / G; };
  const bool col_ok = l16 < ncol;
  const int Pq = col_pos(col_ok ? l16 : 0);
  const bool direct = a.nchunk == 1;  // this workgroup writes the output
  if (P < 0 || (W == 0 && P >= C)) {
    if (direct) nan_columns<D, NW, OBF>(a, ncol, col_out);
    return;
  }
  const int last = W > 0 ? min(P, C - 1) : P;  // highest row index that may be visible
  const int r0 = ch * a.chunk;
  if (r0 > last) return;
  const int r1 = min(r0 + a.chunk, last + 1);  // exclusive
  const int nt = (r1 - r0 + TRK - 1) / TRK;
  const int n_rot = a.n_rot;
  unsigned char* const slot0 = tk + w * 2 * KB;

  // query heads as B operands of the score product, dims in kchunk order
  u32x4 qf[NS];
  {
    const uint16_t* qrow = static_cast<const uint16_t*>(a.q) + col_out(col_ok ? l16 : 0);
#pragma unroll
    for (int s = 0; s < NS; ++s) qf[s] = *reinterpret_cast<const u32x4*>(qrow + 8 * kchunk(s, g4));
  }
  const float cs = a.scale_log2e * a.k_scale[hkv];  // score scale, base 2
  const float vsc = a.k_scale[hkv];                 // value scale (K=V)
  const uint8_t* kbase = static_cast<const uint8_t*>(a.k) + ((size_t)b * a.Hkv + hkv) * C * D;

  // the 16 rows of tile i into a slot (rows past r1 read as zeros); every
  // cache row is read once by the launch: non-temporal
  auto issue = [&](int i, unsigned char* dst) {
    const int rr0 = r0 + i * TRK;
    const uint32_t bytes = (uint32_t)min(TRK, r1 - rr0) * D;
    const s32x4 rs = rsrc_words(kbase + (size_t)rr0 * D, bytes);
    constexpr int CPR = D / 16;    // chunks per row
    constexpr int RPI = 64 / CPR;  // rows per direct load
    int ln = lane;
    asm volatile("" : "+v"(ln));
#pragma unroll
    for (int n = 0; n < NLD; ++n) {
      const int row = n * RPI + ln / CPR;
      const uint32_t voff = (uint32_t)row * D + ((uint32_t)((ln % CPR) ^ kswz(row)) << 4);
      lds_dma16_nt_asm(rs, voff, dst + n * 1024);
    }
  };

  for (int t = threadIdx.x; t < RK * 16; t += 64 * NW) gtab[t] = rope_rev_per_pos(t, D, a.log2_theta);
  if (threadIdx.x == 0) tnext = NW;
  __syncthreads();
  auto claim = [&]() -> int {
    int t = 0;
    if (lane == 0) t = atomicAdd(&tnext, 1);
    return __builtin_amdgcn_readfirstlane(t);
  };
  const int tA = w;
  if (tA < nt) issue(tA, slot0);
#pragma unroll
  for (int s = 0; s < NS; ++s) {
    qf[s] = col_ok ? qf[s] : u32x4{0, 0, 0, 0};
    if (s < RK) qf[s] = rotate_chunk_bf16(qf[s], kchunk(s, g4), Pq, n_rot, gtab);
  }

  f32x4 oacc[NB];
#pragma unroll
  for (int i = 0; i < NB; ++i) oacc[i] = f32x4{};
  float m_run = -INFINITY, l_run = 0.f;  // per column, base 2

  // S^T of tile i (register j = key 4*gq + j of column l16), the softmax
  // update, and O^T += V^T P^T, from the tile in LDS at kt
  auto compute = [&](int i, const unsigned char* kt) {
    int ln = lane;
    asm volatile("" : "+v"(ln));
    const int row = ln & 15, gq = ln >> 4;
    f32x4 sacc;
    {
      const int r = min(r0 + i * TRK + row, r1 - 1);  // rows past the end are masked
      const int tpos = W > 0 ? P - (P - r) % C : r;
      const int base = row * D, sw = kswz(row);
      f32x4 s0 = {}, s1 = {};  // even / odd k-steps: two independent chains
#pragma unroll
      for (int u2 = 0; u2 < NS / 2; ++u2) {
        const u32x4 raw = lds_at<u32x4>(const_cast<unsigned char*>(kt), base + (((4 * u2 + gq) ^ sw) << 4));
        // k-step 2*u2 + e: codes 8e .. 8e+7 of the read
        const u32x4 k0 = 2 * u2 < RK ? widen_rotate8<ALL>(raw[0], raw[1], kchunk(2 * u2, gq), tpos,
                                                          n_rot, gtab)
                                     : widen8(raw[0], raw[1]);
        const u32x4 k1 = 2 * u2 + 1 < RK ? widen_rotate8<ALL>(raw[2], raw[3], kchunk(2 * u2 + 1, gq),
                                                              tpos, n_rot, gtab)
                                         : widen8(raw[2], raw[3]);
        s0 = mfma16x16x32(k0, qf[2 * u2], s0);
        s1 = mfma16x16x32(k1, qf[2 * u2 + 1], s1);
      }
      sacc = s0 + s1;
    }
    u32x2 pf;
    {
      const int nrows = min(TRK, r1 - (r0 + i * TRK));
#pragma unroll
      for (int j = 0; j < 4; ++j) sacc[j] = 4 * gq + j < nrows ? sacc[j] : -INFINITY;
      // wave-uniform: each column sees keys up to its own position, and a ring
      // larger than the window holds keys before every column's window
      if (QL > 1 || (W > 0 && C > W)) {
        const int rk = r0 + i * TRK + 4 * gq;     // this lane's first key row
        const int m0 = W > 0 ? (P - rk) % C : 0;  // (P - row) mod C of that row
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int mj = m0 - j;
          const int tp = W > 0 ? P - (mj >= 0 ? mj : mj + C) : rk + j;  // key position
          const bool vis = tp <= Pq && (W == 0 || tp > Pq - W);
          sacc[j] = vis ? sacc[j] : -INFINITY;
        }
      }
      float mx = fmaxf(fmaxf(sacc[0], sacc[1]), fmaxf(sacc[2], sacc[3]));
      mx = fmaxf(mx, __shfl_xor(mx, 16));
      mx = fmaxf(mx, __shfl_xor(mx, 32));
      const float mt = mx * cs;
      if (__any(mt > m_run + 8.f)) {  // wave-uniform; rare after the first tile
        const float mn = fmaxf(m_run, mt);
        // a column that has seen no key yet holds zeros (scaled by 0, not NaN)
        const float al = m_run == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m_run - mn);
#pragma unroll
        for (int db = 0; db < NB; ++db) oacc[db] *= al;
        l_run *= al;
        m_run = mn;
      }
      const float mr = m_run == -INFINITY ? 0.f : m_run;  // no key seen: every p is 0
      float p[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        p[j] = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[j], cs, -mr));
        l_run += p[j];
      }
      pf = u32x2{pack_bf16(p[0], p[1]), pack_bf16(p[2], p[3])};
    }
    {
      // source lane (gq, n) addresses key row 4*gq + (n/2) % 4, bytes
      // 8*(n%2) .. +7 of chunk db; it receives dim 16*db + n of those rows
      const int kr = 4 * gq + ((row >> 1) & 3);
      const unsigned char* vb = kt + kr * D + (row & 1) * 8;
      const int vsw = kswz(kr);
#pragma unroll
      for (int db = 0; db < NB; ++db) {
        const u32x2 raw = lds_read_tr8(vb + ((db ^ vsw) << 4));
        const u32x2 vf = {
            __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(raw[0], 1.0f, false)),
            __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(raw[0], 1.0f, true))};
        oacc[db] = mfma16x16x16(vf, pf, oacc[db]);
      }
    }
  };

  // The wave's tiles are claimed in increasing order; tile k of the wave
  // sits in slot k % 2.  Each step requests the next tile into the other
  // slot (whose tile the previous step finished reading), then waits only
  // for the current tile's loads.
  int t = tA;
  for (int k = 0; t < nt; ++k) {
    const int tn = claim();
    unsigned char* cur = slot0 + (k & 1) * KB;
    unsigned char* nxt = slot0 + ((k + 1) & 1) * KB;
    if (tn < nt) {
      issue(tn, nxt);
      wait_vmcnt<NLD>();
    } else {
      wait_vmcnt<0>();
    }
    compute(t, cur);
    t = tn;
  }

#pragma unroll
  for (int db = 0; db < NB; ++db) oacc[db] *= vsc;
  l_run += __shfl_xor(l_run, 16);
  l_run += __shfl_xor(l_run, 32);
  finish_chunk<D, NW, OBF>(a, oacc, m_run, l_run, ch, ncol, direct,
                           reinterpret_cast<float*>(tk), mls, col_out, col_pos);
}

template <int D, int G, bool OBF>
hipError_t launch_fp8_kv(const DecodeArgs& a, hipStream_t st) {
  const long long n = (long long)a.B * a.Hkv * a.ncb * a.nchunk;
  if (n > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  const dim3 grid((unsigned)n), block(64 * NW8);
  if (a.n_rot == 64)
    hipLaunchKernelGGL((decode_fp8_kv_kernel<D, G, 4, true, OBF>), grid, block, 0, st, a);
  else if (a.n_rot < 64)
    hipLaunchKernelGGL((decode_fp8_kv_kernel<D, G, 4, false, OBF>), grid, block, 0, st, a);
  else if (a.n_rot == D / 2)
    hipLaunchKernelGGL((decode_fp8_kv_kernel<D, G, D / 32, true, OBF>), grid, block, 0, st, a);
  else
    hipLaunchKernelGGL((decode_fp8_kv_kernel<D, G, D / 32, false, OBF>), grid, block, 0, st, a);
  return hipGetLastError();
}

template <int D, int G, bool OBF>
hipError_t launch_fp8(const DecodeArgs& a, hipStream_t st) {
  const long long n = (long long)a.B * a.Hkv * a.ncb * a.nchunk;
  if (n > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  const dim3 grid((unsigned)n), block(64 * NW8);
  if (a.n_rot <= 64)
    hipLaunchKernelGGL((decode_fp8_kernel<D, G, 4, OBF>), grid, block, 0, st, a);
  else
    hipLaunchKernelGGL((decode_fp8_kernel<D, G, D / 32, OBF>), grid, block, 0, st, a);
  return hipGetLastError();
}

template <int D, bool KVS, bool OBF>
hipError_t launch_fp8_g(const DecodeArgs& a, hipStream_t st) {
  if constexpr (KVS) {
    switch (a.Hq / a.Hkv) {
      case 1: return launch_fp8_kv<D, 1, OBF>(a, st);
      case 2: return launch_fp8_kv<D, 2, OBF>(a, st);
      case 4: return launch_fp8_kv<D, 4, OBF>(a, st);
      case 8: return launch_fp8_kv<D, 8, OBF>(a, st);
    }
  } else {
    switch (a.Hq / a.Hkv) {
      case 1: return launch_fp8<D, 1, OBF>(a, st);
      case 2: return launch_fp8<D, 2, OBF>(a, st);
      case 4: return launch_fp8<D, 4, OBF>(a, st);
      case 8: return launch_fp8<D, 8, OBF>(a, st);
    }
  }
  return hipErrorInvalidValue;
}

template <bool OBF>
hipError_t launch_fp8_d(const DecodeArgs& a, bool kv_shared, hipStream_t st) {
  if (a.D == 256) return kv_shared ? launch_fp8_g<256, true, OBF>(a, st) : launch_fp8_g<256, false, OBF>(a, st);
  if (a.D == 512) return kv_shared ? launch_fp8_g<512, true, OBF>(a, st) : launch_fp8_g<512, false, OBF>(a, st);
  return hipErrorInvalidValue;
}

}  // namespace

int decode_fp8_chunk_rows(int capacity, int window) {
  if (window > 0) return (capacity + TR8 - 1) / TR8 * TR8;  // ring: one workgroup per ring
  return 1024;
}

int decode_fp8_num_chunks(int capacity, int window) {
  const int ch = decode_fp8_chunk_rows(capacity, window);
  return (capacity + ch - 1) / ch;
}

hipError_t launch_decode_fp8(const DecodeArgs& a, bool kv_shared, bool out_bf16, hipStream_t st) {
  if ((long long)a.B * a.Hkv == 0) return hipSuccess;
  const hipError_t e = out_bf16 ? launch_fp8_d<true>(a, kv_shared, st)
                                : launch_fp8_d<false>(a, kv_shared, st);
  if (e != hipSuccess) return e;
  if (a.nchunk == 1) return hipSuccess;  // finished in place by the split kernel
  return launch_decode_merge(a, out_bf16, st);
}

}  // namespace g4a
