// Decode attention (one query token per sequence) over a bf16 KV cache,
// split along the cache length, on the gfx950 matrix cores.
//
// What is computed: the last row of causal attention over the tokens the
// cache holds, with each cached key turned at its own position.  A cache with
// separate values holds its keys already turned (the fill turns each key
// once), so only the query turns here; with K=V the one tensor stays raw to
// serve as values, and its keys are turned per tile in registers.
// Local layers use a ring cache of `window` slots (position t in slot
// t mod window); global layers a linear K=V cache.  Sources: "Guia visual do
// Gemma 4" (pt.news.hada.io), sections "Intercalacao de camadas de atencao",
// "GQA", "Tecnica K=V", "p-RoPE"; "Visao geral do modelo Gemma 4"
// (ai.google.dev), section "Principais Consideracoes para o planejamento de
// memoria" (the KV cache grows with every token).
//
// Split kernel: one single-wave workgroup per (b, kv head, chunk of `chunk`
// cache rows).  The rows of one (b, kv head) are contiguous; the wave walks
// its chunk in 16-row tiles, each loaded straight into LDS with 16-byte
// direct loads.  A wave keeps one tile slot and the CU runs 8 such waves (2
// per SIMD, 18 KB of LDS each), so while one wave computes, the others' tile
// loads are in flight and the SIMD has a second wave to issue from (measured
// faster than 1 wave per SIMD with a 2- or 3-slot private ring).  Per tile
// the wave
//   - reads the key rows as A operands of the 16x16x32 product (16 rows x 8
//     dims per lane), turns them at their positions in registers (K=V), and
//     forms S^T = K~ Q~^T for the G query heads (padded to 16 columns);
//   - updates the softmax per column (the output is rescaled only when a
//     column's max grows by more than 2^8) and packs P^T straight from the
//     score registers as the B operand of the 16x16x16 product;
//   - forms O^T += V^T P^T with the value operand read by LDS transpose reads
//     (4 consecutive rows of one dim per lane).
// It writes (m, l, O) of its chunk to the workspace; the merge kernel combines
// the chunks of every query head with log-sum-exp weights.  Rows the query may
// not see are never loaded (the load extent stops at the last visible row).
#include "common.hpp"
#include "decode_common.hpp"
#include "kernels.hpp"

namespace g4a {

namespace {

using namespace dec;

constexpr int TR = 16;  // cache rows per tile

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

// D(16x16, fp32) += A(16x16) * B(16x16), bf16 operands.  Lane l holds
// A[l % 16][4*(l/16) .. +3], B[4*(l/16) .. +3][l % 16] and D[4*(l/16) + r][l % 16].
__device__ __forceinline__ f32x4 mfma16x16x16(u32x2 a, u32x2 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(s16x4, a),
                                                   __builtin_bit_cast(s16x4, b), c, 0, 0, 0);
}

__device__ __forceinline__ u32x2 lds_read_tr16(const unsigned char* p) {
  const s16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(p));
  return __builtin_bit_cast(u32x2, v);
}

// 16-byte chunk swizzle of tile row r (chunk c stored at c ^ dswz(r)): a
// bijection on r % 16, so a score read (16 lanes = 16 rows, one chunk) hits 16
// bank groups; rows 0..7 map to even and rows 8..15 to odd values, so a
// transpose read (32 lanes = 8 rows x 2 adjacent chunks) hits 16 as well.
__device__ __forceinline__ int dswz(int r) { return ((r & 7) << 1) | ((r >> 3) & 1); }

// RK = score k-steps (32 dims each) that may hold turning pairs: 4 when
// n_rot <= 64 (dims < 128, e.g. p-RoPE at p = 0.25), else all of them.
// NW = waves per workgroup.  With NW > 1 the waves split the chunk and merge
// their partials in LDS at the end (shorter waves, one partial per chunk);
// when one chunk covers every row the workgroup writes the final output and
// no merge kernel runs.
// Separate K and V at D = 256: one wave; keys load straight into registers
// (already in the score operand layout) two tiles ahead, values into the
// second of two LDS slots one tile ahead, so about a tile and a half is always
// in flight.  Separate K and V at D = 512: one wave whose
// K and V tiles are separate LDS objects; the next keys are requested as soon
// as the scores are done, the next values as soon as the value product is.
template <int D, int G, bool KVS, int RK, int NW, bool OBF>
__global__ void __launch_bounds__(64 * NW) __attribute__((amdgpu_waves_per_eu(2, 2)))
decode_split_kernel(DecodeArgs a) {
  constexpr int NS = D / 32;  // 32-dim k-steps of the score product
  constexpr int NB = D / 16;  // 16-dim blocks of the output
  constexpr int KB = TR * D * 2;     // one tensor's tile, bytes
  constexpr int NLD = KB / 1024;     // direct loads per lane per tensor tile
  constexpr bool KREG = !KVS && D == 256;  // keys through registers
  static_assert(G <= 8 && RK <= NS && NS % 4 == 0 && (KVS || KREG || NW == 1), "shape");
  __shared__ __attribute__((aligned(16))) unsigned char tk[KREG ? 16 : NW * KB];   // K (or K=V) tile per wave
  __shared__ __attribute__((aligned(16))) unsigned char tv[KVS ? 16 : NW * KB];    // V tile per wave
  __shared__ __attribute__((aligned(16))) unsigned char tv2[KREG ? NW * KB : 16];  // second V slot per wave
  __shared__ double gtab[D / 2];
  __shared__ float mls[NW][16][2];
  __shared__ int tnext;  // next unclaimed tile of the chunk (NW > 1)


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
  const int ncol = min(16, G * QL - 16 * cb);  // columns in use
  auto col_out = [&](int n) -> size_t {          // output row of column n
    const int c = 16 * cb + n;
    return (((size_t)b * QL + c / G) * a.Hq + hkv * G + c % G) * D;
  };
  auto col_pos = [&](int n) { return P - QL + 1 + (16 * cb + n) / G; };
  const bool col_ok = l16 < ncol;
  const int Pq = col_pos(col_ok ? l16 : 0);  // this lane's column position
  const bool direct = NW > 1 && a.nchunk == 1;  // this workgroup writes the output
  if (P < 0 || (W == 0 && P >= C)) {  // bad position: NaN rows (else the merge writes them)
    if (direct) nan_columns<D, NW, OBF>(a, ncol, col_out);
    return;
  }
  const int last = W > 0 ? min(P, C - 1) : P;  // highest row index that may be visible
  const int r0 = ch * a.chunk;
  if (r0 > last) return;
  const int r1 = min(r0 + a.chunk, last + 1);  // exclusive
  // Tile t of the chunk holds rows r0 + TR*t .. (clipped at r1).  With several
  // waves, wave w starts on tile w (and, where keys run two tiles ahead, on
  // w + NW) and claims every further tile from a workgroup counter, so waves
  // that stream faster take more tiles and all finish together.  A wave's
  // tiles increase, so its loads are issued in tile order.
  const int nt = (r1 - r0 + TR - 1) / TR;
  const bool stream_loads = a.ncb == 1;  // cache rows read once: non-temporal
  const int n_rot = a.n_rot;
  unsigned char* kt = tk + (KREG ? 0 : w * KB);
  unsigned char* vt0 = tv + (KVS ? 0 : w * KB);
  unsigned char* vt1 = tv2 + (KREG ? w * KB : 0);

  // query heads hkv*G .. +G-1 as B operands of the score product (columns >= G
  // are zero); loaded first, so waiting for them leaves the tile loads below in flight
  u32x4 qf[NS];
  {
    const uint16_t* qrow = static_cast<const uint16_t*>(a.q) + col_out(col_ok ? l16 : 0);
#pragma unroll
    for (int s = 0; s < NS; ++s) qf[s] = *reinterpret_cast<const u32x4*>(qrow + 8 * (4 * s + g4));
  }

  const size_t hoff = ((size_t)b * a.Hkv + hkv) * C * D;
  const uint16_t* kbase = static_cast<const uint16_t*>(a.k) + hoff;
  const uint16_t* vbase = static_cast<const uint16_t*>(a.v) + hoff;

  // 16 rows of tile i of one tensor into an LDS tile; rows past r1 read as zeros
  auto issue = [&](const uint16_t* base, int i, unsigned char* dst) {
    const int rr0 = r0 + i * TR;
    const uint32_t bytes = (uint32_t)min(TR, r1 - rr0) * (2 * D);
    const __amdgpu_buffer_rsrc_t rs = make_rsrc(base + (size_t)rr0 * D, bytes);
    constexpr int CPR = D / 8;       // chunks per row
    constexpr int RPI = 64 / CPR;    // rows per direct load
    int ln = lane;
    asm volatile("" : "+v"(ln));
#pragma unroll
    for (int n = 0; n < TR / RPI; ++n) {
      const int row = n * RPI + ln / CPR;
      const uint32_t voff = (uint32_t)row * (2 * D) + ((uint32_t)((ln % CPR) ^ dswz(row)) << 4);
      lds_dma16(rs, voff, dst + n * 1024, stream_loads);
    }
  };
  // The angle table is shared by the waves of a workgroup.  With several
  // waves the barrier (whose fence waits for every outstanding load) comes
  // before the first tile is requested; a single wave reads its own LDS
  // writes in order and needs no barrier, so its query and tile loads overlap.
  for (int t = threadIdx.x; t < D / 2; t += 64 * NW) gtab[t] = rope_rev_per_pos(t, D, a.log2_theta);
  if constexpr (NW > 1) {
    if (threadIdx.x == 0) tnext = (KREG ? 2 : 1) * NW;
    __syncthreads();
  }
  // next tile for this wave (wave-uniform; only used with several waves)
  auto claim = [&]() -> int {
    int t = 0;
    if (lane == 0) t = atomicAdd(&tnext, 1);
    return __builtin_amdgcn_readfirstlane(t);
  };
  const int tA = NW > 1 ? w : 0, tB = NW > 1 ? w + NW : 1;  // first two tiles of this wave
  // keys of tile i into registers, lane (row = l % 16, gq = l / 16) holding
  // dims 32*s + 8*gq .. +7 of its row for every k-step s; rows past r1 read as zeros
  auto load_keys = [&](int i, u32x4 (&kr)[NS]) {
    const int rr0 = r0 + i * TR;
    const uint32_t bytes = (uint32_t)min(TR, r1 - rr0) * (2 * D);
    const __amdgpu_buffer_rsrc_t rs = make_rsrc(kbase + (size_t)rr0 * D, bytes);
    int ln = lane;
    asm volatile("" : "+v"(ln));
    const uint32_t base = (uint32_t)(ln & 15) * (2 * D) + (uint32_t)(ln >> 4) * 16;
#pragma unroll
    for (int s = 0; s < NS; ++s)
      kr[s] = __builtin_bit_cast(
          u32x4, stream_loads ? __builtin_amdgcn_raw_buffer_load_b128(rs, base + 64 * s, 0, CPOL_NT)
                    : __builtin_amdgcn_raw_buffer_load_b128(rs, base + 64 * s, 0, 0));
  };
  u32x4 kr0[KREG ? NS : 1], kr1[KREG ? NS : 1], kr2[KREG ? NS : 1];
  if (tA < nt) {
    if constexpr (KREG) load_keys(tA, kr0);
    else issue(kbase, tA, kt);
    if constexpr (!KVS) issue(vbase, tA, vt0);
    if constexpr (KREG)
      if (tB < nt) load_keys(tB, kr1);
  }
#pragma unroll
  for (int s = 0; s < NS; ++s) {
    qf[s] = col_ok ? qf[s] : u32x4{0, 0, 0, 0};
    if (s < RK) qf[s] = rotate_chunk_bf16(qf[s], 4 * s + g4, Pq, n_rot, gtab);
  }

  f32x4 oacc[NB];
#pragma unroll
  for (int i = 0; i < NB; ++i) oacc[i] = f32x4{};
  float m_run = -INFINITY, l_run = 0.f;  // per column (query head l16), base 2
  const float cs = a.scale_log2e;

  // scores of tile i from the key tile (or, kr non-null, from key registers):
  // S^T register j = key 4*gq + j of column l16
  auto scores = [&](int i, const u32x4* kr) -> f32x4 {
    const int rr0 = r0 + i * TR;
    int ln = lane;
    asm volatile("" : "+v"(ln));
    const int row = ln & 15, gq = ln >> 4;
    const int r = min(rr0 + row, r1 - 1);  // rows past the tile end are masked
    const int tpos = W > 0 ? P - (P - r) % C : r;
    // chunk c = 4*s + gq of row `row` is stored at 16*(s/4) + ((4*(s%4) + gq) ^ dswz(row))
    const int dsw = dswz(row);
    int koff[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) koff[j] = row * (2 * D) + (((4 * j + gq) ^ dsw) << 4);
    f32x4 sacc0 = {}, sacc1 = {};  // even / odd k-steps: two independent chains
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      u32x4 kf = KREG ? kr[s] : lds_at<u32x4>(kt, koff[s & 3] + 256 * (s >> 2));
      // per-pair select inside; keys of a separate-value cache are cached turned
      if (KVS && s < RK) kf = rotate_chunk_bf16(kf, 4 * s + gq, tpos, n_rot, gtab);
      if (s & 1) sacc1 = mfma16x16x32(kf, qf[s], sacc1);
      else sacc0 = mfma16x16x32(kf, qf[s], sacc0);
    }
    return sacc0 + sacc1;
  };
  // softmax update of the columns; returns P^T as the B operand of the value product
  auto softmax = [&](int i, f32x4 sacc) -> u32x2 {
    const int nrows = min(TR, r1 - (r0 + i * TR));
#pragma unroll
    for (int j = 0; j < 4; ++j) sacc[j] = 4 * g4 + j < nrows ? sacc[j] : -INFINITY;
    // wave-uniform: each column sees keys up to its own position, and a ring
    // larger than the window holds keys before every column's window
    if (QL > 1 || (W > 0 && C > W)) {
      const int rk = r0 + i * TR + 4 * g4;   // this lane's first key row
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
    return u32x2{pack_bf16(p[0], p[1]), pack_bf16(p[2], p[3])};
  };
  // O^T += V^T P^T with V^T by transpose reads: source lane (gq, row) addresses
  // tile row 4*gq + row/4, dims 16*db + 4*(row%4) .. +3, i.e. chunk
  // c = 2*db + (row%4)/2 (half row%2), stored at 16*(db/8) + ((2*(db%8) + (row%4)/2) ^ dswz)
  auto values = [&](const unsigned char* vt, u32x2 pf) {
    int ln = lane;
    asm volatile("" : "+v"(ln));
    const int row = ln & 15, gq = ln >> 4;
    const int trow = 4 * gq + (row >> 2);
    const int tch = (row & 3) >> 1;
    const int tdsw = dswz(trow);
    int voff[8];
#pragma unroll
    for (int j = 0; j < 8; ++j)
      voff[j] = trow * (2 * D) + (row & 1) * 8 + (((2 * j + tch) ^ tdsw) << 4);
#pragma unroll
    for (int db = 0; db < NB; ++db) {
      const u32x2 vf = lds_read_tr16(vt + voff[db & 7] + 256 * (db >> 3));
      oacc[db] = mfma16x16x16(vf, pf, oacc[db]);
    }
  };

  if constexpr (KVS) {
    // one tile slot: the previous tile's LDS reads have completed (its
    // products consumed them) before the next tile's loads are requested
    for (int t = tA; t < nt;) {
      const int tn = claim();
      wait_vmcnt<0>();
      const u32x2 pf = softmax(t, scores(t, nullptr));
      values(kt, pf);
      if (tn < nt) issue(kbase, tn, kt);
      t = tn;
    }
  } else if constexpr (KREG) {
    // The wave's tiles are c, n1, n2, ... in increasing order.  A step
    // requests the values of n1, then the keys of n2, and computes c.  Issue
    // order is V_c, K_n1, V_n1, K_n2, so waiting until only the last three
    // groups are in flight means keys and values of c have landed.  Key sets
    // rotate over 3 register blocks and value slots over 2, so the loop is
    // unrolled by 6; the tile after n2 is claimed when n2 is.
    auto step = [&](int c, int n1, int n2, u32x4 (&kc)[NS], u32x4 (&kn2)[NS],
                    unsigned char* vc, unsigned char* vn) {
      if (n1 < nt) issue(vbase, n1, vn);
      if (n2 < nt) load_keys(n2, kn2);
      if (n2 < nt) wait_vmcnt<2 * NS + NLD>();
      else if (n1 < nt) wait_vmcnt<NS + NLD>();
      else wait_vmcnt<0>();
      const u32x2 pf = softmax(c, scores(c, kc));
      values(vc, pf);
    };
    int t0 = tA, t1 = tB, t2;
    for (;;) {
      if (t0 >= nt) break;
      t2 = claim();
      step(t0, t1, t2, kr0, kr2, vt0, vt1);
      if (t1 >= nt) break;
      t0 = claim();
      step(t1, t2, t0, kr1, kr0, vt1, vt0);
      if (t2 >= nt) break;
      t1 = claim();
      step(t2, t0, t1, kr2, kr1, vt0, vt1);
      if (t0 >= nt) break;
      t2 = claim();
      step(t0, t1, t2, kr0, kr2, vt1, vt0);
      if (t1 >= nt) break;
      t0 = claim();
      step(t1, t2, t0, kr1, kr0, vt0, vt1);
      if (t2 >= nt) break;
      t1 = claim();
      step(t2, t0, t1, kr2, kr1, vt1, vt0);
    }
  } else {
    // one wave takes the chunk's tiles in order: keys of tile i+1 load during
    // the softmax and value product of tile i, values of tile i+1 during the
    // scores of tile i+1
    static_assert(NW == 1, "single wave");
    for (int i = 0; i < nt; ++i) {
      wait_vmcnt<NLD>();  // keys of tile i (its values may still be in flight)
      const f32x4 sacc = scores(i, nullptr);
      const bool more = i + 1 < nt;
      if (more) issue(kbase, i + 1, kt);
      const u32x2 pf = softmax(i, sacc);
      if (more) wait_vmcnt<NLD>();  // values of tile i (next keys may be in flight)
      else wait_vmcnt<0>();
      values(vt0, pf);
      if (more) issue(vbase, i + 1, vt0);
    }
  }

  // ---- partial (m, l, O) of this chunk for the block's columns ----
  l_run += __shfl_xor(l_run, 16);
  l_run += __shfl_xor(l_run, 32);
  finish_chunk<D, NW, OBF>(a, oacc, m_run, l_run, ch, ncol, direct,
                           reinterpret_cast<float*>(KREG ? tv : tk), mls, col_out, col_pos);
}

// Combine the chunk partials of query head h of token j of sequence b:
// weights 2^(m_c - M); a chunk with no visible key has m_c = -inf and weight 0.
// Each of the 128 threads owns 4 dims; the chunk loop keeps 4 loads in flight.
template <bool OBF>
__global__ void __launch_bounds__(128) decode_merge_kernel(DecodeArgs a) {
  __shared__ float red[2][2];
  const int h = blockIdx.x % a.Hq;
  const int tok = blockIdx.x / a.Hq % a.q_len;
  const int b = blockIdx.x / a.Hq / a.q_len;
  const int D = a.D, tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int P = a.pos[b];
  const size_t orow = (((size_t)b * a.q_len + tok) * a.Hq + h) * D;
  if (P < 0 || P - a.q_len + 1 + tok < 0 || (a.window == 0 && P >= a.capacity)) {
    for (int e = tid; e < D; e += 128) {
      if constexpr (OBF) static_cast<uint16_t*>(a.out)[orow + e] = 0x7fc0;
      else static_cast<float*>(a.out)[orow + e] = __builtin_nanf("");
    }
    return;
  }
  const int last = a.window > 0 ? min(P, a.capacity - 1) : P;
  const int nch = last / a.chunk + 1;
  const size_t prow = (((size_t)b * a.q_len + tok) * a.Hq + h) * a.nchunk;
  const float* ml = a.part_ml + prow * 2;
  float M = -INFINITY;
  for (int c = tid; c < nch; c += 128) M = fmaxf(M, ml[2 * c]);
  M = wave_max(M);
  if (lane == 0) red[0][w] = M;
  __syncthreads();
  M = fmaxf(red[0][0], red[0][1]);
  float l = 0.f;
  for (int c = tid; c < nch; c += 128) l += __builtin_amdgcn_exp2f(ml[2 * c] - M) * ml[2 * c + 1];
  l = wave_sum(l);
  if (lane == 0) red[1][w] = l;
  __syncthreads();
  const float inv = 1.f / (red[1][0] + red[1][1]);
  for (int e = 4 * tid; e < D; e += 512) {
    const float* po = a.part_o + prow * D + e;
    f32x4 o = {};
    int c = 0;
    for (; c + 4 <= nch; c += 4) {
      f32x4 v[4];
      float f[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        v[j] = *reinterpret_cast<const f32x4*>(po + (size_t)(c + j) * D);
        f[j] = __builtin_amdgcn_exp2f(ml[2 * (c + j)] - M);
      }
#pragma unroll
      for (int j = 0; j < 4; ++j) o += f[j] * v[j];
    }
    for (; c < nch; ++c)
      o += __builtin_amdgcn_exp2f(ml[2 * c] - M) * *reinterpret_cast<const f32x4*>(po + (size_t)c * D);
    o *= inv;
    if constexpr (OBF) {
      const u32x2 pk = {pack_bf16(o[0], o[1]), pack_bf16(o[2], o[3])};
      *reinterpret_cast<u32x2*>(static_cast<uint16_t*>(a.out) + orow + e) = pk;
    } else {
      *reinterpret_cast<f32x4*>(static_cast<float*>(a.out) + orow + e) = o;
    }
  }
}

// waves per split workgroup (the D = 512 separate-K/V path keeps one)
constexpr int split_waves(int D, bool kv_shared) { return (kv_shared || D == 256) ? 4 : 1; }

template <int D, int G, bool KVS, bool OBF>
hipError_t launch_split(const DecodeArgs& a, hipStream_t st) {
  constexpr int NW = split_waves(D, KVS);
  const long long n = (long long)a.B * a.Hkv * a.ncb * a.nchunk;
  if (n > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  if (a.n_rot <= 64)
    hipLaunchKernelGGL((decode_split_kernel<D, G, KVS, 4, NW, OBF>), dim3((unsigned)n),
                       dim3(64 * NW), 0, st, a);
  else
    hipLaunchKernelGGL((decode_split_kernel<D, G, KVS, D / 32, NW, OBF>), dim3((unsigned)n),
                       dim3(64 * NW), 0, st, a);
  return hipGetLastError();
}

template <int D, bool KVS, bool OBF>
hipError_t launch_split_g(const DecodeArgs& a, hipStream_t st) {
  switch (a.Hq / a.Hkv) {
    case 1: return launch_split<D, 1, KVS, OBF>(a, st);
    case 2: return launch_split<D, 2, KVS, OBF>(a, st);
    case 4: return launch_split<D, 4, KVS, OBF>(a, st);
    case 8: return launch_split<D, 8, KVS, OBF>(a, st);
  }
  return hipErrorInvalidValue;
}

template <bool OBF>
hipError_t launch_split_d(const DecodeArgs& a, bool kv_shared, hipStream_t st) {
  if (a.D == 256) return kv_shared ? launch_split_g<256, true, OBF>(a, st) : launch_split_g<256, false, OBF>(a, st);
  if (a.D == 512) return kv_shared ? launch_split_g<512, true, OBF>(a, st) : launch_split_g<512, false, OBF>(a, st);
  return hipErrorInvalidValue;
}

}  // namespace

int decode_chunk_rows(int D, int capacity, int window, bool f32) {
  (void)D;
  if (f32) return capacity;
  if (window > 0) return (capacity + TR - 1) / TR * TR;  // ring: one 4-wave workgroup per ring
  return 1024;
}

int decode_num_chunks(int D, int capacity, int window, bool f32) {
  const int ch = decode_chunk_rows(D, capacity, window, f32);
  return (capacity + ch - 1) / ch;
}

hipError_t launch_decode_bf16(const DecodeArgs& a, bool kv_shared, bool out_bf16,
                              hipStream_t st) {
  if ((long long)a.B * a.Hkv == 0) return hipSuccess;
  // K=V with several column blocks: one pass over each chunk for all of them
  if (kv_shared && a.ncb >= 2) return launch_decode_mc(a, out_bf16, st);
  const hipError_t e = out_bf16 ? launch_split_d<true>(a, kv_shared, st)
                                : launch_split_d<false>(a, kv_shared, st);
  if (e != hipSuccess) return e;
  // a single chunk per (b, kv head) split over several waves is finished in place
  if (a.nchunk == 1 && split_waves(a.D, kv_shared) > 1) return hipSuccess;
  return launch_decode_merge(a, out_bf16, st);
}

hipError_t launch_decode_merge(const DecodeArgs& a, bool out_bf16, hipStream_t st) {
  const long long n = (long long)a.B * a.q_len * a.Hq;
  if (n > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  if (out_bf16) hipLaunchKernelGGL(decode_merge_kernel<true>, dim3((unsigned)n), dim3(128), 0, st, a);
  else hipLaunchKernelGGL(decode_merge_kernel<false>, dim3((unsigned)n), dim3(128), 0, st, a);
  return hipGetLastError();
}

}  // namespace g4a
