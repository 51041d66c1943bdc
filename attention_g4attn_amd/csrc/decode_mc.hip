// Decode of many query columns per KV head over a K=V cache: the verify step
// of several draft tokens with 8 query heads per KV head (every Gemma 4 size
// ships a draft model: "Visao geral do modelo Gemma 4", section "Recursos";
// global layers: 8 query heads per KV head, keys identical to values, p-RoPE,
// "Guia visual do Gemma 4", sections "GQA", "Tecnica K=V", "p-RoPE").
//
// What is computed is the decode of q_len query tokens (columns = (token,
// head) pairs, G * q_len of them, 17 .. 64) against the cache rows each token
// may see, exactly as the one-block split kernel computes it for up to 16
// columns.  That kernel, run once per 16-column block, streams every chunk of
// the cache once per block; this one reads every tile once for all blocks.
//
// Work decomposition: one 4-wave workgroup per (sequence, KV head, chunk of
// 1024 cache rows), numbered densely over the chunks with a visible row as in
// the split kernel.  The workgroup walks its chunk in 16-row tiles that stream
// from HBM through a 3-deep LDS ring (16-byte direct-to-LDS loads, a
// quarter issued by each wave).  The head dims are split over the waves: wave w takes
// score k-steps s = w, w+4, ... (32 dims each; with p-RoPE at p = 0.25 the
// rotated k-steps 0..3 go one per wave) and output dim blocks db = w, w+4, ...
// (16 dims each).  Per tile:
//   1. every wave forms its partial S^T over its k-steps for every column
//      block (16x16x32 products; keys rotated at their positions) and writes
//      it to LDS;
//   2. wave j sums the four partials of block j, masks, and updates the
//      softmax of block j's columns; it writes P^T (bf16, in the B-operand
//      layout of the value product) and, when a column's max grew by more
//      than 2^8, the factor that rescales that column's outputs;
//   3. every wave applies the factors to its output blocks and forms
//      O^T += V^T P^T for its dim blocks of every column block (16x16x16
//      products, V^T by LDS transpose reads).
// Three barriers per tile separate the phases.  A wave holds 16 columns x
// its D/4 output dims per block (8 f32x4 per block at D = 512), so two waves
// fit per SIMD.  The chunk's (m, l, O) go to the workspace for the merge
// kernel, or, when one chunk covers every row, straight to the output.
#include <type_traits>

#include "common.hpp"
#include "decode_common.hpp"
#include "kernels.hpp"

namespace g4a {

namespace {

using namespace dec;

constexpr int TRM = 16;  // cache rows per tile
constexpr int NWM = 4;   // waves per workgroup

template <int N>
using ICM = std::integral_constant<int, N>;

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

__device__ __forceinline__ f32x4 mfma16x16x16(u32x2 a, u32x2 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(s16x4, a),
                                                   __builtin_bit_cast(s16x4, b), c, 0, 0, 0);
}

__device__ __forceinline__ u32x2 lds_read_tr16(const unsigned char* p) {
  const s16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(p));
  return __builtin_bit_cast(u32x2, v);
}

// 16-byte chunk swizzle of tile row r, the one-block kernel's: a bijection on
// r % 16; a score read (16 lanes = 16 rows, one chunk) and a transpose read
// (32 lanes = 8 rows x 2 adjacent chunks) each hit 16 bank groups.
__device__ __forceinline__ int mswz(int r) { return ((r & 7) << 1) | ((r >> 3) & 1); }

// NCB = column blocks the instance holds (2 or 4); RK = score k-steps that
// may hold turning pairs (4 when n_rot <= 64, else all).  The LDS ring is 3
// deep (two workgroups per CU); a fourth stage measured no faster (1481
// against 1461 us for 64 sequences of 4 draft tokens at G = 8, D = 512).
template <int D, int G, int NCB, int RK, bool OBF>
__global__ void __launch_bounds__(64 * NWM) __attribute__((amdgpu_waves_per_eu(2, 2)))
decode_mc_kernel(DecodeArgs a) {
  constexpr int NS = D / 32;       // score k-steps
  constexpr int NB = D / 16;       // output dim blocks
  constexpr int KSW = NS / NWM;    // k-steps per wave
  constexpr int DBW = NB / NWM;    // dim blocks per wave
  constexpr int KB = TRM * D * 2;  // one tile, bytes
  constexpr int NLD = KB / 1024;   // direct loads per tile
  constexpr int NLW = NLD / NWM;   // per wave
  constexpr int NST = 3;  // LDS ring depth
  static_assert(G <= 8 && NCB <= 4 && RK <= NS && NS % NWM == 0 && NLD % NWM == 0, "shape");
  __shared__ __attribute__((aligned(16))) unsigned char st0[KB];
  __shared__ __attribute__((aligned(16))) unsigned char st1[KB];
  __shared__ __attribute__((aligned(16))) unsigned char st2[KB];
  __shared__ __attribute__((aligned(16))) unsigned char st3[NST > 3 ? KB : 16];
  __shared__ __attribute__((aligned(16))) f32x4 xs[NWM][NCB][64];  // partial scores
  __shared__ __attribute__((aligned(16))) u32x2 pb[NCB][64];        // P^T operands
  __shared__ float alb[NCB][16];                                   // rescale factors
  __shared__ int rsb[NCB];                                         // block rescaled?
  __shared__ float mlb[NCB][16][2];                                // final (m, l)
  __shared__ double gtab[D / 2];
  auto stp = [&](auto s) -> unsigned char* {
    if constexpr (decltype(s)::value == 0) return st0;
    else if constexpr (decltype(s)::value == 1) return st1;
    else if constexpr (decltype(s)::value == 2) return st2;
    else return st3;
  };

  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int l16 = lane & 15, g4 = lane >> 4;
  const Unit u = unit_of_block(a);  // every column block in one workgroup
  if (u.b < 0) return;
  const int ch = u.ch, b = u.b, hkv = u.hkv;
  const int P = a.pos[b];
  const int W = a.window, C = a.capacity, QL = a.q_len;
  const int ncb = min(NCB, (G * QL + 15) / 16);
  // Column n of block j is (token, head) pair c = 16*j + n: query token c / G
  // at position P - QL + 1 + c / G, query head hkv*G + c % G.
  auto ncol_of = [&](int j) { return max(0, min(16, G * QL - 16 * j)); };
  auto col_out = [&](int j, int n) -> size_t {
    const int c = 16 * j + n;
    return (((size_t)b * QL + c / G) * a.Hq + hkv * G + c % G) * D;
  };
  auto col_pos = [&](int j, int n) { return P - QL + 1 + (16 * j + n) / G; };
  const bool direct = a.nchunk == 1;
  if (P < 0 || (W == 0 && P >= C)) {
    if (direct)
      for (int j = 0; j < ncb; ++j)
        nan_columns<D, NWM, OBF>(a, ncol_of(j), [&](int n) { return col_out(j, n); });
    return;
  }
  const int last = W > 0 ? min(P, C - 1) : P;
  const int r0 = ch * a.chunk;
  if (r0 > last) return;
  const int r1 = min(r0 + a.chunk, last + 1);
  const int nt = (r1 - r0 + TRM - 1) / TRM;
  const int n_rot = a.n_rot;

  // this wave's k-steps of the queries of every block, as B operands
  bool col_ok[NCB];
  int pq[NCB];
  u32x4 qf[NCB][KSW];
#pragma unroll
  for (int j = 0; j < NCB; ++j) {
    col_ok[j] = j < ncb && l16 < ncol_of(j);
    pq[j] = col_ok[j] ? col_pos(j, l16) : 0;
    const uint16_t* qrow = static_cast<const uint16_t*>(a.q) + (col_ok[j] ? col_out(j, l16) : col_out(0, 0));
#pragma unroll
    for (int k = 0; k < KSW; ++k) {
      const int s = NWM * k + w;
      qf[j][k] = *reinterpret_cast<const u32x4*>(qrow + 8 * (4 * s + g4));
    }
  }
  const size_t hoff = ((size_t)b * a.Hkv + hkv) * C * D;
  const uint16_t* kbase = static_cast<const uint16_t*>(a.k) + hoff;
  // this wave's quarter of tile i's rows into a stage; rows past r1 read as
  // zeros; every cache row is read once by the launch: non-temporal
  auto issue = [&](int i, unsigned char* dst) {
    const int rr0 = r0 + min(i, nt - 1) * TRM;  // past the last tile: repeat it
    const uint32_t bytes = (uint32_t)min(TRM, r1 - rr0) * (2 * D);
    const __amdgpu_buffer_rsrc_t rs = make_rsrc(kbase + (size_t)rr0 * D, bytes);
    constexpr int CPR = D / 8;
    constexpr int RPI = 64 / CPR;
    int ln = lane;
    asm volatile("" : "+v"(ln));
#pragma unroll
    for (int m = 0; m < NLW; ++m) {
      const int n = NLW * w + m;
      const int row = n * RPI + ln / CPR;
      const uint32_t voff = (uint32_t)row * (2 * D) + ((uint32_t)((ln % CPR) ^ mswz(row)) << 4);
      lds_dma16(rs, voff, dst + n * 1024, true);
    }
  };
  for (int t = threadIdx.x; t < D / 2; t += 64 * NWM) gtab[t] = rope_rev_per_pos(t, D, a.log2_theta);
  __syncthreads();
  // tiles 0 .. NST-2 in flight before the queries are rotated
  issue(0, st0);
  issue(1, st1);
  if constexpr (NST > 3) issue(2, st2);
#pragma unroll
  for (int j = 0; j < NCB; ++j)
#pragma unroll
    for (int k = 0; k < KSW; ++k) {
      const int s = NWM * k + w;
      qf[j][k] = col_ok[j] ? qf[j][k] : u32x4{0, 0, 0, 0};
      if (s < RK) qf[j][k] = rotate_chunk_bf16(qf[j][k], 4 * s + g4, pq[j], n_rot, gtab);
    }

  f32x4 oacc[NCB][DBW];
#pragma unroll
  for (int j = 0; j < NCB; ++j)
#pragma unroll
    for (int k = 0; k < DBW; ++k) oacc[j][k] = f32x4{};
  // softmax state of block w's columns (wave w < ncb owns block w)
  float m_run = -INFINITY, l_run = 0.f;
  const float cs = a.scale_log2e;
  const int jo = w;  // the block this wave owns

  auto step = [&](int i, auto s) {
    constexpr int S0 = decltype(s)::value;
    unsigned char* kt = stp(s);
    // ---- 1. partial scores of this wave's k-steps, every block ----
    {
      int ln = lane;
      asm volatile("" : "+v"(ln));
      const int row = ln & 15, gq = ln >> 4;
      const int rr = min(r0 + i * TRM + row, r1 - 1);
      const int tpos = W > 0 ? P - (P - rr) % C : rr;
      const int dsw = mswz(row);
      f32x4 ps[NCB] = {};
#pragma unroll
      for (int k = 0; k < KSW; ++k) {
        const int sk = NWM * k + w;  // k-step: chunk 4*sk + gq of the row
        const int c = 4 * sk + gq;
        u32x4 kf = lds_at<u32x4>(kt, row * (2 * D) + 256 * (c >> 4) + (((c & 15) ^ dsw) << 4));
        if (sk < RK) kf = rotate_chunk_bf16(kf, c, tpos, n_rot, gtab);
#pragma unroll
        for (int j = 0; j < NCB; ++j)
          if (j < ncb) ps[j] = mfma16x16x32(kf, qf[j][k], ps[j]);
      }
#pragma unroll
      for (int j = 0; j < NCB; ++j)
        if (j < ncb) xs[w][j][lane] = ps[j];
    }
    __syncthreads();
    // tile i+NST-1 goes into the stage tile i-1 used (every wave is past its reads)
    if (i + NST - 1 < nt) issue(i + NST - 1, stp(ICM<(S0 + NST - 1) % NST>{}));
    // ---- 2. softmax of the owned block ----
    if (jo < ncb) {
      f32x4 sacc = xs[0][jo][lane];
#pragma unroll
      for (int v = 1; v < NWM; ++v) sacc += xs[v][jo][lane];
      const int nrows = min(TRM, r1 - (r0 + i * TRM));
#pragma unroll
      for (int r = 0; r < 4; ++r) sacc[r] = 4 * g4 + r < nrows ? sacc[r] : -INFINITY;
      if (QL > 1) {  // each column sees keys up to its own position
        const int Pq = col_pos(jo, l16);
        const int rk = r0 + i * TRM + 4 * g4;
        const int m0 = W > 0 ? (P - rk) % C : 0;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int mj = m0 - r;
          const int tp = W > 0 ? P - (mj >= 0 ? mj : mj + C) : rk + r;
          const bool vis = tp <= Pq && (W == 0 || tp > Pq - W);
          sacc[r] = vis ? sacc[r] : -INFINITY;
        }
      }
      float mx = fmaxf(fmaxf(sacc[0], sacc[1]), fmaxf(sacc[2], sacc[3]));
      mx = fmaxf(mx, __shfl_xor(mx, 16));
      mx = fmaxf(mx, __shfl_xor(mx, 32));
      const float mt = mx * cs;
      const bool grow = __any(mt > m_run + 8.f);  // wave-uniform; rare after the first tile
      float al = 1.f;
      if (grow) {
        const float mn = fmaxf(m_run, mt);
        al = m_run == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m_run - mn);
        l_run *= al;
        m_run = mn;
      }
      const float mr = m_run == -INFINITY ? 0.f : m_run;
      float p[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        p[r] = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[r], cs, -mr));
        l_run += p[r];
      }
      pb[jo][lane] = u32x2{pack_bf16(p[0], p[1]), pack_bf16(p[2], p[3])};
      if (g4 == 0) alb[jo][l16] = al;
      if (lane == 0) rsb[jo] = grow;
    }
    __syncthreads();
    // ---- 3. rescale and value products of this wave's dim blocks ----
    {
      int ln = lane;
      asm volatile("" : "+v"(ln));
      const int row = ln & 15, gq = ln >> 4;
      const int trow = 4 * gq + (row >> 2);
      const int tch = (row & 3) >> 1;
      const int tdsw = mswz(trow);
      u32x2 pf[NCB];
#pragma unroll
      for (int j = 0; j < NCB; ++j) {
        if (j < ncb) {
          if (__builtin_amdgcn_readfirstlane(rsb[j])) {  // wave-uniform
            const float f = alb[j][l16];
#pragma unroll
            for (int k = 0; k < DBW; ++k) oacc[j][k] *= f;
          }
          pf[j] = pb[j][lane];
        }
      }
#pragma unroll
      for (int k = 0; k < DBW; ++k) {
        const int db = NWM * k + w;  // chunk c = 2*db + tch of row trow
        const int c = 2 * db + tch;
        const u32x2 vf = lds_read_tr16(kt + trow * (2 * D) + (row & 1) * 8 + 256 * (c >> 4) +
                                       (((c & 15) ^ tdsw) << 4));
#pragma unroll
        for (int j = 0; j < NCB; ++j)
          if (j < ncb) oacc[j][k] = mfma16x16x16(vf, pf[j], oacc[j][k]);
      }
    }
    // tile i+1 must have landed in every wave's part before the next step;
    // this wave's loads of tiles i+2 .. i+NST-1 may still run
    if (i + NST - 1 < nt) wait_vmcnt<(NST - 2) * NLW>();
    else wait_vmcnt<0>();
    __syncthreads();
  };
  wait_vmcnt<(NST - 2) * NLW>();  // this wave's part of tile 0
  __syncthreads();
  for (int i = 0; i < nt; i += NST) {
    step(i, ICM<0>{});
    if (i + 1 >= nt) break;
    step(i + 1, ICM<1>{});
    if (i + 2 >= nt) break;
    step(i + 2, ICM<2 % NST>{});
    if constexpr (NST > 3) {
      if (i + 3 >= nt) break;
      step(i + 3, ICM<3 % NST>{});
    }
  }

  // ---- the chunk's (m, l, O): owners publish (m, l), every wave its dims ----
  if (jo < ncb) {
    l_run += __shfl_xor(l_run, 16);
    l_run += __shfl_xor(l_run, 32);
    if (g4 == 0) {
      mlb[jo][l16][0] = m_run;
      mlb[jo][l16][1] = l_run;
    }
  }
  __syncthreads();
#pragma unroll
  for (int j = 0; j < NCB; ++j) {
    if (j >= ncb || l16 >= ncol_of(j)) continue;
    const float m = mlb[j][l16][0], l = mlb[j][l16][1];
    if (direct) {
      // every column sees its own key unless its position is negative
      const bool ok = col_pos(j, l16) >= 0;
      const float inv = 1.f / l;
      const size_t orow = col_out(j, l16);
#pragma unroll
      for (int k = 0; k < DBW; ++k) {
        const int e = 16 * (NWM * k + w) + 4 * g4;
        const f32x4 o = ok ? oacc[j][k] * inv
                           : f32x4{__builtin_nanf(""), __builtin_nanf(""), __builtin_nanf(""),
                                   __builtin_nanf("")};
        if constexpr (OBF) {
          const u32x2 pk = {pack_bf16(o[0], o[1]), pack_bf16(o[2], o[3])};
          *reinterpret_cast<u32x2*>(static_cast<uint16_t*>(a.out) + orow + e) = pk;
        } else {
          *reinterpret_cast<f32x4*>(static_cast<float*>(a.out) + orow + e) = o;
        }
      }
    } else {
      const size_t prow = (col_out(j, l16) / D) * a.nchunk + ch;
#pragma unroll
      for (int k = 0; k < DBW; ++k) {
        const int e = 16 * (NWM * k + w) + 4 * g4;
        *reinterpret_cast<f32x4*>(a.part_o + prow * D + e) = oacc[j][k];
      }
      if (w == 0 && g4 == 0) {
        a.part_ml[prow * 2 + 0] = m;
        a.part_ml[prow * 2 + 1] = l;
      }
    }
  }
}

template <int D, int G, int NCB, bool OBF>
hipError_t launch_mc_rk(const DecodeArgs& a, hipStream_t st) {
  DecodeArgs a1 = a;
  a1.ncb = 1;  // one workgroup per unit holds every column block
  const long long n = (long long)a.B * a.Hkv * a.nchunk;
  if (n > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  if (a.n_rot <= 64)
    hipLaunchKernelGGL((decode_mc_kernel<D, G, NCB, 4, OBF>), dim3((unsigned)n), dim3(64 * NWM), 0,
                       st, a1);
  else
    hipLaunchKernelGGL((decode_mc_kernel<D, G, NCB, D / 32, OBF>), dim3((unsigned)n),
                       dim3(64 * NWM), 0, st, a1);
  return hipGetLastError();
}

template <int D, int G, bool OBF>
hipError_t launch_mc_g(const DecodeArgs& a, hipStream_t st) {
  if (a.ncb <= 2) return launch_mc_rk<D, G, 2, OBF>(a, st);
  return launch_mc_rk<D, G, 4, OBF>(a, st);
}

template <int D, bool OBF>
hipError_t launch_mc_d(const DecodeArgs& a, hipStream_t st) {
  switch (a.Hq / a.Hkv) {  // G = 1, 2 never need more than one block (q_len <= 8)
    case 4: return launch_mc_g<D, 4, OBF>(a, st);
    case 8: return launch_mc_g<D, 8, OBF>(a, st);
  }
  return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_decode_mc(const DecodeArgs& a, bool out_bf16, hipStream_t st) {
  hipError_t e;
  if (a.D == 256) e = out_bf16 ? launch_mc_d<256, true>(a, st) : launch_mc_d<256, false>(a, st);
  else if (a.D == 512) e = out_bf16 ? launch_mc_d<512, true>(a, st) : launch_mc_d<512, false>(a, st);
  else return hipErrorInvalidValue;
  if (e != hipSuccess || a.nchunk == 1) return e;  // one chunk: written in place
  return launch_decode_merge(a, out_bf16, st);
}

}  // namespace g4a
