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
// Work decomposition: one workgroup per (sequence, KV head, chunk of 1024
// cache rows), numbered densely over the chunks with a visible row as in the
// split kernel, with one wave per 16-column block.  The waves share the
// chunk's 16-row tiles, which stream from HBM into a ring of NSL LDS slots
// (16-byte direct-to-LDS loads, each wave issuing its share of a tile); apart
// from that every wave works alone, as a wave of the split kernel does on its
// block: S^T = K~ Q~^T over the whole head (keys rotated at their positions),
// the softmax of its 16 columns, and O^T += V^T P^T over every output dim.
// One barrier per tile: after it, tile i+1 is in LDS and the slot of tile i
// is free for tile i+NSL.
//
// The head dims could be split over the waves instead (each wave a quarter
// of the k-steps and output dims of every block, partial scores summed
// through LDS), which needs three barriers per tile with the softmax of each
// block on one wave between two of them: with shader-clock stamps a tile took
// about 4800 cycles that way (scores 1150, softmax 1360, values 930, the rest
// barriers and load issue), and 64 sequences of 4 draft tokens at G = 8,
// D = 512 took 1200 us.
//
// With 2 blocks (17 to 32 columns) a workgroup is 2 waves with a 2-slot ring,
// four workgroups per CU; with 3 or 4 blocks, 4 waves with a 4-slot ring, two
// per CU.  Either way a CU holds 8 waves and 8 tile slots, as the split
// kernel does for one block.
#include "common.hpp"
#include "decode_common.hpp"
#include "kernels.hpp"

namespace g4a {

namespace {

using namespace dec;

constexpr int TRM = 16;  // cache rows per tile

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

// 16-byte chunk swizzle of tile row r, the split kernel's: a bijection on
// r % 16; a score read (16 lanes = 16 rows, one chunk) and a transpose read
// (32 lanes = 8 rows x 2 adjacent chunks) each hit 16 bank groups.
__device__ __forceinline__ int mswz(int r) { return ((r & 7) << 1) | ((r >> 3) & 1); }

// NCB = column blocks (= waves) of the instance, NSL = LDS tile slots; RK =
// score k-steps that may hold turning pairs (4 when n_rot <= 64, else all).
//
// Key rotation.  Every block's scores need the same rotated keys, and the
// rotation (an fp64 angle reduction and a hardware sine and cosine per pair)
// costs more than the score products: timed without it, the 4-token decode
// above ran in 950 instead of 1135 us.  With RK = 4 (p-RoPE at p <= 0.25:
// dims below 128) the waves therefore rotate the tile once between them,
// each the rows of its own share, into an LDS copy of those 128 dims, and a
// second barrier per tile publishes it.  With every dim turning (RK = NS)
// that copy would be a second tile; each wave rotates what it reads.
template <int D, int G, int NCB, int NSL, int RK, bool OBF>
__global__ void __launch_bounds__(64 * NCB) __attribute__((amdgpu_waves_per_eu(2, 2)))
decode_mc_kernel(DecodeArgs a) {
  constexpr int NS = D / 32;       // score k-steps
  constexpr int NB = D / 16;       // output dim blocks
  constexpr int KB = TRM * D * 2;  // one tile, bytes
  constexpr int NLD = KB / 1024;   // direct loads per tile
  constexpr int NLW = NLD / NCB;   // per wave
  static_assert(G <= 8 && NCB <= 4 && RK <= NS && NLD % NCB == 0 && NSL >= 2, "shape");
  constexpr bool COOP = RK == 4;                    // rotate the tile once, together
  constexpr int RW = TRM / NCB;                     // rows of a wave's share
  static_assert(!COOP || (RW * 16) % 64 == 0, "rotation share");
  __shared__ __attribute__((aligned(16))) unsigned char ring[NSL * KB];  // tile i in slot i % NSL
  __shared__ __attribute__((aligned(16))) unsigned char rotk[COOP ? TRM * 256 : 16];  // dims < 128, rotated
  __shared__ double gtab[COOP ? 64 : D / 2];

  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // = column block
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
        nan_columns<D, NCB, OBF>(a, ncol_of(j), [&](int n) { return col_out(j, n); });
    return;
  }
  const int last = W > 0 ? min(P, C - 1) : P;
  const int r0 = ch * a.chunk;
  if (r0 > last) return;
  const int r1 = min(r0 + a.chunk, last + 1);
  const int nt = (r1 - r0 + TRM - 1) / TRM;
  const int n_rot = a.n_rot;
  const bool active = w < ncb;  // wave-uniform: this block has columns
  const bool col_ok = l16 < ncol_of(w);
  const int Pq = col_ok ? col_pos(w, l16) : 0;  // this lane's column position

  // the block's queries as B operands of the score product (columns past the
  // block's last are zero)
  u32x4 qf[NS];
  {
    const uint16_t* qrow =
        static_cast<const uint16_t*>(a.q) + (col_ok ? col_out(w, l16) : col_out(0, 0));
#pragma unroll
    for (int s = 0; s < NS; ++s) qf[s] = *reinterpret_cast<const u32x4*>(qrow + 8 * (4 * s + g4));
  }
  const size_t hoff = ((size_t)b * a.Hkv + hkv) * C * D;
  const uint16_t* kbase = static_cast<const uint16_t*>(a.k) + hoff;
  // this wave's share of tile i's rows into a slot (past the last tile: the
  // last tile again); rows past r1 read as zeros; every cache row is read
  // once by the launch: non-temporal
  auto issue = [&](int i, unsigned char* dst) {
    const int rr0 = r0 + min(i, nt - 1) * TRM;
    const uint32_t bytes = (uint32_t)min(TRM, r1 - rr0) * (2 * D);
    const s32x4 rs = rsrc_words(kbase + (size_t)rr0 * D, bytes);
    constexpr int CPR = D / 8;     // chunks per row
    constexpr int RPI = 64 / CPR;  // rows per direct load
    int ln = lane;
    asm volatile("" : "+v"(ln));
#pragma unroll
    for (int m = 0; m < NLW; ++m) {
      const int n = NLW * w + m;
      const int row = n * RPI + ln / CPR;
      const uint32_t voff = (uint32_t)row * (2 * D) + ((uint32_t)((ln % CPR) ^ mswz(row)) << 4);
      lds_dma16_nt_asm(rs, voff, dst + n * 1024);
    }
  };
  for (int t = threadIdx.x; t < (COOP ? 64 : D / 2); t += 64 * NCB)
    gtab[t] = rope_rev_per_pos(t, D, a.log2_theta);
  __syncthreads();
  // tiles 0 .. NSL-2 in flight before the queries are rotated (all NSL-1
  // issued, so the wait below counts them whatever nt is)
#pragma unroll
  for (int t = 0; t < NSL - 1; ++t) issue(t, ring + t * KB);
#pragma unroll
  for (int s = 0; s < NS; ++s) {
    qf[s] = col_ok ? qf[s] : u32x4{0, 0, 0, 0};
    if (s < RK) qf[s] = rotate_chunk_bf16(qf[s], 4 * s + g4, Pq, n_rot, gtab);
  }

  f32x4 oacc[NB];
#pragma unroll
  for (int i = 0; i < NB; ++i) oacc[i] = f32x4{};
  float m_run = -INFINITY, l_run = 0.f;  // per column (l16), base 2
  const float cs = a.scale_log2e;

  // S^T of tile i (register j = key 4*gq + j of column l16), the softmax
  // update, and O^T += V^T P^T, from the tile in LDS at kt
  auto compute = [&](int i, const unsigned char* kt) {
    int ln = lane;
    asm volatile("" : "+v"(ln));
    const int row = ln & 15, gq = ln >> 4;
    f32x4 sacc;
    {
      const int r = min(r0 + i * TRM + row, r1 - 1);  // rows past the tile end are masked
      const int tpos = W > 0 ? P - (P - r) % C : r;
      (void)tpos;
      const int dsw = mswz(row);
      f32x4 s0 = {}, s1 = {};  // even / odd k-steps: two independent chains
#pragma unroll
      for (int s = 0; s < NS; ++s) {
        const int c = 4 * s + gq;  // chunk of the row
        u32x4 kf;
        if (COOP && s < 4) {  // chunk c < 16: from the rotated copy
          kf = *reinterpret_cast<const u32x4*>(rotk + row * 256 + ((c ^ dsw) << 4));
        } else {
          kf = *reinterpret_cast<const u32x4*>(kt + row * (2 * D) + 256 * (c >> 4) +
                                              (((c & 15) ^ dsw) << 4));
          if (!COOP && s < RK) kf = rotate_chunk_bf16(kf, c, tpos, n_rot, gtab);
        }
        if (s & 1) s1 = mfma16x16x32(kf, qf[s], s1);
        else s0 = mfma16x16x32(kf, qf[s], s0);
      }
      sacc = s0 + s1;
    }
    u32x2 pf;
    {
      const int nrows = min(TRM, r1 - (r0 + i * TRM));
#pragma unroll
      for (int j = 0; j < 4; ++j) sacc[j] = 4 * gq + j < nrows ? sacc[j] : -INFINITY;
      // each column sees keys up to its own position (in a ring, only the
      // window before it)
      const int rk = r0 + i * TRM + 4 * gq;     // this lane's first key row
      const int m0 = W > 0 ? (P - rk) % C : 0;  // (P - row) mod C of that row
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int mj = m0 - j;
        const int tp = W > 0 ? P - (mj >= 0 ? mj : mj + C) : rk + j;  // key position
        const bool vis = tp <= Pq && (W == 0 || tp > Pq - W);
        sacc[j] = vis ? sacc[j] : -INFINITY;
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
      // V^T by transpose reads: source lane (gq, row) addresses tile row
      // 4*gq + row/4, dims 16*db + 4*(row%4) .. +3 (chunk 2*db + (row%4)/2)
      const int trow = 4 * gq + (row >> 2);
      const int tch = (row & 3) >> 1;
      const int tdsw = mswz(trow);
      const unsigned char* vb = kt + trow * (2 * D) + (row & 1) * 8;
#pragma unroll
      for (int db = 0; db < NB; ++db) {
        const int c = 2 * db + tch;
        const u32x2 vf = lds_read_tr16(vb + 256 * (c >> 4) + (((c & 15) ^ tdsw) << 4));
        oacc[db] = mfma16x16x16(vf, pf, oacc[db]);
      }
    }
  };

  // the first 128 dims of this wave's rows of tile i, rotated at their
  // positions, into rotk (same row swizzle as the tile); rows past r1 are
  // zeros and stay zeros
  auto rotate_share = [&](int i, const unsigned char* kt) {
#pragma unroll
    for (int m = 0; m < RW * 16 / 64; ++m) {
      const int idx = 64 * m + lane;
      const int row = RW * w + idx / 16, c = idx % 16;
      const int r = min(r0 + i * TRM + row, r1 - 1);
      const int tpos = W > 0 ? P - (P - r) % C : r;
      const int sw = (c ^ mswz(row)) << 4;
      const u32x4 kf = *reinterpret_cast<const u32x4*>(kt + row * (2 * D) + sw);
      *reinterpret_cast<u32x4*>(rotk + row * 256 + sw) = rotate_chunk_bf16(kf, c, tpos, n_rot, gtab);
    }
  };

  wait_vmcnt<(NSL - 2) * NLW>();  // this wave's share of tile 0
  lds_barrier();
  for (int i = 0; i < nt; ++i) {
    // tile i+NSL-1 goes into the slot tile i-1 used (every wave passed the
    // barrier that ended step i-1)
    const bool more = i + NSL - 1 < nt;
    if (more) issue(i + NSL - 1, ring + ((i + NSL - 1) % NSL) * KB);
    if constexpr (COOP) {  // rotk was last read in step i-1, before its end barrier
      rotate_share(i, ring + (i % NSL) * KB);
      lds_barrier();
    }
    if (active) compute(i, ring + (i % NSL) * KB);
    // tile i+1 must have landed in every wave's share before the next step;
    // this wave's loads of tiles i+2 .. i+NSL-1 may still run
    if (more) wait_vmcnt<(NSL - 2) * NLW>();
    else wait_vmcnt<0>();
    lds_barrier();
  }
  if (!active) return;

  // ---- the chunk's (m, l, O) for this block's columns ----
  l_run += __shfl_xor(l_run, 16);
  l_run += __shfl_xor(l_run, 32);
  if (!col_ok) return;
  if (direct) {
    // every column sees its own key unless its position is negative
    const bool ok = Pq >= 0;
    const float inv = 1.f / l_run;
    const size_t orow = col_out(w, l16);
#pragma unroll
    for (int db = 0; db < NB; ++db) {
      const int e = 16 * db + 4 * g4;
      const f32x4 o = ok ? oacc[db] * inv
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
    const size_t prow = (col_out(w, l16) / D) * a.nchunk + ch;
    float* po = a.part_o + prow * D + 4 * g4;
#pragma unroll
    for (int db = 0; db < NB; ++db) *reinterpret_cast<f32x4*>(po + 16 * db) = oacc[db];
    if (g4 == 0) {
      a.part_ml[prow * 2 + 0] = m_run;
      a.part_ml[prow * 2 + 1] = l_run;
    }
  }
}

template <int D, int G, int NCB, int NSL, bool OBF>
hipError_t launch_mc_rk(const DecodeArgs& a, hipStream_t st) {
  DecodeArgs a1 = a;
  a1.ncb = 1;  // one workgroup per unit holds every column block
  const long long n = (long long)a.B * a.Hkv * a.nchunk;
  if (n > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  if (a.n_rot <= 64)
    hipLaunchKernelGGL((decode_mc_kernel<D, G, NCB, NSL, 4, OBF>), dim3((unsigned)n),
                       dim3(64 * NCB), 0, st, a1);
  else
    hipLaunchKernelGGL((decode_mc_kernel<D, G, NCB, NSL, D / 32, OBF>), dim3((unsigned)n),
                       dim3(64 * NCB), 0, st, a1);
  return hipGetLastError();
}

template <int D, int G, bool OBF>
hipError_t launch_mc_g(const DecodeArgs& a, hipStream_t st) {
  if (a.ncb <= 2) return launch_mc_rk<D, G, 2, 2, OBF>(a, st);
  return launch_mc_rk<D, G, 4, 4, OBF>(a, st);
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
