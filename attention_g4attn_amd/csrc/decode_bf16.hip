// Decode attention (one query token per sequence) over a KV cache of raw bf16
// keys/values, split along the cache length, on the gfx950 matrix cores.
//
// What is computed: the last row of causal attention over the tokens the
// cache holds, with each cached key rotated at its own position (the cache
// keeps raw keys; with K=V the one tensor must stay raw to serve as values).
// Local layers use a ring cache of `window` slots (position t in slot
// t mod window); global layers a linear K=V cache.  Sources: "Guia visual do
// Gemma 4" (pt.news.hada.io), sections "Intercalacao de camadas de atencao",
// "GQA", "Tecnica K=V", "p-RoPE"; "Visao geral do modelo Gemma 4"
// (ai.google.dev), section "Principais Consideracoes para o planejamento de
// memoria" (the KV cache grows with every token).
//
// Split kernel: one workgroup per (b, kv head, chunk of `chunk` cache rows);
// its 4 waves take equal slices of the chunk in 32-row tiles.  Per tile a wave
//   - loads the rows straight into registers in the A-operand layout of the
//     16x16x32 product (16 rows x 8 dims per lane), rotates them, and forms
//     S^T = K~ Q~^T for the G query heads (padded to 16 columns);
//   - writes the raw rows transposed into its own LDS slice and forms
//     O^T += V^T P^T, P taken straight from the score registers;
// then the 4 waves merge through LDS and write (m, l, O) of the chunk to the
// workspace.  The merge kernel combines the chunks of every query head with
// log-sum-exp weights.  Rows the query may not see are never loaded.
#include "common.hpp"
#include "kernels.hpp"

namespace g4a {

namespace {

constexpr int DW = 4;        // waves per workgroup
constexpr int TR = 32;       // cache rows per tile

template <int D>
struct DLds {
  static constexpr int VP = TR * 2;           // transposed value row pitch (bytes)
  static constexpr int WAVE = D * VP;         // one wave's transposed tile
  static constexpr int GTAB = (D / 2) * 8;
  static constexpr int TOTAL = DW * WAVE + GTAB;
};

// Position held by cache row r, or -1 if the query may not see it.
__device__ __forceinline__ int row_position(int r, int P, int window) {
  if (window > 0) {
    const int t = P - (((P - r) % window) + window) % window;
    return t;  // negative when the ring is not yet full
  }
  return r <= P ? r : -1;
}

// Byte offset of key k (0..31) within a 64-byte row of the transposed tile:
// the 8 keys lane group q = (k & 15) >> 2 feeds are [4q .. 4q+3, 16+4q .. 16+4q+3],
// stored as one 16-byte chunk, chunk index XOR-swizzled by dim.
__device__ __forceinline__ int vt_key_off(int dim, int k) {
  const int q = (k & 15) >> 2;
  const int slot = (k & 3) + ((k >> 4) << 2);
  return dim * (TR * 2) + ((q ^ ((dim >> 1) & 3)) << 4) + (slot << 1);
}

__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

template <int D, int G, bool KVS>
__global__ void __launch_bounds__(DW * 64, 1) decode_split_kernel(DecodeArgs a) {
  constexpr int NS = D / 32;  // 32-dim k-steps of the score product
  constexpr int NB = D / 16;  // 16-dim blocks of the output
  using L = DLds<D>;
  __shared__ __attribute__((aligned(16))) unsigned char smem[L::TOTAL];

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int l16 = lane & 15, q4 = lane >> 4;
  const int ch = blockIdx.x % a.nchunk;
  const int bh = blockIdx.x / a.nchunk;
  const int b = bh / a.Hkv, hkv = bh % a.Hkv;
  const int P = a.pos[b];
  const int W = a.window, C = a.capacity;
  if (P < 0 || (W == 0 && P >= C)) return;  // the merge writes NaN rows
  const int last = W > 0 ? min(P, W - 1) : P;  // highest row index that may be visible
  const int r0 = ch * a.chunk;
  if (r0 > last) return;

  double* gtab = reinterpret_cast<double*>(smem + DW * L::WAVE);
  for (int t = tid; t < D / 2; t += DW * 64) gtab[t] = rope_rev_per_pos(t, D, a.log2_theta);
  __syncthreads();
  const int n_rot = a.n_rot;

  // query heads hkv*G .. +G-1 as B operands (columns >= G are zero)
  u32x4 qf[NS];
  {
    const int h = hkv * G + (l16 < G ? l16 : 0);
    const uint16_t* qrow = static_cast<const uint16_t*>(a.q) + ((size_t)b * a.Hq + h) * D;
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      const u32x4 x = *reinterpret_cast<const u32x4*>(qrow + 8 * (4 * s + q4));
      qf[s] = l16 < G ? x : u32x4{0, 0, 0, 0};
    }
#pragma unroll
    for (int s = 0; s < NS; ++s)
      if (16 * s < n_rot) qf[s] = rotate_chunk_bf16(qf[s], 4 * s + q4, P, n_rot, gtab);
  }

  const uint16_t* kb = static_cast<const uint16_t*>(a.k) + ((size_t)b * a.Hkv + hkv) * C * D;
  const uint16_t* vb = static_cast<const uint16_t*>(a.v) + ((size_t)b * a.Hkv + hkv) * C * D;
  unsigned char* vt = smem + w * L::WAVE;

  f32x4 oacc[NB];
#pragma unroll
  for (int i = 0; i < NB; ++i) oacc[i] = f32x4{};
  float m_run = -1e30f, l_run = 0.f;
  const float cs = a.scale_log2e;

  const int rows_per_wave = a.chunk / DW;
  const int wr0 = r0 + w * rows_per_wave;
  const int wr1 = min(wr0 + rows_per_wave, last + 1);  // exclusive
  for (int tb = wr0; tb < wr1; tb += TR) {
    // ---- load 32 rows (2 blocks of 16) in A-operand layout ----
    u32x4 kr[2][NS];
    u32x4 vr[KVS ? 1 : 2][KVS ? 1 : NS];
    int tpos[2];
    bool ok[2];
#pragma unroll
    for (int kb2 = 0; kb2 < 2; ++kb2) {
      const int r = tb + 16 * kb2 + l16;
      const int t = r < wr1 ? row_position(r, P, W) : -1;
      ok[kb2] = t >= 0;
      tpos[kb2] = t;
      const size_t ro = (size_t)(ok[kb2] ? r : wr0) * D;  // unseen rows are never read
#pragma unroll
      for (int s = 0; s < NS; ++s) {
        kr[kb2][s] = *reinterpret_cast<const u32x4*>(kb + ro + 8 * (4 * s + q4));
        if constexpr (!KVS) vr[kb2][s] = *reinterpret_cast<const u32x4*>(vb + ro + 8 * (4 * s + q4));
      }
    }
#pragma unroll
    for (int kb2 = 0; kb2 < 2; ++kb2)
#pragma unroll
      for (int s = 0; s < NS; ++s) {
        kr[kb2][s] = ok[kb2] ? kr[kb2][s] : u32x4{0, 0, 0, 0};
        if constexpr (!KVS) vr[kb2][s] = ok[kb2] ? vr[kb2][s] : u32x4{0, 0, 0, 0};
      }

    // ---- raw values, transposed, into this wave's LDS slice ----
#pragma unroll
    for (int kb2 = 0; kb2 < 2; ++kb2) {
      const int k = 16 * kb2 + l16;
#pragma unroll
      for (int s = 0; s < NS; ++s) {
        u32x4 x;
        if constexpr (KVS) x = kr[kb2][s]; else x = vr[kb2][s];
        const int d0 = 8 * (4 * s + q4);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          *reinterpret_cast<uint16_t*>(vt + vt_key_off(d0 + 2 * i, k)) = (uint16_t)(x[i] & 0xffffu);
          *reinterpret_cast<uint16_t*>(vt + vt_key_off(d0 + 2 * i + 1, k)) = (uint16_t)(x[i] >> 16);
        }
      }
    }

    // ---- scores S^T (16 rows x 16 heads) per block ----
    f32x4 sacc[2];
#pragma unroll
    for (int kb2 = 0; kb2 < 2; ++kb2) {
      sacc[kb2] = f32x4{};
#pragma unroll
      for (int s = 0; s < NS; ++s) {
        u32x4 kf = kr[kb2][s];
        if (16 * s < n_rot) kf = rotate_chunk_bf16(kf, 4 * s + q4, tpos[kb2], n_rot, gtab);
        sacc[kb2] = mfma16x16x32(kf, qf[s], sacc[kb2]);
      }
    }
    // rows (keys) of the score registers: block kb2, rows 4*q4 + i
    float mx = -INFINITY;
#pragma unroll
    for (int kb2 = 0; kb2 < 2; ++kb2)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = tb + 16 * kb2 + 4 * q4 + i;
        const bool vis = r < wr1 && row_position(r, P, W) >= 0;
        sacc[kb2][i] = vis ? sacc[kb2][i] : -INFINITY;
        mx = fmaxf(mx, sacc[kb2][i]);
      }
    mx = fmaxf(mx, __shfl_xor(mx, 16));
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    const float m_new = fmaxf(m_run, mx * cs);
    const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
    m_run = m_new;
    l_run *= alpha;
#pragma unroll
    for (int i = 0; i < NB; ++i) oacc[i] *= alpha;
    float p[2][4];
#pragma unroll
    for (int kb2 = 0; kb2 < 2; ++kb2)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        p[kb2][i] = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[kb2][i], cs, -m_run));
        l_run += p[kb2][i];
      }
    const u32x4 pf = {pack_bf16(p[0][0], p[0][1]), pack_bf16(p[0][2], p[0][3]),
                      pack_bf16(p[1][0], p[1][1]), pack_bf16(p[1][2], p[1][3])};

    wave_lds_sync();
    // ---- O^T += V^T P^T ----
#pragma unroll
    for (int db = 0; db < NB; ++db) {
      const int dim = 16 * db + l16;
      const u32x4 vf = *reinterpret_cast<const u32x4*>(
          vt + dim * (TR * 2) + ((q4 ^ ((dim >> 1) & 3)) << 4));
      oacc[db] = mfma16x16x32(vf, pf, oacc[db]);
    }
    wave_lds_sync();
  }

  // ---- merge the 4 waves of this workgroup through LDS ----
  l_run += __shfl_xor(l_run, 16);
  l_run += __shfl_xor(l_run, 32);
  __syncthreads();
  float* ow = reinterpret_cast<float*>(smem);  // [DW][G][D] then [DW][G][2]
  float* mlw = ow + DW * G * D;
  if (l16 < G) {
#pragma unroll
    for (int db = 0; db < NB; ++db)
#pragma unroll
      for (int i = 0; i < 4; ++i) ow[(w * G + l16) * D + 16 * db + 4 * q4 + i] = oacc[db][i];
    if (q4 == 0) {
      mlw[(w * G + l16) * 2 + 0] = m_run;
      mlw[(w * G + l16) * 2 + 1] = l_run;
    }
  }
  __syncthreads();
  for (int idx = tid; idx < G * D; idx += DW * 64) {
    const int h = idx / D, e = idx % D;
    float M = -INFINITY;
#pragma unroll
    for (int ww = 0; ww < DW; ++ww) M = fmaxf(M, mlw[(ww * G + h) * 2]);
    float o = 0.f, l = 0.f;
#pragma unroll
    for (int ww = 0; ww < DW; ++ww) {
      const float f = __builtin_amdgcn_exp2f(mlw[(ww * G + h) * 2] - M);
      o += f * ow[(ww * G + h) * D + e];
      l += f * mlw[(ww * G + h) * 2 + 1];
    }
    const size_t prow = ((size_t)b * a.Hq + hkv * G + h) * a.nchunk + ch;
    a.part_o[prow * D + e] = o;
    if (e == 0) {
      a.part_ml[prow * 2 + 0] = M;
      a.part_ml[prow * 2 + 1] = l;
    }
  }
}

// Combine the chunk partials of query head (b, h): weights 2^(m_c - M).
template <bool OBF>
__global__ void __launch_bounds__(256) decode_merge_kernel(DecodeArgs a) {
  const int b = blockIdx.x / a.Hq, h = blockIdx.x % a.Hq;
  const int D = a.D;
  const int P = a.pos[b];
  const size_t orow = ((size_t)b * a.Hq + h) * D;
  if (P < 0 || (a.window == 0 && P >= a.capacity)) {
    for (int e = threadIdx.x; e < D; e += 256) {
      if constexpr (OBF) static_cast<uint16_t*>(a.out)[orow + e] = 0x7fc0;
      else static_cast<float*>(a.out)[orow + e] = __builtin_nanf("");
    }
    return;
  }
  const int last = a.window > 0 ? min(P, a.window - 1) : P;
  const int nch = last / a.chunk + 1;
  const size_t prow = ((size_t)b * a.Hq + h) * a.nchunk;
  float M = -INFINITY;
  for (int c = 0; c < nch; ++c) M = fmaxf(M, a.part_ml[(prow + c) * 2]);
  for (int e = threadIdx.x; e < D; e += 256) {
    float o = 0.f, l = 0.f;
    for (int c = 0; c < nch; ++c) {
      const float f = __builtin_amdgcn_exp2f(a.part_ml[(prow + c) * 2] - M);
      o += f * a.part_o[(prow + c) * D + e];
      l += f * a.part_ml[(prow + c) * 2 + 1];
    }
    const float r = o / l;
    if constexpr (OBF) static_cast<uint16_t*>(a.out)[orow + e] = (uint16_t)(pack_bf16(r, 0.f) & 0xffffu);
    else static_cast<float*>(a.out)[orow + e] = r;
  }
}

template <int D, int G, bool KVS>
hipError_t launch_split(const DecodeArgs& a, hipStream_t st) {
  const long long n = (long long)a.B * a.Hkv * a.nchunk;
  if (n > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL((decode_split_kernel<D, G, KVS>), dim3((unsigned)n), dim3(DW * 64), 0, st, a);
  return hipGetLastError();
}

template <int D, bool KVS>
hipError_t launch_split_g(const DecodeArgs& a, hipStream_t st) {
  switch (a.Hq / a.Hkv) {
    case 1: return launch_split<D, 1, KVS>(a, st);
    case 2: return launch_split<D, 2, KVS>(a, st);
    case 4: return launch_split<D, 4, KVS>(a, st);
    case 8: return launch_split<D, 8, KVS>(a, st);
  }
  return hipErrorInvalidValue;
}

}  // namespace

int decode_chunk_rows(int D, int capacity, int window, bool f32) {
  (void)D;
  if (f32) return capacity;
  if (window > 0) return 128;  // ring: 4 chunks of a 512-slot window
  return 2048;
}

int decode_num_chunks(int D, int capacity, int window, bool f32) {
  const int ch = decode_chunk_rows(D, capacity, window, f32);
  return (capacity + ch - 1) / ch;
}

hipError_t launch_decode_bf16(const DecodeArgs& a, bool kv_shared, bool out_bf16,
                              hipStream_t st) {
  if ((long long)a.B * a.Hkv == 0) return hipSuccess;
  hipError_t e;
  if (a.D == 256) e = kv_shared ? launch_split_g<256, true>(a, st) : launch_split_g<256, false>(a, st);
  else if (a.D == 512) e = kv_shared ? launch_split_g<512, true>(a, st) : launch_split_g<512, false>(a, st);
  else return hipErrorInvalidValue;
  if (e != hipSuccess) return e;
  const long long n = (long long)a.B * a.Hq;
  if (out_bf16) hipLaunchKernelGGL(decode_merge_kernel<true>, dim3((unsigned)n), dim3(256), 0, st, a);
  else hipLaunchKernelGGL(decode_merge_kernel<false>, dim3((unsigned)n), dim3(256), 0, st, a);
  return hipGetLastError();
}

}  // namespace g4a
