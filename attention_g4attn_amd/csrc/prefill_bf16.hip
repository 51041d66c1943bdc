// Causal (sliding-window or global) prefill attention for bf16 inputs on the
// gfx950 matrix cores.
//
// What is computed: for every query row (b, i, h), softmax over the visible
// keys of the rotated scores, times the raw values (local layers: separate
// K and V; global layers: K=V, one tensor).  Sources: "Guia visual do Gemma
// 4" (pt.news.hada.io), sections "Intercalacao de camadas de atencao"
// (window / whole-sequence layers), "GQA" (query heads sharing one KV head),
// "Tecnica K=V" and "p-RoPE" (rotate only the first pairs).
//
// Work decomposition (one workgroup = 4 waves = 128 query rows):
//   - The M tile packs the G query heads of TQ = 128/G consecutive tokens that
//     share KV head hkv, so every staged KV tile feeds all G heads.  Row r of
//     the tile is token t0 + r/G, head hkv*G + r%G; wave w owns rows 32w..32w+31.
//   - KV tiles of 32 keys stream through LDS, double buffered.  Each tile is
//     read from HBM once and written to LDS twice: a score copy (pairs < n_rot
//     rotated at the key's position) and a transposed raw copy for the value
//     product; rows of both are padded by 16 bytes so the fragment reads of
//     consecutive rows fall in different banks.  For K=V both copies come
//     from the same loaded bytes.
//   - Scores are computed transposed, S^T = K~ Q~^T (32 keys x 32 rows per
//     wave), so each lane ends up owning one query row: the softmax max/sum
//     need one exchange with lane l^32 and the rescale of the output is a
//     per-lane scalar.  P goes straight from the score registers into the
//     B operand of O^T += V^T P^T.
//   - Online softmax in fp32 (base 2, scale folded with log2 e); the output is
//     only rescaled when the running max grows by more than 2^8.
//   - Tiles wholly outside a wave's causal band are skipped; only edge tiles
//     are masked.
//   - Grid order: KV heads fastest, then query tiles from the longest causal
//     row down, so the 8 XCDs each stream one KV head's tiles in step.
#include "common.hpp"
#include "kernels.hpp"

namespace g4a {

namespace {

constexpr int NW = 4;    // waves per workgroup
constexpr int RW = 32;   // query rows per wave
constexpr int BN = 32;   // keys per KV tile

template <int D>
struct PLds {
  static constexpr int KP = 2 * D + 16;  // score copy row pitch (bytes), padded
  static constexpr int VP = 2 * BN + 16; // value copy row pitch (bytes), padded
  static constexpr int KS = BN * KP;     // score copy  [BN][D] bf16
  static constexpr int VT = D * VP;      // value copy  [D][BN] bf16 (transposed)
  static constexpr int STAGE = KS + VT;
  static constexpr int GTAB = (D / 2) * 8;
  static constexpr int TOTAL = 2 * STAGE + GTAB;
};

// Byte offset of the dword holding keys (j, j+1), j even, in a row of the
// transposed value copy.  Within each 16-key group the keys are stored in the
// order 0-3, 8-11 | 4-7, 12-15, which is the key order the score registers of
// lanes 0-31 | 32-63 hold, so P feeds the value product without a shuffle.
__device__ __forceinline__ int vt_slot_off(int j) {
  const int jj = j & 15;
  const int lc = ((j >> 4) << 1) | ((jj >> 2) & 1);
  const int slot = ((jj >> 3) << 2) | (jj & 3);
  return (lc << 4) + ((slot >> 1) << 2);
}

template <int D, int G, bool KVS, bool OBF>
__global__ void __launch_bounds__(NW * 64, 1) prefill_bf16_kernel(PrefillArgs a) {
  constexpr int M = NW * RW;
  constexpr int TQ = M / G;
  constexpr int NDS = D / 16;   // k-steps of the score product
  constexpr int NDB = D / 32;   // 32-dim blocks of the output
  constexpr int UPT = D / 128;  // staging units (2 keys x 16 B) per thread
  using L = PLds<D>;
  __shared__ __attribute__((aligned(16))) unsigned char smem[L::TOTAL];

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int l32 = lane & 31, hl = lane >> 5;
  const int S = a.S;

  const int hb = blockIdx.x % a.nheads;
  const int qt = a.nq - 1 - blockIdx.x / a.nheads;
  const int b = hb / a.Hkv, hkv = hb % a.Hkv;
  const int t0 = qt * TQ;
  const int t_end = min(t0 + TQ, S);

  double* gtab = reinterpret_cast<double*>(smem + 2 * L::STAGE);
  for (int t = tid; t < D / 2; t += NW * 64) gtab[t] = rope_rev_per_pos(t, D, a.log2_theta);
  __syncthreads();

  // ---- this lane's query row, rotated, as B operands of S^T = K~ Q~^T ----
  const int row = w * RW + l32;
  const int tq = t0 + row / G;
  const int hq = hkv * G + row % G;
  const bool row_ok = tq < S;
  const int n_rot = a.n_rot;
  u32x4 qf[NDS];
  {
    const int tqc = row_ok ? tq : S - 1;  // rows past the end read a valid row, zeroed below
    const int qpos = a.pos[(size_t)b * S + tqc];
    const uint16_t* qrow = static_cast<const uint16_t*>(a.q) + (((size_t)b * S + tqc) * a.Hq + hq) * D;
#pragma unroll
    for (int s = 0; s < NDS; ++s) {
      const u32x4 x = *reinterpret_cast<const u32x4*>(qrow + 8 * (2 * s + hl));
      qf[s] = row_ok ? x : u32x4{0, 0, 0, 0};
    }
#pragma unroll
    for (int s = 0; s < NDS; ++s)
      if (8 * s < n_rot)  // wave-uniform: chunk 2s holds pairs 8s .. 8s+3
        qf[s] = rotate_chunk_bf16(qf[s], 2 * s + hl, qpos, n_rot, gtab);
  }

  // rows of this wave, as tokens
  const int tw0 = t0 + (w * RW) / G;
  const int tw1 = min(t0 + (w * RW + RW - 1) / G, S - 1);
  const bool wave_ok = tw0 < S;
  const int W = a.window;

  const int klo = W > 0 ? max(0, t0 - W + 1) : 0;
  const int kt0 = klo / BN, kt1 = (t_end - 1) / BN;

  // ---- staging: thread owns dim chunks c = 16m + c16 of keys 2kp, 2kp+1 ----
  const int c16 = tid & 15, kp = tid >> 4;
  const uint16_t* kbase = static_cast<const uint16_t*>(a.k) + ((size_t)b * S * a.Hkv + hkv) * D;
  const uint16_t* vbase = static_cast<const uint16_t*>(a.v) + ((size_t)b * S * a.Hkv + hkv) * D;
  const size_t kstride = (size_t)a.Hkv * D;
  u32x4 kst[UPT][2];
  u32x4 vst[KVS ? 1 : UPT][2];

  // keys past the end of the sequence are staged as zeros (their scores are
  // masked; zero values keep 0 * V finite)
  auto load_tile = [&](int kt) {
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      const int j = kt * BN + 2 * kp + e;
      const size_t jr = (size_t)min(j, S - 1) * kstride;
#pragma unroll
      for (int m = 0; m < UPT; ++m) {
        const int c = 16 * m + c16;
        kst[m][e] = *reinterpret_cast<const u32x4*>(kbase + jr + 8 * c);
        if constexpr (!KVS) vst[m][e] = *reinterpret_cast<const u32x4*>(vbase + jr + 8 * c);
      }
    }
  };
  auto zero_tail = [&](int kt) {
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      const bool ok = kt * BN + 2 * kp + e < S;
#pragma unroll
      for (int m = 0; m < UPT; ++m) {
        kst[m][e] = ok ? kst[m][e] : u32x4{0, 0, 0, 0};
        if constexpr (!KVS) vst[m][e] = ok ? vst[m][e] : u32x4{0, 0, 0, 0};
      }
    }
  };

  auto store_tile = [&](int kt, int stage) {
    unsigned char* ks = smem + stage * L::STAGE;
    unsigned char* vt = ks + L::KS;
    const int j0 = 2 * kp;
    if (kt * BN + BN > S) zero_tail(kt);
    int kpos[2];
#pragma unroll
    for (int e = 0; e < 2; ++e) kpos[e] = a.pos[(size_t)b * S + min(kt * BN + j0 + e, S - 1)];
#pragma unroll
    for (int m = 0; m < UPT; ++m) {
      const int c = 16 * m + c16;
#pragma unroll
      for (int e = 0; e < 2; ++e) {
        u32x4 r = kst[m][e];
        if (64 * m < n_rot)  // wave-uniform: chunks 16m .. 16m+15 hold pairs 64m ..
          r = rotate_chunk_bf16(r, c, kpos[e], n_rot, gtab);
        *reinterpret_cast<u32x4*>(ks + (j0 + e) * L::KP + 16 * c) = r;
      }
      u32x4 v0, v1;
      if constexpr (KVS) {
        v0 = kst[m][0];
        v1 = kst[m][1];
      } else {
        v0 = vst[m][0];
        v1 = vst[m][1];
      }
      unsigned char* vrow = vt + (8 * c) * L::VP + vt_slot_off(j0);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const uint32_t lo = (v0[i] & 0xffffu) | (v1[i] << 16);
        const uint32_t hi = (v0[i] >> 16) | (v1[i] & 0xffff0000u);
        *reinterpret_cast<uint32_t*>(vrow + (2 * i) * L::VP) = lo;
        *reinterpret_cast<uint32_t*>(vrow + (2 * i + 1) * L::VP) = hi;
      }
    }
  };

  f32x16 oacc[NDB];
#pragma unroll
  for (int i = 0; i < NDB; ++i) oacc[i] = f32x16{};
  float m_run = -1e30f, l_run = 0.f;
  const float cs = a.scale_log2e;

  auto compute = [&](int kt, int stage) {
    const int kv0 = kt * BN;
    if (!wave_ok || kv0 > tw1) return;
    if (W > 0 && kv0 + BN - 1 <= tw0 - W) return;
    const unsigned char* ks = smem + stage * L::STAGE + l32 * L::KP + 16 * hl;
    const unsigned char* vt = smem + stage * L::STAGE + L::KS + l32 * L::VP + 16 * hl;

    // S^T = K~ Q~^T: fragments stream from LDS in groups of 4, one group ahead
    f32x16 sacc = f32x16{};
    {
      constexpr int NG = NDS / 4;
      u32x4 kf[2][4];
#pragma unroll
      for (int i = 0; i < 4; ++i) kf[0][i] = *reinterpret_cast<const u32x4*>(ks + 32 * i);
#pragma unroll
      for (int g = 0; g < NG; ++g) {
        if (g + 1 < NG) {
#pragma unroll
          for (int i = 0; i < 4; ++i)
            kf[(g + 1) & 1][i] = *reinterpret_cast<const u32x4*>(ks + 32 * (4 * (g + 1) + i));
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) sacc = mfma32x32x16(kf[g & 1][i], qf[4 * g + i], sacc);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    const bool need_mask = (kv0 + BN - 1 > tw0) || (W > 0 && kv0 <= tw1 - W);
    if (need_mask) {  // wave-uniform
      const int lo = W > 0 ? tq - W + 1 : 0;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int j = kv0 + 8 * (r >> 2) + 4 * hl + (r & 3);
        sacc[r] = (j <= tq && j >= lo) ? sacc[r] : -INFINITY;
      }
    }
    float mx = sacc[0];
#pragma unroll
    for (int r = 1; r < 16; ++r) mx = fmaxf(mx, sacc[r]);
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    const float m_tile = mx * cs;
    if (__any(m_tile > m_run + 8.f)) {
      const float m_new = fmaxf(m_run, m_tile);
      const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
      l_run *= alpha;
#pragma unroll
      for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) oacc[db][r] *= alpha;
      m_run = m_new;
    }
    u32x4 pf[2];
    float lsum = 0.f;
#pragma unroll
    for (int k2 = 0; k2 < 2; ++k2)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float p0 = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[8 * k2 + 2 * i], cs, -m_run));
        const float p1 =
            __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[8 * k2 + 2 * i + 1], cs, -m_run));
        lsum += p0 + p1;
        pf[k2][i] = pack_bf16(p0, p1);
      }
    l_run += lsum;
    __builtin_amdgcn_sched_barrier(0);

    // O^T += V^T P^T: 2 fragments per 32-dim block, two blocks per group
    {
      constexpr int NG = NDB / 2;
      u32x4 vf[2][4];
#pragma unroll
      for (int i = 0; i < 4; ++i)
        vf[0][i] = *reinterpret_cast<const u32x4*>(vt + (i >> 1) * 32 * L::VP + 32 * (i & 1));
#pragma unroll
      for (int g = 0; g < NG; ++g) {
        if (g + 1 < NG) {
#pragma unroll
          for (int i = 0; i < 4; ++i)
            vf[(g + 1) & 1][i] = *reinterpret_cast<const u32x4*>(
                vt + (2 * (g + 1) + (i >> 1)) * 32 * L::VP + 32 * (i & 1));
        }
#pragma unroll
        for (int i = 0; i < 4; ++i)
          oacc[2 * g + (i >> 1)] = mfma32x32x16(vf[g & 1][i], pf[i & 1], oacc[2 * g + (i >> 1)]);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  };

  // ---- KV loop, double buffered ----
  load_tile(kt0);
  store_tile(kt0, 0);
  __syncthreads();
  for (int kt = kt0; kt <= kt1; ++kt) {
    const int stage = (kt - kt0) & 1;
    if (kt < kt1) load_tile(kt + 1);
    compute(kt, stage);
    if (kt < kt1) store_tile(kt + 1, stage ^ 1);
    __syncthreads();
  }

  // ---- epilogue: O / l ----
  const float lt = l_run + __shfl_xor(l_run, 32);
  if (row_ok) {
    const float inv = 1.f / lt;
    const size_t obase = (((size_t)b * S + tq) * a.Hq + hq) * D;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        const int dim = 32 * db + 8 * g4 + 4 * hl;
        const float o0 = oacc[db][4 * g4 + 0] * inv, o1 = oacc[db][4 * g4 + 1] * inv;
        const float o2 = oacc[db][4 * g4 + 2] * inv, o3 = oacc[db][4 * g4 + 3] * inv;
        if constexpr (OBF) {
          u32x2 pk = {pack_bf16(o0, o1), pack_bf16(o2, o3)};
          *reinterpret_cast<u32x2*>(static_cast<uint16_t*>(a.out) + obase + dim) = pk;
        } else {
          *reinterpret_cast<f32x4*>(static_cast<float*>(a.out) + obase + dim) =
              f32x4{o0, o1, o2, o3};
        }
      }
  }
}

template <int D, int G, bool KVS, bool OBF>
hipError_t launch_one(const PrefillArgs& a, hipStream_t st) {
  constexpr int TQ = NW * RW / G;
  PrefillArgs x = a;
  x.nq = (a.S + TQ - 1) / TQ;
  x.nheads = a.B * a.Hkv;
  const long long nblk = (long long)x.nq * x.nheads;
  if (nblk == 0) return hipSuccess;
  if (nblk > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL((prefill_bf16_kernel<D, G, KVS, OBF>), dim3((unsigned)nblk), dim3(NW * 64),
                     0, st, x);
  return hipGetLastError();
}

template <int D, bool KVS, bool OBF>
hipError_t launch_g(const PrefillArgs& a, int G, hipStream_t st) {
  switch (G) {
    case 1: return launch_one<D, 1, KVS, OBF>(a, st);
    case 2: return launch_one<D, 2, KVS, OBF>(a, st);
    case 4: return launch_one<D, 4, KVS, OBF>(a, st);
    case 8: return launch_one<D, 8, KVS, OBF>(a, st);
  }
  return hipErrorInvalidValue;
}

template <bool KVS, bool OBF>
hipError_t launch_d(const PrefillArgs& a, int G, hipStream_t st) {
  if (a.D == 256) return launch_g<256, KVS, OBF>(a, G, st);
  if (a.D == 512) return launch_g<512, KVS, OBF>(a, G, st);
  return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_prefill_bf16(const PrefillArgs& a, bool kv_shared, bool out_bf16,
                               hipStream_t st) {
  const int G = a.Hq / a.Hkv;
  if (kv_shared) return out_bf16 ? launch_d<true, true>(a, G, st) : launch_d<true, false>(a, G, st);
  return out_bf16 ? launch_d<false, true>(a, G, st) : launch_d<false, false>(a, G, st);
}

}  // namespace g4a
