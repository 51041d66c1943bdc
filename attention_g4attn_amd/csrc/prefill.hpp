// Causal (sliding-window or global) prefill attention for bf16 inputs on the
// gfx950 matrix cores.
//
// What is computed: for every query row (b, i, h), the softmax over the
// visible keys of the rotated scores, times the raw values.  Local layers:
// separate K and V, window W, full rotation.  Global layers: K=V (one tensor
// is rotated for the scores and read raw as the values) with only the first
// n_rot pairs rotated (p-RoPE).  Sources: "Guia visual do Gemma 4"
// (pt.news.hada.io), sections "Intercalacao de camadas de atencao", "GQA",
// "Tecnica K=V" and "p-RoPE".
//
// Work decomposition: one workgroup = 4 waves = M = 128*MB query rows.
//   - The M tile packs the G query heads of TQ = M/G consecutive tokens that
//     share one KV head, so every staged KV tile feeds all G heads.  Row r is
//     token t0 + r/G, head hkv*G + r%G; wave w owns rows RW*w .. RW*w+RW-1,
//     as MB blocks of 32 that share every K/V fragment read from LDS.
//   - Keys are rotated once, before the attention kernel, by a pass that
//     writes the first SW dims of every key, rotated, into a workspace slab
//     (SW = 128 when only pairs < 64 turn, as for p-RoPE at d = 512; else d).
//     Queries are rotated in registers when the workgroup loads them.
//   - KV tiles of 32 keys (slab rows, plus the raw rows the scores or values
//     still need) stream from HBM straight into an NST-deep LDS ring (16-byte
//     direct-to-LDS loads, no staging registers), requested two tiles ahead
//     when NST = 3.  Rows are stored with 16-byte chunks XOR-swizzled by row
//     so both read patterns below are free of bank conflicts.
//   - Scores are computed transposed, S^T = K~ Q~^T, so each lane owns one
//     query row per block: the softmax needs one exchange with lane l^32 and
//     the row statistics are per-lane scalars; P goes from the score registers
//     straight into the B operand of O^T += V^T P^T.
//   - The value operand V^T is read from the raw row-major tile with the LDS
//     transpose read (ds_read_b64_tr_b16): 4 consecutive keys of one dim per
//     lane per read.  For K=V this is the same raw tile the scores read.
//   - Softmax in fp32 (base 2, scale folded with log2 e) against a reference
//     max fixed at the first tile a row sees, so O is never rescaled; a row
//     whose scores later exceed that reference by 2^64 is recomputed exactly.
//   - A wave skips tiles none of its rows can see; only edge tiles are
//     masked.  Grid order: KV heads fastest, then query tiles from the longest
//     causal row down, so each XCD streams one KV head's tiles in step.
//   - VIS instances compute the vision encoder's attention instead: 2D RoPE
//     (half c of the head dims is a RoPE of dim d/2 driven by component c of
//     the patch position (w, h)) and no causal mask, every patch of an image
//     seeing the image's first lengths[b] patches ("Guia visual do Gemma 4",
//     sections "Encoder de visao" and "Suporte a proporcao variavel").
#pragma once
#include <type_traits>

#include "common.hpp"
#include "kernels.hpp"

namespace g4a {
namespace pf {

constexpr int NW = 4;   // waves per workgroup
constexpr int BN = 32;  // keys per KV tile
constexpr int FG = 2;   // LDS fragments per software-pipelined group

// 16-byte chunk swizzle of row r: chunk c of the row is stored at chunk
// c ^ swz(r).  The 64 LDS banks of gfx950 span 256 bytes (16 chunks), and a
// 16-byte read is served 16 lanes at a time, an 8-byte read 32 lanes at a time.
// swz is a bit swap of r % 16, so (a) one chunk of 16 consecutive rows lands on
// 16 different bank groups (score operand: lane = key row), and (b) 4
// consecutive rows (r % 4 == 0) put 4 aligned adjacent chunks into 16 different
// bank groups (value operand: transpose reads, 4 rows x 4 chunks per 32 lanes).
__device__ __forceinline__ int swz(int r) { return ((r & 3) << 2) | ((r >> 2) & 3); }

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

// Score products with the accumulator in VGPRs.  The compiler puts every MFMA
// result of a kernel in AGPRs once the output accumulators need them, and the
// 16 score registers then push an output block out of the AGPRs on every
// tile.  Written as instructions, the score chain keeps its accumulator in
// VGPRs, where the softmax reads it directly.  A dependent chain needs no
// wait states between its products; a VALU read of the result needs 12 on
// gfx950 (the compiler's own figure for this product), given by score_ready.
__device__ __forceinline__ void score_first(f32x16& c, u32x4 a, u32x4 b) {
  asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, 0" : "=&v"(c) : "v"(a), "v"(b));
}
__device__ __forceinline__ void score_next(f32x16& c, u32x4 a, u32x4 b) {
  asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+v"(c) : "v"(a), "v"(b));
}
__device__ __forceinline__ void score_ready(f32x16& c) {
  asm volatile("s_nop 7\n\ts_nop 7" : "+v"(c));
}

// max of x over lanes l and l ^ 32, in registers (v_permlane32_swap exchanges
// the upper half of one operand with the lower half of the other)
__device__ __forceinline__ float max_xor32(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

__device__ __forceinline__ u32x2 lds_read_tr16(const unsigned char* p) {
  const s16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(p));
  return __builtin_bit_cast(u32x2, v);
}

// Buffer resource over [base, base + bytes): loads past the end return zeros.
// base and bytes must be the same in every lane; they are moved to scalar
// registers explicitly so the loads need no per-lane loop.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  const uint64_t p = reinterpret_cast<uint64_t>(base);
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)p);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(p >> 32));
  const uint32_t n = __builtin_amdgcn_readfirstlane(bytes);
  void* u = reinterpret_cast<void*>(((uint64_t)hi << 32) | lo);
  return __builtin_amdgcn_make_buffer_rsrc(u, (short)0, (int)n, 0x00020000);
}

// Direct load into LDS: each lane's `size` bytes at rsrc + voff land at
// ldst + lane * size (ldst wave-uniform).
__device__ __forceinline__ void lds_dma16(__amdgpu_buffer_rsrc_t rs, uint32_t voff,
                                          uint32_t soff, unsigned char* ldst) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (__attribute__((address_space(3))) void*)(ldst),
                                           16, voff, soff, 0, 0);
}

// wait until at most n vector-memory operations of this wave are in flight
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// LDS layout.  Every ring stage is its own __shared__ object, so the compiler
// can tell the stage being read from the stages the direct loads are filling
// and does not wait for those loads before reading.  A stage holds one KV tile:
//   [slab]  the first SW dims of the 32 keys, already rotated (from the
//           workspace written by rope_keys_kernel), BN x SW bf16;
//   [raw K] the raw key rows (K=V: the one tensor, read raw as the values),
//           needed when SW < D (score dims >= SW) or for K=V;
//   [raw V] the raw value rows when K and V are separate.
template <int D, bool KVS, int SW, int NST>
struct Lds {
  static constexpr int RAW = BN * D * 2;    // one raw tile, bytes
  static constexpr int SLAB = BN * SW * 2;  // one rotated slab tile
  static constexpr int NRAW = KVS ? 1 : (SW < D ? 2 : 1);
  static constexpr int KOFF = SLAB;                                     // raw K rows
  static constexpr int VOFF = KVS ? SLAB : (SW < D ? SLAB + RAW : SLAB);  // raw V rows
  static constexpr int STAGE = SLAB + NRAW * RAW;
  static constexpr int NLD = STAGE / (1024 * NW);  // direct loads per lane per tile
  static constexpr int TOTAL = NST * STAGE;  // the angle table lives in the last stage
  static_assert(STAGE >= (D / 2) * 8, "angle table fits one stage");
};

template <int N>
using IC = std::integral_constant<int, N>;

// Workgroups per CU the instance is built for.  The d = 256 instance with one
// 32-row block per wave and a 2-stage ring fits two: 64 KiB of LDS, and at
// most 256 registers per wave once the per-lane LDS offsets are recomputed
// per tile, so each SIMD runs two waves and one wave's softmax overlaps the
// other's products.  The others hold 256 + 256 registers per wave (the
// output accumulators of 32*MB rows of d dims and the query operands).
template <int D, int MB, int NST>
constexpr int wg_per_cu() {
  return (D == 256 && MB == 1 && NST == 2) ? 2 : 1;
}

template <class T>
__device__ __forceinline__ T& lds_at(unsigned char* base, int off) {
  return *reinterpret_cast<T*>(base + off);
}

// Revolutions per unit of position of pair t: theta^(-2t/D) / (2 pi); for
// the 2D rotation of the vision encoder, pair t of half t / (D/4) at
// frequency index t % (D/4) of a RoPE of dim D/2.
template <bool VIS>
__device__ __forceinline__ double pair_rev(int t, int D, double log2_theta) {
  if constexpr (VIS) return rope_rev_per_pos(t % (D / 4), D / 2, log2_theta);
  else return rope_rev_per_pos(t, D, log2_theta);
}

// Rotated key slab, one pass over the keys: ws[row][0 .. SW) = the first SW
// dims of k[row] with pair t < n_rot turned by pos * theta^(-2t/D), rounded to
// bf16; row = (b*S + j)*Hkv + hkv.  One 16-byte chunk (4 pairs) per thread.
// The angle is reduced in fp64 and its sine and cosine come from the
// hardware instructions, as for the queries and the decode's keys (the
// library sincospif made the pass compute-bound: 0.52 ms for the 2 GiB of a
// local layer at S = 262144).
// VIS: pos is [B*S, 2] and the pairs of the chunk (all in one half) turn by
// the component of their half.
template <int SW, bool VIS = false>
__global__ void __launch_bounds__(256) rope_keys_kernel(const uint16_t* __restrict__ k,
                                                       uint16_t* __restrict__ ws,
                                                       const int32_t* __restrict__ pos,
                                                       long long nchunks, int Hkv, int D, int n_rot,
                                                       double log2_theta) {
  constexpr int CPR = SW / 8;  // chunks per slab row
  static_assert(256 % CPR == 0, "the grid stride keeps each thread on one chunk column");
  // A thread's chunk column c is the same in every iteration (the stride is a
  // multiple of CPR), so the frequencies of its 4 pairs are computed once:
  // recomputing them per chunk (an fp64 exponential each) made the pass
  // compute-bound.
  const int c = (int)(threadIdx.x % CPR);
  double g[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) g[e] = pair_rev<VIS>(4 * c + e, D, log2_theta);
  for (long long i = blockIdx.x * 256ll + threadIdx.x; i < nchunks;
       i += (long long)gridDim.x * 256) {
    const long long row = i / CPR;
    u32x4 x = *reinterpret_cast<const u32x4*>(k + row * D + 8 * c);
    if (4 * c < n_rot) {
      const int p = VIS ? pos[(row / Hkv) * 2 + (4 * c >= D / 4)] : pos[row / Hkv];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int t = 4 * c + e;
        float cs, sn;
        rope_cs_fast(p, g[e], cs, sn);
        const float x0 = bf_lo(x[e]), x1 = bf_hi(x[e]);
        const uint32_t r = pack_bf16(x0 * cs - x1 * sn, x0 * sn + x1 * cs);
        x[e] = t < n_rot ? r : x[e];
      }
    }
    *reinterpret_cast<u32x4*>(ws + row * SW + 8 * c) = x;
  }
}

// Exact attention row (token t, query head h) for a wave: every key's score
// is a wave-wide reduction (wave-uniform), so the running max and the
// rescaling of the sums when it grows are uniform too.  Lane e owns dims
// e*(D/64) .. +D/64-1.  Keys are read raw and rotated here.
// VIS: keys 0 .. nv-1 (no causal mask), positions per half from pos [B*S, 2].
template <int D, bool OBF, bool VIS = false>
__device__ __noinline__ void exact_row(const uint16_t* qp, const uint16_t* kp, const uint16_t* vp,
                                       void* outp, const int32_t* posp, int S, int Hq, int Hkv,
                                       int W, int n_rot, float scale_log2e, int b, int hkv, int t,
                                       int h, double log2_theta, int nv = 0) {
  constexpr int E = D / 64;  // dims per lane, even
  const int lane = threadIdx.x & 63;
  double gl[E / 2];  // revolutions per position of the lane's pairs
#pragma unroll
  for (int e = 0; e < E; e += 2) gl[e / 2] = pair_rev<VIS>((lane * E + e) / 2, D, log2_theta);
  const uint16_t* qr = qp + (((size_t)b * S + t) * Hq + h) * D;
  // position of pair d0/2 of token j
  auto ppos = [&](int j, int d0) {
    if constexpr (VIS) return posp[((size_t)b * S + j) * 2 + (d0 >= D / 2)];
    else return posp[(size_t)b * S + j];
  };
  float qv[E];
#pragma unroll
  for (int e = 0; e < E; e += 2) {
    const int d0 = lane * E + e;
    float x0 = bf_lo(qr[d0]), x1 = bf_lo(qr[d0 + 1]);
    if (d0 / 2 < n_rot) {
      float c, s;
      rope_cs_accurate(ppos(t, d0), gl[e / 2], c, s);
      const float y0 = x0 * c - x1 * s, y1 = x0 * s + x1 * c;
      x0 = y0;
      x1 = y1;
    }
    qv[e] = x0;
    qv[e + 1] = x1;
  }
  float o[E], l = 0.f, m = -INFINITY;
#pragma unroll
  for (int e = 0; e < E; ++e) o[e] = 0.f;
  const int lo = VIS ? 0 : (W > 0 ? max(0, t - W + 1) : 0);
  const int hi = VIS ? nv - 1 : t;
  for (int j = lo; j <= hi; ++j) {
    const size_t row = ((size_t)b * S + j) * Hkv + hkv;
    const uint16_t* kr = kp + row * D;
    const uint16_t* vr = vp + row * D;
    float part = 0.f;
#pragma unroll
    for (int e = 0; e < E; e += 2) {
      const int d0 = lane * E + e;
      float x0 = bf_lo(kr[d0]), x1 = bf_lo(kr[d0 + 1]);
      if (d0 / 2 < n_rot) {
        float c, s;
        rope_cs_accurate(ppos(j, d0), gl[e / 2], c, s);
        const float y0 = x0 * c - x1 * s, y1 = x0 * s + x1 * c;
        x0 = y0;
        x1 = y1;
      }
      part += qv[e] * x0 + qv[e + 1] * x1;
    }
    const float sc = wave_sum(part) * scale_log2e;
    if (sc > m) {  // wave-uniform
      const float c = __builtin_amdgcn_exp2f(m - sc);
      l *= c;
#pragma unroll
      for (int e = 0; e < E; ++e) o[e] *= c;
      m = sc;
    }
    const float p = __builtin_amdgcn_exp2f(sc - m);
    l += p;
#pragma unroll
    for (int e = 0; e < E; ++e) o[e] += p * bf_lo(vr[lane * E + e]);
  }
  const size_t ob = (((size_t)b * S + t) * Hq + h) * D + lane * E;
#pragma unroll
  for (int e = 0; e < E; ++e) {
    if constexpr (OBF)
      static_cast<uint16_t*>(outp)[ob + e] = (uint16_t)(pack_bf16(o[e] / l, 0.f) & 0xffffu);
    else
      static_cast<float*>(outp)[ob + e] = o[e] / l;
  }
}

// SW = key dims the score product reads from the rotated slab: 128 (only
// pairs < 64 may turn, e.g. p = 0.25 at D = 512) or D (any p).  Score k-steps
// s < SW/16 read the slab, the others the raw key tile.
// NST = LDS ring depth (2 or 3): each tile is computed whole (scores,
// softmax, value product) while the next one or two tiles load.
// SPREAD: the software-pipelined loop of the global K=V instances.  The loads
// of tile kt+NST-1 are issued one at a time inside the score products of tile
// kt+1, and pairs of waves share their 64 rows' value products (each wave
// keeps half of the output dims).  Every wave must then compute every tile
// that holds a visible key for any wave of the workgroup, which holds
// without a window when a workgroup's tokens fit in one tile.
template <int D, int G, bool KVS, bool OBF, int SW, int NST, int MB, bool SPREAD, bool VIS>
__global__ void __launch_bounds__(NW * 64, (wg_per_cu<D, MB, NST>())) prefill_kernel(PrefillArgs a) {
  constexpr int RW = 32 * MB;          // rows per wave
  constexpr int M = NW * RW;           // rows per workgroup
  constexpr int TQ = M / G;            // tokens per workgroup
  constexpr int NDS = D / 16;          // k-steps of the score product
  constexpr int NSS = SW / 16;         // k-steps read from the slab
  constexpr int NDB = D / 32;          // 32-dim blocks of the output
  using L = Lds<D, KVS, SW, NST>;
  static_assert(L::TOTAL + (SPREAD ? 2 * NW * 2 * 1024 : 0) <= 160 * 1024, "LDS budget");
  static_assert(!SPREAD || (D == 512 && NW == 4), "pairs of waves split the 512 output dims");
  static_assert(SW >= 128 && SW <= D && NDS % 8 == 0 && NSS % 8 == 0, "tile shape");
  static_assert(L::STAGE % (1024 * NW) == 0, "stage = whole direct loads per wave");
  static_assert(NST >= 2 && NST <= 4, "ring");
  static_assert(!SPREAD || ((NST == 3 || NST == 4) && TQ <= BN && MB == 1),
                "the pipelined loop needs a 3- or 4-deep ring, TQ <= BN and one block per wave");
  static_assert(NST != 4 || SPREAD, "the 4-deep ring is the pipelined loop's");
  static_assert(!VIS || (!SPREAD && SW == D && D % 64 == 0), "vision: full slab, halves of whole chunks");
  // With two query blocks per wave, or at two workgroups per CU, the score
  // and output accumulators leave few registers: the lane parts of LDS
  // offsets are then recomputed per tile from an opaque copy of the lane id
  // instead of staying live across the loop.  Otherwise they fit and stay live.
  constexpr bool RECOMP = MB == 2 || wg_per_cu<D, MB, NST>() == 2;
  __shared__ __attribute__((aligned(16))) unsigned char st0[L::STAGE];
  __shared__ __attribute__((aligned(16))) unsigned char st1[L::STAGE];
  __shared__ __attribute__((aligned(16))) unsigned char st2[NST >= 3 ? L::STAGE : 16];
  __shared__ __attribute__((aligned(16))) unsigned char st3[NST >= 4 ? L::STAGE : 16];
  // pipelined instances: P of each wave's rows, passed to the other wave of
  // its pair ([step parity][wave][key half][lane], 16 bytes each)
  constexpr int PXB = SPREAD ? 2 * NW * 2 * 1024 : 16;
  __shared__ __attribute__((aligned(16))) unsigned char pxb[PXB];
  // ring stage s (a compile-time constant) -> its LDS object
  auto stp = [&](auto s) -> unsigned char* {
    if constexpr (decltype(s)::value == 0) return st0;
    else if constexpr (decltype(s)::value == 1) return st1;
    else if constexpr (decltype(s)::value == 2) return st2;
    else return st3;
  };
  // Angle table of the query rotation: in the last ring stage, which receives
  // its first tile only after the barrier that ends the prologue.
  double* gtab = reinterpret_cast<double*>(stp(IC<NST - 1>{}));

  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave index, in a scalar register
  const int l32 = lane & 31, hl = lane >> 5;
  const int S = a.S;
  const int W = a.window;
  const int n_rot = a.n_rot;

  const int hb = blockIdx.x % a.nheads;
  const int qt = a.nq - 1 - blockIdx.x / a.nheads;
  const int b = hb / a.Hkv, hkv = hb % a.Hkv;
  const int t0 = qt * TQ;
  const int t_end = min(t0 + TQ, S);

  for (int t = tid; t < D / 2; t += NW * 64) gtab[t] = pair_rev<VIS>(t, D, a.log2_theta);
  __syncthreads();
  // vision: the image's valid patches (keys past them are not attended to)
  int nv = S;
  if constexpr (VIS) nv = a.lengths ? min(max(a.lengths[b], 0), S) : S;

  // ---- query rows of this lane (one per block), rotated, as B operands ----
  int tq[MB], hq[MB];
  bool row_ok[MB];
  u32x4 qf[MB][NDS];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) {
    const int row = RW * w + 32 * mb + l32;
    tq[mb] = t0 + row / G;
    hq[mb] = hkv * G + row % G;
    row_ok[mb] = tq[mb] < S;
    const int tqc = row_ok[mb] ? tq[mb] : S - 1;
    // VIS: component 0 (w) for the first half of the dims, 1 (h) for the second
    const int qpos = VIS ? a.pos[((size_t)b * S + tqc) * 2] : a.pos[(size_t)b * S + tqc];
    const int qpos1 = VIS ? a.pos[((size_t)b * S + tqc) * 2 + 1] : qpos;
    const uint16_t* qrow =
        static_cast<const uint16_t*>(a.q) + (((size_t)b * S + tqc) * a.Hq + hq[mb]) * D;
#pragma unroll
    for (int s = 0; s < NDS; ++s) {
      const u32x4 x = *reinterpret_cast<const u32x4*>(qrow + 8 * (2 * s + hl));
      qf[mb][s] = row_ok[mb] ? x : u32x4{0, 0, 0, 0};
    }
#pragma unroll
    for (int s = 0; s < NSS; ++s)  // chunk 2s + hl lies in the second half iff s >= D/32
      if (8 * s < n_rot)
        qf[mb][s] = rotate_chunk_bf16(qf[mb][s], 2 * s + hl, (VIS && s >= D / 32) ? qpos1 : qpos,
                                      n_rot, gtab);
  }

  // token span of this wave's rows
  const int tw0 = t0 + (RW * w) / G;
  const int tw1 = min(t0 + (RW * w + RW - 1) / G, S - 1);
  const bool wave_ok = tw0 < (VIS ? nv : S);  // vision: waves of padding rows only skip
  const int klo = (!VIS && W > 0) ? max(0, t0 - W + 1) : 0;
  const int kt0 = klo / BN, kt1 = VIS ? (nv - 1) / BN : (t_end - 1) / BN;

  // ---- direct HBM -> LDS loads of one tile ----
  // Per tile a buffer resource covers the rows kv0 .. kv0+rows-1 of this KV
  // head (and the matching slab rows); each lane's 32-bit offset is fixed.
  const uint32_t row_bytes = (uint32_t)(a.Hkv * D * 2);
  const uint32_t srow_bytes = (uint32_t)(a.Hkv * SW * 2);
  const uint16_t* kbase = static_cast<const uint16_t*>(a.k) + ((size_t)b * S * a.Hkv + hkv) * D;
  const uint16_t* vbase = static_cast<const uint16_t*>(a.v) + ((size_t)b * S * a.Hkv + hkv) * D;
  const uint16_t* sbase_g = static_cast<const uint16_t*>(a.ws) + ((size_t)b * S * a.Hkv + hkv) * SW;
  // The loads of one tile: buffer resources over its rows (scalar, made once
  // per tile), then one 16-byte-per-lane direct load per call, so that the
  // loads can be spread over the tile's score products instead of queueing
  // behind each other at the address unit all at once.
  // Lane part of the direct-load offsets of rows of RB bytes (see load_part):
  // a = chunk ^ (row-in-load << 2), lrb = row-in-load * row stride.
  struct LaneLd {
    uint32_t a, lrb;
  };
  auto lane_ld = [&](auto rbc, uint32_t rbytes) -> LaneLd {
    constexpr int CPR = decltype(rbc)::value / 16;  // chunks per row
    uint32_t ln = (uint32_t)lane;
    if constexpr (RECOMP) asm volatile("" : "+v"(ln));
    const uint32_t lr = ln / CPR;
    const uint32_t rb = __builtin_amdgcn_readfirstlane(rbytes);
    LaneLd r{(ln % CPR) ^ (lr << 2), (uint32_t)__umul24(lr, rb)};
    // keeps the wave-uniform part of the row offset a separate scalar term
    asm volatile("" : "+v"(r.lrb));
    return r;
  };
  struct TileSrc {
    __amdgpu_buffer_rsrc_t s, k, v;
    LaneLd ls, lk;  // slab rows, raw rows
  };
  auto tile_src = [&](int kt) {
    // padding tiles past the sequence reload its last tile: finite data whose
    // keys are all masked for this workgroup's rows
    const int kv0 = min(kt * BN, ((S - 1) / BN) * BN);
    const int rows = min(S - kv0, BN);  // >= 1
    const size_t toff = (size_t)kv0 * a.Hkv;
    TileSrc t;
    t.s = make_rsrc(sbase_g + toff * SW, rows * srow_bytes - (srow_bytes - 2 * SW));
    t.k = make_rsrc(kbase + toff * D, rows * row_bytes - (row_bytes - 2 * D));
    t.v = make_rsrc(vbase + toff * D, rows * row_bytes - (row_bytes - 2 * D));
    t.ls = lane_ld(IC<2 * SW>{}, srow_bytes);
    if constexpr (SW == D) t.lk = t.ls;  // same row size and stride
    else t.lk = lane_ld(IC<2 * D>{}, row_bytes);
    return t;
  };
  // direct load n of this wave for one tensor: rows of RB bytes in HBM
  // (stride rbytes), placed at dst with 16-byte chunks swizzled by row.
  // Lane ln fetches chunk c = ln % CPR of row r = r0 + lr, lr = ln / CPR, with
  // r0 = (w * LPW + n) * RPI a multiple of RPI <= 4.  The low two bits of r
  // are then (r0 & 3) | lr and bits 2-3 are those of r0, so swz(r) =
  // swz(r0) ^ (lr << 2): the lane part A = c ^ (lr << 2) and lr * rb are the
  // same for every load and tile, and a load adds only the wave-uniform
  // swz(r0) and r0 * rb (three vector instructions per load).
  auto load_part = [&](auto rbc, const __amdgpu_buffer_rsrc_t& rs, uint32_t rbytes,
                       const LaneLd& ll, int n, unsigned char* dst) {
    constexpr int RB = decltype(rbc)::value;  // bytes per row in LDS
    constexpr int RPI = 1024 / RB;            // rows per direct load
    constexpr int LPW = BN / RPI / NW;        // direct loads per wave
    static_assert(RPI >= 1 && RPI <= 4, "the lane part of the row stays in bits 0-1");
    const uint32_t rb = __builtin_amdgcn_readfirstlane(rbytes);
    const int r0 = (w * LPW + n) * RPI;  // first row of this load, wave-uniform
    // rows < BN and rb <= Hkv * D * 2 < 2^24: r0 * rb fits 32 bits
    const uint32_t voff = ((ll.a ^ (uint32_t)swz(r0)) << 4) + ll.lrb + (uint32_t)r0 * rb;
    lds_dma16(rs, voff, 0, dst + r0 * RB);
  };
  // loads per wave per tile: slab, raw keys (when the slab does not hold
  // every key dimension, or keys are values), raw values (separate caches)
  constexpr int NL_S = BN / (1024 / (2 * SW)) / NW;
  constexpr int NL_K = (KVS || SW < D) ? BN / (1024 / (2 * D)) / NW : 0;
  constexpr int NL_V = !KVS ? BN / (1024 / (2 * D)) / NW : 0;
  static_assert(NL_S + NL_K + NL_V == L::NLD, "loads per wave");
  // load j (0 <= j < L::NLD) of a tile; j is a constant after unrolling
  auto load_one = [&](const TileSrc& t, auto stage, int j) {
    unsigned char* sp = stp(stage);
    if (j < NL_S) load_part(IC<2 * SW>{}, t.s, srow_bytes, t.ls, j, sp);
    else if (j < NL_S + NL_K) load_part(IC<2 * D>{}, t.k, row_bytes, t.lk, j - NL_S, sp + L::KOFF);
    else load_part(IC<2 * D>{}, t.v, row_bytes, t.lk, j - NL_S - NL_K, sp + L::VOFF);
  };
  auto issue_loads = [&](int kt, auto stage) {
    const TileSrc t = tile_src(kt);
#pragma unroll
    for (int j = 0; j < L::NLD; ++j) load_one(t, stage, j);
  };

  f32x16 oacc[MB][NDB];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb)
#pragma unroll
    for (int i = 0; i < NDB; ++i) oacc[mb][i] = f32x16{};
  // Softmax state per row (base 2, scores scaled by log2(e)/sqrt(d)).  The
  // reference max m_ref is fixed at the first tile where the row sees a key,
  // when O is still zero, so O never needs rescaling.  If a later score ever
  // exceeds m_ref by more than 64 (P = 2^(s - m_ref) could overflow P or O),
  // the row is flagged in ovf and recomputed exactly after the epilogue.
  constexpr float UNSET = -1e30f;
  float m_ref[MB], l_run[MB];
  int ovf = 0;  // bit mb: row of block mb overflowed its reference
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) {
    m_ref[mb] = UNSET;
    l_run[mb] = 0.f;
  }
  const float cs = a.scale_log2e;

  // ---- scores S^T = K~ Q~^T of one tile (fragments stream in groups of FG, one group ahead) ----
  // side(g) and then fill(g) run after group g (the pipelined loop issues
  // direct loads of a later tile there).
  auto scores = [&](auto stage, f32x16 (&sacc)[MB], auto&& side, auto&& fill) {
    unsigned char* sp = stp(stage);
    uint32_t ln = (uint32_t)lane;
    if constexpr (RECOMP) asm volatile("" : "+v"(ln));
    const uint32_t l32 = ln & 31, hl = ln >> 5;
    // score operand (key l32, chunk c = 2s + hl) sits at chunk position
    // 16*(s/8) + ((2*(s%8) + hl) ^ swz(l32)) of its row.  With i = s % 8 and
    // swz = 2*sh + s0, (2i + hl) ^ swz = 2*(i ^ sh) + (hl ^ s0), so the byte
    // offset is P ^ (i << 5) + 256*(s/8) with P = row + 16*(hl ^ s0) + 32*sh:
    // rows start at multiples of 256 bytes, so the XOR only touches bits 5-7
    // and commutes with the row, stage and 256-byte block offsets.
    const uint32_t sw = (uint32_t)swz((int)l32);
    const uint32_t lo = (((hl ^ sw) & 1) << 4) | ((sw >> 1) << 5);
    const uint32_t ps = l32 * (2 * SW) + lo;  // slab rows
    const uint32_t pk = l32 * (2 * D) + lo;   // raw key rows
    // k-step s lives in the slab for s < NSS, in the raw key tile otherwise
    auto frag = [&](int s) -> u32x4 {
      const uint32_t x = (uint32_t)(s & 7) << 5;
      if (s < NSS) return lds_at<u32x4>(sp, (int)((ps ^ x) + 256 * (s >> 3)));
      return lds_at<u32x4>(sp, L::KOFF + (int)((pk ^ x) + 256 * (s >> 3)));
    };
    constexpr int NG = NDS / FG;
    u32x4 kf[2][FG];
#pragma unroll
    for (int i = 0; i < FG; ++i) kf[0][i] = frag(i);
#pragma unroll
    for (int g = 0; g < NG; ++g) {
      if (g + 1 < NG) {
#pragma unroll
        for (int i = 0; i < FG; ++i) kf[(g + 1) & 1][i] = frag(FG * (g + 1) + i);
      }
#pragma unroll
      for (int i = 0; i < FG; ++i)
#pragma unroll
        for (int mb = 0; mb < MB; ++mb)
          if (g == 0 && i == 0) score_first(sacc[mb], kf[g & 1][i], qf[mb][FG * g + i]);
          else score_next(sacc[mb], kf[g & 1][i], qf[mb][FG * g + i]);
      side(g);
      fill(g);
      __builtin_amdgcn_sched_barrier(0);
    }
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) score_ready(sacc[mb]);
  };

  // ---- causal / band mask of tile kt (edge tiles only) ----
  auto mask = [&](int kt, f32x16 (&sacc)[MB]) {
    const int kv0 = kt * BN;
    if constexpr (VIS) {  // keys past the image's patches only
      if (kv0 + BN > nv) {
#pragma unroll
        for (int mb = 0; mb < MB; ++mb)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int j = kv0 + 8 * (r >> 2) + 4 * hl + (r & 3);
            sacc[mb][r] = j < nv ? sacc[mb][r] : -INFINITY;
          }
      }
      return;
    }
    const bool need_mask = (kv0 + BN - 1 > tw0) || (W > 0 && kv0 <= tw1 - W);
    if (need_mask) {  // wave-uniform
      // key j is visible iff 0 <= tq - j < W (W = 0: 0 <= tq - j), i.e. the
      // unsigned difference is below W (below 2^31 without a window)
      const uint32_t wl = W > 0 ? (uint32_t)W : 0x80000000u;
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) {
        const int d0 = tq[mb] - kv0 - 4 * hl;  // tq - j for register 0
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const uint32_t dj = (uint32_t)(d0 - (8 * (r >> 2) + (r & 3)));
          sacc[mb][r] = dj < wl ? sacc[mb][r] : -INFINITY;
        }
      }
    }
  };

  // ---- reference max of block mb's rows that have none yet ----
  // The tile max is needed only until every row of the wave has fixed its
  // reference (wave-uniform test; after the first tiles it is skipped).
  auto ref_max = [&](const f32x16 (&sacc)[MB], int mb) {
    if (__builtin_amdgcn_ballot_w64(m_ref[mb] == UNSET)) {
      // balanced tree over the lane's 16 scores, then the other half-wave
      const f32x16& v = sacc[mb];
      const float a0 = fmaxf(fmaxf(v[0], v[1]), v[2]), a1 = fmaxf(fmaxf(v[3], v[4]), v[5]);
      const float a2 = fmaxf(fmaxf(v[6], v[7]), v[8]), a3 = fmaxf(fmaxf(v[9], v[10]), v[11]);
      const float a4 = fmaxf(fmaxf(v[12], v[13]), v[14]);
      const float mx = max_xor32(fmaxf(fmaxf(fmaxf(a0, a1), a2), fmaxf(fmaxf(a3, a4), v[15])));
      const float m_tile = mx * cs;  // -inf when the row sees no key here
      m_ref[mb] = m_ref[mb] == UNSET ? fmaxf(m_tile, UNSET) : m_ref[mb];
    }
  };

  // ---- softmax of masked scores -> P^T as B operands of the value product ----
  // half k2 computes P for keys 16*k2 .. 16*k2+15 of the tile (the row max
  // and the reference with the first half)
  auto softmax = [&](const f32x16 (&sacc)[MB], u32x4 (&pf)[MB][2], auto k2c) {
    constexpr int K2 = decltype(k2c)::value;
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
      if constexpr (K2 == 0) ref_max(sacc, mb);
      const float mr = m_ref[mb] == UNSET ? 0.f : m_ref[mb];
      float lsum = 0.f;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float p0 = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[mb][8 * K2 + 2 * i], cs, -mr));
        const float p1 =
            __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[mb][8 * K2 + 2 * i + 1], cs, -mr));
        lsum += p0 + p1;
        pf[mb][K2][i] = pack_bf16(p0, p1);
      }
      // a score more than 2^64 above the reference makes this sum exceed
      // 2^64 (infinity included): the row is recomputed exactly
      ovf |= (lsum > 0x1p64f) << mb;
      l_run[mb] += lsum;
    }
  };

  // ---- O^T += V^T P^T, V^T fragments by transpose reads of the raw value tile ----
  // make_p(pf, IC<k2>) produces P^T for keys 16*k2 .. +15.  The products go
  // key half by key half (fragment f: keys 16*(f/NDB).., dims 32*(f%NDB)..):
  // the first half of P is made after the first value reads are issued, the
  // second half under the first group's products.
  // side(g) runs after group g (the pipelined loop issues direct loads there).
  auto values = [&](auto stage, auto&& make_p, auto&& side) {
    unsigned char* sp = stp(stage);
    uint32_t ln = (uint32_t)lane;
    if constexpr (RECOMP) asm volatile("" : "+v"(ln));
    // value operand by transpose reads: lane (g = ln/16, i = ln%16) reads row
    // 4*(g/2) + i/4 (then +8 rows for the upper 4 keys, +16*k2) at dims
    // 32*db + 16*(g%2) + 4*(i%4), i.e. chunk 4*db + tr_x, byte 8*(i%2).
    // For row r = tr_row + 8h, swz(r) = swz(tr_row) ^ 2h, and 4e + tr_x =
    // 4e ^ tr_x (disjoint bits), so the chunk position of block db (e = db%4)
    // is 4e ^ Q_h with Q_h = tr_x ^ swz(tr_row) ^ 2h: the byte offset is
    // V_h ^ (e << 6), where V_h holds the row, the byte and Q_h << 4 (bits
    // 4-7; the row and the 8-byte half sit in other bits), and
    // V_1 = (V_0 ^ 32) + 8 rows.
    const uint32_t tr_i = ln & 15, tr_g = ln >> 4;
    const uint32_t tr_row = 4 * (tr_g >> 1) + (tr_i >> 2);
    const uint32_t tr_x = 2 * (tr_g & 1) + ((tr_i & 3) >> 1);
    const uint32_t v0 = tr_row * (2 * D) + (tr_i & 1) * 8 + ((tr_x ^ (uint32_t)swz((int)tr_row)) << 4);
    const uint32_t v1 = (v0 ^ 32u) + 8 * (2 * D);
    auto vfrag = [&](int db, int k2) -> u32x4 {
      const int off = L::VOFF + 256 * (db >> 2) + (16 * k2) * (2 * D);
      const uint32_t x = (uint32_t)(db & 3) << 6;
      const u32x2 lo = lds_read_tr16(sp + off + (v0 ^ x));
      const u32x2 hi = lds_read_tr16(sp + off + (v1 ^ x));
      return u32x4{lo[0], lo[1], hi[0], hi[1]};
    };
    constexpr int NG = 2 * NDB / FG;
    static_assert(NDB % FG == 0, "a group stays within one key half");
    u32x4 vf[2][FG];
#pragma unroll
    for (int i = 0; i < FG; ++i) vf[0][i] = vfrag(i % NDB, i / NDB);
    __builtin_amdgcn_sched_barrier(0);
    u32x4 pf[MB][2];
    make_p(pf, IC<0>{});
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int g = 0; g < NG; ++g) {
      if (g + 1 < NG) {
#pragma unroll
        for (int i = 0; i < FG; ++i) {
          const int f = FG * (g + 1) + i;
          vf[(g + 1) & 1][i] = vfrag(f % NDB, f / NDB);
        }
      }
#pragma unroll
      for (int i = 0; i < FG; ++i) {
        const int f = FG * g + i;
#pragma unroll
        for (int mb = 0; mb < MB; ++mb)
          oacc[mb][f % NDB] = mfma32x32x16(vf[g & 1][i], pf[mb][f / NDB], oacc[mb][f % NDB]);
      }
      if (g == 0) make_p(pf, IC<1>{});
      side(g);
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  // one whole tile
  // With two workgroups per CU, a wave issuing matrix products runs at wave
  // priority 1 and drops to 0 for the mask and the first softmax half, so the
  // SIMD's other wave yields issue slots to the products while it is in its
  // own softmax (window-1024 layer at S = 32768: 0.84 -> 0.82 ms, same box).
  constexpr bool PRIO = wg_per_cu<D, MB, NST>() == 2;
  auto compute = [&](int kt, auto stage, auto&& side) {
    f32x16 sacc[MB];
    if constexpr (PRIO) __builtin_amdgcn_s_setprio(1);
    scores(stage, sacc, side, [](int) {});
    if constexpr (PRIO) __builtin_amdgcn_s_setprio(0);
    mask(kt, sacc);
    values(stage, [&](u32x4 (&pf)[MB][2], auto k2c) {
      softmax(sacc, pf, k2c);
      if constexpr (PRIO && decltype(k2c)::value == 0) __builtin_amdgcn_s_setprio(1);
    }, [](int) {});
    if constexpr (PRIO) __builtin_amdgcn_s_setprio(0);
  };
  // a wave skips tiles where none of its rows sees a key (past its last
  // token, before its window, or padding)
  auto visible = [&](int kt) {
    const int kv0 = kt * BN;
    if constexpr (VIS) return wave_ok && kv0 < nv;
    return (SPREAD || wave_ok) && kv0 <= tw1 && !(W > 0 && kv0 + BN - 1 <= tw0 - W);
  };
  // vision: an image with no valid patch has only zero rows (and no tile to load)
  if (VIS && nv == 0) {
    for (int idx = tid; idx < M * D / 4; idx += NW * 64) {
      const int r = idx / (D / 4), tk = t0 + r / G;
      if (tk >= S) continue;
      const size_t o = (((size_t)b * S + tk) * a.Hq + hkv * G + r % G) * D + 4 * (idx % (D / 4));
      if constexpr (OBF) *reinterpret_cast<u32x2*>(static_cast<uint16_t*>(a.out) + o) = u32x2{0, 0};
      else *reinterpret_cast<f32x4*>(static_cast<float*>(a.out) + o) = f32x4{};
    }
    return;
  }

  // ---- KV loop, unrolled by the ring depth so every stage is a fixed object ----
  // The tile count is padded up to a multiple of the ring depth; padding tiles
  // lie past the last query token, so every key in them is masked.
  const int ktp = kt0 + (kt1 - kt0 + NST) / NST * NST - 1;  // last (padded) tile
  if constexpr (SPREAD) {
    static_assert(L::NLD <= NDS / FG, "one load per score group");
    // Software-pipelined loop (SPREAD instances: K=V, no window, TQ <= BN, so
    // every wave computes every tile up to the workgroup's last token kt1).
    // Same-box timings against one wave per row block on a 4-deep ring
    // (outputs bit for bit the same): S = 32768 at 32/4 heads 26.55 against
    // 27.19-27.30 ms, S = 262144 at 16/2 heads 842 against 861 ms.  The
    // 3-deep ring alone measured the same as the 4-deep one: the fence of
    // each barrier makes every load land within the step that issues it.
    //
    // Waves 2m and 2m+1 form a pair that shares their 64 query rows: each
    // wave computes the scores and P of its own 32 rows, and keeps the output
    // of all 64 rows for half of the 512 dims (half = w & 1).  Each value
    // fragment read from LDS then feeds two products (own rows, partner's
    // rows), so a wave reads 16 KiB of value operands per tile instead of 32;
    // the partner's P (2 KiB) comes through LDS.  Every output element sums
    // the same products in the same order as with one wave per row block.
    //
    // Step kt enters with P of tile kt made and stored in the exchange buffer
    // and tiles kt, kt+1 in LDS.  It runs the score products of tile kt+1
    // with the loads of tile kt+NST-1 issued one per group, then the value
    // products of tile kt (both waves' P of tile kt read back from the
    // buffer, so no P stays in registers across the score products) with the
    // softmax of tile kt+1 made two score registers per group of value
    // products, and stores that P.  The barrier at the
    // end frees the stage of tile kt and publishes the new P.  Loads past the
    // last tile repeat it (clamped) and are drained at the end.
    const int half = w & 1;  // output dims 256*half .. +255, wave-uniform
    auto pslot = [&](int par, int wave, int k2) -> unsigned char* {
      return pxb + ((par * NW + wave) * 2 + k2) * 1024 + lane * 16;
    };
    auto put_p = [&](int par, const u32x4 (&pd)[MB][2]) {
#pragma unroll
      for (int k2 = 0; k2 < 2; ++k2) *reinterpret_cast<u32x4*>(pslot(par, w, k2)) = pd[0][k2];
    };
    auto get_p = [&](int par, int wave, u32x4 (&pd)[MB][2]) {
#pragma unroll
      for (int k2 = 0; k2 < 2; ++k2) pd[0][k2] = *reinterpret_cast<const u32x4*>(pslot(par, wave, k2));
    };
    // Softmax of one tile's scores sc into P: mask and reference first, then
    // begin_tile; part(g) makes P for score register g (the pair (g-1, g) is
    // packed once g is odd); end_tile adds the tile's sums.  The sums of the
    // two key halves are kept apart and added in the order of the unpipelined
    // loop, so both loops give bit-identical rows.
    float mr[MB], pe[MB], lp[MB][2];
    auto begin_tile = [&](int kt, f32x16 (&sc)[MB]) {
      mask(kt, sc);
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) {
        ref_max(sc, mb);
        mr[mb] = m_ref[mb] == UNSET ? 0.f : m_ref[mb];
        pe[mb] = 0.f;
        lp[mb][0] = lp[mb][1] = 0.f;
      }
    };
    auto part = [&](int g, const f32x16 (&sc)[MB], u32x4 (&pd)[MB][2]) {
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) {
        const float p = __builtin_amdgcn_exp2f(__builtin_fmaf(sc[mb][g], cs, -mr[mb]));
        if (g & 1) {
          pd[mb][g >> 3][(g & 7) >> 1] = pack_bf16(pe[mb], p);
          lp[mb][g >> 3] += pe[mb] + p;
        } else {
          pe[mb] = p;
        }
      }
    };
    auto end_tile = [&]() {
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) {
#pragma unroll
        for (int k2 = 0; k2 < 2; ++k2) {
          // a score more than 2^64 above the reference makes a half's sum
          // exceed 2^64 (infinity included): the row is recomputed exactly
          ovf |= (lp[mb][k2] > 0x1p64f) << mb;
          l_run[mb] += lp[mb][k2];
        }
      }
    };
    // O^T += V^T P^T for this wave's half of the dims, own rows in output
    // blocks 0..7 and the partner's rows in blocks 8..15, with both P read
    // from the exchange buffer of parity par; side(g) runs after group g of
    // value fragments
    auto values_pair = [&](auto stage, int par, auto&& side) {
      u32x4 pown[MB][2], ppar[MB][2];
      get_p(par, w, pown);
      get_p(par, w ^ 1, ppar);
      // dims 256*half start 512 bytes into each raw row, a whole number of
      // 256-byte swizzle blocks
      unsigned char* sp = stp(stage) + 512 * half;
      uint32_t ln = (uint32_t)lane;
      const uint32_t tr_i = ln & 15, tr_g = ln >> 4;
      const uint32_t tr_row = 4 * (tr_g >> 1) + (tr_i >> 2);
      const uint32_t tr_x = 2 * (tr_g & 1) + ((tr_i & 3) >> 1);
      const uint32_t v0 = tr_row * (2 * D) + (tr_i & 1) * 8 + ((tr_x ^ (uint32_t)swz((int)tr_row)) << 4);
      const uint32_t v1 = (v0 ^ 32u) + 8 * (2 * D);
      auto vfrag = [&](int db, int k2) -> u32x4 {
        const int off = L::VOFF + 256 * (db >> 2) + (16 * k2) * (2 * D);
        const uint32_t x = (uint32_t)(db & 3) << 6;
        const u32x2 lo = lds_read_tr16(sp + off + (v0 ^ x));
        const u32x2 hi = lds_read_tr16(sp + off + (v1 ^ x));
        return u32x4{lo[0], lo[1], hi[0], hi[1]};
      };
      constexpr int NH = NDB / 2;   // 32-dim blocks of this wave's half
      constexpr int NG = 2 * NH / FG;
      static_assert(NH % FG == 0, "a group stays within one key half");
      u32x4 vf[2][FG];
#pragma unroll
      for (int i = 0; i < FG; ++i) vf[0][i] = vfrag(i % NH, i / NH);
#pragma unroll
      for (int g = 0; g < NG; ++g) {
        if (g + 1 < NG) {
#pragma unroll
          for (int i = 0; i < FG; ++i) {
            const int f = FG * (g + 1) + i;
            vf[(g + 1) & 1][i] = vfrag(f % NH, f / NH);
          }
        }
#pragma unroll
        for (int i = 0; i < FG; ++i) {
          const int f = FG * g + i;
          oacc[0][f % NH] = mfma32x32x16(vf[g & 1][i], pown[0][f / NH], oacc[0][f % NH]);
          oacc[0][NH + f % NH] = mfma32x32x16(vf[g & 1][i], ppar[0][f / NH], oacc[0][NH + f % NH]);
        }
        side(g);
        __builtin_amdgcn_sched_barrier(0);
      }
    };
    issue_loads(kt0, IC<0>{});
    issue_loads(kt0 + 1, IC<1>{});
    if constexpr (NST == 4) issue_loads(kt0 + 2, IC<2>{});
    wait_vmcnt<(NST - 2) * L::NLD>();
    __syncthreads();
    {
      f32x16 s0[MB];
      u32x4 p0[MB][2];
      scores(IC<0>{}, s0, [](int) {}, [](int) {});
      begin_tile(kt0, s0);
#pragma unroll
      for (int g = 0; g < 16; ++g) part(g, s0, p0);
      end_tile();
      put_p(0, p0);
    }
    wait_vmcnt<(NST - 3) * L::NLD>();
    __syncthreads();
    auto step = [&](int kt, auto s, auto parc) {
      constexpr int S0 = decltype(s)::value;
      constexpr int PAR = decltype(parc)::value;
      if (kt > kt1) return;  // padding steps of the unrolled loop
      const bool more = kt < kt1;  // wave-uniform
      u32x4 pnxt[MB][2];
      f32x16 nxt[MB];
      const TileSrc t = tile_src(kt + NST - 1);
      if (more) {
        scores(IC<(S0 + 1) % NST>{}, nxt, [&](int g) {
          if (g < L::NLD) load_one(t, IC<(S0 + NST - 1) % NST>{}, g);
        }, [](int) {});
        begin_tile(kt + 1, nxt);
      } else {
        // last tile: the parts below run on zeros and their sums are dropped
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) nxt[mb] = f32x16{};
      }
      values_pair(s, PAR, [&](int g) {
        part(2 * g, nxt, pnxt);
        part(2 * g + 1, nxt, pnxt);
      });
      if (more) {
        end_tile();
        put_p(PAR ^ 1, pnxt);
      }
      wait_vmcnt<(NST - 3) * L::NLD>();
      __syncthreads();
    };
    // unrolled by a multiple of the ring depth and of 2 (the P buffers)
    constexpr int U = NST == 4 ? 4 : 6;
    for (int kt = kt0; kt <= kt1; kt += U) {
      step(kt, IC<0>{}, IC<0>{});
      step(kt + 1, IC<1 % NST>{}, IC<1>{});
      step(kt + 2, IC<2 % NST>{}, IC<0>{});
      step(kt + 3, IC<3 % NST>{}, IC<1>{});
      if constexpr (U == 6) {
        step(kt + 4, IC<4 % NST>{}, IC<0>{});
        step(kt + 5, IC<5 % NST>{}, IC<1>{});
      }
    }
    wait_vmcnt<0>();
  } else if constexpr (NST == 3) {
    // tile kt+2 is requested while tile kt is computed; at the end of the
    // step only tile kt+1 must have landed (vmcnt <= one tile's loads)
    issue_loads(kt0, IC<0>{});
    issue_loads(kt0 + 1, IC<1>{});
    wait_vmcnt<L::NLD>();
    __syncthreads();
    auto step = [&](int kt, auto s) {
      constexpr int S0 = decltype(s)::value;
      const bool more = kt + 2 <= ktp;
      if (more) issue_loads(kt + 2, IC<(S0 + 2) % 3>{});
      if (visible(kt)) compute(kt, s, [](int) {});
      if (more) wait_vmcnt<L::NLD>();
      else wait_vmcnt<0>();
      __syncthreads();
    };
    for (int kt = kt0; kt <= ktp; kt += 3) {
      step(kt, IC<0>{});
      step(kt + 1, IC<1>{});
      step(kt + 2, IC<2>{});
    }
  } else {
    // Tile order: the n tiles of the (padded) span are visited starting at
    // the one whose index is a multiple of n, wrapping round, so tile kt is
    // computed at step (kt - kt0 + off) mod n with off = -kt0 mod n.  With
    // a window every full span has the same length, so the workgroups that
    // run together (consecutive query tiles of one KV head on one XCD) read
    // each shared tile in the same step: L2 then holds a few tiles per step
    // instead of the spans of all running windows, where the plain order
    // reads a shared tile two steps later per query tile.  Window-1024 layer
    // at S = 262144: 5.59 -> 5.51 ms with the key pass, same box.  Without a
    // window kt0 = 0 and the order is the plain one.  The d = 512 instances
    // keep the plain order: the rotation's registers make them spill.
    constexpr bool ROT = D == 256 && !VIS;
    const int n = ktp - kt0 + 1;
    const int off = ROT ? (n - kt0 % n) % n : 0;
    auto tile_at = [&](int i) {
      if constexpr (!ROT) return kt0 + i;
      const int j = i + off;
      return kt0 + (j >= n ? j - n : j);
    };
    issue_loads(tile_at(0), IC<0>{});
    wait_vmcnt<0>();
    __syncthreads();
    // (Issuing the next tile's loads one per score group instead, which
    // needs every wave to compute every tile of the span, measured slower:
    // 5.74 against 5.57 ms for the window-1024 layer at S = 262144.  A split
    // ring with the score part of each tile requested two tiles ahead, three
    // score parts and two value parts in 80 KiB, timed 2% slower than this
    // loop: the loads cost about 12% of the kernel, as measured by leaving
    // them out, but not through their latency.)
    auto step = [&](int i, auto s) {
      constexpr int S0 = decltype(s)::value;
      if (i + 1 < n) issue_loads(tile_at(i + 1), IC<1 - S0>{});
      const int kt = tile_at(i);
      if (visible(kt)) compute(kt, s, [](int) {});
      wait_vmcnt<0>();
      __syncthreads();
    };
    for (int i = 0; i < n; i += 2) {
      step(i, IC<0>{});
      step(i + 1, IC<1>{});
    }
  }

  // ---- epilogue: O / l (vision: padding rows are zero) ----
  if constexpr (D == 256) {
    // The rows leave through LDS, 16 per wave at a time, so that each store
    // writes one whole output row (64 lanes x 16 bytes) instead of 32 bytes in
    // each of 32 rows, and the stores are non-temporal, so the output streams
    // out without displacing the key and value tiles that the neighbouring
    // workgroups still read from L2.  Written straight from the accumulators
    // the stores took about 10% of the local-layer kernel's time (measured by
    // leaving them out); this way the window-1024 layer at S = 262144 went
    // from 6.38 to 6.01 ms (6.17 ms with the staging alone).  The ring stages
    // are free: the loop ended with a barrier after its last reads.  Wave w uses 16 KiB of stage w / 2; chunk c (16 bytes) of row r
    // sits at c ^ r, so the writes (16 rows, one chunk each) and the row reads
    // (one row, 64 chunks) both spread over all banks.  One wave writes and
    // reads its own region in order, so no barrier is needed.
    static_assert(L::STAGE >= 2 * 16 * D * 4, "two waves' 16-row output blocks per stage");
    unsigned char* ob = (w < 2 ? st0 : st1) + (w & 1) * (16 * D * 4);
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
      const float lt = l_run[mb] + __shfl_xor(l_run[mb], 32);
      const float inv = (VIS && tq[mb] >= nv) ? 0.f : 1.f / lt;
      // rows to store (bit l32 of the lower half-wave): in range and not flagged
      const unsigned long long okm = __ballot(row_ok[mb] && !((ovf >> mb) & 1));
#pragma unroll
      for (int p = 0; p < 2; ++p) {
        const int rr = l32 - 16 * p;  // this lane's row within the pass
        if (rr >= 0 && rr < 16) {
#pragma unroll
          for (int db = 0; db < NDB; ++db)
#pragma unroll
            for (int g4 = 0; g4 < 4; ++g4) {
              const int c = 8 * db + 2 * g4 + hl;  // dims 4c .. 4c+3
              *reinterpret_cast<f32x4*>(ob + rr * (D * 4) + ((c ^ rr) << 4)) =
                  f32x4{oacc[mb][db][4 * g4 + 0] * inv, oacc[mb][db][4 * g4 + 1] * inv,
                        oacc[mb][db][4 * g4 + 2] * inv, oacc[mb][db][4 * g4 + 3] * inv};
            }
        }
        for (int r = 0; r < 16; ++r) {
          if (!((okm >> (16 * p + r)) & 1)) continue;  // wave-uniform
          const f32x4 o = *reinterpret_cast<const f32x4*>(ob + r * (D * 4) + ((lane ^ r) << 4));
          const int rw = RW * w + 32 * mb + 16 * p + r;  // row within the workgroup
          const size_t orow = (((size_t)b * S + t0 + rw / G) * a.Hq + hkv * G + rw % G) * D;
          if constexpr (OBF) {
            __builtin_nontemporal_store(
                u32x2{pack_bf16(o[0], o[1]), pack_bf16(o[2], o[3])},
                reinterpret_cast<u32x2*>(static_cast<uint16_t*>(a.out) + orow + 4 * lane));
          } else {
            __builtin_nontemporal_store(
                o, reinterpret_cast<f32x4*>(static_cast<float*>(a.out) + orow + 4 * lane));
          }
        }
      }
    }
  } else if constexpr (SPREAD) {
    // each wave writes its half of the dims for its own rows (blocks 0..7)
    // and the partner's rows (blocks 8..15); the row sums and overflow flags
    // of the partner's rows come through LDS (the loop ended with a barrier
    // after the last reads of the exchange buffer)
    const float lt = l_run[0] + __shfl_xor(l_run[0], 32);
    ovf |= __shfl_xor(ovf, 32);
    float* xl = reinterpret_cast<float*>(pxb);
    int* xo = reinterpret_cast<int*>(pxb + NW * 64 * 4);
    xl[w * 64 + lane] = lt;
    xo[w * 64 + lane] = ovf;
    __syncthreads();
    const float lt_p = xl[(w ^ 1) * 64 + lane];
    const int ovf_p = xo[(w ^ 1) * 64 + lane];
    const int rp = RW * (w ^ 1) + l32;  // the partner's row of this lane
    const int tp = t0 + rp / G, hp = hkv * G + rp % G;
    const int hf = w & 1;
#pragma unroll
    for (int rb = 0; rb < 2; ++rb) {
      const bool ok = rb ? (tp < S && !(ovf_p & 1)) : (row_ok[0] && !(ovf & 1));
      if (!ok) continue;
      const float inv = 1.f / (rb ? lt_p : lt);
      const size_t obase = rb ? (((size_t)b * S + tp) * a.Hq + hp) * D
                              : (((size_t)b * S + tq[0]) * a.Hq + hq[0]) * D;
#pragma unroll
      for (int db = 0; db < NDB / 2; ++db)
#pragma unroll
        for (int g4 = 0; g4 < 4; ++g4) {
          const int dim = 256 * hf + 32 * db + 8 * g4 + 4 * hl;
          const f32x16& o = oacc[0][(NDB / 2) * rb + db];
          const float o0 = o[4 * g4 + 0] * inv, o1 = o[4 * g4 + 1] * inv;
          const float o2 = o[4 * g4 + 2] * inv, o3 = o[4 * g4 + 3] * inv;
          if constexpr (OBF) {
            u32x2 pk = {pack_bf16(o0, o1), pack_bf16(o2, o3)};
            *reinterpret_cast<u32x2*>(static_cast<uint16_t*>(a.out) + obase + dim) = pk;
          } else {
            *reinterpret_cast<f32x4*>(static_cast<float*>(a.out) + obase + dim) =
                f32x4{o0, o1, o2, o3};
          }
        }
    }
  } else {
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
      const float lt = l_run[mb] + __shfl_xor(l_run[mb], 32);
      if (!row_ok[mb] || ((ovf >> mb) & 1)) continue;
      const float inv = (VIS && tq[mb] >= nv) ? 0.f : 1.f / lt;
      const size_t obase = (((size_t)b * S + tq[mb]) * a.Hq + hq[mb]) * D;
#pragma unroll
      for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int g4 = 0; g4 < 4; ++g4) {
          const int dim = 32 * db + 8 * g4 + 4 * hl;
          const float o0 = oacc[mb][db][4 * g4 + 0] * inv, o1 = oacc[mb][db][4 * g4 + 1] * inv;
          const float o2 = oacc[mb][db][4 * g4 + 2] * inv, o3 = oacc[mb][db][4 * g4 + 3] * inv;
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

  // ---- rows flagged above: exact recompute with the known row max ----
  // One wave per row, lanes over head dims; taken only when some row's score
  // grew 2^64 past its first visible tile (never for normalised data).
  ovf |= __shfl_xor(ovf, 32);
  if (__any(ovf)) {
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
      unsigned long long rows = __ballot(((ovf >> mb) & 1) && row_ok[mb]) & 0xffffffffull;
      while (rows) {
        const int src_lane = __builtin_ctzll(rows);
        rows &= rows - 1;
        const int t = __shfl(tq[mb], src_lane), h = __shfl(hq[mb], src_lane);
        exact_row<D, OBF, VIS>(static_cast<const uint16_t*>(a.q),
                               static_cast<const uint16_t*>(a.k),
                               static_cast<const uint16_t*>(a.v), a.out, a.pos, S, a.Hq, a.Hkv,
                               W, n_rot, cs, b, hkv, t, h, a.log2_theta, nv);
      }
    }
  }
}

// Rotated key slab for slab width SW, then the attention kernel, on stream st.
template <int D, int G, bool KVS, bool OBF, int SW, int NST, int MB, bool SPREAD = false,
          bool VIS = false>
hipError_t launch(const PrefillArgs& a, hipStream_t st) {
  constexpr int TQ = NW * 32 * MB / G;
  PrefillArgs x = a;
  x.nq = (a.S + TQ - 1) / TQ;
  x.nheads = a.B * a.Hkv;
  const long long nblk = (long long)x.nq * x.nheads;
  if (nblk == 0) return hipSuccess;
  if (nblk > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  const long long nchunks = (long long)a.B * a.S * a.Hkv * (SW / 8);
  const long long rblk = (nchunks + 255) / 256;
  hipLaunchKernelGGL((rope_keys_kernel<SW, VIS>), dim3((unsigned)(rblk < 65536 ? rblk : 65536)),
                     dim3(256), 0, st, static_cast<const uint16_t*>(a.k),
                     static_cast<uint16_t*>(a.ws), a.pos, nchunks, a.Hkv, D, a.n_rot,
                     a.log2_theta);
  if (SPREAD && a.window != 0) return hipErrorInvalidValue;
  hipLaunchKernelGGL((prefill_kernel<D, G, KVS, OBF, SW, NST, MB, SPREAD, VIS>), dim3((unsigned)nblk),
                     dim3(NW * 64), 0, st, x);
  return hipGetLastError();
}

}  // namespace pf
}  // namespace g4a
