// Pieces shared by the split-KV decode kernels (bf16 cache and fp8 cache):
// buffer resources and 16-byte direct-to-LDS loads, the grid -> (column
// block, chunk, sequence, KV head) mapping, and the end of a chunk (partial
// (m, l, O) to the workspace, or the merge of a workgroup's waves in LDS).
#pragma once
#include "common.hpp"
#include "kernels.hpp"

namespace g4a {
namespace dec {

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  const uint64_t p = reinterpret_cast<uint64_t>(base);
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)p);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(p >> 32));
  const uint32_t n = __builtin_amdgcn_readfirstlane(bytes);
  void* u = reinterpret_cast<void*>(((uint64_t)hi << 32) | lo);
  return __builtin_amdgcn_make_buffer_rsrc(u, (short)0, (int)n, 0x00020000);
}

// Cache policy of the cache-row loads.  With one column block per chunk every
// cache row is read once per launch, so it is loaded non-temporal: keeping it
// in L2 helps nothing, and the batch-64 decodes ran at 55.4-57.0 us (local)
// and 792-807 us (global) with the default policy against 52.4-52.5 and
// 708-769 us non-temporal (same box).  With several column blocks in
// separate workgroups (several query tokens over separate K and V caches)
// the later blocks of a chunk read it again from L2, and non-temporal loads
// made the 4-token global decode slower when it still ran that way (1448 ->
// 1643 us), so those keep the default policy.  K=V caches with more than 16
// columns read each tile once for every block (decode_mc.hip).
constexpr int CPOL_NT = 2;

// 16 bytes at voff of the resource into LDS at ldst + 16 * lane (reads past
// the resource's size return zeros); nt: non-temporal (wave-uniform)
__device__ __forceinline__ void lds_dma16(__amdgpu_buffer_rsrc_t rs, uint32_t voff,
                                          unsigned char* ldst, bool nt) {
  auto* l = (__attribute__((address_space(3))) void*)(ldst);
  if (nt) __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, l, 16, voff, 0, 0, CPOL_NT);
  else __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, l, 16, voff, 0, 0, 0);
}

// Workgroup barrier that leaves the tile loads in flight: this wave's LDS
// writes have completed, its vector-memory operations are not waited for.
// (__syncthreads' release fence waits for every outstanding load, the
// direct-to-LDS tile loads included, so with it no tile stays in flight
// across a step.)  The memory clobber keeps the compiler from moving LDS
// accesses across it.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// Buffer resource as four scalar words (base, stride 0, size in bytes, raw
// 32-bit dwords), for loads issued from inline assembly.
typedef uint32_t s32x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ s32x4 rsrc_words(const void* base, uint32_t bytes) {
  const uint64_t p = reinterpret_cast<uint64_t>(base);
  return s32x4{(uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)p),
               (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)(p >> 32)) & 0xffffu,
               (uint32_t)__builtin_amdgcn_readfirstlane(bytes), 0x00020000u};
}

// Non-temporal 16-byte direct load into LDS (lane l's bytes at ldst + 16 l),
// issued from inline assembly.  The compiler's wait insertion cannot tell
// which LDS object a builtin direct load writes, so after one it waits for
// every outstanding load before the next LDS read, which drains a ring of
// tiles each step.  It does not see this one: the kernel orders the tile
// reads itself (wait_vmcnt, and a barrier where waves share a tile).  The
// instruction writes no register.
__device__ __forceinline__ void lds_dma16_nt_asm(s32x4 rs, uint32_t voff, unsigned char* ldst) {
  // the low 32 bits of a generic address in the LDS aperture are the LDS
  // offset (the aperture is 4 GiB aligned)
  const uint32_t m = __builtin_amdgcn_readfirstlane((uint32_t)reinterpret_cast<uintptr_t>(ldst));
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dwordx4 %1, %2, 0 offen nt lds"
               :: "s"(m), "v"(voff), "s"(rs) : "memory", "m0");
}

template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

template <class T>
__device__ __forceinline__ T& lds_at(unsigned char* base, int off) {
  return *reinterpret_cast<T*>(base + off);
}

// Work unit of a split workgroup: column block cb (16 (query token, head)
// columns), chunk ch of the cache rows, sequence b, KV head hkv.  b < 0: the
// workgroup has no unit and returns at once.
struct Unit {
  int cb, ch, b, hkv;
};

// Chunks of sequence b that hold a row its queries may see.  A sequence whose
// position is out of range has none: the merge kernel writes its NaN rows.
__device__ __forceinline__ int active_chunks(const DecodeArgs& a, int P) {
  if (P < 0 || (a.window == 0 && P >= a.capacity)) return 0;
  const int last = a.window > 0 ? min(P, a.capacity - 1) : P;
  return min(last / a.chunk + 1, a.nchunk);
}

// Inclusive prefix sum over the 64 lanes of a wave.
__device__ __forceinline__ int wave_scan_incl(int v) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int t = __shfl_up(v, d);
    v += lane >= d ? t : 0;
  }
  return v;
}

// Grid index -> unit.  Units are the (sequence, KV head, chunk) triples with
// a visible row, chunk fastest, numbered densely: the grid is sized for every
// chunk of the capacity, and the blocks past the active units (sequences
// shorter than the capacity leave many) all sit at the end of the grid and
// return at once.  With the empty blocks interleaved among the working ones
// (a fixed block per chunk of the capacity), shader-clock probes of a batch-64
// K=V decode found working waves in only about 61% of the wave slots over the
// launch, against 90% with the dense numbering, and the lower XCDs received
// more units than the upper ones.
// Units go in groups of 8; the column blocks of the units of a group take
// grid indices 8 apart (r apart in a last, smaller group of r units).
// Workgroups are dealt to the 8 XCDs in grid order, so every column block of
// a chunk runs on the same XCD at about the same time and its later reads of
// the chunk hit that XCD's L2; and each XCD receives the same number of units.
// One chunk per sequence (rings): every (sequence, KV head) is a unit, so the
// workgroup of a sequence with a bad position writes its NaN rows itself.
__device__ __forceinline__ Unit unit_of_block(const DecodeArgs& a) {
  const int lane = threadIdx.x & 63;
  int nunit;
  if (a.nchunk == 1) {
    nunit = a.B * a.Hkv;
  } else {
    int total = 0;
    for (int b0 = 0; b0 < a.B; b0 += 64) {
      const int b = b0 + lane;
      total += __shfl(wave_scan_incl(b < a.B ? active_chunks(a, a.pos[b]) : 0), 63);
    }
    nunit = __builtin_amdgcn_readfirstlane(total) * a.Hkv;
  }
  const int grp = blockIdx.x / (8 * a.ncb);
  const int gsz = min(8, nunit - 8 * grp);  // units in this group
  if (gsz <= 0) return Unit{0, 0, -1, 0};
  const int within = blockIdx.x - grp * 8 * a.ncb;
  if (within >= gsz * a.ncb) return Unit{0, 0, -1, 0};  // past the last unit's blocks
  const int unit = 8 * grp + within % gsz;
  const int cb = within / gsz;
  if (a.nchunk == 1) return Unit{cb, 0, unit / a.Hkv, unit % a.Hkv};
  // the sequence whose units [acc + excl, acc + incl) hold `unit`
  int acc = 0;
  for (int b0 = 0; b0 < a.B; b0 += 64) {
    const int b = b0 + lane;
    const int n = b < a.B ? active_chunks(a, a.pos[b]) : 0;
    const int incl = wave_scan_incl(n * a.Hkv);
    const unsigned long long hit = __ballot(acc + incl > unit);
    if (hit) {
      const int l = __builtin_ctzll(hit);
      const int nb = __builtin_amdgcn_readfirstlane(__shfl(n, l));
      const int rem = unit - acc - __builtin_amdgcn_readfirstlane(__shfl(incl, l)) + nb * a.Hkv;
      return Unit{cb, rem % nb, b0 + l, rem / nb};
    }
    acc += __builtin_amdgcn_readfirstlane(__shfl(incl, 63));
  }
  return Unit{0, 0, -1, 0};
}

// End of a chunk.  oacc holds O^T of this wave (lane (g4, l16): dims
// 16*db + 4*g4 + r of column l16), m_run / l_run the column's running max
// (base 2) and sum, already summed over the lanes of the column.
//   NW == 1: the wave writes its partial (m, l, O) to the workspace.
//   NW > 1: the waves merge through LDS (ow: NW * 8 * D floats, mls: (m, l)
//   per wave and column); the merged chunk goes to the workspace, or, when
//   `direct` (one chunk covers every row), is normalised into the output.
// Columns go in passes of 8 so a wave's LDS share holds 8 columns of D floats.
template <int D, int NW, bool OBF, class ColOut, class ColPos>
__device__ __forceinline__ void finish_chunk(const DecodeArgs& a, const f32x4 (&oacc)[D / 16],
                                             float m_run, float l_run, int ch, int ncol,
                                             bool direct, float* ow, float (*mls)[16][2],
                                             ColOut col_out, ColPos col_pos) {
  constexpr int NB = D / 16;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int l16 = lane & 15, g4 = lane >> 4;
  const bool col_ok = l16 < ncol;
  if constexpr (NW == 1) {
    if (col_ok) {
      const size_t prow = (col_out(l16) / D) * a.nchunk + ch;
      float* po = a.part_o + prow * D + 4 * g4;
#pragma unroll
      for (int db = 0; db < NB; ++db) *reinterpret_cast<f32x4*>(po + 16 * db) = oacc[db];
      if (g4 == 0) {
        a.part_ml[prow * 2 + 0] = m_run;
        a.part_ml[prow * 2 + 1] = l_run;
      }
    }
  } else {
    constexpr int MC = 8;
    if (col_ok && g4 == 0) {
      mls[w][l16][0] = m_run;
      mls[w][l16][1] = l_run;
    }
    for (int c0 = 0; c0 < ncol; c0 += MC) {
      __syncthreads();
      if (col_ok && l16 >= c0 && l16 < c0 + MC) {
#pragma unroll
        for (int db = 0; db < NB; ++db)
          *reinterpret_cast<f32x4*>(ow + ((size_t)w * MC + l16 - c0) * D + 16 * db + 4 * g4) =
              oacc[db];
      }
      __syncthreads();
      const int nc = min(MC, ncol - c0);
      for (int idx = threadIdx.x; idx < nc * D / 4; idx += 64 * NW) {
        const int n = c0 + idx / (D / 4), e = 4 * (idx % (D / 4));
        float M = -INFINITY;
#pragma unroll
        for (int v = 0; v < NW; ++v) M = fmaxf(M, mls[v][n][0]);
        f32x4 o = {};
        float l = 0.f;
#pragma unroll
        for (int v = 0; v < NW; ++v) {
          // 0 for a wave that saw no key of this column (and for all, if none did)
          const float f = M == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(mls[v][n][0] - M);
          o += f * *reinterpret_cast<const f32x4*>(ow + ((size_t)v * MC + n - c0) * D + e);
          l += f * mls[v][n][1];
        }
        if (direct) {
          // every column sees its own key unless its position is negative
          o = col_pos(n) >= 0 ? o * (1.f / l) : f32x4{__builtin_nanf(""), __builtin_nanf(""),
                                                        __builtin_nanf(""), __builtin_nanf("")};
          const size_t orow = col_out(n) + e;
          if constexpr (OBF) {
            const u32x2 pk = {pack_bf16(o[0], o[1]), pack_bf16(o[2], o[3])};
            *reinterpret_cast<u32x2*>(static_cast<uint16_t*>(a.out) + orow) = pk;
          } else {
            *reinterpret_cast<f32x4*>(static_cast<float*>(a.out) + orow) = o;
          }
        } else {
          const size_t prow = (col_out(n) / D) * a.nchunk + ch;
          *reinterpret_cast<f32x4*>(a.part_o + prow * D + e) = o;
          if (e == 0) {
            a.part_ml[prow * 2 + 0] = M;
            a.part_ml[prow * 2 + 1] = l;
          }
        }
      }
    }
  }
}

// NaN rows of the block's columns (a sequence whose position is out of range)
template <int D, int NW, bool OBF, class ColOut>
__device__ __forceinline__ void nan_columns(const DecodeArgs& a, int ncol, ColOut col_out) {
  for (int idx = threadIdx.x; idx < ncol * D; idx += 64 * NW) {
    const size_t o = col_out(idx / D) + idx % D;
    if constexpr (OBF) static_cast<uint16_t*>(a.out)[o] = 0x7fc0;
    else static_cast<float*>(a.out)[o] = __builtin_nanf("");
  }
}

}  // namespace dec
}  // namespace g4a
