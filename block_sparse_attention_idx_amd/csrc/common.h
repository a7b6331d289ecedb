// Shared device helpers for the MSA kernels (gfx950 / CDNA4).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace msa {

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef int i32x4 __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;
constexpr float kNegInf = -__builtin_inff();

// 32x32 MFMA tile traits.  Operand layout (checked on gfx950): lane l holds
// A[l % 32][(l / 32) * KPL + e] and B[(l / 32) * KPL + e][l % 32] for
// e < KPL; the 32x32 fp32 result has C[(j / 4) * 8 + (l / 32) * 4 + j % 4][l % 32]
// in register j of lane l.
template <typename T>
struct Mma;

template <>
struct Mma<bf16> {
  static constexpr int KPL = 8;    // k elements per lane per instruction
  static constexpr int KSTEP = 16; // k per instruction
  typedef bf16x8 frag;
  __device__ static inline f32x16 mma(frag a, frag b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
  }
  __device__ static inline frag zero() { return frag{}; }
};

template <>
struct Mma<float> {
  static constexpr int KPL = 1;
  static constexpr int KSTEP = 2;
  typedef float frag;
  __device__ static inline f32x16 mma(frag a, frag b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, 0, 0, 0);
  }
  __device__ static inline frag zero() { return 0.0f; }
};

// row index (within the 32-row tile) held by register j of a lane in half h
__device__ __forceinline__ constexpr int c_row(int j, int h) { return (j / 4) * 8 + h * 4 + (j % 4); }

__device__ __forceinline__ float to_f32(float x) { return x; }
__device__ __forceinline__ float to_f32(bf16 x) { return (float)x; }

template <typename T>
__device__ __forceinline__ T from_f32(float x);
template <>
__device__ __forceinline__ float from_f32<float>(float x) { return x; }
template <>
__device__ __forceinline__ bf16 from_f32<bf16>(float x) { return (bf16)x; }  // round to nearest even

__device__ __forceinline__ float wave_max_xor32(float x) { return fmaxf(x, __shfl_xor(x, 32)); }

struct alignas(16) Chunk16 {
  uint32_t w[4];
};

// Element vector of a 16-byte chunk.
template <typename T> struct Vec16;
template <> struct Vec16<bf16> { typedef bf16x8 type; };
template <> struct Vec16<float> { typedef f32x4 type; };

// E x E transpose of 16-byte rows (E = 16 / sizeof(T)), in registers.  Native
// vector types throughout, so nothing is placed in scratch memory.
template <typename T, int E>
__device__ __forceinline__ void transpose_tile(const i32x4 (&in)[E], i32x4 (&out)[E]) {
  typedef typename Vec16<T>::type V;
  V a[E], o[E];
#pragma unroll
  for (int r = 0; r < E; ++r) a[r] = __builtin_bit_cast(V, in[r]);
#pragma unroll
  for (int c = 0; c < E; ++c)
#pragma unroll
    for (int r = 0; r < E; ++r) o[c][r] = a[r][c];
#pragma unroll
  for (int c = 0; c < E; ++c) out[c] = __builtin_bit_cast(i32x4, o[c]);
}

// One OCP FP8 E4M3 (e4m3fn) value as stored in a KV or index-key cache: sign,
// 4 exponent bits (bias 7), 3 mantissa bits; no infinities, NaN = 0x7f / 0xff.
struct e4m3 {
  uint8_t bits;
};

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// Four e4m3 values (one 32-bit word, lowest byte first) as four bf16 values
// (two 32-bit words).  Every e4m3 value, subnormals included, is a bf16 value,
// so the conversion (v_cvt_scalef32_pk_bf16_fp8 with scale 1) is exact.
__device__ __forceinline__ uint2 e4m3x4_to_bf16(uint32_t w) {
  const bf16x2 lo = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, false);
  const bf16x2 hi = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, true);
  return make_uint2(__builtin_bit_cast(uint32_t, lo), __builtin_bit_cast(uint32_t, hi));
}

// A run of E = 16 / sizeof(T) consecutive cache elements of storage type S,
// loaded raw and later widened to one 16-byte chunk of T.  For S == T that is a
// plain 16-byte load; for e4m3 (T = bf16) an 8-byte load converted exactly.
// Loads and conversions are separate steps so that a kernel can issue all its
// loads before the first conversion waits on one.
template <typename T, typename S>
struct ChunkIO {
  typedef i32x4 raw;
  __device__ static __forceinline__ raw load(const S* p) { return *(const i32x4*)p; }
  __device__ static __forceinline__ i32x4 widen(raw x) { return x; }
};

template <>
struct ChunkIO<bf16, e4m3> {
  typedef uint2 raw;
  __device__ static __forceinline__ raw load(const e4m3* p) { return *(const uint2*)p; }
  __device__ static __forceinline__ i32x4 widen(raw x) {
    const uint2 a = e4m3x4_to_bf16(x.x), b = e4m3x4_to_bf16(x.y);
    return i32x4{(int)a.x, (int)a.y, (int)b.x, (int)b.y};
  }
};

// Top-k order: the higher block score first, on equal scores the lower block.
__device__ __forceinline__ bool ranks_before(float s1, int i1, float s2, int i2) {
  return s1 > s2 || (s1 == s2 && i1 < i2);
}

// x combined with the value of the lane O = 16 or 32 away (lane index xor O)
// by the lane-group swaps, without an LDS round trip: each lane receives its
// own and its partner's value in some order, and sum and max do not care.
template <int O>
__device__ __forceinline__ float xor_sum(float x) {
  static_assert(O == 16 || O == 32, "lane-group swaps");
  const auto p = O == 16 ? __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false)
                         : __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(p[0]) + __uint_as_float(p[1]);
}
template <int O>
__device__ __forceinline__ float xor_max(float x) {
  static_assert(O == 16 || O == 32, "lane-group swaps");
  const auto p = O == 16 ? __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false)
                         : __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(p[0]), __uint_as_float(p[1]));
}

// One butterfly step of a wave-wide "best (score, block id)" reduction: the
// better of this lane's pair and that of its partner, the lane whose index
// differs in bit O and agrees above it.  O < 16 by DPP (quad permutes, then
// the half-row and row mirrors, which pair lanes the same way), O = 16 and 32
// by the lane-group swaps, which hand each lane its own and its partner's
// value in some order -- enough for a symmetric choice.  No LDS round trip.
template <int O>
__device__ __forceinline__ void best_step(float& s, int& i) {
  float os;
  int oi;
  if constexpr (O < 16) {
    constexpr int ctrl = O == 1 ? 0xB1 : O == 2 ? 0x4E : O == 4 ? 0x141 : 0x140;
    os = __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(s), ctrl, 0xF, 0xF, false));
    oi = __builtin_amdgcn_update_dpp(0, i, ctrl, 0xF, 0xF, false);
  } else {
    const auto ps = O == 16 ? __builtin_amdgcn_permlane16_swap(__float_as_uint(s), __float_as_uint(s), false, false)
                            : __builtin_amdgcn_permlane32_swap(__float_as_uint(s), __float_as_uint(s), false, false);
    const auto pi = O == 16 ? __builtin_amdgcn_permlane16_swap((unsigned)i, (unsigned)i, false, false)
                            : __builtin_amdgcn_permlane32_swap((unsigned)i, (unsigned)i, false, false);
    s = __uint_as_float(ps[0]);
    i = (int)pi[0];
    os = __uint_as_float(ps[1]);
    oi = (int)pi[1];
  }
  if (ranks_before(os, oi, s, i)) {
    s = os;
    i = oi;
  }
}

// This lane's entry of a merged selection row: position pos (ascending block
// ids) holds block id; pos = -1 for lanes past the row's selected blocks.
struct MergedSlot {
  int pos, id;
};

// One wave merges the partial top lists of one (query row, group): nl lists of
// cap entries at gs / gi (scores, block ids; each list ordered by ranks_before,
// empty entries id -1 last; a block id appears in at most one list), staged
// through the wave's LDS ss / si (nl * cap entries each; nl <= 128).  The
// first `take` blocks by rank are kept (fewer when the lists hold fewer) and
// the local block L is added.  Lane j < n returns the j-th pick's position
// among the n picks in ascending id order, lane n returns L at position n, the
// other lanes pos = -1.
__device__ inline MergedSlot merge_row_lists(const float* gs, const int32_t* gi, int nl, int cap, int take, int L,
                                             float* ss, int* si, int lane) {
  // the lists in batches of 8 loads per lane, all in flight before any is stored
  for (int e0 = 0; e0 < nl * cap; e0 += 64 * 8) {
    float vs[8];
    int vi[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int e = min(e0 + u * 64 + lane, nl * cap - 1);
      vs[u] = gs[e];
      vi[u] = gi[e];
    }
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int e = e0 + u * 64 + lane;
      if (e < nl * cap) {
        ss[e] = vs[u];
        si[e] = vi[u];
      }
    }
  }
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");

  // take rounds of a wave-wide argmax over the list heads (lists lane and lane + 64)
  int pos0 = 0, pos1 = 0;
  int mywin = 0x7fffffff;
  for (int it = 0; it < take; ++it) {
    float bs = kNegInf;
    int bi = 0x7fffffff, bl = -1;
    if (lane < nl && pos0 < cap) {
      const float s = ss[lane * cap + pos0];
      const int id = si[lane * cap + pos0];
      if (id >= 0) {
        bs = s;
        bi = id;
        bl = 0;
      }
    }
    if (lane + 64 < nl && pos1 < cap) {
      const float s = ss[(lane + 64) * cap + pos1];
      const int id = si[(lane + 64) * cap + pos1];
      if (id >= 0 && ranks_before(s, id, bs, bi)) {
        bs = s;
        bi = id;
        bl = 1;
      }
    }
    float ws = bs;
    int wi = bi;
    best_step<1>(ws, wi);
    best_step<2>(ws, wi);
    best_step<4>(ws, wi);
    best_step<8>(ws, wi);
    best_step<16>(ws, wi);
    best_step<32>(ws, wi);
    // block ids are unique across the lists, so exactly one lane owns the winner
    if (bl >= 0 && bi == wi) {
      if (bl == 0) ++pos0;
      else ++pos1;
    }
    if (lane == it) mywin = wi;
  }
  // rounds that found no entry (lists shorter than take) leave the sentinel
  const int n = __popcll(__ballot(lane < take && mywin != 0x7fffffff));
  int rank = 0;
  for (int m = 0; m < n; ++m) rank += (__builtin_amdgcn_readlane(mywin, m) < mywin) ? 1 : 0;
  if (lane < n) return MergedSlot{rank, mywin};
  if (lane == n) return MergedSlot{n, L};
  return MergedSlot{-1, -1};
}

}  // namespace msa
