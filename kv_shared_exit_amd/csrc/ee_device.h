// Device helpers shared by the gfx950 kernels: bf16 conversions, the bf16 dot
// product, the cross-lane transpose-reduce and the (max, sum exp) / top-2
// merges used by the vocabulary reductions.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <math.h>

#include <type_traits>

namespace ee {

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

typedef unsigned u32x4_t __attribute__((ext_vector_type(4)));

// Streaming 16-byte load that does not allocate in the caches (weights are
// read once per launch).
__device__ __forceinline__ uint4 ld_stream(const void* p) {
  return __builtin_bit_cast(uint4, __builtin_nontemporal_load((const u32x4_t*)p));
}

__device__ __forceinline__ float bf2f(uint32_t b) { return __uint_as_float(b << 16); }

// float32 -> bf16 bits, round to nearest, ties to even (inputs are finite)
__device__ __forceinline__ uint32_t f2bf(float f) {
  const uint32_t u = __float_as_uint(f);
  return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

__device__ __forceinline__ float dot2(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a),
                                         __builtin_bit_cast(bf16x2_t, b), c, false);
}

// The value held by lane ^ M (M = 1, 2, 4, 8, 16 or 32) without an LDS round
// trip: within a row of 16 lanes through the DPP modifier (quad permutes for 1
// and 2; for 4, a shift left by 4 into the lanes whose bit 2 is clear and a
// shift right into the others, chosen by the bank mask; a rotation by 8 for
// 8), across rows with the gfx950 permlane swaps (each returns the lower half
// of the pair duplicated and the upper half duplicated: the partner is the
// other half).  Every lane of the wave must be active.
template <int M>
__device__ __forceinline__ int xor_lane(int v, int lane) {
  static_assert(M == 1 || M == 2 || M == 4 || M == 8 || M == 16 || M == 32, "lane offset");
  if constexpr (M == 1) {
    return __builtin_amdgcn_mov_dpp(v, 0xB1, 0xF, 0xF, false);
  } else if constexpr (M == 2) {
    return __builtin_amdgcn_mov_dpp(v, 0x4E, 0xF, 0xF, false);
  } else if constexpr (M == 4) {
    const int t = __builtin_amdgcn_update_dpp(v, v, 0x104, 0xF, 0x5, false);
    return __builtin_amdgcn_update_dpp(t, v, 0x114, 0xF, 0xA, false);
  } else if constexpr (M == 8) {
    return __builtin_amdgcn_mov_dpp(v, 0x128, 0xF, 0xF, false);
  } else if constexpr (M == 16) {
    const auto r = __builtin_amdgcn_permlane16_swap((unsigned)v, (unsigned)v, false, false);
    return (int)((lane & 16) ? r[0] : r[1]);
  } else {
    const auto r = __builtin_amdgcn_permlane32_swap((unsigned)v, (unsigned)v, false, false);
    return (int)((lane & 32) ? r[0] : r[1]);
  }
}

template <int M>
__device__ __forceinline__ float xor_lane(float v, int lane) {
  return __int_as_float(xor_lane<M>(__float_as_int(v), lane));
}

// f(std::integral_constant<int, M>) for M = FROM, 2 FROM, ..., up to 32
template <int FROM, typename F>
__device__ __forceinline__ void each_offset_up(F&& f) {
  if constexpr (FROM <= 32) {
    f(std::integral_constant<int, FROM>{});
    each_offset_up<2 * FROM>(f);
  }
}

// f(std::integral_constant<int, M>) for M = 32, 16, ..., down to TO
template <int TO, int M = 32, typename F>
__device__ __forceinline__ void each_offset_down(F&& f) {
  if constexpr (M >= TO) {
    f(std::integral_constant<int, M>{});
    each_offset_down<TO, M / 2>(f);
  }
}

// Lane exchange within a row of 16 lanes through the DPP modifier (no LDS
// round trip): C is the DPP control (0xB1 quad_perm [1,0,3,2], 0x4E quad_perm
// [2,3,0,1], 0x141 row_half_mirror, 0x140 row_mirror).
template <int C>
__device__ __forceinline__ float dpp_f(float v) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), C, 0xF, 0xF, false));
}

// Sum over each aligned group of N adjacent lanes (N = 1, 2, 4, 8 or 16),
// left in every lane of the group: exchanges with lane ^ 1 and lane ^ 2, then
// with the mirrored lane of the 8- and the 16-lane half (after the quads hold
// their sums, the mirrored lane holds the other quad's, or the other half's).
template <int N>
__device__ __forceinline__ float group_sum_dpp(float v) {
  static_assert(N == 1 || N == 2 || N == 4 || N == 8 || N == 16, "group of 1..16 lanes");
  if constexpr (N >= 2) v += dpp_f<0xB1>(v);
  if constexpr (N >= 4) v += dpp_f<0x4E>(v);
  if constexpr (N >= 8) v += dpp_f<0x141>(v);
  if constexpr (N >= 16) v += dpp_f<0x140>(v);
  return v;
}

// ---------------------------------------------------------------------------
// Cross-lane "transpose-reduce": V partial sums per lane, summed over the 64
// lanes of the wave.  Each halving stage keeps half of the values and trades
// the other half with the partner lane, so the total work is ~2V exchanges
// instead of 6V.  Afterwards lane l holds the sum for value index xidx<V>(l)
// (lanes >= V hold copies).
// ---------------------------------------------------------------------------
template <int V, int S>
struct XRed {
  __device__ __forceinline__ static void run(float* v, int lane) {
    if constexpr ((1 << S) < V) {
      constexpr int half = V >> (S + 1);
      const bool hi = (lane >> S) & 1;
#pragma unroll
      for (int i = 0; i < half; ++i) {
        const float keep = hi ? v[half + i] : v[i];
        const float send = hi ? v[i] : v[half + i];
        v[i] = keep + xor_lane<(1 << S)>(send, lane);
      }
      XRed<V, S + 1>::run(v, lane);
    } else if constexpr (S < 6) {
      v[0] += xor_lane<(1 << S)>(v[0], lane);
      XRed<V, S + 1>::run(v, lane);
    }
  }
};

template <int V>
__device__ __forceinline__ int xidx(int lane) {
  int idx = 0;
#pragma unroll
  for (int s = 0; (1 << s) < V; ++s)
    if ((lane >> s) & 1) idx += V >> (s + 1);
  return idx;
}

__device__ __forceinline__ void lse_merge(float& m, float& s, float m2, float s2) {
  const float M = fmaxf(m, m2);
  if (M == -INFINITY) return;
  s = s * __expf(m - M) + s2 * __expf(m2 - M);
  m = M;
}

struct Top2 {
  float v1;
  int i1;
  float v2;
};

__device__ __forceinline__ void top2_merge(Top2& a, const Top2& o) {
  if (o.v1 > a.v1 || (o.v1 == a.v1 && o.i1 < a.i1)) {
    a.v2 = fmaxf(o.v2, a.v1);
    a.v1 = o.v1;
    a.i1 = o.i1;
  } else {
    a.v2 = fmaxf(a.v2, o.v1);
  }
}

}  // namespace ee
