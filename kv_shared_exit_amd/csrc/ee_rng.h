// Counter-based random draws of sampled decoding: Philox4x64 with 10 rounds
// (Salmon, Moraes, Dror, Shaw, "Parallel random numbers: as easy as 1, 2, 3",
// SC 2011).  Each vocabulary entry v of a draw takes word v % 4 of the block
// with counter (v / 4, sequence, position, stream) and key (seed, 0), so any
// thread draws any entry's number without state.  A word x gives the uniform
// u = ((x >> 41) + 0.5) / 2^23 in (0, 1), exact in float32; a Gumbel variate
// is -log(-log(u)).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ee {

__device__ __forceinline__ uint64_t philox_word(uint64_t seed, uint64_t pos, uint64_t seq, uint64_t stream,
                                                uint64_t v) {
  constexpr uint64_t M0 = 0xD2E7470EE14C6C93ull, M1 = 0xCA5A826395121157ull;
  constexpr uint64_t W0 = 0x9E3779B97F4A7C15ull, W1 = 0xBB67AE8584CAA73Bull;
  uint64_t x0 = v >> 2, x1 = seq, x2 = pos, x3 = stream;
  uint64_t k0 = seed, k1 = 0;
#pragma unroll
  for (int r = 0; r < 10; ++r) {
    if (r) {
      k0 += W0;
      k1 += W1;
    }
    const uint64_t hi0 = __umul64hi(M0, x0), lo0 = M0 * x0;
    const uint64_t hi1 = __umul64hi(M1, x2), lo1 = M1 * x2;
    const uint64_t y0 = hi1 ^ x1 ^ k0, y2 = hi0 ^ x3 ^ k1;
    x0 = y0;
    x1 = lo1;
    x2 = y2;
    x3 = lo0;
  }
  const int w = (int)(v & 3);
  return w == 0 ? x0 : w == 1 ? x1 : w == 2 ? x2 : x3;
}

__device__ __forceinline__ float philox_uniform(uint64_t x) { return ((float)(x >> 41) + 0.5f) * 0x1p-23f; }

// Above every Gumbel value these uniforms give (the largest, 1 - 2^-24, gives
// -log(-log u) = 16.64): an entry whose score is more than this below the best
// perturbed score so far cannot win a draw, so its noise is not computed.
constexpr float kGumbelMax = 16.7f;

__device__ __forceinline__ float gumbel_noise(uint32_t seed, int pos, int seq, int stream, int v) {
  const float u = philox_uniform(philox_word(seed, (uint64_t)pos, (uint64_t)seq, (uint64_t)stream, (uint64_t)v));
  return -logf(-logf(u));
}

}  // namespace ee
