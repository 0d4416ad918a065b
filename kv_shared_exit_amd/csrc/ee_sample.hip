// Sampled decoding with AdaDecode's verification (AdaDecode explainer,
// section 3.1): the token a sequence predicts at its exit layer is a draft,
// accepted with probability min(1, p_final / p_draft); a rejected draft is
// replaced by a draw from the normalised relu(p_final - p_draft).  With
// temperature tau, p_draft = softmax(exit-head logits / tau) at the exit layer
// (section 2.2: the draft is made where the head's confidence passes the
// threshold) and p_final = softmax(final logits / tau); a sequence that runs
// every layer has no draft and draws from p_final.  Draws are Gumbel-max over
// counter-based noise (ee_rng.h), so every workgroup of a vocabulary pass keeps
// only its best perturbed score; the acceptance uniform is word 0 of the block
// (0, sequence, position, STREAM_ACCEPT).
//
// Partials (per workgroup k and sequence b, kPartS floats at part_s[k][b]):
//   after EPI_LSE_S:    max and sum exp of logit / tau, best perturbed score,
//                       its index, the logit at that index
//   after EPI_ARGMAX_S: the same for the final logits, the final logit at the
//                       draft's index in the 5th float (-inf elsewhere)
//   after EPI_RESAMPLE: best perturbed score and index of the residual draw
#include "ee_internal.h"
#include "ee_device.h"
#include "ee_rng.h"

#include <stdexcept>

namespace ee {

namespace {

constexpr int kThreads = 512;  // one wave per sequence
constexpr int kWavesS = kThreads / 64;
constexpr int kPer = kNwgMax / 64;  // partials per lane

struct Merged {
  float m, s;   // max and sum exp (log sum exp = m + log s)
  float best;   // best perturbed score
  int idx;      // its index (lowest on ties)
  float logit;  // the largest 5th float
};

// Merges the nwg partials of sequence b across the wave (all loads issued
// before any is used); every lane returns the result.
__device__ Merged merge_parts(const float* part_s, int nwg, int b, int lane) {
  float4 v[kPer];
  float l5[kPer];
#pragma unroll
  for (int j = 0; j < kPer; ++j) {
    const int k = min(lane + 64 * j, nwg - 1);
    const float* p = part_s + ((size_t)k * kMaxBatch + b) * kPartS;
    v[j] = *(const float4*)p;
    l5[j] = p[4];
  }
  Merged r{-INFINITY, 0.0f, -INFINITY, 0x7fffffff, -INFINITY};
#pragma unroll
  for (int j = 0; j < kPer; ++j) {
    if (lane + 64 * j >= nwg) continue;
    lse_merge(r.m, r.s, v[j].x, v[j].y);
    const int i = __float_as_int(v[j].w);
    if (v[j].z > r.best || (v[j].z == r.best && i < r.idx)) {
      r.best = v[j].z;
      r.idx = i;
    }
    r.logit = fmaxf(r.logit, l5[j]);
  }
  each_offset_up<1>([&](auto mc) {
    constexpr int M = decltype(mc)::value;
    lse_merge(r.m, r.s, xor_lane<M>(r.m, lane), xor_lane<M>(r.s, lane));
    const float b2 = xor_lane<M>(r.best, lane);
    const int i2 = xor_lane<M>(r.idx, lane);
    if (b2 > r.best || (b2 == r.best && i2 < r.idx)) {
      r.best = b2;
      r.idx = i2;
    }
    r.logit = fmaxf(r.logit, xor_lane<M>(r.logit, lane));
  });
  return r;
}

}  // namespace

// The draft of each sequence that left the backbone after `layer` (forced or
// not): Gumbel-max of its exit logits / tau, that logit, and the log sum exp;
// its z row (the exit head's input to E) is kept for the resampling pass.
__global__ __launch_bounds__(kThreads) void sample_draft_kernel(StepState* st, const float* part_s, int nwg,
                                                                int layer, int B, const uint16_t* z, uint16_t* zx,
                                                                int d) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  for (int b = w; b < B; b += kWavesS) {
    if (st->e[b] != layer) continue;  // uniform over the wave
    const Merged r = merge_parts(part_s, nwg, b, lane);
    if (lane == 0) {
      st->draft_tok[b] = r.idx;
      st->draft_logit[b] = r.logit;
      st->draft_lse[b] = r.m + logf(r.s);
    }
    const uint4* src = (const uint4*)(z + (size_t)b * d);
    uint4* dst = (uint4*)(zx + (size_t)b * d);
    for (int i = lane; i < d / 8; i += 64) dst[i] = src[i];
  }
}

// The emitted token of every sequence: without a draft, the final
// distribution's Gumbel-max; with one, the draft if u p_draft < p_final,
// otherwise the sequence is queued for the resampling pass as the row pair
// (b, 64 + b).
__global__ __launch_bounds__(kThreads) void sample_final_kernel(StepState* st, const float* part_s, int nwg, int B,
                                                                int L, int V, const int32_t* lens, float itau,
                                                                uint32_t seed) {
  __shared__ int rejected[kMaxBatch];
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  for (int b = w; b < B; b += kWavesS) {
    const Merged r = merge_parts(part_s, nwg, b, lane);
    if (lane == 0) {
      const float lse = r.m + logf(r.s);
      st->lse_f[b] = lse;
      int tok = (r.idx >= 0 && r.idx < V) ? r.idx : 0;
      int rej = 0;
      const int dt = st->draft_tok[b];
      if (st->e[b] < L && dt >= 0) {
        const float pf = __expf(r.logit * itau - lse);
        const float pd = __expf(st->draft_logit[b] * itau - st->draft_lse[b]);
        const float u = philox_uniform(philox_word(seed, (uint64_t)lens[b], (uint64_t)b, STREAM_ACCEPT, 0));
        if (u * pd < pf) {
          tok = dt;
        } else {
          rej = 1;
        }
      }
      rejected[b] = rej;
      st->out_tok[b] = tok;
      st->tok[b] = tok;
    }
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    int n = 0;
    for (int b = 0; b < B; ++b)
      if (rejected[b]) {
        st->rej[n++] = b;
        st->rej[n++] = kMaxBatch + b;
      }
    st->n_rej = n;
  }
}

// The resampled tokens of the rejected sequences; then every length advances
// and the drafts are cleared for the next step.
__global__ __launch_bounds__(kThreads) void resample_final_kernel(StepState* st, const float* part_s, int nwg,
                                                                  int B, int V, int32_t* lens) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int n = min(max(st->n_rej, 0), 2 * kMaxBatch);
  for (int i = 2 * w; i < n; i += 2 * kWavesS) {
    const int b = st->rej[i];
    float bv[kPer];
    int bi[kPer];
#pragma unroll
    for (int j = 0; j < kPer; ++j) {
      const int k = min(lane + 64 * j, nwg - 1);
      const float* p = part_s + ((size_t)k * kMaxBatch + b) * kPartS;
      bv[j] = p[0];
      bi[j] = __float_as_int(p[1]);
    }
    float best = -INFINITY;
    int idx = 0x7fffffff;
#pragma unroll
    for (int j = 0; j < kPer; ++j)
      if (lane + 64 * j < nwg && (bv[j] > best || (bv[j] == best && bi[j] < idx))) {
        best = bv[j];
        idx = bi[j];
      }
    each_offset_up<1>([&](auto mc) {
      constexpr int M = decltype(mc)::value;
      const float b2 = xor_lane<M>(best, lane);
      const int i2 = xor_lane<M>(idx, lane);
      if (b2 > best || (b2 == best && i2 < idx)) {
        best = b2;
        idx = i2;
      }
    });
    if (lane == 0) {
      const int tok = (idx >= 0 && idx < V) ? idx : 0;  // an empty residual cannot be drawn from: token 0
      st->out_tok[b] = tok;
      st->tok[b] = tok;
    }
  }
  __syncthreads();
  if ((int)threadIdx.x < B) {
    lens[threadIdx.x] += 1;
    st->draft_tok[threadIdx.x] = -1;
  }
}

void launch_sample_draft(StepState* st, const float* part_s, int nwg, int layer, int B, const uint16_t* z,
                         uint16_t* zx, int d, hipStream_t s) {
  if (nwg < 1 || nwg > kNwgMax || B < 1 || B > kMaxBatch || d % 8 || !part_s || !z || !zx)
    throw std::logic_error("sample_draft: bad arguments");
  hipLaunchKernelGGL(sample_draft_kernel, dim3(1), dim3(kThreads), 0, s, st, part_s, nwg, layer, B, z, zx, d);
}

void launch_sample_final(StepState* st, const float* part_s, int nwg, int B, int L, int V, const int32_t* lens,
                         float itau, uint32_t seed, hipStream_t s) {
  if (nwg < 1 || nwg > kNwgMax || B < 1 || B > kMaxBatch || !part_s || !(itau > 0.0f))
    throw std::logic_error("sample_final: bad arguments");
  hipLaunchKernelGGL(sample_final_kernel, dim3(1), dim3(kThreads), 0, s, st, part_s, nwg, B, L, V, lens, itau,
                     seed);
}

void launch_resample_final(StepState* st, const float* part_s, int nwg, int B, int V, int32_t* lens,
                           hipStream_t s) {
  if (nwg < 1 || nwg > kNwgMax || B < 1 || B > kMaxBatch || !part_s)
    throw std::logic_error("resample_final: bad arguments");
  hipLaunchKernelGGL(resample_final_kernel, dim3(1), dim3(kThreads), 0, s, st, part_s, nwg, B, V, lens);
}

}  // namespace ee
