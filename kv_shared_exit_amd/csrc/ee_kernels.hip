// gfx950 kernels of the KV-shared early-exit decode step.
//
// The step (River-LLM explainer sections 4.1-4.3; AdaDecode explainer sections
// 2.1-2.2; CALM explainer sections 2.2 and 3.3) is built from these kernels:
//   init       embed the input tokens into the float32 residual, reset the
//              per-step exit state and the row lists
//   rmsnorm    bf16(h * rsqrt(mean(h^2) + eps) * g)
//   proj       the projections: one launch serves the rows still on the
//              backbone (bf16 weights) and the rows that exited (int4 exit
//              copy of the same layer); fused epilogues store bf16, add into
//              the residual, apply SwiGLU, or reduce vocabulary logits to
//              per-workgroup (max, sum exp) or (argmax, top-2) partials
//   rope_kv    rotate q and k, write k and v into the shared cache slot of the
//              position (the same slot for either weight copy)
//   attention  grouped-query decode attention, split over 256-position chunks;
//              K/V tiles staged in LDS, scores on MFMA, softmax per wave, and a
//              combine kernel merging the chunks
//   decide     finish the exit head (p = 1 / sum exp(l - max)), compare with
//              gamma or apply a forced exit, rebuild the backbone/exit row lists
//              with a wave ballot (active-sequence compaction)
//   final      argmax of the LM head, top-2 gap, next input token
//   quantize   build the int4 exit copies (setup)
#include "ee_internal.h"

#include <math.h>

namespace ee {

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

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
        v[i] = keep + __shfl_xor(send, 1 << S);
      }
      XRed<V, S + 1>::run(v, lane);
    } else if constexpr (S < 6) {
      v[0] += __shfl_xor(v[0], 1 << S);
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

// ---------------------------------------------------------------------------
// Projection GEMV
// ---------------------------------------------------------------------------
template <int EPI>
struct EpiTraits {
  static constexpr int R = (EPI == EPI_LSE || EPI == EPI_ARGMAX) ? 8 : 2;  // rows per wave tile
  static constexpr int P = (EPI == EPI_SWIGLU) ? 2 : 1;                     // matrices per tile
};

__device__ __forceinline__ const uint16_t* bf_row(const ProjArgs& a, int n) {
  int s = 0, start = 0;
  if (n >= a.seg_end[0]) {
    s = (n >= a.seg_end[1]) ? 2 : 1;
    start = a.seg_end[s - 1];
  }
  return a.wb[s] + (size_t)(n - start) * a.K;
}

// acc[r * NB + b] += sum_k W_r[k] x_b[k]; lanes own 8-element slices, 512 per step.
template <int RP, int NB>
__device__ __forceinline__ void dot_bf16(const uint16_t* const (&w)[RP], const uint16_t* const (&x)[NB],
                                         int K, int lane, float (&acc)[RP * NB]) {
  for (int k = lane * 8; k < K; k += 512) {
    uint4 wv[RP];
#pragma unroll
    for (int r = 0; r < RP; ++r) wv[r] = *(const uint4*)(w[r] + k);
#pragma unroll
    for (int b = 0; b < NB; ++b) {
      const uint4 xv = *(const uint4*)(x[b] + k);
#pragma unroll
      for (int r = 0; r < RP; ++r) {
        float t = acc[r * NB + b];
        t = dot2(wv[r].x, xv.x, t);
        t = dot2(wv[r].y, xv.y, t);
        t = dot2(wv[r].z, xv.z, t);
        t = dot2(wv[r].w, xv.w, t);
        acc[r * NB + b] = t;
      }
    }
  }
}

// One int4 dword (8 codes) times 8 inputs of each batch row.  The codes are
// offset binary (u = q + 8); OR-ing a nibble into bf16 0x4300 gives 128 + u =
// 136 + q exactly, so the products below are (136 + q) x.  The 136 * sum(x)
// part is removed per group afterwards (i4_correct), leaving sum q x; the
// group's scale multiplies the dword's partial sum.
template <int RP, int NB>
__device__ __forceinline__ void i4_word(const uint32_t (&word)[RP], const float (&sc)[RP],
                                        const uint16_t* const (&x)[NB], int e0,
                                        float (&acc)[RP * NB]) {
  uint32_t pr[RP][4];
#pragma unroll
  for (int r = 0; r < RP; ++r) {
#pragma unroll
    for (int i = 0; i < 4; ++i) pr[r][i] = ((word[r] >> (4 * i)) & 0x000F000Fu) | 0x43004300u;
  }
#pragma unroll
  for (int b = 0; b < NB; ++b) {
    const uint4 xv = *(const uint4*)(x[b] + e0);
#pragma unroll
    for (int r = 0; r < RP; ++r) {
      float t = dot2(pr[r][0], xv.x, 0.0f);
      t = dot2(pr[r][1], xv.y, t);
      t = dot2(pr[r][2], xv.z, t);
      t = dot2(pr[r][3], xv.w, t);
      acc[r * NB + b] = fmaf(sc[r], t, acc[r * NB + b]);
    }
  }
}

// Codes of a row: K/8 dwords.  Within each full 2048-element block the dword
// holding elements [8t, 8t+8) (t = blk*256 + j*64 + lane) is stored at
// blk*256 + lane*4 + j, so one 16-byte load per lane fetches its four dwords;
// the tail (K mod 2048) keeps natural order.
template <int RP, int NB>
__device__ __forceinline__ void dot_i4(const uint32_t* const (&q)[RP], const uint16_t* const (&s)[RP],
                                       const uint16_t* const (&x)[NB], int K, int G, int lane,
                                       float (&acc)[RP * NB]) {
  const int words = K >> 3;
  const int nblk = K / kNib;
  for (int blk = 0; blk < nblk; ++blk) {
    uint4 cw[RP];
#pragma unroll
    for (int r = 0; r < RP; ++r) cw[r] = *(const uint4*)(q[r] + blk * 256 + lane * 4);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int e0 = (blk * 256 + j * 64 + lane) * 8;
      uint32_t word[RP];
      float sc[RP];
#pragma unroll
      for (int r = 0; r < RP; ++r) {
        word[r] = j == 0 ? cw[r].x : j == 1 ? cw[r].y : j == 2 ? cw[r].z : cw[r].w;
        sc[r] = bf2f(s[r][e0 / G]);
      }
      i4_word<RP, NB>(word, sc, x, e0, acc);
    }
  }
  for (int t = nblk * 256 + lane; t < words; t += 64) {
    uint32_t word[RP];
    float sc[RP];
#pragma unroll
    for (int r = 0; r < RP; ++r) {
      word[r] = q[r][t];
      sc[r] = bf2f(s[r][(t * 8) / G]);
    }
    i4_word<RP, NB>(word, sc, x, t * 8, acc);
  }
}

// acc -= 136 * s_g * sum_{k in g} x_k for the groups this lane owns.
template <int RP, int NB>
__device__ __forceinline__ void i4_correct(const uint16_t* const (&s)[RP], const float* xg, int ngr,
                                           int lane, float (&acc)[RP * NB]) {
  for (int g = lane; g < ngr; g += 64) {
#pragma unroll
    for (int r = 0; r < RP; ++r) {
      const float c = -136.0f * bf2f(s[r][g]);
#pragma unroll
      for (int b = 0; b < NB; ++b) acc[r * NB + b] = fmaf(c, xg[b * ngr + g], acc[r * NB + b]);
    }
  }
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

template <int EPI, bool XL, int NB>
__device__ __forceinline__ void proj_chunk(const ProjArgs& a, int fmt, int nb, const int32_t* list,
                                           int c0, const uint16_t* xs, const float* xg, float* red) {
  constexpr int R = EpiTraits<EPI>::R;
  constexpr int P = EpiTraits<EPI>::P;
  constexpr int RP = R * P;
  constexpr int V = RP * NB;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int gw = blockIdx.x * 4 + wave;
  const int nw = gridDim.x * 4;
  const int N = a.N, K = a.K;
  const int ntiles = (N + R - 1) / R;

  const uint16_t* x[NB];
#pragma unroll
  for (int b = 0; b < NB; ++b) {
    const int bb = b < nb ? b : nb - 1;
    x[b] = XL ? xs + bb * K : a.x + (size_t)list[c0 + bb] * a.x_stride;
  }
  const int idx = xidx<V>(lane);
  const int rr = idx / NB;
  const int bsel = idx - rr * NB;
  const bool lane_ok = lane < V && bsel < nb;
  const int ngr = K / a.G;

  // running reduction state of this lane (vocabulary epilogues)
  float lm = -INFINITY, ls = 0.0f;
  Top2 tp{-INFINITY, 0x7fffffff, -INFINITY};

  for (int t = gw; t < ntiles; t += nw) {
    const int n0 = t * R;
    float acc[V];
#pragma unroll
    for (int i = 0; i < V; ++i) acc[i] = 0.0f;
    if (fmt == 0) {
      const uint16_t* w[RP];
#pragma unroll
      for (int r = 0; r < R; ++r) {
        const int n = min(n0 + r, N - 1);
        w[r] = bf_row(a, n);
        if constexpr (P == 2) w[R + r] = a.wb2 + (size_t)n * K;
      }
      dot_bf16<RP, NB>(w, x, K, lane, acc);
    } else {
      const uint32_t* q[RP];
      const uint16_t* s[RP];
#pragma unroll
      for (int r = 0; r < R; ++r) {
        const int n = min(n0 + r, N - 1);
        q[r] = a.q4 + (size_t)n * (K >> 3);
        s[r] = a.s4 + (size_t)n * ngr;
        if constexpr (P == 2) {
          q[R + r] = a.q4b + (size_t)n * (K >> 3);
          s[R + r] = a.s4b + (size_t)n * ngr;
        }
      }
      dot_i4<RP, NB>(q, s, x, K, a.G, lane, acc);
      i4_correct<RP, NB>(s, xg, ngr, lane, acc);
    }
    XRed<V, 0>::run(acc, lane);
    const float v = acc[0];

    if constexpr (EPI == EPI_SWIGLU) {
      const float u = __shfl_xor(v, 1);
      const int n = n0 + rr;  // bit 0 clear: gate half
      if (lane_ok && (lane & 1) == 0 && n < N) {
        const int seq = list[c0 + bsel];
        const float g = v;
        const float act = g / (1.0f + __expf(-g)) * u;
        ((uint16_t*)a.y)[(size_t)seq * a.y_stride + n] = (uint16_t)f2bf(act);
      }
    } else {
      const int n = n0 + rr;
      if (lane_ok && n < N) {
        if constexpr (EPI == EPI_BF16) {
          const int seq = list[c0 + bsel];
          ((uint16_t*)a.y)[(size_t)seq * a.y_stride + n] = (uint16_t)f2bf(v);
        } else if constexpr (EPI == EPI_RESID) {
          const int seq = list[c0 + bsel];
          float* yp = (float*)a.y + (size_t)seq * a.y_stride + n;
          const float nv = *yp + v;
          *yp = nv;
          if (a.y2) a.y2[(size_t)seq * a.y2_stride + n] = (uint16_t)f2bf(nv);
        } else if constexpr (EPI == EPI_LSE) {
          lse_merge(lm, ls, v, 1.0f);
        } else if constexpr (EPI == EPI_ARGMAX) {
          if (a.logits) a.logits[(size_t)list[c0 + bsel] * a.logits_stride + n] = v;
          if (v > tp.v1) {
            tp.v2 = tp.v1;
            tp.v1 = v;
            tp.i1 = n;
          } else if (v > tp.v2) {
            tp.v2 = v;
          }
        }
      }
    }
  }

  if constexpr (EPI == EPI_LSE || EPI == EPI_ARGMAX) {
    float* rw = red + (wave * 64 + lane) * 4;
    if constexpr (EPI == EPI_LSE) {
      rw[0] = lm;
      rw[1] = ls;
    } else {
      rw[0] = tp.v1;
      rw[1] = __int_as_float(tp.i1);
      rw[2] = tp.v2;
    }
    __syncthreads();
    const int tid = threadIdx.x;
    if (tid < nb) {
      float* out = a.part + ((size_t)blockIdx.x * kMaxBatch + (c0 + tid)) * 4;
      if constexpr (EPI == EPI_LSE) {
        float m = -INFINITY, s = 0.0f;
        for (int w = 0; w < 4; ++w)
          for (int l = 0; l < V; ++l)
            if (xidx<V>(l) % NB == tid) {
              const float* src = red + (w * 64 + l) * 4;
              lse_merge(m, s, src[0], src[1]);
            }
        out[0] = m;
        out[1] = s;
      } else {
        Top2 best{-INFINITY, 0x7fffffff, -INFINITY};
        for (int w = 0; w < 4; ++w)
          for (int l = 0; l < V; ++l)
            if (xidx<V>(l) % NB == tid) {
              const float* src = red + (w * 64 + l) * 4;
              top2_merge(best, Top2{src[0], __float_as_int(src[1]), src[2]});
            }
        out[0] = best.v1;
        out[1] = __int_as_float(best.i1);
        out[2] = best.v2;
      }
    }
  }
}

template <int EPI, bool XL>
__global__ __launch_bounds__(kProjThreads) void proj_kernel(const ProjArgs a) {
  __shared__ __attribute__((aligned(16))) uint16_t xs[XL ? kXLdsElems : 8];
  __shared__ float xg[kXgElems];
  __shared__ float red[4 * 64 * 4];
  const int K = a.K;
  for (int fmt = 0; fmt < 2; ++fmt) {
    const int32_t* cntp = fmt ? a.cnt_i4 : a.cnt_bf;
    const int n = cntp ? min(max(*cntp, 0), kMaxBatch) : 0;
    const int32_t* list = fmt ? a.list_i4 : a.list_bf;
    for (int c0 = 0; c0 < n; c0 += 8) {
      const int nb = min(8, n - c0);
      __syncthreads();
      if constexpr (XL) {
        const int k8 = K >> 3;
        for (int i = threadIdx.x; i < nb * k8; i += kProjThreads) {
          const int b = i / k8;
          const int kk = i - b * k8;
          *(uint4*)&xs[b * K + kk * 8] =
              *(const uint4*)(a.x + (size_t)list[c0 + b] * a.x_stride + kk * 8);
        }
      }
      if (fmt == 1) {
        __syncthreads();
        const int ngr = K / a.G;
        for (int i = threadIdx.x; i < nb * ngr; i += kProjThreads) {
          const int b = i / ngr;
          const int g = i - b * ngr;
          const uint16_t* src = XL ? xs + b * K + g * a.G
                                   : a.x + (size_t)list[c0 + b] * a.x_stride + g * a.G;
          float sum = 0.0f;
          for (int e = 0; e < a.G; ++e) sum += bf2f(src[e]);
          xg[b * ngr + g] = sum;
        }
      }
      __syncthreads();
      if (nb == 1)
        proj_chunk<EPI, XL, 1>(a, fmt, nb, list, c0, xs, xg, red);
      else if (nb == 2)
        proj_chunk<EPI, XL, 2>(a, fmt, nb, list, c0, xs, xg, red);
      else if (nb <= 4)
        proj_chunk<EPI, XL, 4>(a, fmt, nb, list, c0, xs, xg, red);
      else
        proj_chunk<EPI, XL, 8>(a, fmt, nb, list, c0, xs, xg, red);
    }
  }
}

template <int EPI>
static void launch_proj_t(const ProjArgs& a, int nwg, hipStream_t s) {
  if (a.K * 8 <= kXLdsElems)
    hipLaunchKernelGGL((proj_kernel<EPI, true>), dim3(nwg), dim3(kProjThreads), 0, s, a);
  else
    hipLaunchKernelGGL((proj_kernel<EPI, false>), dim3(nwg), dim3(kProjThreads), 0, s, a);
}

void launch_proj(int epi, const ProjArgs& a, int nwg, hipStream_t s) {
  switch (epi) {
    case EPI_BF16: launch_proj_t<EPI_BF16>(a, nwg, s); break;
    case EPI_RESID: launch_proj_t<EPI_RESID>(a, nwg, s); break;
    case EPI_SWIGLU: launch_proj_t<EPI_SWIGLU>(a, nwg, s); break;
    case EPI_LSE: launch_proj_t<EPI_LSE>(a, nwg, s); break;
    case EPI_ARGMAX: launch_proj_t<EPI_ARGMAX>(a, nwg, s); break;
  }
}

// ---------------------------------------------------------------------------
// Step setup: embedding rows into the residual, exit state, row lists.
// ---------------------------------------------------------------------------
__global__ void init_kernel(StepState* st, const int32_t* prompt, int P, int t, int B, int L,
                            const uint16_t* emb, int d, int V, float* h, float* p_rec) {
  const int b = blockIdx.x;
  int tok = prompt ? prompt[(size_t)b * P + t] : st->tok[b];
  tok = min(max(tok, 0), V - 1);  // host-validated; a device-produced token is always < V
  const uint16_t* src = emb + (size_t)tok * d;
  for (int i = threadIdx.x; i < d; i += blockDim.x) h[(size_t)b * d + i] = bf2f(src[i]);
  if (p_rec)
    for (int l = threadIdx.x; l < L - 1; l += blockDim.x) p_rec[l * kMaxBatch + b] = __int_as_float(0x7fc00000);
  if (b == 0) {
    for (int i = threadIdx.x; i < B; i += blockDim.x) {
      st->exited[i] = 0;
      st->e[i] = L;
      st->act[i] = i;
      st->all[i] = i;
    }
    if (threadIdx.x == 0) {
      st->n_act = B;
      st->n_ex = 0;
      st->n_all = B;
    }
  }
}

void launch_init(StepState* st, const int32_t* prompt, int P, int t, int B, int L,
                 const uint16_t* emb, int d, int V, float* h, float* p_rec, hipStream_t s) {
  hipLaunchKernelGGL(init_kernel, dim3(B), dim3(256), 0, s, st, prompt, P, t, B, L, emb, d, V, h, p_rec);
}

// ---------------------------------------------------------------------------
// RMSNorm: one workgroup per row, fixed reduction order.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void rmsnorm_kernel(const float* h, const uint16_t* g, uint16_t* x,
                                                      int d, float eps) {
  __shared__ float wsum[4];
  const int b = blockIdx.x;
  const float* hr = h + (size_t)b * d;
  float ss = 0.0f;
  for (int i = threadIdx.x; i < d; i += 256) ss = fmaf(hr[i], hr[i], ss);
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) ss += __shfl_xor(ss, o);
  if ((threadIdx.x & 63) == 0) wsum[threadIdx.x >> 6] = ss;
  __syncthreads();
  const float tot = (wsum[0] + wsum[1]) + (wsum[2] + wsum[3]);
  const float r = 1.0f / sqrtf(tot / (float)d + eps);
  uint16_t* xr = x + (size_t)b * d;
  for (int i = threadIdx.x; i < d; i += 256) xr[i] = (uint16_t)f2bf(hr[i] * r * bf2f(g[i]));
}

void launch_rmsnorm(const float* h, const uint16_t* g, uint16_t* x, int B, int d, float eps,
                    hipStream_t s) {
  hipLaunchKernelGGL(rmsnorm_kernel, dim3(B), dim3(256), 0, s, h, g, x, d, eps);
}

// ---------------------------------------------------------------------------
// RoPE on q and k, and the shared-slot K/V write of the current position.
// ---------------------------------------------------------------------------
__global__ void rope_kv_kernel(const uint16_t* qkv, uint16_t* qrot, uint16_t* Kl, uint16_t* Vl,
                               uint8_t* occ_l, const int32_t* lens, const float* cosT,
                               const float* sinT, int H, int Hkv, int hd, int S) {
  const int b = blockIdx.x;
  const int pos = lens[b];
  const int half = hd >> 1;
  const uint16_t* row = qkv + (size_t)b * (H + 2 * Hkv) * hd;
  const float* cr = cosT + (size_t)pos * half;
  const float* sr = sinT + (size_t)pos * half;
  for (int i = threadIdx.x; i < (H + Hkv) * half; i += blockDim.x) {
    const int head = i / half;
    const int e = i - head * half;
    const uint16_t* src = row + head * hd;
    const float x1 = bf2f(src[e]);
    const float x2 = bf2f(src[e + half]);
    const float c = cr[e], sn = sr[e];
    const uint16_t o1 = (uint16_t)f2bf(x1 * c - x2 * sn);
    const uint16_t o2 = (uint16_t)f2bf(x2 * c + x1 * sn);
    uint16_t* dst;
    if (head < H)
      dst = qrot + ((size_t)b * H + head) * hd;
    else
      dst = Kl + (((size_t)b * Hkv + (head - H)) * S + pos) * hd;
    dst[e] = o1;
    dst[e + half] = o2;
  }
  const uint16_t* vsrc = row + (size_t)(H + Hkv) * hd;
  for (int i = threadIdx.x; i < Hkv * hd; i += blockDim.x) {
    const int kh = i / hd;
    const int e = i - kh * hd;
    Vl[(((size_t)b * Hkv + kh) * S + pos) * hd + e] = vsrc[i];
  }
  if (occ_l && threadIdx.x == 0) occ_l[(size_t)b * S + pos] += 1;
}

void launch_rope_kv(const uint16_t* qkv, uint16_t* qrot, uint16_t* Kl, uint16_t* Vl, uint8_t* occ_l,
                    const int32_t* lens, const float* cosT, const float* sinT, int B, int H, int Hkv,
                    int hd, int S, int Bmax, hipStream_t s) {
  (void)Bmax;
  hipLaunchKernelGGL(rope_kv_kernel, dim3(B), dim3(256), 0, s, qkv, qrot, Kl, Vl, occ_l, lens, cosT,
                     sinT, H, Hkv, hd, S);
}

// ---------------------------------------------------------------------------
// Grouped-query decode attention over the shared cache.
// Block (chunk c, kv head j, sequence b): positions [256c, 256c+256) of the
// sequence's context; wave w owns 64 of them.  Per wave: stage the K tile in
// LDS (rows padded by 16 bytes), scores S[t][i] = K[t] . q_i on MFMA
// (16 positions x 16 padded q heads x 32 head dims per instruction), softmax
// statistics per q head, stage the V tile into the same LDS, accumulate
// o_i = sum_t p[t][i] V[t] on the vector ALUs, merge the four waves, and write
// the chunk's (m, l, o) partial.  attn_combine merges the chunks in order.
// ---------------------------------------------------------------------------
template <int HD>
__device__ __forceinline__ void stage_tile(uint16_t* tile, const uint16_t* src, int nval, int lane) {
  constexpr int CPR = HD / 8;  // 16-byte chunks per row
  constexpr int LD = HD + 8;
  for (int i = lane; i < 64 * CPR; i += 64) {
    const int row = i / CPR;
    const int ch = i - row * CPR;
    uint4 v = make_uint4(0, 0, 0, 0);
    if (row < nval) v = *(const uint4*)(src + (size_t)row * HD + ch * 8);
    *(uint4*)(tile + row * LD + ch * 8) = v;
  }
}

template <int HD, int GQ>
__global__ __launch_bounds__(256) void attn_kernel(const AttnArgs a) {
  constexpr int LD = HD + 8;
  constexpr int KK = HD / 32;
  constexpr int DPL = 2;             // head dims per lane in the PV pass
  constexpr int LPR = HD / DPL;      // lanes per position row
  constexpr int NPG = 64 / LPR;      // position groups per wave
  __shared__ __attribute__((aligned(16))) uint16_t tile[4][64 * LD];
  __shared__ float pb[4][64][GQ];
  __shared__ float mw[4][GQ], lw[4][GQ];
  __shared__ float ow[4][GQ][HD];

  const int c = blockIdx.x, j = blockIdx.y, b = blockIdx.z;
  const int ctx = a.lens[b] + 1;
  const int start = c * kAttnChunk;
  if (start >= ctx) return;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int g = a.H / a.Hkv;
  const int t0 = start + w * 64;
  const int nval = max(0, min(64, ctx - t0));
  const size_t rowbase = (((size_t)b * a.Hkv + j) * a.S + t0) * HD;
  uint16_t* tw = tile[w];

  const int hh = lane & 15;
  uint4 qv[KK];
#pragma unroll
  for (int kk = 0; kk < KK; ++kk) {
    qv[kk] = make_uint4(0, 0, 0, 0);
    if (hh < g)
      qv[kk] = *(const uint4*)(a.q + ((size_t)b * a.H + j * g + hh) * HD + (lane >> 4) * 8 + 32 * kk);
  }

  stage_tile<HD>(tw, a.K + rowbase, nval, lane);
  __syncthreads();

  float m = -INFINITY, l = 0.0f;
  if (nval > 0) {
    float sc[4][4];
#pragma unroll
    for (int pt = 0; pt < 4; ++pt) {
      f32x4_t acc = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
      for (int kk = 0; kk < KK; ++kk) {
        const uint4 av = *(const uint4*)(tw + (pt * 16 + (lane & 15)) * LD + (lane >> 4) * 8 + 32 * kk);
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, av),
                                                      __builtin_bit_cast(bf16x8_t, qv[kk]), acc, 0, 0, 0);
      }
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int p = pt * 16 + (lane >> 4) * 4 + r;
        sc[pt][r] = p < nval ? acc[r] * a.scale : -INFINITY;
        m = fmaxf(m, sc[pt][r]);
      }
    }
    m = fmaxf(m, __shfl_xor(m, 16));
    m = fmaxf(m, __shfl_xor(m, 32));
#pragma unroll
    for (int pt = 0; pt < 4; ++pt)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float p = __expf(sc[pt][r] - m);
        l += p;
        if (hh < GQ) pb[w][pt * 16 + (lane >> 4) * 4 + r][hh] = p;
      }
    l += __shfl_xor(l, 16);
    l += __shfl_xor(l, 32);
  }
  if (lane < GQ) {
    mw[w][lane] = m;
    lw[w][lane] = l;
  }
  __syncthreads();
  stage_tile<HD>(tw, a.V + rowbase, nval, lane);
  __syncthreads();

  float o[GQ][DPL];
#pragma unroll
  for (int i = 0; i < GQ; ++i)
#pragma unroll
    for (int d = 0; d < DPL; ++d) o[i][d] = 0.0f;
  const int pg = lane / LPR, dl = lane - pg * LPR;
  for (int t = pg; t < nval; t += NPG) {
    const uint32_t vv = *(const uint32_t*)(tw + t * LD + dl * DPL);
    const float v0 = bf2f(vv & 0xffffu), v1 = bf2f(vv >> 16);
#pragma unroll
    for (int i = 0; i < GQ; ++i) {
      const float p = pb[w][t][i];
      o[i][0] = fmaf(p, v0, o[i][0]);
      o[i][1] = fmaf(p, v1, o[i][1]);
    }
  }
#pragma unroll
  for (int sft = LPR; sft < 64; sft <<= 1)
#pragma unroll
    for (int i = 0; i < GQ; ++i) {
      o[i][0] += __shfl_xor(o[i][0], sft);
      o[i][1] += __shfl_xor(o[i][1], sft);
    }
  if (pg == 0) {
#pragma unroll
    for (int i = 0; i < GQ; ++i) {
      ow[w][i][dl * DPL] = o[i][0];
      ow[w][i][dl * DPL + 1] = o[i][1];
    }
  }
  __syncthreads();
  for (int idx = threadIdx.x; idx < g * HD; idx += 256) {
    const int i = idx / HD;
    const int dd = idx - i * HD;
    float M = -INFINITY;
    for (int ww = 0; ww < 4; ++ww) M = fmaxf(M, mw[ww][i]);
    float L = 0.0f, O = 0.0f;
    for (int ww = 0; ww < 4; ++ww) {
      if (mw[ww][i] == -INFINITY) continue;
      const float f = __expf(mw[ww][i] - M);
      L = fmaf(lw[ww][i], f, L);
      O = fmaf(ow[ww][i][dd], f, O);
    }
    float* out = a.part + ((((size_t)b * a.H + j * g + i) * a.nch) + c) * (HD + 2);
    out[dd] = O;
    if (dd == 0) {
      out[HD] = M;
      out[HD + 1] = L;
    }
  }
}

__global__ void attn_combine_kernel(const AttnArgs a) {
  const int h = blockIdx.x, b = blockIdx.y;
  const int hd = a.hd;
  const int ctx = a.lens[b] + 1;
  const int nc = (ctx + kAttnChunk - 1) / kAttnChunk;
  const float* base = a.part + (((size_t)b * a.H + h) * a.nch) * (hd + 2);
  float M = -INFINITY;
  for (int c = 0; c < nc; ++c) M = fmaxf(M, base[c * (hd + 2) + hd]);
  for (int d = threadIdx.x; d < hd; d += blockDim.x) {
    float L = 0.0f, O = 0.0f;
    for (int c = 0; c < nc; ++c) {
      const float* p = base + c * (hd + 2);
      const float f = __expf(p[hd] - M);
      L = fmaf(p[hd + 1], f, L);
      O = fmaf(p[d], f, O);
    }
    a.out[((size_t)b * a.H + h) * hd + d] = (uint16_t)f2bf(O / L);
  }
}

template <int HD, int GQ>
static void launch_attn_t(const AttnArgs& a, hipStream_t s) {
  hipLaunchKernelGGL((attn_kernel<HD, GQ>), dim3(a.nch, a.Hkv, a.B), dim3(256), 0, s, a);
}

template <int HD>
static void launch_attn_hd(const AttnArgs& a, hipStream_t s) {
  const int g = a.H / a.Hkv;
  if (g <= 1) launch_attn_t<HD, 1>(a, s);
  else if (g <= 2) launch_attn_t<HD, 2>(a, s);
  else if (g <= 4) launch_attn_t<HD, 4>(a, s);
  else if (g <= 8) launch_attn_t<HD, 8>(a, s);
  else launch_attn_t<HD, 16>(a, s);
}

void launch_attention(const AttnArgs& a, hipStream_t s) {
  switch (a.hd) {
    case 32: launch_attn_hd<32>(a, s); break;
    case 64: launch_attn_hd<64>(a, s); break;
    default: launch_attn_hd<128>(a, s); break;
  }
  hipLaunchKernelGGL(attn_combine_kernel, dim3(a.H, a.B), dim3(128), 0, s, a);
}

// ---------------------------------------------------------------------------
// Exit decision and active-sequence compaction.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void decide_kernel(StepState* st, const float* part, int nwg,
                                                     const float* gamma, int layer, int L, int B,
                                                     float* p_rec) {
  __shared__ int sx[kMaxBatch];
  __shared__ int sn;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  if (threadIdx.x < B) sx[threadIdx.x] = st->exited[threadIdx.x];
  if (threadIdx.x == 0) sn = min(max(st->n_act, 0), B);
  __syncthreads();
  const int n = sn;
  for (int i = w; i < n; i += 4) {
    const int b = st->act[i];
    float m = -INFINITY, s = 0.0f;
    for (int k = lane; k < nwg; k += 64) {
      const float* p = part + ((size_t)k * kMaxBatch + i) * 4;
      lse_merge(m, s, p[0], p[1]);
    }
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const float m2 = __shfl_xor(m, o), s2 = __shfl_xor(s, o);
      lse_merge(m, s, m2, s2);
    }
    if (lane == 0) {
      const float p = 1.0f / s;
      const int f = st->forced[b];
      const bool ex = f > 0 ? (layer == f) : (p > gamma[layer - 1]);
      if (p_rec) p_rec[(layer - 1) * kMaxBatch + b] = p;
      if (ex) {
        sx[b] = 1;
        st->e[b] = layer;
      }
    }
  }
  __syncthreads();
  if (w == 0) {
    const bool valid = lane < B;
    const bool fl = valid && sx[lane] != 0;
    const unsigned long long mex = __ballot(fl);
    const unsigned long long mact = __ballot(valid && !fl);
    const unsigned long long below = (1ull << lane) - 1ull;
    if (valid) {
      st->exited[lane] = fl ? 1 : 0;
      if (fl)
        st->ex[__popcll(mex & below)] = lane;
      else
        st->act[__popcll(mact & below)] = lane;
    }
    if (lane == 0) {
      st->n_act = __popcll(mact);
      st->n_ex = __popcll(mex);
    }
  }
}

void launch_decide(StepState* st, const float* part, int nwg, const float* gamma, int layer, int L,
                   int B, float* p_rec, hipStream_t s) {
  hipLaunchKernelGGL(decide_kernel, dim3(1), dim3(256), 0, s, st, part, nwg, gamma, layer, L, B, p_rec);
}

// ---------------------------------------------------------------------------
// Final LM head: merge argmax partials, emit the token, advance the sequence.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void final_kernel(StepState* st, const float* part, int nwg, int B,
                                                    int V, int32_t* lens, int advance) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  for (int b = w; b < B; b += 4) {
    Top2 t{-INFINITY, 0x7fffffff, -INFINITY};
    for (int k = lane; k < nwg; k += 64) {
      const float* p = part + ((size_t)k * kMaxBatch + b) * 4;
      top2_merge(t, Top2{p[0], __float_as_int(p[1]), p[2]});
    }
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      Top2 u{__shfl_xor(t.v1, o), __shfl_xor(t.i1, o), __shfl_xor(t.v2, o)};
      top2_merge(t, u);
    }
    if (lane == 0) {
      const int tok = (t.i1 >= 0 && t.i1 < V) ? t.i1 : 0;  // no finite logit: token 0
      st->out_tok[b] = tok;
      st->tok[b] = tok;
      st->gap[b] = t.v1 - t.v2;
      if (advance) lens[b] += 1;
    }
  }
}

void launch_final(StepState* st, const float* part, int nwg, int B, int V, int32_t* lens, int advance,
                  hipStream_t s) {
  hipLaunchKernelGGL(final_kernel, dim3(1), dim3(256), 0, s, st, part, nwg, B, V, lens, advance);
}

__global__ void advance_kernel(int32_t* lens, int B) {
  if ((int)threadIdx.x < B) lens[threadIdx.x] += 1;
}

void launch_advance(int32_t* lens, int B, hipStream_t s) {
  hipLaunchKernelGGL(advance_kernel, dim3(1), dim3(64), 0, s, lens, B);
}

// ---------------------------------------------------------------------------
// int4 exit copies: one thread per (row, group).
//   s = bf16(max|w| / 7) (IEEE float32 division, then round to bf16)
//   q = clamp(rint(w / s), -8, 7), or 0 when s == 0; stored as q + 8.
// ---------------------------------------------------------------------------
__device__ __forceinline__ int stored_word(int t, int nblk) {
  if (t < nblk * 256) return (t & ~255) + (t & 63) * 4 + ((t & 255) >> 6);
  return t;
}

__global__ void quantize_kernel(const uint16_t* w, int N, int K, int G, uint32_t* codes,
                                uint16_t* scales) {
  const int ngr = K / G;
  const long long gid = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  if (gid >= (long long)N * ngr) return;
  const int n = (int)(gid / ngr);
  const int g = (int)(gid - (long long)n * ngr);
  const uint16_t* src = w + (size_t)n * K + (size_t)g * G;
  float amax = 0.0f;
  for (int e = 0; e < G; ++e) amax = fmaxf(amax, fabsf(bf2f(src[e])));
  const uint32_t sb = f2bf(amax / 7.0f);
  const float s = bf2f(sb);
  const int words = K >> 3, nblk = K / kNib;
  for (int dw = 0; dw < G / 8; ++dw) {
    uint32_t word = 0;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      int q = 0;
      if (s != 0.0f) {
        q = (int)rintf(bf2f(src[dw * 8 + e]) / s);
        q = min(7, max(-8, q));
      }
      word |= (uint32_t)(q + 8) << (4 * (e >> 1) + 16 * (e & 1));
    }
    const int t = (g * G) / 8 + dw;
    codes[(size_t)n * words + stored_word(t, nblk)] = word;
  }
  scales[(size_t)n * ngr + g] = (uint16_t)sb;
}

void launch_quantize(const uint16_t* w, int N, int K, int G, uint32_t* codes, uint16_t* scales,
                     hipStream_t s) {
  const long long n = (long long)N * (K / G);
  const int threads = 256;
  const long long blocks = (n + threads - 1) / threads;
  hipLaunchKernelGGL(quantize_kernel, dim3((unsigned)blocks), dim3(threads), 0, s, w, N, K, G, codes, scales);
}

__global__ void unpack_kernel(const uint32_t* codes, int K, int row0, int nrows, int8_t* out) {
  const long long i = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= (long long)nrows * K) return;
  const int r = (int)(i / K);
  const int k = (int)(i - (long long)r * K);
  const int t = k >> 3, e = k & 7;
  const uint32_t word = codes[(size_t)(row0 + r) * (K >> 3) + stored_word(t, K / kNib)];
  const int u = (word >> (4 * (e >> 1) + 16 * (e & 1))) & 15;
  out[i] = (int8_t)(u - 8);
}

void launch_unpack_codes(const uint32_t* codes, int N, int K, int row0, int nrows, int8_t* out,
                         hipStream_t s) {
  (void)N;
  const long long n = (long long)nrows * K;
  hipLaunchKernelGGL(unpack_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, codes, K, row0,
                     nrows, out);
}

}  // namespace ee
