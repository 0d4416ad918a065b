// Projection GEMVs of the decode step and the int4 exit-copy packer (gfx950).
//
// One launch of proj_kernel computes y = W x for the rows of a step that are
// still on the backbone (bf16 W, list "bf") and for the rows that already exited
// (the int4 exit copy of the same layer, list "i4"): River-LLM explainer,
// section 4.1-4.2 (exit layers are 4-bit copies of every layer) and CALM
// explainer, section 3.3 (sequences of a batch leave at different layers, so
// each layer serves both kinds of rows; the row lists remove the divergence).
//
// Layout of the work
//   * The input rows (at most 8 per pass) are staged in LDS (64 KB) when they
//     fit; wider inputs (the down projection) are read from L2 directly.  There
//     is no split-K: a cross-workgroup reduction needs device-scope fences,
//     which on gfx950 write back and invalidate the L2.
//   * bf16 rows: each wave owns R weight rows; a lane reads 16 contiguous bytes
//     per row per step (a wave reads 1 KB contiguous per row), double-buffered,
//     and accumulates bf16 pairs with v_dot2_f32_bf16 against the inputs; a
//     transpose-reduce finishes the sums across lanes.  HBM-bound at B <= 8.
//     The first weights are requested before the inputs are staged.
//   * int4 rows: the dequantise-and-multiply is ALU-heavy on the vector unit
//     (8 products per 4 bytes per batch row), so it runs on MFMA
//     (v_mfma_f32_16x16x32_bf16): a workgroup owns 16 weight rows, its 8 waves
//     split K, each lane unpacks one dword of codes (8 weights) into the A
//     operand in registers (nibble | 0x4300 is the bf16 value 136 + q), the
//     inputs are the B operand (batch rows padded to 16 with zeros), and a
//     second MFMA with A = 136 everywhere yields 136 * sum(x) per step, which is
//     removed before each group of G inputs is scaled by its bf16 scale.
#include "ee_internal.h"
#include "ee_device.h"

#include <algorithm>

namespace ee {

constexpr int kWaves = kProjThreads / 64;

template <int EPI>
struct Ep {
  static constexpr int P = EPI == EPI_SWIGLU ? 2 : 1;                     // matrices per tile
  static constexpr int R = EPI == EPI_SWIGLU ? 1 : 2;
};

__device__ __forceinline__ const uint16_t* bf_row(const ProjArgs& a, int n) {
  int s = 0, start = 0;
  if (n >= a.seg_end[0]) {
    s = (n >= a.seg_end[1]) ? 2 : 1;
    start = a.seg_end[s - 1];
  }
  return a.wb[s] + (size_t)(n - start) * a.K;
}

__device__ __forceinline__ float silu_mul(float g, float u) { return g / (1.0f + __expf(-g)) * u; }

// Epilogue of one finished output value v (row n, sequence seq).
template <int EPI>
__device__ __forceinline__ void store_out(const ProjArgs& a, int seq, int n, float v) {
  if constexpr (EPI == EPI_BF16) {
    ((uint16_t*)a.y)[(size_t)seq * a.y_stride + n] = (uint16_t)f2bf(v);
  } else if constexpr (EPI == EPI_RESID) {
    float* yp = (float*)a.y + (size_t)seq * a.y_stride + n;
    const float nv = *yp + v;
    *yp = nv;
    if (a.y2) a.y2[(size_t)seq * a.y2_stride + n] = (uint16_t)f2bf(nv);
  }
}

// Stages input rows list[c0 .. c0+nb) into LDS (row stride K).
__device__ __forceinline__ void stage_x(const ProjArgs& a, const int32_t* list, int c0, int nb, uint16_t* xs) {
  const int k8 = a.K >> 3;
  for (int i = threadIdx.x; i < nb * k8; i += kProjThreads) {
    const int b = i / k8;
    const int kk = i - b * k8;
    *(uint4*)&xs[b * a.K + kk * 8] = *(const uint4*)(a.x + (size_t)list[c0 + b] * a.x_stride + kk * 8);
  }
}

// ---------------------------------------------------------------------------
// bf16 rows (vector ALU, dot2)
// ---------------------------------------------------------------------------
// One 512-element step of a bf16 wave tile: acc[r*NB+b] += W_r . x_b over this
// lane's 8 elements.  Inputs are read in groups of four to bound registers.
template <int RP, int NB, bool XL>
__device__ __forceinline__ void bf16_step(const uint4 (&wv)[RP], const uint16_t* xs, const uint16_t* xg,
                                          const int (&xo)[NB], int k, float (&acc)[RP * NB]) {
  constexpr int BG = NB < 4 ? NB : 4;
#pragma unroll
  for (int b0 = 0; b0 < NB; b0 += BG) {
    uint4 xv[BG];
#pragma unroll
    for (int b = 0; b < BG; ++b)
      xv[b] = XL ? *(const uint4*)(xs + xo[b0 + b] + k) : *(const uint4*)(xg + (size_t)xo[b0 + b] + k);
#pragma unroll
    for (int b = 0; b < BG; ++b)
#pragma unroll
      for (int r = 0; r < RP; ++r) {
        float s = acc[r * NB + b0 + b];
        s = dot2(wv[r].x, xv[b].x, s);
        s = dot2(wv[r].y, xv[b].y, s);
        s = dot2(wv[r].z, xv[b].z, s);
        s = dot2(wv[r].w, xv[b].w, s);
        acc[r * NB + b0 + b] = s;
      }
  }
}

template <int EPI, bool XL, int NB>
__device__ __forceinline__ void bf16_pass(const ProjArgs& a, int nb, const int32_t* list, int c0,
                                          uint16_t* xs, float* red) {
  constexpr int P = Ep<EPI>::P;
  constexpr int R = Ep<EPI>::R;
  constexpr int RP = R * P;
  constexpr int V = RP * NB;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wid = blockIdx.x * kWaves + wave;
  const int nwc = gridDim.x * kWaves;
  const int N = a.N, K = a.K;
  const int ntiles = (N + R - 1) / R;
  const int idx = xidx<V>(lane);
  const int rr = idx / NB;
  const int bsel = idx - rr * NB;
  const bool lane_ok = lane < V && bsel < nb;

  int xo[NB];  // element offset of each input row (LDS or global)
#pragma unroll
  for (int b = 0; b < NB; ++b) {
    const int bb = b < nb ? b : nb - 1;
    xo[b] = XL ? bb * K : list[c0 + bb] * a.x_stride;
  }

  float lm = -INFINITY, ls = 0.0f;
  Top2 tp{-INFINITY, 0x7fffffff, -INFINITY};

  // request the first tile's first weights before the inputs are staged
  const int nfull = K >> 9;                  // full 512-element steps (every lane active)
  const int kt = nfull * 512 + lane * 8;     // this lane's element in the ragged tail
  int t = wid;
  const uint16_t* w[RP];
  uint4 cur[RP];
  auto set_rows = [&](int tt) {
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const int n = min(tt * R + r, N - 1);
      w[r] = bf_row(a, n) + lane * 8;
      if constexpr (P == 2) w[R + r] = a.wb2 + (size_t)n * K + lane * 8;
    }
  };
  if (t < ntiles && nfull > 0) {
    set_rows(t);
#pragma unroll
    for (int r = 0; r < RP; ++r) cur[r] = ld_stream(w[r]);
  }
  if constexpr (XL) stage_x(a, list, c0, nb, xs);
  __syncthreads();

  for (; t < ntiles; t += nwc) {
    const int n0 = t * R;
    if (t != wid || nfull == 0) {
      set_rows(t);
      if (nfull > 0) {
#pragma unroll
        for (int r = 0; r < RP; ++r) cur[r] = ld_stream(w[r]);
      }
    }
    float acc[V];
#pragma unroll
    for (int i = 0; i < V; ++i) acc[i] = 0.0f;
    // software pipeline with two register sets: one step's weights are in
    // flight while the other step computes
    int st = 0;
    uint4 alt[RP];
    for (; st + 2 < nfull; st += 2) {
#pragma unroll
      for (int r = 0; r < RP; ++r) alt[r] = ld_stream(w[r] + (st + 1) * 512);
      bf16_step<RP, NB, XL>(cur, xs, a.x, xo, lane * 8 + st * 512, acc);
#pragma unroll
      for (int r = 0; r < RP; ++r) cur[r] = ld_stream(w[r] + (st + 2) * 512);
      bf16_step<RP, NB, XL>(alt, xs, a.x, xo, lane * 8 + (st + 1) * 512, acc);
    }
    if (st + 1 < nfull) {
#pragma unroll
      for (int r = 0; r < RP; ++r) alt[r] = ld_stream(w[r] + (st + 1) * 512);
      bf16_step<RP, NB, XL>(cur, xs, a.x, xo, lane * 8 + st * 512, acc);
      bf16_step<RP, NB, XL>(alt, xs, a.x, xo, lane * 8 + (st + 1) * 512, acc);
    } else if (st < nfull) {
      bf16_step<RP, NB, XL>(cur, xs, a.x, xo, lane * 8 + st * 512, acc);
    }
    if (kt < K) {  // ragged tail (K not a multiple of 512)
      uint4 tw[RP];
#pragma unroll
      for (int r = 0; r < RP; ++r) tw[r] = ld_stream(w[r] + nfull * 512);
      bf16_step<RP, NB, XL>(tw, xs, a.x, xo, kt, acc);
    }
    XRed<V, 0>::run(acc, lane);
    const float v = acc[0];
    const int n = n0 + (rr % R);
    if constexpr (EPI == EPI_SWIGLU) {
      const float u = __shfl_xor(v, 1);  // the up row sits in the partner lane
      if (lane_ok && (lane & 1) == 0 && n < N)
        ((uint16_t*)a.y)[(size_t)list[c0 + bsel] * a.y_stride + n] = (uint16_t)f2bf(silu_mul(v, u));
    } else if constexpr (EPI == EPI_LSE) {
      if (lane_ok && n < N) lse_merge(lm, ls, v, 1.0f);
    } else if constexpr (EPI == EPI_ARGMAX) {
      if (lane_ok && n < N) {
        if (a.logits) a.logits[(size_t)list[c0 + bsel] * a.logits_stride + n] = v;
        if (v > tp.v1) {
          tp.v2 = tp.v1;
          tp.v1 = v;
          tp.i1 = n;
        } else if (v > tp.v2) {
          tp.v2 = v;
        }
      }
    } else {
      if (lane_ok && n < N) store_out<EPI>(a, list[c0 + bsel], n, v);
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
        for (int ww = 0; ww < kWaves; ++ww)
          for (int l = 0; l < V; ++l)
            if (xidx<V>(l) % NB == tid) {
              const float* src = red + (ww * 64 + l) * 4;
              lse_merge(m, s, src[0], src[1]);
            }
        out[0] = m;
        out[1] = s;
      } else {
        Top2 best{-INFINITY, 0x7fffffff, -INFINITY};
        for (int ww = 0; ww < kWaves; ++ww)
          for (int l = 0; l < V; ++l)
            if (xidx<V>(l) % NB == tid) {
              const float* src = red + (ww * 64 + l) * 4;
              top2_merge(best, Top2{src[0], __float_as_int(src[1]), src[2]});
            }
        out[0] = best.v1;
        out[1] = __int_as_float(best.i1);
        out[2] = best.v2;
      }
    }
  }
}

// ---------------------------------------------------------------------------
// int4 rows (MFMA)
//
// Codes of a row: K/8 dwords, dword t holding elements [8t, 8t+8) with element
// 8t+2i in bits [4i, 4i+4) and 8t+2i+1 in bits [16+4i, 16+4i+4), value q + 8.
// Within each full 128-element block the four dwords a lane needs for the
// block's four MFMA steps are adjacent: logical dword 16u + 4j + c (step j,
// lane quarter c) is stored at 16u + 4c + j.  A tail (K mod 128 > 0) keeps
// natural order.  Rows are padded to a multiple of 16 with zero codes.
// Scales: [N16/16][K/G][16] bf16 (16 rows of one tile and one group adjacent).
// ---------------------------------------------------------------------------
__device__ __forceinline__ bf16x8_t unpack8(uint32_t w) {
  uint4 o;
  o.x = (w & 0x000F000Fu) | 0x43004300u;
  o.y = ((w >> 4) & 0x000F000Fu) | 0x43004300u;
  o.z = ((w >> 8) & 0x000F000Fu) | 0x43004300u;
  o.w = ((w >> 12) & 0x000F000Fu) | 0x43004300u;
  return __builtin_bit_cast(bf16x8_t, o);
}

__device__ __forceinline__ uint32_t pick(const uint4& v, int j) {
  return j == 0 ? v.x : j == 1 ? v.y : j == 2 ? v.z : v.w;
}

// tot += s_row * (C - C136) for the 4 rows of this lane
__device__ __forceinline__ void i4_group_scale(const uint16_t* stile, int g, int q, const f32x4_t& cg,
                                               const f32x4_t& c136, f32x4_t& tot) {
  const uint2 sv = *(const uint2*)(stile + g * 16 + 4 * q);
  tot[0] = fmaf(bf2f(sv.x & 0xffffu), cg[0] - c136[0], tot[0]);
  tot[1] = fmaf(bf2f(sv.x >> 16), cg[1] - c136[1], tot[1]);
  tot[2] = fmaf(bf2f(sv.y & 0xffffu), cg[2] - c136[2], tot[2]);
  tot[3] = fmaf(bf2f(sv.y >> 16), cg[3] - c136[3], tot[3]);
}

template <int P>
__device__ __forceinline__ void i4_step(const uint32_t (&word)[P], const uint4& bv, f32x4_t (&cg)[P],
                                        f32x4_t& c136) {
  const bf16x8_t b8 = __builtin_bit_cast(bf16x8_t, bv);
  const uint4 k136 = make_uint4(0x43084308u, 0x43084308u, 0x43084308u, 0x43084308u);
  c136 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, k136), b8, c136, 0, 0, 0);
#pragma unroll
  for (int p = 0; p < P; ++p) cg[p] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(unpack8(word[p]), b8, cg[p], 0, 0, 0);
}

template <int EPI, bool XL>
__device__ __forceinline__ void i4_pass(const ProjArgs& a, int nb, const int32_t* list, int c0,
                                        uint16_t* xs, float* red) {
  constexpr int P = Ep<EPI>::P;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int m = lane & 15, q = lane >> 4;
  const int N = a.N, K = a.K, G = a.G;
  const int ntiles = (N + 15) / 16;
  const int ngr = K / G;
  const int mpg = G / 32;             // MFMA steps per group
  const int nfull = K >> 7;
  const int ntail = (K & 127) >> 5;   // MFMA steps in the tail
  const int b0 = wave * nfull / kWaves, b1 = (wave + 1) * nfull / kWaves;
  const bool bok = m < nb;
  const bool tail_here = wave == kWaves - 1 && ntail > 0;
  const uint16_t* xrow = XL ? xs + (bok ? m : 0) * K : a.x + (size_t)list[c0 + (bok ? m : 0)] * a.x_stride;

  // request the first tile's first codes before the inputs are staged
  int t = blockIdx.x;
  uint4 cw0[P];
  if (t < ntiles && b0 < b1) {
#pragma unroll
    for (int p = 0; p < P; ++p)
      cw0[p] = ld_stream((p == 0 ? a.q4 : a.q4b) + (size_t)(t * 16 + m) * (K >> 3) + b0 * 16 + q * 4);
  }
  if constexpr (XL) stage_x(a, list, c0, nb, xs);
  __syncthreads();

  for (; t < ntiles; t += gridDim.x) {
    const uint32_t* crow[P];
    const uint16_t* stile[P];
#pragma unroll
    for (int p = 0; p < P; ++p) {
      crow[p] = (p == 0 ? a.q4 : a.q4b) + (size_t)(t * 16 + m) * (K >> 3);
      stile[p] = (p == 0 ? a.s4 : a.s4b) + (size_t)t * ngr * 16;
    }
    f32x4_t tot[P];
#pragma unroll
    for (int p = 0; p < P; ++p) tot[p] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
    for (int u = b0; u < b1; ++u) {
      uint4 cw[P];
      if (u == b0 && t == (int)blockIdx.x) {
#pragma unroll
        for (int p = 0; p < P; ++p) cw[p] = cw0[p];
      } else {
#pragma unroll
        for (int p = 0; p < P; ++p) cw[p] = ld_stream(crow[p] + u * 16 + q * 4);
      }
      f32x4_t cg[P];
      f32x4_t c136 = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
      for (int p = 0; p < P; ++p) cg[p] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int ka = u * 128 + 32 * j;
        uint4 bv = *(const uint4*)(xrow + ka + 8 * q);
        if (!bok) bv = make_uint4(0, 0, 0, 0);
        uint32_t word[P];
#pragma unroll
        for (int p = 0; p < P; ++p) word[p] = pick(cw[p], j);
        i4_step<P>(word, bv, cg, c136);
        if (j % mpg == mpg - 1) {
#pragma unroll
          for (int p = 0; p < P; ++p) {
            i4_group_scale(stile[p], ka / G, q, cg[p], c136, tot[p]);
            cg[p] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
          }
          c136 = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
        }
      }
    }
    if (tail_here) {
      f32x4_t cg[P];
      f32x4_t c136 = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
      for (int p = 0; p < P; ++p) cg[p] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
      for (int j = 0; j < ntail; ++j) {
        const int ka = nfull * 128 + 32 * j;
        uint4 bv = *(const uint4*)(xrow + ka + 8 * q);
        if (!bok) bv = make_uint4(0, 0, 0, 0);
        uint32_t word[P];
#pragma unroll
        for (int p = 0; p < P; ++p) word[p] = crow[p][nfull * 16 + 4 * j + q];
        i4_step<P>(word, bv, cg, c136);
        if (j % mpg == mpg - 1) {
#pragma unroll
          for (int p = 0; p < P; ++p) {
            i4_group_scale(stile[p], ka / G, q, cg[p], c136, tot[p]);
            cg[p] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
          }
          c136 = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
        }
      }
    }
    // sum the waves' K slices in wave order
    float vals[P][4];
#pragma unroll
    for (int p = 0; p < P; ++p) {
      float* rw = red + (wave * 64 + lane) * 4;
      rw[0] = tot[p][0];
      rw[1] = tot[p][1];
      rw[2] = tot[p][2];
      rw[3] = tot[p][3];
      __syncthreads();
      if (wave == 0) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          float s = 0.0f;
          for (int ww = 0; ww < kWaves; ++ww) s += red[(ww * 64 + lane) * 4 + i];
          vals[p][i] = s;
        }
      }
      __syncthreads();
    }
    if (wave != 0 || !bok) continue;
    // lane (q, m) holds rows t*16 + 4q + i of batch column m
    const int seq = list[c0 + m];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int n = t * 16 + 4 * q + i;
      if (n >= N) continue;
      if constexpr (EPI == EPI_SWIGLU)
        ((uint16_t*)a.y)[(size_t)seq * a.y_stride + n] = (uint16_t)f2bf(silu_mul(vals[0][i], vals[P - 1][i]));
      else
        store_out<EPI>(a, seq, n, vals[0][i]);
    }
  }
}

template <int EPI, bool XL>
__global__ __launch_bounds__(kProjThreads, 4) void proj_kernel(const ProjArgs a) {
  __shared__ __attribute__((aligned(16))) uint16_t xs[XL ? kXLdsElems : 8];
  __shared__ __attribute__((aligned(16))) float red[kWaves * 64 * 4];
  for (int fmt = 0; fmt < 2; ++fmt) {
    if constexpr (EPI == EPI_LSE || EPI == EPI_ARGMAX) {
      if (fmt == 1) break;
    }
    const int32_t* cntp = fmt ? a.cnt_i4 : a.cnt_bf;
    const int n = cntp ? min(max(*cntp, 0), kMaxBatch) : 0;
    const int32_t* list = fmt ? a.list_i4 : a.list_bf;
    for (int c0 = 0; c0 < n; c0 += 8) {
      const int nb = min(8, n - c0);
      __syncthreads();  // the previous pass is done with xs and red
      if (fmt == 0) {
        if (nb == 1)
          bf16_pass<EPI, XL, 1>(a, nb, list, c0, xs, red);
        else if (nb == 2)
          bf16_pass<EPI, XL, 2>(a, nb, list, c0, xs, red);
        else if (nb <= 4)
          bf16_pass<EPI, XL, 4>(a, nb, list, c0, xs, red);
        else
          bf16_pass<EPI, XL, 8>(a, nb, list, c0, xs, red);
      } else {
        if constexpr (EPI != EPI_LSE && EPI != EPI_ARGMAX) i4_pass<EPI, XL>(a, nb, list, c0, xs, red);
      }
    }
  }
}

template <int EPI>
static void launch_epi(const ProjArgs& a, int g, hipStream_t s) {
  if ((long long)8 * a.K <= kXLdsElems)
    hipLaunchKernelGGL((proj_kernel<EPI, true>), dim3(g), dim3(kProjThreads), 0, s, a);
  else
    hipLaunchKernelGGL((proj_kernel<EPI, false>), dim3(g), dim3(kProjThreads), 0, s, a);
}

void launch_proj(int epi, const ProjArgs& a, int nwg, hipStream_t s) {
  // the vocabulary epilogues write one partial per workgroup (kNwgMax of them)
  const int g = std::max(1, std::min(nwg, kNwgMax));
  switch (epi) {
    case EPI_BF16: launch_epi<EPI_BF16>(a, g, s); break;
    case EPI_RESID: launch_epi<EPI_RESID>(a, g, s); break;
    case EPI_SWIGLU: launch_epi<EPI_SWIGLU>(a, g, s); break;
    case EPI_LSE: launch_epi<EPI_LSE>(a, g, s); break;
    case EPI_ARGMAX: launch_epi<EPI_ARGMAX>(a, g, s); break;
  }
}

// ---------------------------------------------------------------------------
// int4 exit copies: one thread per (row, group) of a matrix written into rows
// [row0, row0 + N) of a packed buffer.
//   s = bf16(max|w| / 7) (IEEE float32 division, then round to bf16)
//   q = clamp(rint(w / s), -8, 7), or 0 when s == 0; stored as q + 8.
// ---------------------------------------------------------------------------
__device__ __forceinline__ int stored_word(int t, int words) {
  const int full = (words >> 4) << 4;
  if (t < full) return (t & ~15) + (t & 3) * 4 + ((t & 15) >> 2);
  return t;
}

__global__ void quantize_kernel(const uint16_t* w, int N, int K, int G, int row0, uint32_t* codes,
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
  const int words = K >> 3;
  const int r = row0 + n;
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
    codes[(size_t)r * words + stored_word(t, words)] = word;
  }
  scales[((size_t)(r >> 4) * ngr + g) * 16 + (r & 15)] = (uint16_t)sb;
}

void launch_quantize(const uint16_t* w, int N, int K, int G, int row0, uint32_t* codes, uint16_t* scales,
                     hipStream_t s) {
  const long long n = (long long)N * (K / G);
  const long long blocks = (n + 255) / 256;
  hipLaunchKernelGGL(quantize_kernel, dim3((unsigned)blocks), dim3(256), 0, s, w, N, K, G, row0, codes,
                     scales);
}

__global__ void unpack_kernel(const uint32_t* codes, const uint16_t* scales, int K, int G, int row0,
                              int nrows, int8_t* out, uint16_t* sout) {
  const long long i = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= (long long)nrows * K) return;
  const int r = (int)(i / K);
  const int k = (int)(i - (long long)r * K);
  const int t = k >> 3, e = k & 7;
  const int row = row0 + r;
  const uint32_t word = codes[(size_t)row * (K >> 3) + stored_word(t, K >> 3)];
  const int u = (word >> (4 * (e >> 1) + 16 * (e & 1))) & 15;
  out[i] = (int8_t)(u - 8);
  if (k % G == 0) {
    const int ngr = K / G;
    sout[(size_t)r * ngr + k / G] = scales[((size_t)(row >> 4) * ngr + k / G) * 16 + (row & 15)];
  }
}

void launch_unpack(const uint32_t* codes, const uint16_t* scales, int K, int G, int row0, int nrows,
                   int8_t* out, uint16_t* sout, hipStream_t s) {
  const long long n = (long long)nrows * K;
  hipLaunchKernelGGL(unpack_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, codes, scales, K, G,
                     row0, nrows, out, sout);
}

}  // namespace ee
