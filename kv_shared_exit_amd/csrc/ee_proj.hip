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
//   * The input rows (at most 8 per pass) are staged in LDS (64 KB).  A launch
//     with the partial-sum epilogue splits the columns into ranges that each
//     fit the stage; every workgroup works on one range and writes float32
//     partial sums, which the finish kernel adds to the residual in a fixed
//     order (no cross-workgroup synchronisation, bitwise reproducible).
//   * bf16 rows: each wave owns R weight rows; a lane reads 16 contiguous bytes
//     per row per step (a wave reads 1 KB contiguous per row), double-buffered,
//     and accumulates bf16 pairs with v_dot2_f32_bf16 against the inputs; a
//     transpose-reduce finishes the sums across lanes.  HBM-bound at B <= 8.
//     The first weights are requested before the inputs are staged.
//   * int4 rows: the dequantise-and-multiply is ALU-heavy on the vector unit
//     (8 products per 4 bytes per batch row), so it runs on MFMA
//     (v_mfma_f32_16x16x32_bf16): a 16-row tile is shared by up to 8 waves
//     that split its columns, each lane unpacks one dword of codes (8 weights)
//     into the A operand in registers (nibble | 0x4300 is the bf16 value
//     136 + q), the inputs are the B operand (batch rows padded to 16 with
//     zeros); the input stage sums every staged row over each scale group,
//     and 136 times that sum is removed before each group of G products is
//     scaled by its bf16 scale.
#include "ee_internal.h"
#include "ee_device.h"
#include "ee_epi.h"
#include "ee_rng.h"

#include <hip/hip_ext.h>

#include <algorithm>
#include <stdexcept>

namespace ee {

constexpr int kWaves = kProjThreads / 64;
// bf16 rows on MFMA (true) or on the vector ALU with dot2 (false).  With the
// row-major weights a 16-row MFMA operand load touches 16 rows x 64 bytes, and
// the vocabulary GEMV measured 219 us against 159-178 us on the vector ALU, so
// the MFMA path is kept only as the measured alternative.
constexpr bool kBf16Mfma = false;
// share of a range's workgroups given to the bf16 rows when both formats have
// rows, in 1/256 (bf16 streams ~4x the bytes of its int4 copy; measured)
constexpr int kBfShare = 176;     // QKV, O
constexpr int kBfShareFfn = 128;  // gate/up, down

template <int EPI>
struct Ep {
  static constexpr int P = EPI == EPI_SWIGLU ? 2 : 1;  // matrices per tile
  static constexpr int R = EPI == EPI_SWIGLU ? 1 : 2;  // bf16 rows per wave tile
  // the vocabulary passes (one partial per workgroup and row)
  static constexpr bool VOCAB = EPI == EPI_LSE || EPI == EPI_ARGMAX || EPI == EPI_LSE_S || EPI == EPI_ARGMAX_S ||
                                EPI == EPI_RESAMPLE;
  static constexpr bool SAMPLED = EPI == EPI_LSE_S || EPI == EPI_ARGMAX_S || EPI == EPI_RESAMPLE;
  static constexpr int RW = SAMPLED ? 8 : 4;  // floats per lane in the cross-wave reduction
};

// The share of a launch one workgroup works on: its column range and its
// index among the workgroups of that range.
struct Work {
  int K, k0;    // columns of the range and the first of them
  int wg, nwg;  // workgroup index within the range, workgroups per range
  int chunk;    // range index
};

// Rows of a QKV tile: each tile pairs rotation rows c and c + hd/2 of one head
// (RoPE rotates element i with element i + hd/2), so both halves of every pair
// finish in the same wave.  A tile of 2*half rows covers c0 .. c0+half-1 and
// their partners.
template <int HALF>
__device__ __forceinline__ int qkv_row(const ProjArgs& a, int t, int m) {
  constexpr int L2 = HALF == 1 ? 1 : HALF == 2 ? 2 : HALF == 4 ? 3 : 4;  // log2(2 * HALF)
  const int sh = a.hd_log2 - L2;  // log2(tiles per head)
  const int head = t >> sh;
  const int c0 = (t & ((1 << sh) - 1)) * HALF;
  return (head << a.hd_log2) + (m >= HALF ? a.hd / 2 : 0) + c0 + (m % HALF);
}

__device__ __forceinline__ const uint16_t* bf_row(const ProjArgs& a, const Work& w, int n) {
  int s = 0, start = 0;
  if (n >= a.seg_end[0]) {
    s = (n >= a.seg_end[1]) ? 2 : 1;
    start = a.seg_end[s - 1];
  }
  return a.wb[s] + (size_t)(n - start) * a.K + w.k0;
}

// Epilogue of one finished output value v (row n, sequence seq).
template <int EPI>
__device__ __forceinline__ void store_out(const ProjArgs& a, const Work& w, int seq, int n, float v) {
  if constexpr (EPI == EPI_BF16) {
    ((uint16_t*)a.y)[(size_t)seq * a.y_stride + n] = (uint16_t)f2bf(v);
  } else if constexpr (EPI == EPI_PART) {
    ((float*)a.y)[(size_t)w.chunk * a.y_cstride + (size_t)seq * a.y_stride + n] = v;
  }
}

// Staging of the input rows list[c0 .. c0+nb) of this workgroup's column range
// into LDS (row stride w.K).  stage_rows puts the rows' sequence ids in LDS and
// is called before the first weights are requested, so that its load is not
// queued behind them; stage_x then copies the rows.  Every thread issues all
// of its loads (at most kItems items of 8 elements) before storing any, so the
// copy costs one memory latency.
constexpr int kItems = kXLdsElems / 8 / kProjThreads;

// LDS row stride of the staged inputs: K plus 16 bytes, so that the MFMA B
// operand reads (16 rows, 16 bytes each, in groups of 8 lanes) fall in
// different banks.
__device__ __forceinline__ int xstride(int K) { return K + 8; }

// A chunk's sequence ids into LDS (padded with the chunk's last id).  The
// first chunk's are read through the scalar cache (a uniform address) and
// written after the pass has issued its first weight loads: vector loads of
// them queued behind the weight loads the other waves of the CU had already
// issued (measured: ~3.4 us of an 11 us int4 pass went to wave 0 waiting for
// its ids before requesting its own weights).  Later chunks read the list
// with vector loads.  stage_x's first barrier publishes the ids.  Every list
// holds at least 8 entries (launch_proj points an absent one at kNoRows).
using cint = const int32_t __attribute__((address_space(4)));
__device__ __forceinline__ void stage_rows(const int32_t* list, int c0, int nb, int* seq) {
  if (c0 == 0) {
    if (threadIdx.x < 8) {
      const cint* lp = (const cint*)list;
      const int e = min((int)threadIdx.x, nb - 1);
      int v = lp[0];
#pragma unroll
      for (int k = 1; k < 8; ++k) {
        const int w = lp[k];
        v = e == k ? w : v;
      }
      seq[threadIdx.x] = v;
    }
  } else if (threadIdx.x < 8) {
    seq[threadIdx.x] = list[c0 + min((int)threadIdx.x, nb - 1)];
  }
}

// With PPG > 0 (the int4 pass: PPG = G / 8 items per scale group) the stage
// also writes gs[b * (K / G) + g] = the float32 sum of row b over scale group g
// of the range: the 136 * sum(x) each group's codes carry (see the int4 pass)
// is then taken from here instead of being computed by every wave.  The items
// of a group sit in PPG consecutive threads (aligned: K is a multiple of G),
// summed by a butterfly over those lanes.
template <int PPG = 0>
__device__ __forceinline__ void stage_x(const ProjArgs& a, const Work& w, int nb, const int* seq, uint16_t* xs,
                                        float* gs = nullptr) {
  __syncthreads();  // seq is in LDS
  const int k8 = w.K >> 3;
  const int n = nb * k8;  // items; item i = (row b, column group kk) goes to xs[b * xstride(K) + kk*8]
  int tid = threadIdx.x;
  asm volatile("" : "+v"(tid));  // keeps the per-item index math here (not hoisted and held live)
  // row of item i: i / k8 from a float reciprocal, corrected to the exact quotient
  const float inv = 1.0f / (float)k8;
  auto row_of = [&](int i) {
    int b = (int)((float)i * inv);
    b += (b + 1) * k8 <= i;
    b -= b * k8 > i;
    return b;
  };
  uint4 v[kItems];
#pragma unroll
  for (int j = 0; j < kItems; ++j) {
    const int i = min(tid + j * kProjThreads, n - 1);
    const int b = row_of(i);
    v[j] = *(const uint4*)(a.x + (size_t)seq[b] * a.x_stride + w.k0 + (i - b * k8) * 8);
  }
#pragma unroll
  for (int j = 0; j < kItems; ++j) {
    const int i = tid + j * kProjThreads;
    if constexpr (PPG > 0) {
      // a group lies wholly below n or wholly above it (n and i are aligned
      // to PPG), so every lane of a group takes part in its butterfly
      if (j * kProjThreads < n) {
        constexpr uint32_t kOnes = 0x3F803F80u;  // bf16 (1, 1)
        float t = dot2(v[j].x, kOnes, 0.0f);
        t = dot2(v[j].y, kOnes, t);
        t = dot2(v[j].z, kOnes, t);
        t = dot2(v[j].w, kOnes, t);
        t = group_sum_dpp<PPG>(t);
        if (i < n && (i & (PPG - 1)) == 0) gs[i / PPG] = t;
      }
    }
    if (i < n) {
      const int b = row_of(i);
      *(uint4*)&xs[b * xstride(w.K) + (i - b * k8) * 8] = v[j];
    }
  }
}

// ---------------------------------------------------------------------------
// bf16 rows (vector ALU, dot2)
// ---------------------------------------------------------------------------
// One 512-element step of a bf16 wave tile: acc[r*NB+b] += W_r . x_b over this
// lane's 8 elements.  Inputs are read from LDS in groups of four to bound
// registers.
template <int RP, int NB>
__device__ __forceinline__ void bf16_step(const uint4 (&wv)[RP], const uint16_t* xs, const int (&xo)[NB], int k,
                                          float (&acc)[RP * NB]) {
  constexpr int BG = NB < 4 ? NB : 4;
#pragma unroll
  for (int b0 = 0; b0 < NB; b0 += BG) {
    uint4 xv[BG];
#pragma unroll
    for (int b = 0; b < BG; ++b) xv[b] = *(const uint4*)(xs + xo[b0 + b] + k);
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

template <int EPI, int NB>
__device__ __forceinline__ void bf16_pass(const ProjArgs& a, const Work& wk, int nb, const int32_t* list, int c0,
                                          int* seq, uint16_t* xs, float* red) {
  constexpr int P = Ep<EPI>::P;
  constexpr int R = Ep<EPI>::R;
  constexpr int RP = R * P;
  constexpr int V = RP * NB;
  int lane = threadIdx.x & 63;
  asm volatile("" : "+v"(lane));  // lane-derived values are computed per pass, not held across passes
  const int wave = threadIdx.x >> 6;
  const int wid = wk.wg * kWaves + wave;
  const int nwc = wk.nwg * kWaves;
  const int N = a.N, K = wk.K;
  const int ntiles = (N + R - 1) / R;
  const int idx = xidx<V>(lane);
  const int rr = idx / NB;
  const int bsel = idx - rr * NB;
  const bool lane_ok = lane < V && bsel < nb;

  int xo[NB];  // LDS element offset of each input row
#pragma unroll
  for (int b = 0; b < NB; ++b) xo[b] = (b < nb ? b : nb - 1) * xstride(K);

  float lm = -INFINITY, ls = 0.0f;
  Top2 tp{-INFINITY, 0x7fffffff, -INFINITY};
  // sampled passes: (max, sum exp) of logit / tau, the best Gumbel-perturbed
  // score with its index, and one logit (the draft's, or the final logit at
  // the draft's index)
  float lmt = -INFINITY, lst = 0.0f, pb = -INFINITY, pl = -INFINITY;
  int pi = 0x7fffffff;

  // request the first tile's first weights before the inputs are staged
  const int nfull = K >> 9;                  // full 512-element steps (every lane active)
  const int kt = nfull * 512 + lane * 8;     // this lane's element in the ragged tail
  int t = wid;
  const uint16_t* w[RP];
  uint4 cur[RP];
  auto set_rows = [&](int tt) {
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const int n = EPI == EPI_QKV ? qkv_row<R / 2>(a, tt, r) : min(tt * R + r, N - 1);
      w[r] = bf_row(a, wk, n) + lane * 8;
      if constexpr (P == 2) w[R + r] = a.wb2 + (size_t)n * a.K + wk.k0 + lane * 8;
    }
  };
  if (t < ntiles && nfull > 0) {
    set_rows(t);
#pragma unroll
    for (int r = 0; r < RP; ++r) cur[r] = ld_stream(w[r]);
  }
  stage_rows(list, c0, nb, seq);
  stage_x(a, wk, nb, seq, xs);
  __syncthreads();
  // QKV: the position of this lane's sequence (seq is padded to 8 ids)
  const int pos = EPI == EPI_QKV ? a.lens[seq[bsel]] : 0;

  for (; t < ntiles; t += nwc) {
    const int n0 = t * R;
    if (t != wid || nfull == 0) {
      set_rows(t);
      if (nfull > 0) {
#pragma unroll
        for (int r = 0; r < RP; ++r) cur[r] = ld_stream(w[r]);
      }
    }
    QkvPre pre{};
    if constexpr (EPI == EPI_QKV) pre = qkv_pre(a, seq[bsel], qkv_row<R / 2>(a, t, rr), pos);
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
      bf16_step<RP, NB>(cur, xs, xo, lane * 8 + st * 512, acc);
#pragma unroll
      for (int r = 0; r < RP; ++r) cur[r] = ld_stream(w[r] + (st + 2) * 512);
      bf16_step<RP, NB>(alt, xs, xo, lane * 8 + (st + 1) * 512, acc);
    }
    if (st + 1 < nfull) {
#pragma unroll
      for (int r = 0; r < RP; ++r) alt[r] = ld_stream(w[r] + (st + 1) * 512);
      bf16_step<RP, NB>(cur, xs, xo, lane * 8 + st * 512, acc);
      bf16_step<RP, NB>(alt, xs, xo, lane * 8 + (st + 1) * 512, acc);
    } else if (st < nfull) {
      bf16_step<RP, NB>(cur, xs, xo, lane * 8 + st * 512, acc);
    }
    if (kt < K) {  // ragged tail (K not a multiple of 512)
      uint4 tw[RP];
#pragma unroll
      for (int r = 0; r < RP; ++r) tw[r] = ld_stream(w[r] + nfull * 512);
      bf16_step<RP, NB>(tw, xs, xo, kt, acc);
    }
    XRed<V, 0>::run(acc, lane);
    const float v = acc[0];
    const int n = EPI == EPI_QKV ? qkv_row<R / 2>(a, t, rr) : n0 + (rr % R);
    if constexpr (EPI == EPI_QKV) {
      const float u = xor_lane<1>(v, lane);  // the RoPE partner row sits in the partner lane
      if (lane_ok) qkv_out(a, seq[bsel], n, v, u, pos, pre);
    } else if constexpr (EPI == EPI_SWIGLU) {
      const float u = xor_lane<1>(v, lane);  // the up row sits in the partner lane
      if (lane_ok && (lane & 1) == 0 && n < N)
        ((uint16_t*)a.y)[(size_t)seq[bsel] * a.y_stride + n] = (uint16_t)f2bf(silu_mul(v, u));
    } else if constexpr (EPI == EPI_LSE) {
      if (lane_ok && n < N) lse_merge(lm, ls, v, 1.0f);
    } else if constexpr (EPI == EPI_LSE_S) {
      if (lane_ok && n < N) {
        const int sq = seq[bsel];
        lse_merge(lm, ls, v, 1.0f);
        const float sv = v * a.itau;
        lse_merge(lmt, lst, sv, 1.0f);
        if (sv + kGumbelMax >= pb) {  // else no noise value can lift it above the best
          const float sc = sv + gumbel_noise(a.seed, a.lens[sq], sq, STREAM_DRAFT, n);
          if (sc > pb) {  // rows ascend per lane: the lowest index wins ties
            pb = sc;
            pi = n;
            pl = v;
          }
        }
      }
    } else if constexpr (EPI == EPI_ARGMAX_S) {
      if (lane_ok && n < N) {
        const int sq = seq[bsel];
        if (a.logits) a.logits[(size_t)sq * a.logits_stride + n] = v;
        if (v > tp.v1) {
          tp.v2 = tp.v1;
          tp.v1 = v;
          tp.i1 = n;
        } else if (v > tp.v2) {
          tp.v2 = v;
        }
        const float sv = v * a.itau;
        lse_merge(lmt, lst, sv, 1.0f);
        if (sv + kGumbelMax >= pb) {
          const float sc = sv + gumbel_noise(a.seed, a.lens[sq], sq, STREAM_FINAL, n);
          if (sc > pb) {
            pb = sc;
            pi = n;
          }
        }
        if (n == a.st->draft_tok[sq]) pl = v;
      }
    } else if constexpr (EPI == EPI_RESAMPLE) {
      // rows come in pairs (final input of sequence b, its exit layer's z at
      // row 64 + b): the pair's two values sit in lanes l and l ^ (V / 2)
      const float u = xor_lane<V / 2>(v, lane);
      if (lane_ok && (bsel & 1) == 0 && n < N) {
        const int sq = seq[bsel];
        const float r = __expf(v * a.itau - a.st->lse_f[sq]) - __expf(u * a.itau - a.st->draft_lse[sq]);
        if (r > 0.0f && __logf(r) + kGumbelMax >= pb) {
          const float sc = __logf(r) + gumbel_noise(a.seed, a.lens[sq], sq, STREAM_RESAMPLE, n);
          if (sc > pb) {
            pb = sc;
            pi = n;
          }
        }
      }
    } else if constexpr (EPI == EPI_ARGMAX) {
      if (lane_ok && n < N) {
        if (a.logits) a.logits[(size_t)seq[bsel] * a.logits_stride + n] = v;
        if (v > tp.v1) {
          tp.v2 = tp.v1;
          tp.v1 = v;
          tp.i1 = n;
        } else if (v > tp.v2) {
          tp.v2 = v;
        }
      }
    } else {
      if (lane_ok && n < N) store_out<EPI>(a, wk, seq[bsel], n, v);
    }
  }

  if constexpr (Ep<EPI>::SAMPLED) {
    // 10 floats per lane: reduced through the input stage's LDS (every wave is
    // done with the inputs after this barrier), which keeps the kernel's LDS
    // at two workgroups per CU
    static_assert(kXLdsElems * 2 >= kWaves * 64 * 10 * 4, "the input stage holds the sampled reduction");
    __syncthreads();
    float* rd = reinterpret_cast<float*>(xs);
    float* rw = rd + (wave * 64 + lane) * 8;
    rw[0] = lm;
    rw[1] = ls;
    rw[2] = tp.v1;
    rw[3] = __int_as_float(tp.i1);
    rw[4] = tp.v2;
    rw[5] = lmt;
    rw[6] = lst;
    rw[7] = pl;
    float* rp = rd + kWaves * 64 * 8 + (wave * 64 + lane) * 2;  // the perturbed best and its index
    rp[0] = pb;
    rp[1] = __int_as_float(pi);
    __syncthreads();
    const int tid = threadIdx.x;
    if (tid < nb && (EPI != EPI_RESAMPLE || (tid & 1) == 0)) {
      float m = -INFINITY, sm = 0.0f, mt = -INFINITY, st = 0.0f, lg = -INFINITY, best = -INFINITY;
      int bi = 0x7fffffff;
      Top2 g2{-INFINITY, 0x7fffffff, -INFINITY};
      for (int ww = 0; ww < kWaves; ++ww)
        for (int l = 0; l < V; ++l)
          if (xidx<V>(l) % NB == tid) {
            const float* src = rd + (ww * 64 + l) * 8;
            const float* sp = rd + kWaves * 64 * 8 + (ww * 64 + l) * 2;
            lse_merge(m, sm, src[0], src[1]);
            top2_merge(g2, Top2{src[2], __float_as_int(src[3]), src[4]});
            lse_merge(mt, st, src[5], src[6]);
            lg = fmaxf(lg, src[7]);
            const int si = __float_as_int(sp[1]);
            if (sp[0] > best || (sp[0] == best && si < bi)) {
              best = sp[0];
              bi = si;
            }
          }
      // by list position (what decide and final merge), and by sequence
      float* out = a.part + ((size_t)blockIdx.x * kMaxBatch + (c0 + tid)) * 4;
      float* os = a.part_s + ((size_t)blockIdx.x * kMaxBatch + seq[tid]) * kPartS;
      if constexpr (EPI == EPI_LSE_S) {
        out[0] = m;
        out[1] = sm;
      } else if constexpr (EPI == EPI_ARGMAX_S) {
        out[0] = g2.v1;
        out[1] = __int_as_float(g2.i1);
        out[2] = g2.v2;
      }
      if constexpr (EPI == EPI_RESAMPLE) {
        os[0] = best;
        os[1] = __int_as_float(bi);
      } else {
        os[0] = mt;
        os[1] = st;
        os[2] = best;
        os[3] = __int_as_float(bi);
        os[4] = lg;
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
//
// Work split: a 16-row tile is shared by WPT waves (1, 2, 4 or 8, chosen so
// each wave owns about D blocks of 128 columns); a workgroup works on 8/WPT
// tiles at a time.  Each wave keeps D blocks of codes and their scales in
// flight in a register ring, refilled as blocks are consumed; the refills run
// on into the workgroup's next tiles, so one tile's reduction overlaps the
// next tile's loads.  A ring slot past the wave's work loads from the scale
// array (always valid) and contributes zero.
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

// tot += (sl * s_row) * (C - corr) for the 4 rows of this lane (sv: their 4
// scales; corr = 136 * the group's input sum; sl is 1, or 0 for a slot
// without work)
__device__ __forceinline__ void i4_group_scale(const uint2& sv, float sl, const f32x4_t& cg, float corr,
                                               f32x4_t& tot) {
  tot[0] = fmaf(sl * bf2f(sv.x & 0xffffu), cg[0] - corr, tot[0]);
  tot[1] = fmaf(sl * bf2f(sv.x >> 16), cg[1] - corr, tot[1]);
  tot[2] = fmaf(sl * bf2f(sv.y & 0xffffu), cg[2] - corr, tot[2]);
  tot[3] = fmaf(sl * bf2f(sv.y >> 16), cg[3] - corr, tot[3]);
}

// Ring depth (blocks of 128 columns in flight per wave): bf16 blocks are 64
// bytes per lane (four MFMA A operands), int4 blocks 16 bytes of codes plus
// the scales; within 128 VGPRs.
template <bool BF, int P, int NG>
struct MmaRing {
  static constexpr int D = BF ? (P == 2 ? 1 : 2) : (P == 2 ? (NG == 1 ? 2 : 1) : NG == 4 ? 2 : 4);
};

// Waves sharing a 16-row tile (splitting its 128-column blocks), a power of
// two up to the block count: the split with the fewest block steps per wave
// over the whole pass (rounds of the range's waves x blocks per wave), and of
// those the fewest rounds (each round waits out a memory latency and a
// cross-wave reduction).
__host__ __device__ inline int mma_wpt(int nfull, int ntiles, int nwaves) {
  int best = 1;
  long long best_cost = -1, best_rounds = 0;
  for (int w = 1; w <= kWaves && w <= nfull; w *= 2) {
    const long long rounds = ((long long)ntiles * w + nwaves - 1) / nwaves;
    const long long cost = rounds * ((nfull + w - 1) / w);
    if (best_cost < 0 || cost < best_cost || (cost == best_cost && rounds < best_rounds)) {
      best = w;
      best_cost = cost;
      best_rounds = rounds;
    }
  }
  return best;
}

// MFMA pass over 16-row tiles for one weight format: BF true reads the bf16
// rows straight into the A operands (lane (m, q) holds row m, columns
// 8q..8q+7 of each 32-column step); BF false unpacks int4 codes (see above).
// The inputs are the B operand (batch rows padded to 16 with zeros).
template <int EPI, int NG, bool BF>
__device__ __forceinline__ void mma_pass(const ProjArgs& a, const Work& wk, int wpt, int nb, const int32_t* list,
                                         int c0, int* seq, uint16_t* xs, float* red, float* gs) {
  constexpr int P = Ep<EPI>::P;
  constexpr int D = MmaRing<BF, P, NG>::D;
  constexpr int SL = BF ? 4 : 1;  // 16-byte loads per block and matrix
  int lane = threadIdx.x & 63;
  asm volatile("" : "+v"(lane));  // lane-derived values are computed per pass, not held across passes
  const int wave = threadIdx.x >> 6;
  const int m = lane & 15, q = lane >> 4;
  // (no integer division below: the group size follows from NG, the wave
  // split is a power of two; each wave repeats this setup)
  constexpr int G = 128 / NG;
  const int N = a.N, K = wk.K;
  const int ntiles = (N + 15) >> 4;
  const int ldc = a.K >> 3;             // dwords per code row
  const int ngr = a.K / G;              // scale groups per row of the whole matrix
  const int gk0 = wk.k0 / G;            // first group of this range
  const int nfull = K >> 7;
  const int ntail = (K & 127) >> 5;     // MFMA steps in the tail
  // (wpt = mma_wpt(nfull, ntiles, wk.nwg * kWaves), computed by launch_proj)
  const int lw = __builtin_ctz(wpt);
  const int tpi = kWaves >> lw;         // tiles per workgroup iteration
  const int ws = wave & (wpt - 1);      // this wave's K slice of its tile
  const int b0 = (ws * nfull) >> lw;
  const int nbw = (((ws + 1) * nfull) >> lw) - b0;
  const int nbp = (((nfull + wpt - 1) >> lw) + D - 1) / D * D;  // ring rounds per tile, same for all waves
  const int nit = (ntiles + tpi - 1) >> (3 - lw);              // workgroup iterations in the range
  const bool bok = m < nb;
  const bool tail_here = ws == wpt - 1 && ntail > 0;
  const uint16_t* xrow = xs + (bok ? m : 0) * xstride(K);
  const float* gsr = gs + (bok ? m : 0) * (K / G);  // int4: this column's group sums

  // weight row of MFMA A row mm of tile tt (the QKV epilogue pairs RoPE rows)
  // (bf16 rows past N read row N-1; int4 rows are padded to a multiple of 16)
  auto arow = [&](int tt, int mm) {
    return EPI == EPI_QKV ? qkv_row<8>(a, tt, mm) : BF ? min(tt * 16 + mm, N - 1) : tt * 16 + mm;
  };
  auto tile_of = [&](int j) { return (wk.wg + j * wk.nwg) * tpi + (wave >> lw); };
  auto has_iter = [&](int j) { return wk.wg + j * wk.nwg < nit; };
  // where a tile's loads start for this lane: bf16 row pointers (first
  // block of the slice), or int4 code and scale offsets; ok false: no tile
  struct TileAt {
    const uint16_t* w0;
    const uint16_t* w1;
    int code, scale;
    bool ok;
  };
  auto tile_at = [&](int j) {
    TileAt r{a.wb[0], a.wb[0], 0, 0, false};
    const int t = tile_of(j);
    if (!has_iter(j) || t >= ntiles) return r;
    r.ok = true;
    const int n = arow(t, m);
    if constexpr (BF) {
      r.w0 = bf_row(a, wk, n) + b0 * 128 + q * 8;
      if constexpr (P == 2) r.w1 = a.wb2 + (size_t)n * a.K + wk.k0 + b0 * 128 + q * 8;
    } else {
      const int r0 = arow(t, 4 * q);
      r.code = n * ldc + (wk.k0 >> 3) + b0 * 16 + q * 4;
      r.scale = ((r0 >> 4) * ngr + gk0 + b0 * NG) * 16 + (r0 & 15);
    }
    return r;
  };

  uint4 ra[P][D][SL];
  uint2 sc[P][D][NG];
  // a slot without work loads a line of its own (spread, so the idle loads
  // of all waves do not queue on one L2 channel) and contributes zero
  const int gwave = (wk.chunk * wk.nwg + wk.wg) * kWaves + wave;
  const int ispan = BF ? min(ntiles * 16, N * a.K) : ntiles * 16 * ngr;  // elements that may be read
  const int imask = (1 << (31 - __builtin_clz(ispan))) - 1;              // power of two <= ispan, minus 1
  const uint16_t* idle = (BF ? a.wb[0] : a.s4) + ((gwave * (BF ? 64 : 32)) & imask);
  // issue the loads of block kk of the wave's slice of tile c (here) or n
  // into ring slot i (member-wise selects keep everything in registers)
  auto issue = [&](const TileAt& c, const TileAt& nx, bool here, int kk, int i) {
    const bool ok = here ? c.ok : nx.ok;
    const bool real = ok && kk < nbw;
#pragma unroll
    for (int p = 0; p < P; ++p) {
      if constexpr (BF) {
        const uint16_t* base = p == 0 ? (here ? c.w0 : nx.w0) : (here ? c.w1 : nx.w1);
        const uint16_t* src = real ? base + kk * 128 : idle;
#pragma unroll
        for (int st = 0; st < 4; ++st) ra[p][i][st] = ld_stream(src + (real ? st * 32 : 0));
      } else {
        const uint32_t* cb = p == 0 ? a.q4 : a.q4b;
        const uint16_t* sb = p == 0 ? a.s4 : a.s4b;
        const int code = here ? c.code : nx.code;
        const int scale = here ? c.scale : nx.scale;
        // cached load: a block's codes are half of a 128-byte line per row, the
        // other half being the next block; a streaming load fetched the line
        // twice (measured 1.37x the algorithmic bytes for gate/up, 1.035x cached)
        ra[p][i][0] = *(const uint4*)(real ? (const void*)(cb + code + kk * 16) : (const void*)idle);
#pragma unroll
        for (int g = 0; g < NG; ++g) sc[p][i][g] = *(const uint2*)(real ? sb + scale + (kk * NG + g) * 16 : idle);
      }
    }
  };
  TileAt at_cur = tile_at(0);
  if (nfull > 0) {
#pragma unroll
    for (int i = 0; i < D; ++i) issue(at_cur, at_cur, true, i, i);
  }
  stage_rows(list, c0, nb, seq);
  stage_x<BF ? 0 : G / 8>(a, wk, nb, seq, xs, gs);
  __syncthreads();
  // QKV: the position of this column's sequence, read while the tiles run
  const int pos = EPI == EPI_QKV ? a.lens[seq[bok ? m : 0]] : 0;

  float lm = -INFINITY, ls = 0.0f;            // EPI_LSE: running (max, sum exp) of column m
  Top2 tp{-INFINITY, 0x7fffffff, -INFINITY};  // EPI_ARGMAX
  for (int j = 0; has_iter(j); ++j) {
    const int t = tile_of(j);
    const int r0 = arow(t, 4 * q);
    const TileAt at_nxt = tile_at(j + 1);
    f32x4_t tot[P];
#pragma unroll
    for (int p = 0; p < P; ++p) tot[p] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
    for (int kk = 0; kk < nbp; kk += D) {
#pragma unroll
      for (int i = 0; i < D; ++i) {
        // straight-line ring body (a branch around it would make the
        // compiler wait for every load in flight): a slot past this wave's
        // blocks computes on in-bounds data and is multiplied by 0
        const bool live = kk + i < nbw && t < ntiles;
        const float sl = live ? 1.0f : 0.0f;
        const int u = min(b0 + kk + i, max(nfull - 1, 0));
        if constexpr (BF) {
#pragma unroll
          for (int p = 0; p < P; ++p) {
            f32x4_t cg = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
            for (int st = 0; st < 4; ++st) {
              uint4 bv = *(const uint4*)(xrow + u * 128 + 32 * st + 8 * q);
              if (!bok) bv = make_uint4(0, 0, 0, 0);
              cg = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, ra[p][i][st]),
                                                           __builtin_bit_cast(bf16x8_t, bv), cg, 0, 0, 0);
            }
#pragma unroll
            for (int e = 0; e < 4; ++e) tot[p][e] = fmaf(sl, cg[e], tot[p][e]);
          }
        } else {
          constexpr int MPG = 4 / NG;  // MFMA steps per scale group
          // the group's 136 * sum(x) for this lane's batch column (0 for a
          // padding column, whose inputs are zero)
          float corr[NG];
#pragma unroll
          for (int g = 0; g < NG; ++g) corr[g] = bok ? 136.0f * gsr[u * NG + g] : 0.0f;
#pragma unroll
          for (int p = 0; p < P; ++p) {
            f32x4_t cg = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
            for (int st = 0; st < 4; ++st) {
              uint4 bv = *(const uint4*)(xrow + u * 128 + 32 * st + 8 * q);
              if (!bok) bv = make_uint4(0, 0, 0, 0);
              cg = __builtin_amdgcn_mfma_f32_16x16x32_bf16(unpack8(pick(ra[p][i][0], st)),
                                                           __builtin_bit_cast(bf16x8_t, bv), cg, 0, 0, 0);
              if (st % MPG == MPG - 1) {
                i4_group_scale(sc[p][i][st / MPG], sl, cg, corr[st / MPG], tot[p]);
                cg = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
              }
            }
          }
        }
        // refill with the block D ahead, in this tile or the next (a select,
        // not a branch, so the loads stay unconditional)
        const bool here = kk + i + D < nbp;
        issue(at_cur, at_nxt, here, here ? kk + i + D : kk + i + D - nbp, i);
      }
    }
    if (tail_here && t < ntiles) {  // K mod 128: steps of 32 columns, last wave of the tile
      f32x4_t cgt[P];
#pragma unroll
      for (int p = 0; p < P; ++p) cgt[p] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
      for (int st = 0; st < ntail; ++st) {
        const int ka = nfull * 128 + 32 * st;
        uint4 bv = *(const uint4*)(xrow + ka + 8 * q);
        if (!bok) bv = make_uint4(0, 0, 0, 0);
        const bf16x8_t b8 = __builtin_bit_cast(bf16x8_t, bv);
        if constexpr (BF) {
#pragma unroll
          for (int p = 0; p < P; ++p) {
            const int n = arow(t, m);
            const uint16_t* wr = p == 0 ? bf_row(a, wk, n) : a.wb2 + (size_t)n * a.K + wk.k0;
            const uint4 av = *(const uint4*)(wr + ka + 8 * q);
            tot[p] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, av), b8, tot[p], 0, 0, 0);
          }
        } else {
          // the tail holds whole scale groups (K is a multiple of G): the
          // group's products accumulate over its steps and are scaled at its
          // last step
#pragma unroll
          for (int p = 0; p < P; ++p) {
            const uint32_t* cb = p == 0 ? a.q4 : a.q4b;
            const uint32_t word = cb[(size_t)arow(t, m) * ldc + ((wk.k0 + ka) >> 3) + q];
            cgt[p] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(unpack8(word), b8, cgt[p], 0, 0, 0);
          }
          if ((st + 1) % (G / 32) == 0) {
            const float corr = bok ? 136.0f * gsr[ka / G] : 0.0f;
#pragma unroll
            for (int p = 0; p < P; ++p) {
              const uint16_t* sb = p == 0 ? a.s4 : a.s4b;
              const uint2 sv = *(const uint2*)(sb + ((size_t)(r0 >> 4) * ngr + gk0 + ka / G) * 16 + (r0 & 15));
              i4_group_scale(sv, 1.0f, cgt[p], corr, tot[p]);
              cgt[p] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
            }
          }
        }
      }
    }
    at_cur = at_nxt;
    // with several waves per tile, sum their K slices in slice order; wave
    // (tile index) tt of the iteration finishes tile tt
    float vals[P][4];
#pragma unroll
    for (int p = 0; p < P; ++p)
#pragma unroll
      for (int i = 0; i < 4; ++i) vals[p][i] = tot[p][i];
    const bool fin = wave < tpi;
    if (wpt > 1) {
#pragma unroll
      for (int p = 0; p < P; ++p) {
        float* rw = red + (wave * 64 + lane) * 4;
        rw[0] = tot[p][0];
        rw[1] = tot[p][1];
        rw[2] = tot[p][2];
        rw[3] = tot[p][3];
        __syncthreads();
        if (fin) {
          // slices in order (wpt is an even power of two here), two reads
          // in flight
          float s0 = 0.0f, s1 = 0.0f, s2 = 0.0f, s3 = 0.0f;
          const float* rs = red + ((wave * wpt) * 64 + lane) * 4;
          for (int ww = 0; ww < wpt; ww += 2) {
            const float4 u = *(const float4*)(rs + ww * 256);
            const float4 v = *(const float4*)(rs + (ww + 1) * 256);
            s0 = (s0 + u.x) + v.x;
            s1 = (s1 + u.y) + v.y;
            s2 = (s2 + u.z) + v.z;
            s3 = (s3 + u.w) + v.w;
          }
          vals[p][0] = s0;
          vals[p][1] = s1;
          vals[p][2] = s2;
          vals[p][3] = s3;
        }
        __syncthreads();
      }
    }
    if (!fin) continue;
    const int tf = (wk.wg + j * wk.nwg) * tpi + wave;  // the tile this wave finishes
    if (tf >= ntiles) continue;
    if constexpr (EPI == EPI_QKV) {
      // lane (q, m) holds rows arow(tf, 4q + i); the RoPE partners sit in lane ^ 32
      float u[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) u[i] = xor_lane<32>(vals[0][i], lane);
      if (!bok) continue;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int n = arow(tf, 4 * q + i);
        qkv_out(a, seq[m], n, vals[0][i], u[i], pos, qkv_pre(a, seq[m], n, pos));
      }
      continue;
    }
    if (!bok) continue;
    // lane (q, m) holds rows tf*16 + 4q + i of batch column m
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int n = tf * 16 + 4 * q + i;
      if (n >= N) continue;
      const float v = vals[0][i];
      if constexpr (EPI == EPI_SWIGLU) {
        ((uint16_t*)a.y)[(size_t)seq[m] * a.y_stride + n] = (uint16_t)f2bf(silu_mul(v, vals[P - 1][i]));
      } else if constexpr (EPI == EPI_LSE) {
        lse_merge(lm, ls, v, 1.0f);
      } else if constexpr (EPI == EPI_ARGMAX) {
        if (a.logits) a.logits[(size_t)seq[m] * a.logits_stride + n] = v;
        if (v > tp.v1) {  // rows arrive in increasing order within a lane: ties keep the lowest
          tp.v2 = tp.v1;
          tp.v1 = v;
          tp.i1 = n;
        } else if (v > tp.v2) {
          tp.v2 = v;
        }
      } else {
        store_out<EPI>(a, wk, seq[m], n, v);
      }
    }
  }

  if constexpr (EPI == EPI_LSE || EPI == EPI_ARGMAX) {
    // per column m: merge the 4 lanes (q) of every wave, waves in order
    __syncthreads();  // the tile reductions are done with red
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
        float mm = -INFINITY, s = 0.0f;
        for (int ww = 0; ww < kWaves; ++ww)
          for (int qq = 0; qq < 4; ++qq) {
            const float* src = red + (ww * 64 + qq * 16 + tid) * 4;
            lse_merge(mm, s, src[0], src[1]);
          }
        out[0] = mm;
        out[1] = s;
      } else {
        Top2 best{-INFINITY, 0x7fffffff, -INFINITY};
        for (int ww = 0; ww < kWaves; ++ww)
          for (int qq = 0; qq < 4; ++qq) {
            const float* src = red + (ww * 64 + qq * 16 + tid) * 4;
            top2_merge(best, Top2{src[0], __float_as_int(src[1]), src[2]});
          }
        out[0] = best.v1;
        out[1] = __int_as_float(best.i1);
        out[2] = best.v2;
      }
    }
  }
}

// Zero rows: stands in for an absent row list or count (its address on each
// device is resolved by no_rows()).
__device__ int32_t kNoRows[8] = {0, 0, 0, 0, 0, 0, 0, 0};

template <int EPI, int NG>
__global__ __launch_bounds__(kProjThreads, 4) void proj_kernel(const ProjArgs a) {
  __shared__ __attribute__((aligned(16))) uint16_t xs[kXLdsElems + 8 * 8];
  __shared__ __attribute__((aligned(16))) float red[kWaves * 64 * 4];
  __shared__ int seqc[8];  // sequence ids of the staged rows of a later chunk
  // int4 pass: sums of the staged rows over each scale group of the range
  constexpr bool kI4 = EPI == EPI_PART || EPI == EPI_SWIGLU || EPI == EPI_QKV;
  __shared__ float gsum[kI4 ? kXLdsElems / (128 / NG) : 1];
  Work wk;
  wk.nwg = a.nwg_r;
  wk.chunk = 0;
  while ((wk.chunk + 1) * wk.nwg <= (int)blockIdx.x) ++wk.chunk;
  wk.wg = blockIdx.x - wk.chunk * wk.nwg;
  wk.k0 = wk.chunk * a.kc;
  wk.K = min(a.kc, a.K - wk.k0);
  // Row counts, read through the scalar cache (uniform addresses) before
  // anything else; launch_proj points an absent list or count at kNoRows, so
  // nothing here branches on a pointer.  Each pass stages its own ids.
  __shared__ int seq0[2][8];
  // (the resampling pass's list holds row pairs: up to 2 * kMaxBatch entries)
  const int n_bf = min(max(*(const cint*)a.cnt_bf, 0), EPI == EPI_RESAMPLE ? 2 * kMaxBatch : kMaxBatch);
  const int n_i4 = min(max(*(const cint*)a.cnt_i4, 0), kMaxBatch);
  if constexpr (EPI == EPI_RESAMPLE) {
    if (n_bf == 0) return;  // nothing rejected
  }
  // When both weight formats have rows, the workgroups of each column range
  // split between them (the int4 share above its share of the bytes, since
  // that pass is latency-bound) and the two passes run side by side instead
  // of one after the other.  The bf16 share (of 256) was measured per
  // projection kind: QKV and O (at most 2 ranges) 176, the FFN (gate/up,
  // down) 128.
  int fmt_lo = 0, fmt_hi = 1;
  int wsel = wk.chunk == a.nkc - 1 ? 1 : 0;  // int4 wave split: last range or not
  if constexpr (EPI == EPI_PART || EPI == EPI_QKV || EPI == EPI_SWIGLU) {
    if (n_bf == 0) {
      // only exited rows: a smaller grid works (measured at the 8B widths,
      // 256 against 512 workgroups: O 10.3 -> 9.2 us, QKV 12.5 -> 10.6, down
      // 15.3 -> 14.2, gate/up 20.2 -> 19.6; fewer workgroups stage fewer
      // copies of the inputs).  The first nkc * nwg_i4 workgroups take the
      // work (so the dispatcher spreads them over the CUs as it would a grid
      // of that size); the rest return at once.
      const int nw4 = a.nwg_i4;
      if ((int)blockIdx.x >= a.nkc * nw4) return;
      wk.nwg = nw4;
      wk.chunk = 0;
      while ((wk.chunk + 1) * nw4 <= (int)blockIdx.x) ++wk.chunk;
      wk.wg = blockIdx.x - wk.chunk * nw4;
      wk.k0 = wk.chunk * a.kc;
      wk.K = min(a.kc, a.K - wk.k0);
      wsel = wk.chunk == a.nkc - 1 ? 1 : 0;
    } else if (n_i4 > 0 && wk.nwg >= 2) {
      const int nbf = a.nbf_mix;
      wsel += 2;
      if (wk.wg < nbf) {
        fmt_hi = 0;
        wk.nwg = nbf;
      } else {
        fmt_lo = 1;
        wk.wg -= nbf;
        wk.nwg -= nbf;
      }
    }
  }
  const int wpt = a.wpt4[wsel];
  bool first = true;  // the first pass needs no barrier: nothing in LDS is in use yet
  for (int fmt = fmt_lo; fmt <= fmt_hi; ++fmt) {
    if constexpr (Ep<EPI>::VOCAB || EPI == EPI_BF16) {
      if (fmt == 1) break;  // these run on backbone rows only
    }
    const int n = fmt ? n_i4 : n_bf;
    const int32_t* list = fmt ? a.list_i4 : a.list_bf;

    for (int c0 = 0; c0 < n; c0 += 8) {
      const int nb = min(8, n - c0);
      if (!first) __syncthreads();  // the previous pass is done with xs, red and seq
      first = false;
      int* seq = c0 == 0 ? seq0[fmt] : seqc;
      if (fmt == 0) {
        if constexpr (kBf16Mfma) {
          mma_pass<EPI, NG, true>(a, wk, wpt, nb, list, c0, seq, xs, red, gsum);
        } else {
          if (nb == 1)
            bf16_pass<EPI, 1>(a, wk, nb, list, c0, seq, xs, red);
          else if (nb == 2)
            bf16_pass<EPI, 2>(a, wk, nb, list, c0, seq, xs, red);
          else if (nb <= 4)
            bf16_pass<EPI, 4>(a, wk, nb, list, c0, seq, xs, red);
          else
            bf16_pass<EPI, 8>(a, wk, nb, list, c0, seq, xs, red);
        }
      } else {
        if constexpr (EPI == EPI_PART || EPI == EPI_SWIGLU || EPI == EPI_QKV)
          mma_pass<EPI, NG, false>(a, wk, wpt, nb, list, c0, seq, xs, red, gsum);
      }
    }
  }
}

bool proj_fits(int K, int batch) { return (long long)std::min(8, batch) * K <= kXLdsElems; }

template <int EPI, int NG>
static void launch_k(const ProjArgs& a, int g, hipStream_t s, hipEvent_t ev0, hipEvent_t ev1) {
  if (ev0)
    hipExtLaunchKernelGGL((proj_kernel<EPI, NG>), dim3(g), dim3(kProjThreads), 0, s, ev0, ev1, 0, a);
  else
    hipLaunchKernelGGL((proj_kernel<EPI, NG>), dim3(g), dim3(kProjThreads), 0, s, a);
}

template <int EPI>
static void launch_ng(const ProjArgs& a, int g, hipStream_t s, hipEvent_t ev0, hipEvent_t ev1) {
  if constexpr (EPI == EPI_PART || EPI == EPI_SWIGLU || EPI == EPI_QKV) {
    if (a.G == 32) return launch_k<EPI, 4>(a, g, s, ev0, ev1);
    if (a.G == 64) return launch_k<EPI, 2>(a, g, s, ev0, ev1);
  }
  launch_k<EPI, 1>(a, g, s, ev0, ev1);
}

int proj_ranges(int K, int N, int nwg, int batch, int* kc) {
  // whole 128-column blocks that fit the stage, and enough ranges that the
  // 16-row int4 tiles of all ranges cover the grid (ranges of >= 8 blocks)
  const int rows = std::min(8, batch);
  const int g = std::max(1, std::min(nwg, kNwgMax));
  const int blocks = (K + 127) / 128;
  const int cmax = (kXLdsElems / rows) / 128;  // blocks per range at most
  const int nmin = (blocks + cmax - 1) / cmax;
  const int want = std::min(4, g * 16 / std::max(N, 1));
  const int n = std::max(1, std::max(nmin, std::min(want, blocks / 8)));
  const int kcb = (blocks + n - 1) / n;
  if (kc) *kc = kcb * 128;
  return (blocks + kcb - 1) / kcb;
}

const int32_t* no_rows() {
  constexpr int kMaxDevices = 64;
  static const int32_t* addr[kMaxDevices] = {};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices)
    throw std::runtime_error("no_rows: no current HIP device");
  if (!addr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(kNoRows)) != hipSuccess || !p)
      throw std::runtime_error("no_rows: hipGetSymbolAddress failed");
    addr[dev] = (const int32_t*)p;
  }
  return addr[dev];
}

int launch_proj(int epi, const ProjArgs& a0, int nwg, int batch, hipStream_t s, hipEvent_t ev0, hipEvent_t ev1) {
  ProjArgs a = a0;
  if (!a.cnt_bf || !a.list_bf) a.cnt_bf = a.list_bf = no_rows();
  if (!a.cnt_i4 || !a.list_i4) a.cnt_i4 = a.list_i4 = no_rows();
  // the vocabulary epilogues write one partial per workgroup (kNwgMax of them)
  int g = std::max(1, std::min(nwg, kNwgMax));
  a.nkc = 1;
  a.kc = a.K;
  if (epi == EPI_PART) {
    a.nkc = proj_ranges(a.K, a.N, nwg, batch, &a.kc);
    g = std::max(1, g / a.nkc) * a.nkc;
  } else if (!proj_fits(a.K, batch)) {
    throw std::logic_error("projection input too wide for the stage");
  }
  a.nwg_r = g / a.nkc;
  // the workgroup split between the formats and the int4 wave split, as the
  // device would derive them: bf16 share of each range (of 256: measured per
  // projection kind), trimmed so the bf16 waves keep the whole rounds of
  // tiles the share gives them; int4 waves per tile by mma_wpt
  a.nbf_mix = 0;
  a.nwg_i4 = std::max(1, a.nwg_r / 2);
  for (int i = 0; i < 4; ++i) a.wpt4[i] = 1;
  if (epi == EPI_PART || epi == EPI_SWIGLU || epi == EPI_QKV) {
    const int nw = a.nwg_r;
    if (nw >= 2) {
      const int R = epi == EPI_SWIGLU ? 1 : 2;  // bf16 rows per wave tile
      const int share = (epi == EPI_SWIGLU || a.nkc > 2) ? kBfShareFfn : kBfShare;
      int nbf = std::min(nw - 1, std::max(1, (nw * share) >> 8));
      const int tb = (a.N + R - 1) / R;
      const int rounds = (tb + nbf * kWaves - 1) / (nbf * kWaves);
      nbf = std::min(nbf, std::max(1, (tb + rounds * kWaves - 1) / (rounds * kWaves)));
      a.nbf_mix = nbf;
    }
    const int ntiles = (a.N + 15) >> 4;
    for (int mixed = 0; mixed < 2; ++mixed)
      for (int last = 0; last < 2; ++last) {
        const int kr = last ? a.K - (a.nkc - 1) * a.kc : a.kc;
        const int nwr = mixed ? std::max(1, nw - a.nbf_mix) : a.nwg_i4;
        a.wpt4[mixed * 2 + last] = mma_wpt(kr >> 7, ntiles, nwr * kWaves);
      }
  }
  if (epi == EPI_QKV && (a.hd < 32 || (a.hd & (a.hd - 1)) || (1 << a.hd_log2) != a.hd))
    throw std::logic_error("QKV epilogue needs a power-of-two head_dim >= 32 and its log2");
  switch (epi) {
    case EPI_BF16: launch_ng<EPI_BF16>(a, g, s, ev0, ev1); break;
    case EPI_PART: launch_ng<EPI_PART>(a, g, s, ev0, ev1); break;
    case EPI_SWIGLU: launch_ng<EPI_SWIGLU>(a, g, s, ev0, ev1); break;
    case EPI_LSE: launch_ng<EPI_LSE>(a, g, s, ev0, ev1); break;
    case EPI_ARGMAX: launch_ng<EPI_ARGMAX>(a, g, s, ev0, ev1); break;
    case EPI_QKV: launch_ng<EPI_QKV>(a, g, s, ev0, ev1); break;
    case EPI_LSE_S: launch_ng<EPI_LSE_S>(a, g, s, ev0, ev1); break;
    case EPI_ARGMAX_S: launch_ng<EPI_ARGMAX_S>(a, g, s, ev0, ev1); break;
    case EPI_RESAMPLE: launch_ng<EPI_RESAMPLE>(a, g, s, ev0, ev1); break;
    default: throw std::logic_error("projection: unknown epilogue");
  }
  return a.nkc;
}

// ---------------------------------------------------------------------------
// Residual finish: h = hsrc + the partial sums of the column ranges (fixed
// order; hsrc may be h itself), then the RMSNorm of the new residual for the
// next projection (bf16(h * rsqrt(mean(h^2) + eps) * g)) and optionally
// bf16(h).  With STS, also the state transition similarity of the row
// (River-LLM explainer, section 5.1): the cosine between the layer's input
// hin and the new residual, dot / (|hin| |h|) with each norm floored at 1e-12
// (hin is read before h is written, so it may be h).  One workgroup per row.
// ---------------------------------------------------------------------------
constexpr int kFinThreads = 256;
constexpr int kFinVec = 4;    // float4 per thread per row chunk
constexpr int kFinParts = 8;  // column ranges summed with all loads in flight (at most)

// A workgroup owns a row.  Rows up to kFinThreads * kFinVec * 4 columns are
// held in registers between the sum of squares and the normalisation; wider
// rows are processed in chunks and re-read (this workgroup wrote them).  Every
// load of a chunk (residual, partial sums, gains) is issued before any is used.
template <bool STS, int NP>
__global__ __launch_bounds__(kFinThreads) void finish_kernel(float* h, const float* hsrc, const float* parts,
                                                             int nparts, size_t cstride, int d, const uint16_t* gain,
                                                             float eps, uint16_t* x, uint16_t* hb, const float* hin,
                                                             float* sts) {
  const int b = blockIdx.x;
  const int tid = threadIdx.x;
  const int d4 = d >> 2;
  float* hr = h + (size_t)b * d;
  const float* hs = hsrc + (size_t)b * d;
  const float* hi = STS ? hin + (size_t)b * d : hs;
  const int per = kFinThreads * kFinVec;  // float4 per chunk
  const bool one = d4 <= per;
  float ss = 0.0f, si = 0.0f, sd = 0.0f;
  float4 v[kFinVec];
  uint2 g[kFinVec];
  // ranges past nparts reload the last one (or, with none, the source row
  // itself: parts may be null then) and are not added; every load of a chunk
  // is unconditional (a branch around a load makes the compiler wait for the
  // loads before it)
  const float* pbase = nparts > 0 ? parts + (size_t)b * d : hs;
  const size_t pcs = nparts > 0 ? cstride : 0;
  const int plast = max(nparts - 1, 0);
  for (int c0 = 0; c0 < d4; c0 += per) {
    float4 pv[NP][kFinVec];
    float4 vi[kFinVec];
#pragma unroll
    for (int j = 0; j < kFinVec; ++j) {
      const int i = min(c0 + tid + j * kFinThreads, d4 - 1);
      v[j] = *(const float4*)(hs + 4 * i);
      if constexpr (STS) vi[j] = *(const float4*)(hi + 4 * i);
      g[j] = *(const uint2*)(gain + 4 * i);
#pragma unroll
      for (int c = 0; c < NP; ++c) pv[c][j] = *(const float4*)(pbase + min(c, plast) * pcs + 4 * i);
    }
#pragma unroll
    for (int j = 0; j < kFinVec; ++j) {
#pragma unroll
      for (int c = 0; c < NP; ++c) {
        if (c < nparts) {
          v[j].x += pv[c][j].x;
          v[j].y += pv[c][j].y;
          v[j].z += pv[c][j].z;
          v[j].w += pv[c][j].w;
        }
      }
      for (int c = NP; c < nparts; ++c) {  // more ranges than NP (very wide inputs)
        const int i = min(c0 + tid + j * kFinThreads, d4 - 1);
        const float4 p = *(const float4*)(parts + c * cstride + (size_t)b * d + 4 * i);
        v[j].x += p.x;
        v[j].y += p.y;
        v[j].z += p.z;
        v[j].w += p.w;
      }
      const int i = c0 + tid + j * kFinThreads;
      if (i >= d4) continue;
      *(float4*)(hr + 4 * i) = v[j];
      ss = fmaf(v[j].x, v[j].x, ss);
      ss = fmaf(v[j].y, v[j].y, ss);
      ss = fmaf(v[j].z, v[j].z, ss);
      ss = fmaf(v[j].w, v[j].w, ss);
      if constexpr (STS) {
        si = fmaf(vi[j].x, vi[j].x, si);
        si = fmaf(vi[j].y, vi[j].y, si);
        si = fmaf(vi[j].z, vi[j].z, si);
        si = fmaf(vi[j].w, vi[j].w, si);
        sd = fmaf(vi[j].x, v[j].x, sd);
        sd = fmaf(vi[j].y, v[j].y, sd);
        sd = fmaf(vi[j].z, v[j].z, sd);
        sd = fmaf(vi[j].w, v[j].w, sd);
      }
      if (hb) {
        uint2 o;
        o.x = f2bf(v[j].x) | (f2bf(v[j].y) << 16);
        o.y = f2bf(v[j].z) | (f2bf(v[j].w) << 16);
        *(uint2*)(hb + (size_t)b * d + 4 * i) = o;
      }
    }
  }
  constexpr int kW = kFinThreads / 64;
  __shared__ float wsum[3][kW];
  __shared__ float rs;
  each_offset_down<1>([&](auto mc) {
    constexpr int M = decltype(mc)::value;
    ss += xor_lane<M>(ss, tid & 63);
    if constexpr (STS) {
      si += xor_lane<M>(si, tid & 63);
      sd += xor_lane<M>(sd, tid & 63);
    }
  });
  if ((tid & 63) == 0) {
    wsum[0][tid >> 6] = ss;
    wsum[1][tid >> 6] = si;
    wsum[2][tid >> 6] = sd;
  }
  __syncthreads();
  if (tid == 0) {
    float t = 0.0f, ti = 0.0f, td = 0.0f;
    for (int w = 0; w < kW; ++w) {
      t += wsum[0][w];
      ti += wsum[1][w];
      td += wsum[2][w];
    }
    rs = 1.0f / sqrtf(t / (float)d + eps);
    if constexpr (STS) sts[b] = td / (fmaxf(sqrtf(ti), 1e-12f) * fmaxf(sqrtf(t), 1e-12f));
  }
  __syncthreads();
  const float r = rs;
  auto put = [&](int i, const float4& vv, const uint2& gg) {
    uint2 o;
    o.x = f2bf(vv.x * r * bf2f(gg.x & 0xffffu)) | (f2bf(vv.y * r * bf2f(gg.x >> 16)) << 16);
    o.y = f2bf(vv.z * r * bf2f(gg.y & 0xffffu)) | (f2bf(vv.w * r * bf2f(gg.y >> 16)) << 16);
    *(uint2*)(x + (size_t)b * d + 4 * i) = o;
  };
  if (one) {  // the row is still in registers
#pragma unroll
    for (int j = 0; j < kFinVec; ++j) {
      const int i = tid + j * kFinThreads;
      if (i < d4) put(i, v[j], g[j]);
    }
    return;
  }
  for (int c0 = 0; c0 < d4; c0 += per) {
#pragma unroll
    for (int j = 0; j < kFinVec; ++j) {
      const int i = min(c0 + tid + j * kFinThreads, d4 - 1);
      v[j] = *(const float4*)(hr + 4 * i);
      g[j] = *(const uint2*)(gain + 4 * i);
    }
#pragma unroll
    for (int j = 0; j < kFinVec; ++j) {
      const int i = c0 + tid + j * kFinThreads;
      if (i < d4) put(i, v[j], g[j]);
    }
  }
}

void launch_finish(float* h, const float* hsrc, const float* parts, int nparts, size_t cstride, int B, int d,
                   const uint16_t* gain, float eps, uint16_t* x, uint16_t* hb, const float* hin, float* sts,
                   hipStream_t s) {
  if (!h || !hsrc || !gain || !x || (nparts > 0 && !parts) || d % 4 || (!hin != !sts))
    throw std::logic_error("finish: bad arguments");
  // the ranges summed with all loads in flight: the fewest of 1, 2, 4, 8 that
  // cover nparts (a load per range and element, so no more than needed)
  auto go = [&](auto np) {
    constexpr int NP = decltype(np)::value;
    if (sts)
      hipLaunchKernelGGL((finish_kernel<true, NP>), dim3(B), dim3(kFinThreads), 0, s, h, hsrc, parts, nparts,
                         cstride, d, gain, eps, x, hb, hin, sts);
    else
      hipLaunchKernelGGL((finish_kernel<false, NP>), dim3(B), dim3(kFinThreads), 0, s, h, hsrc, parts, nparts,
                         cstride, d, gain, eps, x, hb, hin, sts);
  };
  if (nparts <= 1)
    go(std::integral_constant<int, 1>{});
  else if (nparts <= 2)
    go(std::integral_constant<int, 2>{});
  else if (nparts <= 4)
    go(std::integral_constant<int, 4>{});
  else
    go(std::integral_constant<int, kFinParts>{});
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
