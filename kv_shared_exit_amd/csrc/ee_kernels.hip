// gfx950 kernels of the KV-shared early-exit decode step.
//
// The step (River-LLM explainer sections 4.1-4.3; AdaDecode explainer sections
// 2.1-2.2; CALM explainer sections 2.2 and 3.3) is built from these kernels:
//   init       embed the input tokens into the float32 residual, reset the
//              per-step exit state and the row lists
//   rmsnorm    bf16(h * rsqrt(mean(h^2) + eps) * g)
//   proj       (ee_proj.hip) the projections over both weight copies, and
//              the int4 packer
//   rope_kv    rotate q and k, write k and v into the shared cache slot of the
//              position (the same slot for either weight copy)
//   attention  grouped-query decode attention, split over 256-position chunks;
//              K/V tiles staged in LDS, scores on MFMA, softmax per wave, and a
//              combine kernel merging the chunks
//   decide     finish the exit head (p = 1 / sum exp(l - max)), compare with
//              gamma or apply a forced exit, rebuild the backbone/exit row lists
//              with a wave ballot (active-sequence compaction)
//   final      argmax of the LM head, top-2 gap, next input token
#include "ee_internal.h"
#include "ee_device.h"

#include <math.h>

namespace ee {


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

}  // namespace ee
