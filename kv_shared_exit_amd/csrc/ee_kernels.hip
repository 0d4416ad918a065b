// gfx950 kernels of the KV-shared early-exit decode step.
//
// The step (River-LLM explainer sections 4.1-4.3; AdaDecode explainer sections
// 2.1-2.2; CALM explainer sections 2.2 and 3.3) is built from these kernels:
//   init       embed the input tokens into the float32 residual and normalise
//              them for the first layer, reset the per-step exit state and the
//              row lists
//   proj       (ee_proj.hip) the projections over both weight copies, RoPE plus
//              the write of k and v into the shared cache slot of the position
//              (the same slot for either weight copy) in the QKV epilogue, the
//              residual finish with the RMSNorm of the next input; the int4
//              packer
//   attention  grouped-query decode attention: one wave per run of 64-position
//              tiles of a (sequence, kv head), scores on MFMA, online softmax,
//              and a combine kernel merging the runs
//   decide     finish the exit head (p = 1 / sum exp(l - max)), compare with
//              gamma or apply a forced exit, rebuild the backbone/exit row lists
//              with a wave ballot (active-sequence compaction)
//   final      argmax of the LM head, top-2 gap, next input token
#include "ee_internal.h"
#include "ee_device.h"

#include <math.h>

#include <algorithm>
#include <stdexcept>

namespace ee {

// ---------------------------------------------------------------------------
// Step setup: embedding rows into the residual, exit state, row lists.
// ---------------------------------------------------------------------------
constexpr int kInitThreads = 256;

__global__ __launch_bounds__(kInitThreads) void init_kernel(StepState* st, const int32_t* prompt, int P, int t,
                                                            int B, int L, const uint16_t* emb, int d, int V,
                                                            float* h, float* p_rec, const uint16_t* gain, float eps,
                                                            uint16_t* x) {
  const int b = blockIdx.x;
  const int tid = threadIdx.x;
  int tok = prompt ? prompt[(size_t)b * P + t] : st->tok[b];
  tok = min(max(tok, 0), V - 1);  // host-validated; a device-produced token is always < V
  const uint16_t* src = emb + (size_t)tok * d;
  // h = embedding row (4 columns per item; d is a multiple of 32), then the
  // RMSNorm of the row (same formula as the residual finish) into x
  const int d4 = d >> 2;
  float ss = 0.0f;
  for (int i = tid; i < d4; i += kInitThreads) {
    const uint2 e = *(const uint2*)(src + 4 * i);
    const float4 v = make_float4(bf2f(e.x & 0xffffu), bf2f(e.x >> 16), bf2f(e.y & 0xffffu), bf2f(e.y >> 16));
    *(float4*)(h + (size_t)b * d + 4 * i) = v;
    ss = fmaf(v.x, v.x, ss);
    ss = fmaf(v.y, v.y, ss);
    ss = fmaf(v.z, v.z, ss);
    ss = fmaf(v.w, v.w, ss);
  }
  __shared__ float wsum[kInitThreads / 64];
  __shared__ float rs;
  each_offset_down<1>([&](auto mc) { ss += xor_lane<decltype(mc)::value>(ss, tid & 63); });
  if ((tid & 63) == 0) wsum[tid >> 6] = ss;
  __syncthreads();
  if (tid == 0) {
    float tt = 0.0f;
    for (int w = 0; w < kInitThreads / 64; ++w) tt += wsum[w];
    rs = 1.0f / sqrtf(tt / (float)d + eps);
  }
  __syncthreads();
  const float r = rs;
  for (int i = tid; i < d4; i += kInitThreads) {
    const uint2 e = *(const uint2*)(src + 4 * i);
    const uint2 g = *(const uint2*)(gain + 4 * i);
    uint2 o;
    o.x = f2bf(bf2f(e.x & 0xffffu) * r * bf2f(g.x & 0xffffu)) | (f2bf(bf2f(e.x >> 16) * r * bf2f(g.x >> 16)) << 16);
    o.y = f2bf(bf2f(e.y & 0xffffu) * r * bf2f(g.y & 0xffffu)) | (f2bf(bf2f(e.y >> 16) * r * bf2f(g.y >> 16)) << 16);
    *(uint2*)(x + (size_t)b * d + 4 * i) = o;
  }
  if (p_rec)
    for (int l = tid; l < L - 1; l += kInitThreads) p_rec[l * kMaxBatch + b] = __int_as_float(0x7fc00000);
  if (b == 0) {
    for (int i = tid; i < B; i += kInitThreads) {
      st->exited[i] = 0;
      st->e[i] = L;
      st->act[i] = i;
      st->all[i] = i;
      st->draft_tok[i] = -1;
    }
    if (tid == 0) {
      st->n_act = B;
      st->n_ex = 0;
      st->n_all = B;
    }
  }
}

// Fills n 32-bit words with v (used instead of a memset node, also in code a
// caller may capture into a graph).
__global__ void fill_u32_kernel(uint32_t* p, size_t n, uint32_t v) {
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (size_t)gridDim.x * blockDim.x)
    p[i] = v;
}

void launch_fill_u32(uint32_t* p, size_t n, uint32_t v, hipStream_t s) {
  if (n == 0) return;
  const unsigned blocks = (unsigned)std::min<size_t>((n + 255) / 256, 1024);
  hipLaunchKernelGGL(fill_u32_kernel, dim3(blocks), dim3(256), 0, s, p, n, v);
}

void launch_init(StepState* st, const int32_t* prompt, int P, int t, int B, int L,
                 const uint16_t* emb, int d, int V, float* h, float* p_rec, const uint16_t* gain,
                 float eps, uint16_t* x, hipStream_t s) {
  hipLaunchKernelGGL(init_kernel, dim3(B), dim3(kInitThreads), 0, s, st, prompt, P, t, B, L, emb, d, V, h, p_rec,
                     gain, eps, x);
}

// ---------------------------------------------------------------------------
// Grouped-query decode attention over the shared cache (River-LLM explainer,
// section 3.1: softmax(q K^T / sqrt(d)) V over every cached position).
//
// One wave per (sequence b, kv head j, run of `tpw` 64-position tiles).  For
// each tile the wave reads K straight from HBM into MFMA A operands (16
// positions x 32 head dims per lane group, 16-byte loads) and computes the
// scores of all q heads of the group with v_mfma_f32_16x16x32_bf16 (q heads
// padded to 16 as the B operand, held in registers).  Softmax statistics are
// per q head (online across the wave's tiles); the probabilities go through
// LDS (1 KB) to the PV product, which runs on the vector ALUs with V rows read
// as 16-byte chunks (16 lanes per position row for head_dim 128).
//
// A tile's K and V loads are all issued together (rows are clamped to the
// cache capacity; positions at or past the length are masked: score -inf,
// never multiplied).  Each wave writes one (m, l, o) partial; a wave whose run
// starts at or past the length writes the empty partial (m = -inf, l = 0),
// which the combine kernel skips, so the combine needs no length.
// ---------------------------------------------------------------------------
template <int HD, int GQ>
__global__ __launch_bounds__(64) void attn_kernel(const AttnArgs a) {
  constexpr int KK = HD / 32;          // MFMA steps over the head dim
  constexpr int CPR = HD / 8;          // 16-byte chunks per K/V row
  constexpr int RPI = 64 / CPR;        // rows per V load instruction
  constexpr int NVL = 64 / RPI;        // V loads per 64-row tile
  __shared__ float pb[64][GQ];
  __shared__ float cr[GQ];

  const int c = blockIdx.x, j = blockIdx.y, b = blockIdx.z;
  const int tpw = a.tpw;
  const int tstart = c * tpw * 64;
  const int lane = threadIdx.x;
  const int g = a.H / a.Hkv;
  const int hh = lane & 15;            // q head in the MFMA B / C layouts
  const int qc = lane >> 4;
  const int smax = a.S - 1;            // last row of the cache
  const size_t base = ((size_t)b * a.Hkv + j) * a.S;   // row of position 0
  const uint16_t* Kb = a.K + base * HD;
  const uint16_t* Vb = a.V + base * HD;
  const int vr = lane / CPR, vc = lane - vr * CPR;   // V: row within load, 16-byte chunk

  uint4 kv[4][KK];   // K rows t0 + pt*16 + (lane & 15), head dims qc*8 + 32*kk
  uint4 vv[NVL];     // V rows t0 + vr + i*RPI, chunk vc
  auto load_tile = [&](int t0) {
#pragma unroll
    for (int pt = 0; pt < 4; ++pt) {
      const int row = min(t0 + pt * 16 + (lane & 15), smax);
#pragma unroll
      for (int kk = 0; kk < KK; ++kk) kv[pt][kk] = ld_stream(Kb + (size_t)row * HD + qc * 8 + 32 * kk);
    }
#pragma unroll
    for (int i = 0; i < NVL; ++i) {
      const int row = min(t0 + vr + i * RPI, smax);
      vv[i] = ld_stream(Vb + (size_t)row * HD + vc * 8);
    }
  };
  uint4 qv[KK];
#pragma unroll
  for (int kk = 0; kk < KK; ++kk) {
    qv[kk] = make_uint4(0, 0, 0, 0);
    if (hh < g) qv[kk] = *(const uint4*)(a.q + ((size_t)b * a.H + j * g + hh) * HD + qc * 8 + 32 * kk);
  }
  const int ctx = a.lens[b] + 1;
  const int nw = a.nch;
  if (tstart >= ctx) {  // no position in this run
    if (lane < g) {
      float* out = a.part + ((((size_t)b * a.H + j * g + lane) * nw) + c) * (HD + 2);
      out[HD] = -INFINITY;
      out[HD + 1] = 0.0f;
    }
    return;
  }

  float m = -INFINITY, l = 0.0f;   // per q head hh (replicated over qc)
  float o[GQ][8];
#pragma unroll
  for (int i = 0; i < GQ; ++i)
#pragma unroll
    for (int e = 0; e < 8; ++e) o[i][e] = 0.0f;

  const int tend = min(ctx, tstart + tpw * 64);
  for (int t0 = tstart; t0 < tend; t0 += 64) {
    load_tile(t0);
    const int nval = min(64, ctx - t0);
    // scores S[t][i] for 64 positions
    float sc[4][4];
    float mt = -INFINITY;
#pragma unroll
    for (int pt = 0; pt < 4; ++pt) {
      f32x4_t acc = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
      for (int kk = 0; kk < KK; ++kk)
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, kv[pt][kk]),
                                                      __builtin_bit_cast(bf16x8_t, qv[kk]), acc, 0, 0, 0);
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int p = pt * 16 + qc * 4 + r;
        sc[pt][r] = p < nval ? acc[r] * a.scale : -INFINITY;
        mt = fmaxf(mt, sc[pt][r]);
      }
    }
    mt = fmaxf(mt, xor_lane<16>(mt, lane));
    mt = fmaxf(mt, xor_lane<32>(mt, lane));
    const float mn = fmaxf(m, mt);
    const float corr = __expf(m - mn);   // 0 on the first tile (m = -inf)
    float ls = 0.0f;
#pragma unroll
    for (int pt = 0; pt < 4; ++pt)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float p = __expf(sc[pt][r] - mn);
        ls += p;
        if (hh < GQ) pb[pt * 16 + qc * 4 + r][hh] = p;
      }
    ls += xor_lane<16>(ls, lane);
    ls += xor_lane<32>(ls, lane);
    l = l * corr + ls;
    m = mn;
    if (lane < GQ) cr[lane] = corr;
    __syncthreads();
#pragma unroll
    for (int i = 0; i < GQ; ++i) {
      const float f = cr[i];
#pragma unroll
      for (int e = 0; e < 8; ++e) o[i][e] *= f;
    }
#pragma unroll
    for (int ii = 0; ii < NVL; ++ii) {
      const int t = vr + ii * RPI;
      if (t < nval) {
        const uint4 v4 = vv[ii];
        const float ve[8] = {bf2f(v4.x & 0xffffu), bf2f(v4.x >> 16), bf2f(v4.y & 0xffffu), bf2f(v4.y >> 16),
                             bf2f(v4.z & 0xffffu), bf2f(v4.z >> 16), bf2f(v4.w & 0xffffu), bf2f(v4.w >> 16)};
#pragma unroll
        for (int i = 0; i < GQ; ++i) {
          const float p = pb[t][i];
#pragma unroll
          for (int e = 0; e < 8; ++e) o[i][e] = fmaf(p, ve[e], o[i][e]);
        }
      }
    }
    __syncthreads();
  }
  // sum over the row groups of a V load (lanes with equal vc)
  each_offset_up<CPR>([&](auto mc) {
#pragma unroll
    for (int i = 0; i < GQ; ++i)
#pragma unroll
      for (int e = 0; e < 8; ++e) o[i][e] += xor_lane<decltype(mc)::value>(o[i][e], lane);
  });
  if (vr == 0) {
#pragma unroll
    for (int i = 0; i < GQ; ++i) {
      if (i >= g) break;
      float* out = a.part + ((((size_t)b * a.H + j * g + i) * nw) + c) * (HD + 2);
#pragma unroll
      for (int e = 0; e < 8; ++e) out[vc * 8 + e] = o[i][e];
    }
  }
  if (lane < g) {
    float* out = a.part + ((((size_t)b * a.H + j * g + lane) * nw) + c) * (HD + 2);
    out[HD] = m;
    out[HD + 1] = l;
  }
}

// Merges the (m, l, o) partials of one (sequence, q head) in partial order:
// weights f_c = exp(m_c - max m) and L = sum f_c l_c, then o = sum_c f_c o_c
// / L per head dimension.  Empty partials (m = -inf) have weight 0 and their
// o is not read into the sum.  The partials are taken in batches of kCombBatch
// whose loads are all issued at once, merged online (running max) across
// batches.
constexpr int kCombBatch = 32;

__global__ __launch_bounds__(128) void attn_combine_kernel(const AttnArgs a) {
  const int h = blockIdx.x, b = blockIdx.y;
  const int hd = a.hd;
  const int tid = threadIdx.x;
  const int nc = a.nch;
  const float* base = a.part + (((size_t)b * a.H + h) * nc) * (hd + 2);
  const int d = min(tid, hd - 1);   // this thread's head dimension (threads past hd repeat the last)
  float M = -INFINITY, L = 0.0f, O = 0.0f;
  for (int c0 = 0; c0 < nc; c0 += kCombBatch) {
    float mv[kCombBatch], lv[kCombBatch], ov[kCombBatch];
#pragma unroll
    for (int i = 0; i < kCombBatch; ++i) {
      const int cc = min(c0 + i, nc - 1);
      const float* p = base + (size_t)cc * (hd + 2);
      mv[i] = c0 + i < nc ? p[hd] : -INFINITY;
      lv[i] = p[hd + 1];
      ov[i] = p[d];
    }
    float Mb = M;
#pragma unroll
    for (int i = 0; i < kCombBatch; ++i) Mb = fmaxf(Mb, mv[i]);
    if (Mb == -INFINITY) continue;   // nothing yet
    const float rs = __expf(M - Mb);  // 0 when M = -inf
    L *= rs;
    O *= rs;
#pragma unroll
    for (int i = 0; i < kCombBatch; ++i) {
      const float f = __expf(mv[i] - Mb);   // 0 for empty partials
      L = fmaf(lv[i], f, L);
      O = f > 0.0f ? fmaf(ov[i], f, O) : O;
    }
    M = Mb;
  }
  if (tid < hd) a.out[((size_t)b * a.H + h) * hd + tid] = (uint16_t)f2bf(O / L);
}

// Fused variant: one workgroup of NW waves per (sequence, kv head).  The
// waves take the context's 64-position tiles in turn (wave w: tiles w,
// w + NW, ...), each keeping its own online softmax exactly as
// attn_kernel does for a run; the waves' (m, l, o) then meet in LDS and are
// merged in wave order, as the combine kernel merges partials, and the bf16
// output is written directly: no partial buffer, no second launch.  Inside
// the tile loop a wave only synchronises with itself (its probabilities go
// through its own LDS slice), so waves with fewer tiles never wait at a
// barrier the others reach more often.  NW = 8 up to 511 pairs, 4 from 512
// (at two waves per SIMD, 512 four-wave workgroups are resident at once; at 64
// sequences x 4096 positions 166 against 177 us per layer, at 32 sequences 92
// against 88 us, where four waves would leave half of each CU idle).
template <int HD, int GQ, int NW>
__global__ __launch_bounds__(64 * NW) void attn_fused_kernel(const AttnArgs a) {
  constexpr int KK = HD / 32;
  constexpr int CPR = HD / 8;
  constexpr int RPI = 64 / CPR;
  constexpr int NVL = 64 / RPI;
  __shared__ float pbw[NW][64][GQ];
  __shared__ float crw[NW][GQ];
  __shared__ float pm[NW][GQ], pl[NW][GQ];
  __shared__ float po[NW][GQ][HD];

  const int j = blockIdx.x, b = blockIdx.y;
  const int wave = threadIdx.x >> 6;
  const int lane = threadIdx.x & 63;
  const int g = a.H / a.Hkv;
  const int hh = lane & 15;
  const int qc = lane >> 4;
  const int smax = a.S - 1;
  const size_t base = ((size_t)b * a.Hkv + j) * a.S;
  const uint16_t* Kb = a.K + base * HD;
  const uint16_t* Vb = a.V + base * HD;
  const int vr = lane / CPR, vc = lane - vr * CPR;
  float (*pb)[GQ] = pbw[wave];
  float* cr = crw[wave];

  uint4 kv[4][KK];
  uint4 vv[NVL];
  auto load_tile = [&](int t0) {
#pragma unroll
    for (int pt = 0; pt < 4; ++pt) {
      const int row = min(t0 + pt * 16 + (lane & 15), smax);
#pragma unroll
      for (int kk = 0; kk < KK; ++kk) kv[pt][kk] = ld_stream(Kb + (size_t)row * HD + qc * 8 + 32 * kk);
    }
#pragma unroll
    for (int i = 0; i < NVL; ++i) {
      const int row = min(t0 + vr + i * RPI, smax);
      vv[i] = ld_stream(Vb + (size_t)row * HD + vc * 8);
    }
  };
  uint4 qv[KK];
#pragma unroll
  for (int kk = 0; kk < KK; ++kk) {
    qv[kk] = make_uint4(0, 0, 0, 0);
    if (hh < g) qv[kk] = *(const uint4*)(a.q + ((size_t)b * a.H + j * g + hh) * HD + qc * 8 + 32 * kk);
  }
  const int ctx = a.lens[b] + 1;

  float m = -INFINITY, l = 0.0f;
  float o[GQ][8];
#pragma unroll
  for (int i = 0; i < GQ; ++i)
#pragma unroll
    for (int e = 0; e < 8; ++e) o[i][e] = 0.0f;

  for (int t0 = wave * 64; t0 < ctx; t0 += 64 * NW) {
    load_tile(t0);
    const int nval = min(64, ctx - t0);
    float sc[4][4];
    float mt = -INFINITY;
#pragma unroll
    for (int pt = 0; pt < 4; ++pt) {
      f32x4_t acc = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
      for (int kk = 0; kk < KK; ++kk)
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, kv[pt][kk]),
                                                      __builtin_bit_cast(bf16x8_t, qv[kk]), acc, 0, 0, 0);
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int p = pt * 16 + qc * 4 + r;
        sc[pt][r] = p < nval ? acc[r] * a.scale : -INFINITY;
        mt = fmaxf(mt, sc[pt][r]);
      }
    }
    mt = fmaxf(mt, xor_lane<16>(mt, lane));
    mt = fmaxf(mt, xor_lane<32>(mt, lane));
    const float mn = fmaxf(m, mt);
    const float corr = __expf(m - mn);
    float ls = 0.0f;
#pragma unroll
    for (int pt = 0; pt < 4; ++pt)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float p = __expf(sc[pt][r] - mn);
        ls += p;
        if (hh < GQ) pb[pt * 16 + qc * 4 + r][hh] = p;
      }
    ls += xor_lane<16>(ls, lane);
    ls += xor_lane<32>(ls, lane);
    l = l * corr + ls;
    m = mn;
    if (lane < GQ) cr[lane] = corr;
    // this wave's LDS slice: its stores complete before its loads (LDS
    // operations of a wave are performed in order); the barrier keeps the
    // compiler from moving them across
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
#pragma unroll
    for (int i = 0; i < GQ; ++i) {
      const float f = cr[i];
#pragma unroll
      for (int e = 0; e < 8; ++e) o[i][e] *= f;
    }
#pragma unroll
    for (int ii = 0; ii < NVL; ++ii) {
      const int t = vr + ii * RPI;
      if (t < nval) {
        const uint4 v4 = vv[ii];
        const float ve[8] = {bf2f(v4.x & 0xffffu), bf2f(v4.x >> 16), bf2f(v4.y & 0xffffu), bf2f(v4.y >> 16),
                             bf2f(v4.z & 0xffffu), bf2f(v4.z >> 16), bf2f(v4.w & 0xffffu), bf2f(v4.w >> 16)};
#pragma unroll
        for (int i = 0; i < GQ; ++i) {
          const float p = pb[t][i];
#pragma unroll
          for (int e = 0; e < 8; ++e) o[i][e] = fmaf(p, ve[e], o[i][e]);
        }
      }
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  }
  each_offset_up<CPR>([&](auto mc) {
#pragma unroll
    for (int i = 0; i < GQ; ++i)
#pragma unroll
      for (int e = 0; e < 8; ++e) o[i][e] += xor_lane<decltype(mc)::value>(o[i][e], lane);
  });
  // this wave's partial into LDS (a wave without tiles: m = -inf, l = 0)
  if (vr == 0) {
#pragma unroll
    for (int i = 0; i < GQ; ++i)
#pragma unroll
      for (int e = 0; e < 8; ++e) po[wave][i][vc * 8 + e] = o[i][e];
  }
  if (lane < GQ) {
    pm[wave][lane] = m;
    pl[wave][lane] = l;
  }
  __syncthreads();
  // merge in wave order: weights exp(m_w - max m), empty partials skipped
  for (int idx = threadIdx.x; idx < g * HD; idx += 64 * NW) {
    const int i = idx / HD, dd = idx - i * HD;
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < NW; ++w) M = fmaxf(M, pm[w][i]);
    float L = 0.0f, O = 0.0f;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      const float f = __expf(pm[w][i] - M);  // 0 for an empty partial
      L = fmaf(pl[w][i], f, L);
      O = f > 0.0f ? fmaf(po[w][i][dd], f, O) : O;
    }
    a.out[((size_t)b * a.H + j * g + i) * HD + dd] = (uint16_t)f2bf(O / L);
  }
}

template <int HD, int GQ>
static void launch_attn_t(const AttnArgs& a, hipStream_t s) {
  if (a.fused && (long long)a.B * a.Hkv >= 512)
    hipLaunchKernelGGL((attn_fused_kernel<HD, GQ, 4>), dim3(a.Hkv, a.B), dim3(64 * 4), 0, s, a);
  else if (a.fused)
    hipLaunchKernelGGL((attn_fused_kernel<HD, GQ, 8>), dim3(a.Hkv, a.B), dim3(64 * 8), 0, s, a);
  else
    hipLaunchKernelGGL((attn_kernel<HD, GQ>), dim3(a.nch, a.Hkv, a.B), dim3(64), 0, s, a);
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
  if (!a.fused) hipLaunchKernelGGL(attn_combine_kernel, dim3(a.H, a.B), dim3(128), 0, s, a);
}

// ---------------------------------------------------------------------------
// Exit decision and active-sequence compaction.
// ---------------------------------------------------------------------------
constexpr int kHeadThreads = 512;              // decide: eight waves
constexpr int kHeadWaves = kHeadThreads / 64;
constexpr int kPartPerLane = kNwgMax / 64;    // partials a lane of final merges (nwg <= kNwgMax)
constexpr int kPartPerWave = kNwgMax / kHeadWaves;  // partials one wave of decide merges per position
static_assert(kMaxBatch == 64 && kPartPerWave == 64, "decide: the lane split assumes 64 positions and 64 partials per wave");

// MODE DECIDE_STS: the value of a row is its state transition similarity
// sts[b] instead of the exit head's p; DECIDE_FORCED: no value, only forced
// exits (p_rec is left as it is).
// batch_min: the unforced rows leave together when the smallest of their
// values exceeds the threshold (River-LLM explainer, section 5.2), decided
// by thread 0 over the values in list order.
template <int MODE>
__global__ __launch_bounds__(kHeadThreads) void decide_kernel(StepState* st, const float* part, int nwg,
                                                              const float* gamma, int layer, int L, int B,
                                                              float* p_rec, const float* sts, int batch_min) {
  constexpr bool STS = MODE == DECIDE_STS;
  __shared__ int sx[kMaxBatch];
  __shared__ float pv[kMaxBatch];
  __shared__ float2 red[kHeadWaves][kMaxBatch];
  __shared__ int sact[kMaxBatch], sfrc[kMaxBatch];
  __shared__ float ssts[kMaxBatch];
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  // the step state of every row (lists, forced layers, exit flags, the
  // similarities), the row count and the threshold, requested before the
  // partials so that nothing after the merge waits for memory (every array
  // holds kMaxBatch entries)
  int act_t = 0, frc_t = 0, exi_t = 0;
  float sts_t = 0.0f;
  if ((int)threadIdx.x < kMaxBatch) {
    act_t = st->act[threadIdx.x];
    frc_t = st->forced[threadIdx.x];
    exi_t = st->exited[threadIdx.x];
    if constexpr (STS) sts_t = sts[threadIdx.x];
  }
  const int n_act = st->n_act;
  const float gam = MODE != DECIDE_FORCED ? gamma[layer - 1] : 0.0f;
  // DECIDE_HEAD, the (max, sum exp) partials of every list position into
  // red[wave][position] (merged over the waves below).  All loads are
  // requested before the row count is known (positions below the batch, or
  // below 8, are always in bounds; absent partials merge as no-ops).
  if constexpr (MODE == DECIDE_HEAD) {
    if (B <= kHeadWaves) {
      // wave w takes position w, its lanes the partials k = lane + 64j
      float2 v[kPartPerLane];
#pragma unroll
      for (int j = 0; j < kPartPerLane; ++j) {
        const int k = lane + 64 * j;
        v[j] = k < nwg ? *(const float2*)(part + ((size_t)k * kMaxBatch + w) * 4) : make_float2(-INFINITY, 0.0f);
      }
#pragma unroll
      for (int j = 1; j < kPartPerLane; ++j) lse_merge(v[0].x, v[0].y, v[j].x, v[j].y);
      each_offset_up<1>([&](auto mc) {
        constexpr int M = decltype(mc)::value;
        lse_merge(v[0].x, v[0].y, xor_lane<M>(v[0].x, lane), xor_lane<M>(v[0].y, lane));
      });
      if (lane < kHeadWaves) red[lane][w] = lane == 0 ? v[0] : make_float2(-INFINITY, 0.0f);
    } else {
      // wave w takes the partials k = w + 8t (t < 64) of every position.
      // With Bp the batch rounded up to a power of two, lane (kk, i) =
      // (lane / Bp, lane % Bp) takes position i and t = kk + (64 / Bp) j for
      // j < Bp, so the lanes of one load read adjacent positions of a few
      // workgroups' partials (contiguous runs, not a line per lane); each lane
      // merges its Bp values as a tree, then the 64 / Bp lanes of a position
      // combine theirs.
      const int lg = 32 - __builtin_clz(B - 1);  // log2(Bp), uniform
      const int bp = 1 << lg;
      const int pos = lane & (bp - 1), kk = lane >> lg;
      float2 v[kPartPerWave];
#pragma unroll
      for (int j = 0; j < kPartPerWave; ++j) {
        const int k = w + kHeadWaves * (kk + (64 >> lg) * j);
        v[j] = (j < bp && k < nwg) ? *(const float2*)(part + ((size_t)k * kMaxBatch + pos) * 4)
                                   : make_float2(-INFINITY, 0.0f);
      }
#pragma unroll
      for (int h = kPartPerWave / 2; h >= 1; h >>= 1) {
        if (2 * h <= bp) {  // uniform: the levels of a tree over bp values
#pragma unroll
          for (int j = 0; j < h; ++j) lse_merge(v[j].x, v[j].y, v[j + h].x, v[j + h].y);
        }
      }
      for (int o = bp; o < 64; o <<= 1) {
        const float m2 = __shfl_xor(v[0].x, o), s2 = __shfl_xor(v[0].y, o);
        lse_merge(v[0].x, v[0].y, m2, s2);
      }
      if (kk == 0) red[w][pos] = v[0];
    }
  }
  if ((int)threadIdx.x < kMaxBatch) {
    sx[threadIdx.x] = exi_t;
    sact[threadIdx.x] = act_t;
    sfrc[threadIdx.x] = frc_t;
    if constexpr (STS) ssts[threadIdx.x] = sts_t;
  }
  __syncthreads();
  const int n = min(max(n_act, 0), B);
  // one thread per list position (n <= kMaxBatch < kHeadThreads)
  const int i = threadIdx.x;
  if (i < n) {
    const int b = sact[i];
    float p = 0.0f;
    if constexpr (STS) {
      p = ssts[b];
    } else if constexpr (MODE == DECIDE_HEAD) {
      float m = -INFINITY, sum = 0.0f;
#pragma unroll
      for (int ww = 0; ww < kHeadWaves; ++ww) lse_merge(m, sum, red[ww][i].x, red[ww][i].y);
      p = 1.0f / sum;
    }
    const int f = sfrc[b];
    const bool own = MODE != DECIDE_FORCED && !batch_min && p > gam;
    const bool ex = f > 0 ? (layer == f) : own;
    if (p_rec && MODE != DECIDE_FORCED) p_rec[(layer - 1) * kMaxBatch + b] = p;
    pv[i] = p;
    if (ex) {
      sx[b] = 1;
      st->e[b] = layer;
    }
  }
  if (MODE != DECIDE_FORCED && batch_min) {
    __syncthreads();
    if (threadIdx.x == 0) {
      float mn = INFINITY;
      bool any = false;
      for (int i = 0; i < n; ++i)
        if (sfrc[sact[i]] == 0) {
          mn = fminf(mn, pv[i]);
          any = true;
        }
      if (any && mn > gam)
        for (int i = 0; i < n; ++i) {
          const int b = sact[i];
          if (sfrc[b] == 0) {
            sx[b] = 1;
            st->e[b] = layer;
          }
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

void launch_decide(int mode, bool batch_min, StepState* st, const float* part, int nwg, const float* gamma,
                   int layer, int L, int B, float* p_rec, const float* sts, hipStream_t s) {
  const int bm = batch_min ? 1 : 0;
  if (B < 1 || B > kMaxBatch) throw std::logic_error("decide: batch out of range");
  switch (mode) {
    case DECIDE_STS:
      if (!sts) throw std::logic_error("decide: no similarities");
      hipLaunchKernelGGL(decide_kernel<DECIDE_STS>, dim3(1), dim3(kHeadThreads), 0, s, st, part, nwg, gamma, layer,
                         L, B, p_rec, sts, bm);
      return;
    case DECIDE_FORCED:
      hipLaunchKernelGGL(decide_kernel<DECIDE_FORCED>, dim3(1), dim3(kHeadThreads), 0, s, st, part, nwg, gamma,
                         layer, L, B, p_rec, sts, 0);
      return;
    default:
      if (nwg < 1 || nwg > kNwgMax) throw std::logic_error("decide: partial count out of range");
      hipLaunchKernelGGL(decide_kernel<DECIDE_HEAD>, dim3(1), dim3(kHeadThreads), 0, s, st, part, nwg, gamma,
                         layer, L, B, p_rec, sts, bm);
  }
}

// One wave per row (a workgroup each: the rows are independent).
__global__ __launch_bounds__(64) void final_kernel(StepState* st, const float* part, int nwg, int B, int V,
                                                   int32_t* lens, int advance) {
  const int lane = threadIdx.x & 63;
  {
    const int b = blockIdx.x;
    float4 v[kPartPerLane];
#pragma unroll
    for (int j = 0; j < kPartPerLane; ++j) {
      const int k = lane + 64 * j;
      v[j] = k < nwg ? *(const float4*)(part + ((size_t)k * kMaxBatch + b) * 4)
                     : make_float4(-INFINITY, __int_as_float(0x7fffffff), -INFINITY, 0.0f);
    }
    Top2 t{-INFINITY, 0x7fffffff, -INFINITY};
#pragma unroll
    for (int j = 0; j < kPartPerLane; ++j) top2_merge(t, Top2{v[j].x, __float_as_int(v[j].y), v[j].z});
    each_offset_up<1>([&](auto mc) {
      constexpr int M = decltype(mc)::value;
      top2_merge(t, Top2{xor_lane<M>(t.v1, lane), xor_lane<M>(t.i1, lane), xor_lane<M>(t.v2, lane)});
    });
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
  if (nwg < 1 || nwg > kNwgMax) throw std::logic_error("final: partial count out of range");
  if (B < 1 || B > kMaxBatch) throw std::logic_error("final: batch out of range");
  hipLaunchKernelGGL(final_kernel, dim3(B), dim3(64), 0, s, st, part, nwg, B, V, lens, advance);
}

__global__ void advance_kernel(int32_t* lens, int B, int delta) {
  if ((int)threadIdx.x < B) lens[threadIdx.x] += delta;
}

void launch_advance(int32_t* lens, int B, hipStream_t s, int delta) {
  hipLaunchKernelGGL(advance_kernel, dim3(1), dim3(64), 0, s, lens, B, delta);
}

// out[b] = min over positions t < P of sts[t * B + b] (one wave per sequence).
__global__ void sts_min_kernel(const float* sts, int P, int B, float* out) {
  const int b = blockIdx.x, lane = threadIdx.x;
  float m = INFINITY;
  for (int t = lane; t < P; t += 64) m = fminf(m, sts[(size_t)t * B + b]);
  each_offset_up<1>([&](auto mc) { m = fminf(m, xor_lane<decltype(mc)::value>(m, lane)); });
  if (lane == 0) out[b] = m;
}

void launch_sts_min(const float* sts, int P, int B, float* out, hipStream_t s) {
  if (!sts || !out || P < 1 || B < 1 || B > kMaxBatch) throw std::logic_error("sts_min: bad arguments");
  hipLaunchKernelGGL(sts_min_kernel, dim3(B), dim3(64), 0, s, sts, P, B, out);
}

}  // namespace ee
