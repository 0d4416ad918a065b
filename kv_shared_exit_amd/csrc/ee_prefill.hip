// gfx950 kernels of the prefill ("River-LLM 深度解析", section 6.1: the prompt is
// processed as a whole before tokens are generated one at a time).  The
// prefill runs layer by layer over every prompt position of every sequence at
// once, so each projection is a dense contraction of B*P activation rows with
// the layer's weights and runs on matrix cores:
//   gemm        C = X W^T over the rows of a list of sequences, bf16 weights or
//               the int4 exit copies, with a bf16, residual-add or SwiGLU
//               epilogue
//   rope_kv     RoPE of q and k per position, k and v into the shared cache
//               slots of the positions (the slots the decode step reads)
//   attention   causal attention of every prompt position over the cached
//               positions before it and the prompt positions up to it
//   embed       embedding rows and the first layer's RMSNorm for every position
//   group sums  per-row sums of the activations over each int4 scale group
// Activation rows are position-major: row t * B + b holds position t of
// sequence b.
#include "ee_internal.h"
#include "ee_device.h"
#include "ee_epi.h"

#include <math.h>

#include <algorithm>
#include <stdexcept>

namespace ee {

// ---------------------------------------------------------------------------
// GEMM: for the sequences list[0..n) (n = *cnt), rows r in [0, n * P) are
// position t = r / n of sequence b = list[r % n], physical row t * Bt + b.
// Tile: 128 rows (tokens) x 128 weight rows, K in steps of 64 staged in LDS
// (double-buffered, the next step's global loads in flight during the
// current step's products).  Four waves; wave w computes token rows
// [64 * (w >> 1), +64) against weight rows {32 * (w & 1), +16, 64 + 32 * (w & 1),
// +16} of the tile, so that with the SwiGLU layout (tile rows 0..63 gate rows,
// 64..127 the same up rows) a lane holds gate and up of the same output.
// MFMA v_mfma_f32_16x16x32_bf16 with the weights as the A operand (16 weight
// rows x 32 k) and the tokens as B (32 k x 16 tokens): lane l holds D rows
// (weight rows) 4 (l >> 4) + i, i < 4, of column (token) l & 15.
// int4 weights: each code q (stored q + 8) becomes the bf16 value 136 + q
// (bits 0x4300 | nibble), exact; after every scale group the group's
// products are folded in as s * (sum (136 + q) x - 136 * sum x), with the
// per-row group sums of x precomputed (group_sums_kernel).
// ---------------------------------------------------------------------------
constexpr int kGemmThreads = 256;
constexpr int kGM = 128;   // token rows per tile
constexpr int kGN = 128;   // weight rows per tile
constexpr int kGK = 64;    // k per staged step
constexpr int kGLd = kGK + 8;  // LDS row stride (bf16), padded against bank conflicts

template <int EPI, bool W4>
__global__ __launch_bounds__(kGemmThreads, 2) void gemm_kernel(const GemmArgs a) {
  __shared__ __attribute__((aligned(16))) uint16_t sW[2][kGN * kGLd];
  __shared__ __attribute__((aligned(16))) uint16_t sX[2][kGM * kGLd];
  const int n_seq = min(max(*a.cnt, 0), a.Bt);
  const int rows = n_seq * a.P;
  const int tm = blockIdx.x, tn = blockIdx.y;
  if (tm * kGM >= rows) return;  // uniform: no token rows in this tile
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int wn = wave & 1, wm = wave >> 1;
  const int c16 = lane & 15, g4 = lane >> 4;

  // physical row of compact row r (or -1 past the rows)
  auto phys = [&](int r) -> int {
    if (r >= rows) return -1;
    const int t = r / n_seq;
    return t * a.Bt + a.list[r - t * n_seq];
  };
  // weight row of tile row v: its bf16 row pointer / its row index in the
  // int4 matrix (and which matrix), or invalid
  const bool swi = EPI == GEPI_SWIGLU;
  auto wrow = [&](int v, int& n, int& mat) -> bool {
    if (swi) {
      n = tn * 64 + (v & 63);
      mat = v >> 6;
    } else {
      n = tn * kGN + v;
      mat = 0;
    }
    return n < a.N;
  };

  // global -> register loads of one K step: 4 chunks of 8 k per thread per operand
  uint4 rx[4];
  uint32_t rq[4];
  uint4 rw[4];
  int xrow[4];            // physical rows of this thread's X chunks
  const uint16_t* wptr[4];
  const uint32_t* qptr[4];
  int wvalid[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int c = tid + kGemmThreads * i;
    const int row = c >> 3;
    xrow[i] = phys(tm * kGM + row);
    int n = 0, mat = 0;
    wvalid[i] = wrow(row, n, mat);
    wptr[i] = nullptr;
    qptr[i] = nullptr;
    if (wvalid[i]) {
      if (W4) {
        qptr[i] = (mat ? a.q4b : a.q4) + (size_t)n * (a.K >> 3);
      } else if (swi) {
        wptr[i] = (mat ? a.wb2 : a.wb[0]) + (size_t)n * a.K;
      } else {
        int sgi = 0;
        while (sgi < a.nseg - 1 && n >= a.seg_end[sgi]) ++sgi;
        const int n0 = sgi ? a.seg_end[sgi - 1] : 0;
        wptr[i] = a.wb[sgi] + (size_t)(n - n0) * a.K;
      }
    }
  }
  const int words = a.K >> 3;
  auto load_step = [&](int k0) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int c = tid + kGemmThreads * i;
      const int kc = c & 7;
      const int k = k0 + kc * 8;
      const bool kin = k < a.K;
      rx[i] = make_uint4(0, 0, 0, 0);
      if (xrow[i] >= 0 && kin) rx[i] = *(const uint4*)(a.x + (size_t)xrow[i] * a.ldx + k);
      if (W4) {
        rq[i] = 0x88888888u;  // code 8 = q 0 (contributes 136 * x, removed by the fold; x is 0 past K)
        if (wvalid[i] && kin) {
          const int t = k >> 3;
          const int full = (words >> 4) << 4;
          const int st = t < full ? (t & ~15) + (t & 3) * 4 + ((t & 15) >> 2) : t;
          rq[i] = qptr[i][st];
        }
      } else {
        rw[i] = make_uint4(0, 0, 0, 0);
        if (wvalid[i] && kin) rw[i] = ld_stream(wptr[i] + k);
      }
    }
  };
  auto store_step = [&](int buf) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int c = tid + kGemmThreads * i;
      const int row = c >> 3, kc = c & 7;
      *(uint4*)(&sX[buf][row * kGLd + kc * 8]) = rx[i];
      uint4 w;
      if (W4) {
        const uint32_t d = rq[i];
        w.x = ((d >> 0) & 0x000F000Fu) | 0x43004300u;
        w.y = ((d >> 4) & 0x000F000Fu) | 0x43004300u;
        w.z = ((d >> 8) & 0x000F000Fu) | 0x43004300u;
        w.w = ((d >> 12) & 0x000F000Fu) | 0x43004300u;
      } else {
        w = rw[i];
      }
      *(uint4*)(&sW[buf][row * kGLd + kc * 8]) = w;
    }
  };

  f32x4_t acc[4][4];
  f32x4_t tmp[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      acc[i][j] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
      tmp[i][j] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
    }
  // tile rows of this wave's 4 weight sub-tiles and 4 token sub-tiles
  auto vbase = [&](int ns) { return (ns >> 1) * 64 + wn * 32 + (ns & 1) * 16; };
  auto mbase = [&](int ms) { return wm * 64 + ms * 16; };

  // int4 fold: acc += s * (tmp - 136 * xs) for the group ending at column k_end
  int xrow_m[4];  // physical rows of this lane's token columns
#pragma unroll
  for (int ms = 0; ms < 4; ++ms) xrow_m[ms] = phys(tm * kGM + mbase(ms) + c16);
  const int ngr = W4 ? a.K / a.G : 1;
  auto fold = [&](int g) {
    float xsv[4];
#pragma unroll
    for (int ms = 0; ms < 4; ++ms) xsv[ms] = xrow_m[ms] >= 0 ? a.xs[(size_t)xrow_m[ms] * a.ldxs + g] : 0.0f;
#pragma unroll
    for (int ns = 0; ns < 4; ++ns) {
      int n = 0, mat = 0;
      const int v = vbase(ns) + 4 * g4;
      float sv[4] = {0.0f, 0.0f, 0.0f, 0.0f};
      if (wrow(v, n, mat)) {  // 4 consecutive rows of one 16-row scale block
        const uint16_t* s4 = mat ? a.s4b : a.s4;
        const uint2 sp = *(const uint2*)(s4 + ((size_t)(n >> 4) * ngr + g) * 16 + (n & 15));
        sv[0] = bf2f(sp.x & 0xffffu);
        sv[1] = bf2f(sp.x >> 16);
        sv[2] = bf2f(sp.y & 0xffffu);
        sv[3] = bf2f(sp.y >> 16);
      }
#pragma unroll
      for (int ms = 0; ms < 4; ++ms) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          acc[ns][ms][r] = fmaf(sv[r], tmp[ns][ms][r] - 136.0f * xsv[ms], acc[ns][ms][r]);
          tmp[ns][ms][r] = 0.0f;
        }
      }
    }
  };

  const int nsteps = (a.K + kGK - 1) / kGK;
  load_step(0);
  store_step(0);
  __syncthreads();
  for (int st = 0; st < nsteps; ++st) {
    const int buf = st & 1;
    if (st + 1 < nsteps) load_step((st + 1) * kGK);
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      const int kcol = kk * 32 + g4 * 8;
      uint4 af[4], bfr[4];
#pragma unroll
      for (int ns = 0; ns < 4; ++ns) af[ns] = *(const uint4*)(&sW[buf][(vbase(ns) + c16) * kGLd + kcol]);
#pragma unroll
      for (int ms = 0; ms < 4; ++ms) bfr[ms] = *(const uint4*)(&sX[buf][(mbase(ms) + c16) * kGLd + kcol]);
#pragma unroll
      for (int ns = 0; ns < 4; ++ns)
#pragma unroll
        for (int ms = 0; ms < 4; ++ms) {
          if (W4)
            tmp[ns][ms] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, af[ns]),
                                                                  __builtin_bit_cast(bf16x8_t, bfr[ms]),
                                                                  tmp[ns][ms], 0, 0, 0);
          else
            acc[ns][ms] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, af[ns]),
                                                                  __builtin_bit_cast(bf16x8_t, bfr[ms]),
                                                                  acc[ns][ms], 0, 0, 0);
        }
      if (W4) {
        const int kend = st * kGK + kk * 32 + 32;  // columns done after this sub-step
        if (kend <= a.K && kend % a.G == 0) fold(kend / a.G - 1);
      }
    }
    if (st + 1 < nsteps) {
      store_step(buf ^ 1);
      __syncthreads();
    }
  }

  // epilogue: lane holds weight rows vbase(ns) + 4 g4 + i of token column mbase(ms) + c16
#pragma unroll
  for (int ms = 0; ms < 4; ++ms) {
    const int pr = xrow_m[ms];
    if (pr < 0) continue;
    if (EPI == GEPI_SWIGLU) {
#pragma unroll
      for (int ns = 0; ns < 2; ++ns) {
        const int n = tn * 64 + vbase(ns) + 4 * g4;  // gate rows of sub-tile ns, up rows in ns + 2
        if (n >= a.N) continue;
        uint32_t o[2];
#pragma unroll
        for (int i = 0; i < 2; ++i) {
          const float lo = silu_mul(acc[ns][ms][2 * i], acc[ns + 2][ms][2 * i]);
          const float hi = silu_mul(acc[ns][ms][2 * i + 1], acc[ns + 2][ms][2 * i + 1]);
          o[i] = f2bf(lo) | (f2bf(hi) << 16);
        }
        *(uint2*)(a.ob + (size_t)pr * a.ldo + n) = make_uint2(o[0], o[1]);
      }
    } else {
#pragma unroll
      for (int ns = 0; ns < 4; ++ns) {
        const int n = tn * kGN + vbase(ns) + 4 * g4;
        if (n >= a.N) continue;
        if (EPI == GEPI_BF16) {
          const uint32_t o0 = f2bf(acc[ns][ms][0]) | (f2bf(acc[ns][ms][1]) << 16);
          const uint32_t o1 = f2bf(acc[ns][ms][2]) | (f2bf(acc[ns][ms][3]) << 16);
          *(uint2*)(a.ob + (size_t)pr * a.ldo + n) = make_uint2(o0, o1);
        } else {  // GEPI_RESID: out = src + acc (float32)
          const float4 sv = *(const float4*)(a.src + (size_t)pr * a.ldf + n);
          const float4 ov = make_float4(sv.x + acc[ns][ms][0], sv.y + acc[ns][ms][1], sv.z + acc[ns][ms][2],
                                        sv.w + acc[ns][ms][3]);
          *(float4*)(a.of + (size_t)pr * a.ldf + n) = ov;
        }
      }
    }
  }
}

void launch_gemm(int epi, bool w4, const GemmArgs& a, int max_rows, hipStream_t s) {
  if (a.K % 32 || a.N % 4 || (w4 && (a.G % 32 || a.K % a.G)) || a.Bt < 1 || a.P < 1)
    throw std::logic_error("gemm: unsupported shape");
  const int gm = std::max(1, (max_rows + kGM - 1) / kGM);
  const int gn = epi == GEPI_SWIGLU ? (a.N + 63) / 64 : (a.N + kGN - 1) / kGN;
  const dim3 grid(gm, gn);
#define EE_GEMM(E, W) hipLaunchKernelGGL((gemm_kernel<E, W>), grid, dim3(kGemmThreads), 0, s, a)
  if (epi == GEPI_BF16) {
    if (w4) EE_GEMM(GEPI_BF16, true); else EE_GEMM(GEPI_BF16, false);
  } else if (epi == GEPI_RESID) {
    if (w4) EE_GEMM(GEPI_RESID, true); else EE_GEMM(GEPI_RESID, false);
  } else if (epi == GEPI_SWIGLU) {
    if (w4) EE_GEMM(GEPI_SWIGLU, true); else EE_GEMM(GEPI_SWIGLU, false);
  } else {
    throw std::logic_error("gemm: unknown epilogue");
  }
#undef EE_GEMM
}

// ---------------------------------------------------------------------------
// Per-row sums of x over each scale group of G columns (float32), for the
// rows of the sequences in list (the int4 GEMM's correction term).  One wave
// per (row, run of groups).
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(64) void group_sums_kernel(const uint16_t* x, int ldx, int K, int G, float* xs,
                                                        int ldxs, const int32_t* list, const int32_t* cnt, int P,
                                                        int Bt) {
  const int n_seq = min(max(*cnt, 0), Bt);
  const int r = blockIdx.x;
  if (r >= n_seq * P) return;
  const int t = r / n_seq;
  const int pr = t * Bt + list[r - t * n_seq];
  const int lane = threadIdx.x;
  const int ngr = K / G;
  const int lpg = G / 8 < 64 ? G / 8 : 64;  // lanes per group (8 columns each)
  const int gpi = 64 / lpg;                 // groups per iteration
  for (int g0 = 0; g0 < ngr; g0 += gpi) {
    const int g = g0 + lane / lpg;
    const int k = g * G + (lane % lpg) * 8;
    float sum = 0.0f;
    if (g < ngr) {
      const uint4 v = *(const uint4*)(x + (size_t)pr * ldx + k);
      sum = bf2f(v.x & 0xffffu) + bf2f(v.x >> 16) + bf2f(v.y & 0xffffu) + bf2f(v.y >> 16) +
            bf2f(v.z & 0xffffu) + bf2f(v.z >> 16) + bf2f(v.w & 0xffffu) + bf2f(v.w >> 16);
    }
    for (int o = 1; o < lpg; o <<= 1) sum += __shfl_xor(sum, o);
    if (g < ngr && lane % lpg == 0) xs[(size_t)pr * ldxs + g] = sum;
  }
}

void launch_group_sums(const uint16_t* x, int ldx, int K, int G, float* xs, int ldxs, const int32_t* list,
                       const int32_t* cnt, int P, int Bt, hipStream_t s) {
  if (K % G || G % 8 || G / 8 > 64 || (64 % std::min(G / 8, 64)))
    throw std::logic_error("group sums: unsupported group size");
  hipLaunchKernelGGL(group_sums_kernel, dim3(P * Bt), dim3(64), 0, s, x, ldx, K, G, xs, ldxs, list, cnt, P, Bt);
}

// ---------------------------------------------------------------------------
// RoPE and the shared-slot K/V write for every prompt row: qkv [row][H*hd +
// 2*Hkv*hd] holds bf16(W x); row t * B + b is position pos = lens[b] + t of
// sequence b.  q and k pairs (i, i + hd/2) rotate by pos * theta^(-2i/hd)
// (float32 arithmetic on the bf16 values, then rounded), q to qrot, k and v
// to slot (b, head, pos) of the layer; the slot's write counter + 1.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void rope_kv_kernel(const uint16_t* qkv, int P, int B, int H, int Hkv, int hd,
                                                      const float* cosT, const float* sinT, const int32_t* lens,
                                                      uint16_t* qrot, uint16_t* Kl, uint16_t* Vl, uint8_t* occ_l,
                                                      int S) {
  const int r = blockIdx.x;
  const int t = r / B, b = r - t * B;
  const int pos = lens[b] + t;
  const int half = hd >> 1;
  const int nq = H * hd, nkv = Hkv * hd;
  const uint16_t* src = qkv + (size_t)r * (nq + 2 * nkv);
  for (int i = threadIdx.x; i < (H + Hkv) * half; i += blockDim.x) {
    const int head = i / half, e = i - head * half;
    const float c = cosT[(size_t)pos * half + e], sn = sinT[(size_t)pos * half + e];
    const float x1 = bf2f(src[head * hd + e]), x2 = bf2f(src[head * hd + e + half]);
    const uint16_t o1 = (uint16_t)f2bf(x1 * c - x2 * sn);
    const uint16_t o2 = (uint16_t)f2bf(x2 * c + x1 * sn);
    if (head < H) {
      qrot[(size_t)r * nq + head * hd + e] = o1;
      qrot[(size_t)r * nq + head * hd + e + half] = o2;
    } else {
      const int kh = head - H;
      uint16_t* dst = Kl + (((size_t)b * Hkv + kh) * S + pos) * hd;
      dst[e] = o1;
      dst[e + half] = o2;
    }
  }
  for (int i = threadIdx.x; i < nkv; i += blockDim.x) {
    const int vh = i / hd, e = i - vh * hd;
    Vl[(((size_t)b * Hkv + vh) * S + pos) * hd + e] = src[nq + nkv + i];
  }
  if (occ_l && threadIdx.x == 0) occ_l[(size_t)b * S + pos] += 1;
}

void launch_rope_kv(const uint16_t* qkv, int P, int B, int H, int Hkv, int hd, const float* cosT,
                    const float* sinT, const int32_t* lens, uint16_t* qrot, uint16_t* Kl, uint16_t* Vl,
                    uint8_t* occ_l, int S, hipStream_t s) {
  hipLaunchKernelGGL(rope_kv_kernel, dim3(P * B), dim3(256), 0, s, qkv, P, B, H, Hkv, hd, cosT, sinT, lens, qrot,
                     Kl, Vl, occ_l, S);
}

// ---------------------------------------------------------------------------
// Causal prefill attention.  One wave per (block of 32 prompt positions, q
// head, sequence); position t of sequence b (query row t * B + b, cache
// position lens[b] + t) attends to cache positions 0..lens[b] + t of its kv
// head, in tiles of 32 keys.  Scores S = K q on MFMA (K rows from the cache
// as the A operand, 16 keys x 32 head dims per lane group; the queries as B),
// so lane l holds the scores of query l & 15 against keys 4 (l >> 4) + i of
// each 16-key half.  Online softmax per query in float32.  The PV product
// O = P V contracts over the keys; a lane's own eight probabilities (keys
// 4 (l >> 4) + i of both halves) form its A operand (the key order inside
// the contraction is free), and V is staged transposed in LDS (head dims x
// keys) so the B operand reads the same eight keys of one head dimension.
// P is split into bf16 high and low parts (two products), so the weights
// keep ~16 significant bits.  Output bf16(O / l).
// ---------------------------------------------------------------------------
constexpr int kQB = 32;   // queries per wave
constexpr int kKT = 32;   // keys per tile
constexpr int kVtLd = kKT + 4;

template <int HD>
__global__ __launch_bounds__(64) void prefill_attn_kernel(const uint16_t* q, const uint16_t* K, const uint16_t* V,
                                                          int S, int P, int B, int H, int Hkv,
                                                          const int32_t* lens, float scale, uint16_t* out) {
  constexpr int KK = HD / 32;   // MFMA steps over the head dim (scores)
  constexpr int NT = HD / 16;   // 16-wide head-dim tiles of the output
  constexpr int HC = HD / 8;    // 8-wide head-dim chunks (V staging)
  __shared__ __attribute__((aligned(16))) uint16_t vt[HD * kVtLd];
  const int nqb = (P + kQB - 1) / kQB;
  const int qb = nqb - 1 - (int)blockIdx.x;  // the longest blocks first
  const int h = blockIdx.y, b = blockIdx.z;
  const int j = h / (H / Hkv);
  const int lane = threadIdx.x;
  const int c16 = lane & 15, g4 = lane >> 4;
  const int len0 = lens[b];
  const int t0 = qb * kQB;
  const int qd = H * HD;
  const uint16_t* Kb = K + ((size_t)b * Hkv + j) * S * HD;
  const uint16_t* Vb = V + ((size_t)b * Hkv + j) * S * HD;

  // queries of this lane's B columns: positions t0 + qs * 16 + c16
  uint4 qf[2][KK];
#pragma unroll
  for (int qs = 0; qs < 2; ++qs) {
    const int t = t0 + qs * 16 + c16;
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) {
      qf[qs][kk] = make_uint4(0, 0, 0, 0);
      if (t < P) qf[qs][kk] = *(const uint4*)(q + ((size_t)t * B + b) * qd + h * HD + g4 * 8 + 32 * kk);
    }
  }
  float m[2] = {-INFINITY, -INFINITY}, l[2] = {0.0f, 0.0f};
  f32x4_t o[2][NT];
#pragma unroll
  for (int qs = 0; qs < 2; ++qs)
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) o[qs][nt] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};

  const int tlast = min(t0 + kQB, P) - 1;
  const int kend = len0 + tlast;  // last key of the block's last query
  const int smax = S - 1;
  for (int k0 = 0; k0 <= kend; k0 += kKT) {
    // K rows of the two 16-key halves (A operand); rows past the block's last
    // key (never written, possibly not finite) are zeros, their scores masked
    uint4 kf[2][KK];
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      const int key = k0 + ks * 16 + c16;
      const int row = min(key, smax);
#pragma unroll
      for (int kk = 0; kk < KK; ++kk) {
        kf[ks][kk] = make_uint4(0, 0, 0, 0);
        if (key <= kend) kf[ks][kk] = *(const uint4*)(Kb + (size_t)row * HD + g4 * 8 + 32 * kk);
      }
    }
    // V tile transposed into LDS: items (key quad, head-dim chunk)
    constexpr int ITEMS = (kKT / 4) * HC;
#pragma unroll
    for (int it0 = 0; it0 < ITEMS; it0 += 64) {
      const int it = it0 + lane;
      if (it < ITEMS) {
        const int kq = it / HC, hc = it - kq * HC;
        uint4 vr[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {  // zeros past the last key: 0 * V must stay 0
          const int key = k0 + kq * 4 + i;
          vr[i] = make_uint4(0, 0, 0, 0);
          if (key <= kend) vr[i] = *(const uint4*)(Vb + (size_t)min(key, smax) * HD + hc * 8);
        }
        const uint32_t* w0 = (const uint32_t*)&vr[0];
        const uint32_t* w1 = (const uint32_t*)&vr[1];
        const uint32_t* w2 = (const uint32_t*)&vr[2];
        const uint32_t* w3 = (const uint32_t*)&vr[3];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int sh = (e & 1) * 16;
          const uint32_t a0 = (w0[e >> 1] >> sh) & 0xffffu, a1 = (w1[e >> 1] >> sh) & 0xffffu;
          const uint32_t a2 = (w2[e >> 1] >> sh) & 0xffffu, a3 = (w3[e >> 1] >> sh) & 0xffffu;
          *(uint2*)(&vt[(hc * 8 + e) * kVtLd + kq * 4]) = make_uint2(a0 | (a1 << 16), a2 | (a3 << 16));
        }
      }
    }
    // scores: lane holds keys k0 + ks * 16 + 4 g4 + i against query t0 + qs * 16 + c16
    float sc[2][2][4];
#pragma unroll
    for (int qs = 0; qs < 2; ++qs) {
      const int tq = t0 + qs * 16 + c16;
      const int qpos = len0 + tq;
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        f32x4_t s4 = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int kk = 0; kk < KK; ++kk)
          s4 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, kf[ks][kk]),
                                                       __builtin_bit_cast(bf16x8_t, qf[qs][kk]), s4, 0, 0, 0);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int key = k0 + ks * 16 + 4 * g4 + i;
          sc[qs][ks][i] = key <= qpos ? s4[i] * scale : -INFINITY;
        }
      }
    }
    __syncthreads();  // V tile staged
    uint32_t pa_hi[2][4], pa_lo[2][4];   // bf16 pairs of the A operand (8 keys)
    float corr[2];
#pragma unroll
    for (int qs = 0; qs < 2; ++qs) {
      float mt = -INFINITY;
#pragma unroll
      for (int ks = 0; ks < 2; ++ks)
#pragma unroll
        for (int i = 0; i < 4; ++i) mt = fmaxf(mt, sc[qs][ks][i]);
      mt = fmaxf(mt, __shfl_xor(mt, 16));
      mt = fmaxf(mt, __shfl_xor(mt, 32));
      const float mn = fmaxf(m[qs], mt);
      corr[qs] = mn == -INFINITY ? 1.0f : __expf(m[qs] - mn);
      float ls = 0.0f;
      float p[8];
#pragma unroll
      for (int ks = 0; ks < 2; ++ks)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float pv = mn == -INFINITY ? 0.0f : __expf(sc[qs][ks][i] - mn);
          p[ks * 4 + i] = pv;
          ls += pv;
        }
      ls += __shfl_xor(ls, 16);
      ls += __shfl_xor(ls, 32);
      l[qs] = l[qs] * corr[qs] + ls;
      m[qs] = mn;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const uint32_t h0 = f2bf(p[2 * i]), h1 = f2bf(p[2 * i + 1]);
        const uint32_t l0 = f2bf(p[2 * i] - bf2f(h0)), l1 = f2bf(p[2 * i + 1] - bf2f(h1));
        pa_hi[qs][i] = h0 | (h1 << 16);
        pa_lo[qs][i] = l0 | (l1 << 16);
      }
    }
    // rescale the output rows (queries 4 g4 + i of each half) by their queries' corr
#pragma unroll
    for (int qs = 0; qs < 2; ++qs) {
      float cr[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) cr[i] = __shfl(corr[qs], 4 * g4 + i);
#pragma unroll
      for (int nt = 0; nt < NT; ++nt)
#pragma unroll
        for (int i = 0; i < 4; ++i) o[qs][nt][i] *= cr[i];
    }
    // O += P V: B operand = V[keys of this lane group][head dim c16 + 16 nt]
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      const uint2 v0 = *(const uint2*)(&vt[(nt * 16 + c16) * kVtLd + 4 * g4]);
      const uint2 v1 = *(const uint2*)(&vt[(nt * 16 + c16) * kVtLd + 16 + 4 * g4]);
      const uint4 vb = make_uint4(v0.x, v0.y, v1.x, v1.y);
#pragma unroll
      for (int qs = 0; qs < 2; ++qs) {
        const uint4 ah = make_uint4(pa_hi[qs][0], pa_hi[qs][1], pa_hi[qs][2], pa_hi[qs][3]);
        const uint4 al = make_uint4(pa_lo[qs][0], pa_lo[qs][1], pa_lo[qs][2], pa_lo[qs][3]);
        o[qs][nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, ah),
                                                            __builtin_bit_cast(bf16x8_t, vb), o[qs][nt], 0, 0, 0);
        o[qs][nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, al),
                                                            __builtin_bit_cast(bf16x8_t, vb), o[qs][nt], 0, 0, 0);
      }
    }
    __syncthreads();  // before the next tile overwrites vt
  }
  // out rows: queries t0 + qs * 16 + 4 g4 + i, head dims nt * 16 + c16
#pragma unroll
  for (int qs = 0; qs < 2; ++qs) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float li = __shfl(l[qs], 4 * g4 + i);
      const int t = t0 + qs * 16 + 4 * g4 + i;
      if (t >= P) continue;
      const float inv = 1.0f / li;
      uint16_t* dst = out + ((size_t)t * B + b) * qd + h * HD + c16;
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) dst[nt * 16] = (uint16_t)f2bf(o[qs][nt][i] * inv);
    }
  }
}

void launch_prefill_attention(const uint16_t* q, const uint16_t* K, const uint16_t* V, int S, int P, int B, int H,
                              int Hkv, int hd, const int32_t* lens, uint16_t* out, hipStream_t s) {
  const dim3 grid((P + kQB - 1) / kQB, H, B);
  const float scale = (float)(1.0 / std::sqrt((double)hd));
  switch (hd) {
    case 32: hipLaunchKernelGGL(prefill_attn_kernel<32>, grid, dim3(64), 0, s, q, K, V, S, P, B, H, Hkv, lens, scale, out); break;
    case 64: hipLaunchKernelGGL(prefill_attn_kernel<64>, grid, dim3(64), 0, s, q, K, V, S, P, B, H, Hkv, lens, scale, out); break;
    case 128: hipLaunchKernelGGL(prefill_attn_kernel<128>, grid, dim3(64), 0, s, q, K, V, S, P, B, H, Hkv, lens, scale, out); break;
    default: throw std::logic_error("prefill attention: head_dim must be 32, 64 or 128");
  }
}

// ---------------------------------------------------------------------------
// Embedding of every prompt row (row t * B + b is token prompt[b * P + t])
// into the float32 residual and the RMSNorm of the first layer's input into
// x; the step state's row lists are reset (every sequence on the backbone).
// ---------------------------------------------------------------------------
constexpr int kEmbThreads = 256;

__global__ __launch_bounds__(kEmbThreads) void prefill_embed_kernel(StepState* st, const int32_t* prompt, int P,
                                                                    int B, int L, const uint16_t* emb, int d, int V,
                                                                    float* h, const uint16_t* gain, float eps,
                                                                    uint16_t* x) {
  const int r = blockIdx.x;
  const int t = r / B, b = r - t * B;
  const int tid = threadIdx.x;
  int tok = prompt[(size_t)b * P + t];
  tok = min(max(tok, 0), V - 1);  // host-validated
  const uint16_t* src = emb + (size_t)tok * d;
  float* hr = h + (size_t)r * d;
  float ss = 0.0f;
  for (int i = tid; i < d; i += kEmbThreads) {
    const float v = bf2f(src[i]);
    hr[i] = v;
    ss = fmaf(v, v, ss);
  }
  __shared__ float wsum[kEmbThreads / 64];
  __shared__ float rs;
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) ss += __shfl_xor(ss, o);
  if ((tid & 63) == 0) wsum[tid >> 6] = ss;
  __syncthreads();
  if (tid == 0) {
    float tt = 0.0f;
    for (int w = 0; w < kEmbThreads / 64; ++w) tt += wsum[w];
    rs = 1.0f / sqrtf(tt / (float)d + eps);
  }
  __syncthreads();
  for (int i = tid; i < d; i += kEmbThreads)
    x[(size_t)r * d + i] = (uint16_t)f2bf(bf2f(src[i]) * rs * bf2f(gain[i]));
  if (r == 0) {
    for (int i = tid; i < B; i += kEmbThreads) {
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

void launch_prefill_embed(StepState* st, const int32_t* prompt, int P, int B, int L, const uint16_t* emb, int d,
                          int V, float* h, const uint16_t* gain, float eps, uint16_t* x, hipStream_t s) {
  hipLaunchKernelGGL(prefill_embed_kernel, dim3(P * B), dim3(kEmbThreads), 0, s, st, prompt, P, B, L, emb, d, V, h,
                     gain, eps, x);
}

}  // namespace ee
