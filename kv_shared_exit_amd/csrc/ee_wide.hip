// Vocabulary GEMVs for more than 8 rows on matrix cores (gfx950).
//
// The exit head's vocabulary pass (AdaDecode page, section 2.1: logits of the
// intermediate state against the LM head matrix E, softmax, top-1 probability)
// and the final LM head read E (V x d bf16, 1.05 GB at the 8B shape) once per
// launch.  The vector-ALU pass stages at most 8 input rows, so a batch of 64
// rows would read E eight times.  Here every row of the batch (up to 64) is an
// MFMA B-operand column and E is read once:
//   * E is kept a second time in a tiled order made at model creation: for each
//     16-row tile and each 32-column step, the 1 KB that the 64 lanes of a wave
//     load as the A operand of v_mfma_f32_16x16x32_bf16 are contiguous (lane l
//     holds row l % 16, columns 8 (l / 16) .. +8 of the step), so a wave reads
//     whole cache lines.  Rows past V are zero.
//   * A workgroup (8 waves) owns 8 tiles (128 rows) at a time, one per wave,
//     and takes its next 8 tiles a grid later.  The input rows are staged in
//     LDS 256 columns at a time, double-buffered: the next columns are fetched
//     while the current ones are multiplied.
//   * Each wave keeps 8 steps of its tile's E blocks in flight in a register
//     ring, refilled as they are consumed (two workgroups per CU within 128
//     registers per lane: 128 KB of E in flight per CU).  Measured against
//     two tiles per wave at one workgroup per CU: 175.6 against 182.5 us for
//     64 rows at the 8B shape.
//   * Epilogue as the vector-ALU pass: per row of the batch, the workgroup's
//     (max, sum exp) of its logits, or its top-2 (lowest index on ties); the
//     logits never reach memory (except on request for diagnostics).
// Every workgroup of the grid writes its partial for every row, so the decide
// and final kernels merge the same number of partials as after the vector-ALU
// pass.
#include "ee_internal.h"
#include "ee_device.h"
#include "ee_epi.h"

#include <hip/hip_ext.h>

#include <algorithm>
#include <stdexcept>
#include <type_traits>

namespace ee {

namespace {

constexpr int kWideRows = 64;             // batch rows of one pass (MFMA B columns)
constexpr int kWideCols = 256;            // input columns staged per chunk
constexpr int kWideStride = kWideCols + 16;  // LDS row stride: 32 bytes of padding (no bank conflicts in the operand reads)
constexpr int kWideBuf = kWideRows * kWideStride;
constexpr int kWideWaves = kProjThreads / 64;
constexpr int kWideTiles = 1;             // 16-row tiles per wave
constexpr int kRing = 8;                  // 32-column steps in flight per tile

__device__ __forceinline__ bf16x8_t as_bf16x8(const uint4& v) { return __builtin_bit_cast(bf16x8_t, v); }

// int4 A operand: 8 codes of a dword (q + 8 in each nibble, elements 2i and
// 2i+1 in bits 4i and 16+4i) as the bf16 values 136 + q
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

// Sum of one staged 16-byte piece (8 bf16 inputs: four dot products with
// (1, 1)) over the PPG pieces of its scale group (adjacent lanes of the row's
// 32, summed through DPP), stored by the group's first lane
template <int PPG>
__device__ __forceinline__ void wide_group_sum(const uint4& v, float* row_sums, int tid) {
  constexpr uint32_t kOnes = 0x3F803F80u;  // bf16 (1, 1)
  float t = dot2(v.x, kOnes, 0.0f);
  t = dot2(v.y, kOnes, t);
  t = dot2(v.z, kOnes, t);
  t = dot2(v.w, kOnes, t);
  t = group_sum_dpp<PPG>(t);
  if ((tid & (PPG - 1)) == 0) row_sums[(tid & 31) / PPG] = t;
}

}  // namespace

bool wide_vocab_supported(int d) { return d > 0 && d % kWideCols == 0; }

size_t wide_vocab_elems(int V, int d) { return (size_t)((V + 15) / 16) * 16 * d; }

// Wt[((t * nks + k) * 64 + l) * 8 + j] = W[16 t + l % 16][32 k + 8 (l / 16) + j]
// (zero for rows >= N).  One thread per 16 bytes.
__global__ void tile_rows_kernel(const uint16_t* __restrict__ W, int N, int K, uint16_t* __restrict__ Wt,
                                 size_t pieces) {
  const size_t g = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (g >= pieces) return;
  const int nks = K / 32;
  const int lane = (int)(g & 63);
  const size_t blk = g >> 6;
  const int t = (int)(blk / nks);
  const int k = (int)(blk - (size_t)t * nks);
  const int row = t * 16 + (lane & 15);
  const int col = k * 32 + (lane >> 4) * 8;
  uint4 v = make_uint4(0, 0, 0, 0);
  if (row < N) v = *(const uint4*)(W + (size_t)row * K + col);
  *(uint4*)(Wt + g * 8) = v;
}

void launch_tile_rows(const uint16_t* W, int N, int K, uint16_t* dst, hipStream_t s) {
  if (!wide_vocab_supported(K) || N < 1 || !W || !dst) throw std::logic_error("tiled copy: unsupported shape");
  const size_t pieces = wide_vocab_elems(N, K) / 8;
  const int threads = 256;
  hipLaunchKernelGGL(tile_rows_kernel, dim3((unsigned)((pieces + threads - 1) / threads)), dim3(threads), 0, s, W,
                     N, K, dst, pieces);
}

// The gate/up pair order: tile t holds gate rows 8t..8t+7 (tile rows 0-7) and
// up rows 8t..8t+7 (tile rows 8-15), each tile in the order above, so the
// gate and up values of an output end up in lanes l and l ^ 32 of the MFMA
// result.
__global__ void tile_pair_rows_kernel(const uint16_t* __restrict__ gate, const uint16_t* __restrict__ up, int K,
                                      uint16_t* __restrict__ Wt, size_t pieces) {
  const size_t g = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (g >= pieces) return;
  const int nks = K / 32;
  const int lane = (int)(g & 63);
  const size_t blk = g >> 6;
  const int t = (int)(blk / nks);
  const int k = (int)(blk - (size_t)t * nks);
  const int r = lane & 15;
  const uint16_t* src = (r < 8 ? gate : up) + (size_t)(t * 8 + (r & 7)) * K + k * 32 + (lane >> 4) * 8;
  *(uint4*)(Wt + g * 8) = *(const uint4*)src;
}

void launch_tile_pair_rows(const uint16_t* gate, const uint16_t* up, int F, int K, uint16_t* dst, hipStream_t s) {
  if (!wide_vocab_supported(K) || F < 8 || F % 8 || !gate || !up || !dst)
    throw std::logic_error("tiled gate/up copy: unsupported shape");
  const size_t pieces = (size_t)2 * F * K / 8;
  const int threads = 256;
  hipLaunchKernelGGL(tile_pair_rows_kernel, dim3((unsigned)((pieces + threads - 1) / threads)), dim3(threads), 0, s,
                     gate, up, K, dst, pieces);
}

void launch_tile_vocab(const uint16_t* E, int V, int d, uint16_t* Et, hipStream_t s) {
  launch_tile_rows(E, V, d, Et, s);
}

// a.wb[0]: the tiled E; a.N = V; a.K = d; rows: list_bf / cnt_bf, any count
// from 1 to 64 (the four 16-row batch blocks are computed whatever the count:
// the pass is bound by reading E, so a launch with few rows costs about what
// one with 64 does, and no second launch is needed for small counts).
template <int EPI>
__global__ __launch_bounds__(kProjThreads, 4) void wide_vocab_kernel(const ProjArgs a) {
  __shared__ __attribute__((aligned(16))) uint16_t xs[2 * kWideBuf];
  __shared__ float red[kWideWaves * kWideRows * 4];
  const int n = min(max(*a.cnt_bf, 0), kWideRows);
  if (n == 0) return;  // no row on the backbone
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int V = a.N, d = a.K;
  const int nks = d >> 5;            // 32-column steps
  const int nch = d / kWideCols;     // staged chunks
  const int ntiles = (V + 15) >> 4;
  const int npairs = (ntiles + kWideTiles - 1) / kWideTiles;
  const uint16_t* Et = a.wb[0];

  // staging: thread tid copies rows (tid >> 5) + 16 j, 16-byte column group tid & 31
  const int srow = tid >> 5, scol = (tid & 31) * 8;
  const uint16_t* sx[4];
#pragma unroll
  for (int j = 0; j < 4; ++j)  // rows past the count repeat the last one
    sx[j] = a.x + (size_t)a.list_bf[min(srow + 16 * j, n - 1)] * a.x_stride + scol;
  uint4 s0, s1, s2, s3;  // one chunk of this thread's staged inputs in flight
#define EE_STAGE_LOAD(c)                                  \
  do {                                                    \
    const int co_ = (c) * kWideCols;                      \
    s0 = *(const uint4*)(sx[0] + co_);                    \
    s1 = *(const uint4*)(sx[1] + co_);                    \
    s2 = *(const uint4*)(sx[2] + co_);                    \
    s3 = *(const uint4*)(sx[3] + co_);                    \
  } while (0)
#define EE_STAGE_STORE(buf)                                                   \
  do {                                                                        \
    uint16_t* d_ = xs + (buf) * kWideBuf + srow * kWideStride + scol;         \
    *(uint4*)(d_) = s0;                                                       \
    *(uint4*)(d_ + 16 * kWideStride) = s1;                                    \
    *(uint4*)(d_ + 32 * kWideStride) = s2;                                    \
    *(uint4*)(d_ + 48 * kWideStride) = s3;                                    \
  } while (0)

  // running reductions per batch block (column lane % 16 of block bb)
  float lm[4], ls[4];
  Top2 tp[4];
#pragma unroll
  for (int bb = 0; bb < 4; ++bb) {
    lm[bb] = -INFINITY;
    ls[bb] = 0.0f;
    tp[bb] = Top2{-INFINITY, 0x7fffffff, -INFINITY};
  }
  int seqc[4];  // sequence of each batch column of this lane (diagnostic logits)
#pragma unroll
  for (int bb = 0; bb < 4; ++bb) seqc[bb] = a.list_bf[min(bb * 16 + (lane & 15), n - 1)];

  const int niter = (npairs + gridDim.x * kWideWaves - 1) / (gridDim.x * kWideWaves);
  for (int it = 0; it < niter; ++it) {
    const int pair0 = (it * gridDim.x + blockIdx.x) * kWideWaves;
    if (pair0 >= npairs) break;  // uniform over the workgroup
    const int pair = pair0 + wave;
    int tile[kWideTiles];
    const uint16_t* at[kWideTiles];
#pragma unroll
    for (int t = 0; t < kWideTiles; ++t) {
      tile[t] = pair * kWideTiles + t;
      const int tc = min(tile[t], ntiles - 1);  // a wave past the end reads the last tile, discarded
      at[t] = Et + ((size_t)tc * nks * 64 + lane) * 8;
    }
    uint4 ra[kWideTiles][kRing];
#pragma unroll
    for (int i = 0; i < kRing; ++i)
#pragma unroll
      for (int t = 0; t < kWideTiles; ++t) ra[t][i] = ld_stream(at[t] + (size_t)min(i, nks - 1) * 512);
    EE_STAGE_LOAD(0);
    EE_STAGE_STORE(0);
    EE_STAGE_LOAD(min(1, nch - 1));
    __syncthreads();

    f32x4_t acc[kWideTiles][4];
#pragma unroll
    for (int t = 0; t < kWideTiles; ++t)
#pragma unroll
      for (int bb = 0; bb < 4; ++bb) acc[t][bb] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};

    for (int c = 0; c < nch; ++c) {
      const uint16_t* xb = xs + (c & 1) * kWideBuf + (lane & 15) * kWideStride + (lane >> 4) * 8;
#pragma unroll
      for (int i = 0; i < kWideCols / 32; ++i) {
        const int k = c * (kWideCols / 32) + i;
#pragma unroll
        for (int bb = 0; bb < 4; ++bb) {
          const bf16x8_t bop = as_bf16x8(*(const uint4*)(xb + bb * 16 * kWideStride + i * 32));
#pragma unroll
          for (int t = 0; t < kWideTiles; ++t)
            acc[t][bb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(ra[t][i % kRing]), bop, acc[t][bb], 0, 0, 0);
        }
        const int kn = min(k + kRing, nks - 1);  // past the end: reload the last step (unused)
#pragma unroll
        for (int t = 0; t < kWideTiles; ++t) ra[t][i % kRing] = ld_stream(at[t] + (size_t)kn * 512);
      }
      if (c + 1 < nch) EE_STAGE_STORE((c + 1) & 1);
      __syncthreads();
      EE_STAGE_LOAD(min(c + 2, nch - 1));  // past the end: reload the last chunk (unused)
    }

    // fold this iteration's logits into the running reductions: lane l holds
    // rows 16 t + 4 (l / 16) + r of its tiles for batch column l % 16
#pragma unroll
    for (int t = 0; t < kWideTiles; ++t) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int row = tile[t] * 16 + 4 * (lane >> 4) + r;
        if (tile[t] < ntiles && row < V) {
#pragma unroll
          for (int bb = 0; bb < 4; ++bb) {
            const float v = acc[t][bb][r];
            if constexpr (EPI == EPI_LSE) {
              lse_merge(lm[bb], ls[bb], v, 1.0f);
            } else {
              if (a.logits && bb * 16 + (lane & 15) < n) a.logits[(size_t)seqc[bb] * a.logits_stride + row] = v;
              if (v > tp[bb].v1) {
                tp[bb].v2 = tp[bb].v1;
                tp[bb].v1 = v;
                tp[bb].i1 = row;
              } else if (v > tp[bb].v2) {
                tp[bb].v2 = v;
              }
            }
          }
        }
      }
    }
  }

#undef EE_STAGE_LOAD
#undef EE_STAGE_STORE

  // merge the four lanes of each column, then the waves (fixed order)
#pragma unroll
  for (int bb = 0; bb < 4; ++bb) {
    each_offset_up<16>([&](auto mc) {
      constexpr int M = decltype(mc)::value;
      if constexpr (EPI == EPI_LSE) {
        lse_merge(lm[bb], ls[bb], xor_lane<M>(lm[bb], lane), xor_lane<M>(ls[bb], lane));
      } else {
        top2_merge(tp[bb], Top2{xor_lane<M>(tp[bb].v1, lane), xor_lane<M>(tp[bb].i1, lane),
                                xor_lane<M>(tp[bb].v2, lane)});
      }
    });
    if (lane < 16) {
      float* rw = red + (wave * kWideRows + bb * 16 + lane) * 4;
      if constexpr (EPI == EPI_LSE) {
        rw[0] = lm[bb];
        rw[1] = ls[bb];
      } else {
        rw[0] = tp[bb].v1;
        rw[1] = __int_as_float(tp[bb].i1);
        rw[2] = tp[bb].v2;
      }
    }
  }
  __syncthreads();
  if (tid < n) {
    float* out = a.part + ((size_t)blockIdx.x * kMaxBatch + tid) * 4;
    if constexpr (EPI == EPI_LSE) {
      float m = -INFINITY, s = 0.0f;
      for (int w = 0; w < kWideWaves; ++w) {
        const float* r = red + (w * kWideRows + tid) * 4;
        lse_merge(m, s, r[0], r[1]);
      }
      out[0] = m;
      out[1] = s;
    } else {
      Top2 best{-INFINITY, 0x7fffffff, -INFINITY};
      for (int w = 0; w < kWideWaves; ++w) {
        const float* r = red + (w * kWideRows + tid) * 4;
        top2_merge(best, Top2{r[0], __float_as_int(r[1]), r[2]});
      }
      out[0] = best.v1;
      out[1] = __int_as_float(best.i1);
      out[2] = best.v2;
    }
  }
}

void launch_wide_vocab(int epi, const ProjArgs& a0, int nwg, hipStream_t s, hipEvent_t ev_start,
                       hipEvent_t ev_end) {
  ProjArgs a = a0;
  if (!a.cnt_bf || !a.list_bf) a.cnt_bf = a.list_bf = no_rows();
  if (!wide_vocab_supported(a.K) || a.N < 1 || !a.wb[0] || !a.part)
    throw std::logic_error("wide vocabulary pass: unsupported arguments");
  if (epi != EPI_LSE && epi != EPI_ARGMAX) throw std::logic_error("wide vocabulary pass: epilogue");
  const int g = std::max(1, std::min(nwg, kNwgMax));
  auto kern = epi == EPI_LSE ? wide_vocab_kernel<EPI_LSE> : wide_vocab_kernel<EPI_ARGMAX>;
  if (ev_start || ev_end)
    hipExtLaunchKernelGGL(kern, dim3(g), dim3(kProjThreads), 0, s, ev_start, ev_end, 0, a);
  else
    hipLaunchKernelGGL(kern, dim3(g), dim3(kProjThreads), 0, s, a);
}

// ---------------------------------------------------------------------------
// Projections for more than 8 rows (QKV, O, gate/up, down, the head
// projection T): y[r][seq][n] = sum over the columns of range r of W[n][k]
// x[seq][k], on matrix cores for up to 64 rows at once, so every weight is
// read once per launch (River-LLM explainer, section 4: a layer serves its
// backbone rows with the bf16 weights and its exited rows with the int4 copy;
// both run in the same launch, the workgroups split between the two).
//   * A workgroup owns 128 rows (a 16-row tile per wave) and one column range;
//     the input rows of the range are staged in LDS 256 columns at a time,
//     double-buffered (as in the vocabulary pass).
//   * bf16 rows read the tiled copy (4 or 2 steps of 1 KB in flight per wave,
//     see the end of the kernel).
//   * int4 rows: a lane unpacks a dword of codes (8 weights) into the A
//     operand (nibble | 0x4300 is the bf16 value 136 + q); the 136 * sum(x)
//     of each scale group is computed once per staged row when the inputs are
//     staged (not by a second MFMA per wave) and removed before the group's
//     scale is applied.
//   * The ranges are summed by the epilogue kernels below (or by the finish
//     kernel for O and down), in range order.
// ---------------------------------------------------------------------------
// Column ranges: the most (up to 8) that keep one format's workgroups within
// 256, so a launch with both formats fits the 512 resident workgroups in one
// round (measured at 64 rows, 8B widths: gate/up 1 range 42 us against 54 us
// for 3 with bf16 rows only, 59 against 63 us with 32 rows of each; QKV 4
// ranges 13 against 16 us).
int wide_ranges(int N, int K, int* kr) {
  const int nrb = (N + 127) / 128;
  const int steps = K / kWideCols;
  int nr = std::max(1, std::min(std::min(8, steps), 256 / nrb));
  const int w = (steps + nr - 1) / nr;
  if (kr) *kr = w * kWideCols;
  return (steps + w - 1) / w;
}

template <int NG>
__global__ __launch_bounds__(kProjThreads, 4) void wide_proj_kernel(const WideArgs a) {
  constexpr int G = 128 / NG;   // int4 scale group
  constexpr int PPG = G / 8;    // 16-byte pieces per group
  constexpr int SPG = 4 / NG;   // 32-column steps per group
  __shared__ __attribute__((aligned(16))) uint16_t xs[2 * kWideBuf];
  __shared__ float xsum[2][kWideRows][2 * NG];  // sum of each staged row over each scale group of the chunk
  const bool i4 = (int)blockIdx.x >= a.g_bf;
  const int wg = i4 ? (int)blockIdx.x - a.g_bf : (int)blockIdx.x;
  const int32_t* list = i4 ? a.list_i4 : a.list_bf;
  const int n = min(max(*(i4 ? a.cnt_i4 : a.cnt_bf), 0), kWideRows);
  if (n == 0) return;  // uniform: no rows in this format
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int r = wg % a.nr, rb = wg / a.nr;
  const int k0 = r * a.kr;
  const int kw = min(a.kr, a.K - k0);
  const int nch = kw / kWideCols;
  const int nbb = (n + 15) >> 4;
  const int ntiles = a.N >> 4;
  const int tile = rb * kWideWaves + wave;
  const int tc = min(tile, ntiles - 1);  // a wave past the last tile computes on it and stores nothing

  const int srow = tid >> 5, scol = (tid & 31) * 8;
  const uint16_t* sx[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) sx[j] = a.x + (size_t)list[min(srow + 16 * j, n - 1)] * a.x_stride + k0 + scol;
  uint4 s0, s1{}, s2{}, s3{};
  // (used inside the loop body below: only the NBS blocks of rows are staged)
#define EE_STAGE_LOAD(c)                            \
  do {                                              \
    const int co_ = (c) * kWideCols;                \
    s0 = *(const uint4*)(sx[0] + co_);              \
    if (NBS > 1) s1 = *(const uint4*)(sx[1] + co_); \
    if (NBS > 2) s2 = *(const uint4*)(sx[2] + co_); \
    if (NBS > 3) s3 = *(const uint4*)(sx[3] + co_); \
  } while (0)
#define EE_STAGE_STORE(buf)                                                   \
  do {                                                                        \
    uint16_t* d_ = xs + (buf) * kWideBuf + srow * kWideStride + scol;         \
    *(uint4*)(d_) = s0;                                                       \
    if (NBS > 1) *(uint4*)(d_ + 16 * kWideStride) = s1;                       \
    if (NBS > 2) *(uint4*)(d_ + 32 * kWideStride) = s2;                       \
    if (NBS > 3) *(uint4*)(d_ + 48 * kWideStride) = s3;                       \
    if (i4) {                                                                 \
      wide_group_sum<PPG>(s0, xsum[buf][srow], tid);                          \
      if (NBS > 1) wide_group_sum<PPG>(s1, xsum[buf][srow + 16], tid);        \
      if (NBS > 2) wide_group_sum<PPG>(s2, xsum[buf][srow + 32], tid);        \
      if (NBS > 3) wide_group_sum<PPG>(s3, xsum[buf][srow + 48], tid);        \
    }                                                                         \
  } while (0)

  // At group size 128 the batch blocks (16 rows each) are a template constant
  // of the loop body, so each MFMA and its LDS operand are issued without a
  // branch and the compiler keeps several operand reads in flight (NBB = 0:
  // the count read at run time, for the smaller groups, whose scales leave no
  // registers for it).  RB: 32-column steps of bf16 weights in flight per wave.
  auto run = [&](auto nbb_c, auto rb_c) {
    constexpr int NBS = decltype(nbb_c)::value ? decltype(nbb_c)::value : 4;  // blocks staged
    constexpr int RB = decltype(rb_c)::value;
    const int NBB = decltype(nbb_c)::value ? decltype(nbb_c)::value : nbb;
    f32x4_t acc[4];
#pragma unroll
    for (int bb = 0; bb < 4; ++bb) acc[bb] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};

    if (!i4) {
      const int nks = a.K >> 5;
      const int st0 = k0 >> 5, ns = kw >> 5;  // first step of the range, steps in it
      const uint16_t* at = a.wt + ((size_t)tc * nks * 64 + lane) * 8;
      uint4 ra[RB];
#pragma unroll
      for (int i = 0; i < RB; ++i) ra[i] = ld_stream(at + (size_t)(st0 + min(i, ns - 1)) * 512);
      EE_STAGE_LOAD(0);
      EE_STAGE_STORE(0);
      EE_STAGE_LOAD(min(1, nch - 1));
      __syncthreads();
      for (int c = 0; c < nch; ++c) {
        const uint16_t* xb = xs + (c & 1) * kWideBuf + (lane & 15) * kWideStride + (lane >> 4) * 8;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const bf16x8_t aop = as_bf16x8(ra[i % RB]);  // step c * 8 + i (RB divides 8)
#pragma unroll
          for (int bb = 0; bb < 4; ++bb)
            if (bb < NBB)
              acc[bb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                  aop, as_bf16x8(*(const uint4*)(xb + bb * 16 * kWideStride + i * 32)), acc[bb], 0, 0, 0);
          ra[i % RB] = ld_stream(at + (size_t)(st0 + min(c * 8 + i + RB, ns - 1)) * 512);  // past the end: reload (unused)
          __builtin_amdgcn_sched_barrier(0);
        }
        if (c + 1 < nch) EE_STAGE_STORE((c + 1) & 1);
        __syncthreads();
        EE_STAGE_LOAD(min(c + 2, nch - 1));
      }
    } else if constexpr (RB == 4) {
      const int ngr = a.K / G;
      // this lane's code row (A operand row lane % 16) and the four rows of
      // its scales (result rows 4 (lane / 16) ..): segment and row in it
      int cseg, crow, sseg, srw;
      if (a.pair) {  // gate rows 8 tc .. (tile rows 0-7), then the same up rows
        cseg = (lane & 15) >= 8;
        crow = tc * 8 + (lane & 7);
        sseg = (lane >> 4) >= 2;
        srw = tc * 8 + 4 * ((lane >> 4) & 1);
      } else {
        cseg = sseg = tc * 16 >= a.n0 ? 1 : 0;
        const int ts = tc - (cseg ? a.n0 >> 4 : 0);  // tile within its segment
        crow = ts * 16 + (lane & 15);
        srw = ts * 16 + 4 * (lane >> 4);
      }
      const uint32_t* cp = a.q4[cseg] + (size_t)crow * (a.K >> 3) + (k0 >> 3) + (lane >> 4) * 4;
      // scales: [16-row tile of the segment][group][row of the tile]
      const uint16_t* sp = a.s4[sseg] + ((size_t)(srw >> 4) * ngr + k0 / G) * 16 + (srw & 15);
      const int nbk = kw >> 7;  // 128-column blocks of the range
      // codes of two chunks (RD = 4 blocks) in flight at group size 128: slots
      // 0-1 hold the even chunks' blocks, 2-3 the odd chunks' (the chunk loop is
      // unrolled by two so every slot index is fixed); smaller groups keep one
      // chunk (their scales take the registers).  Cached loads: a block's codes
      // are half of a 128-byte line per row, the other half being the next
      // block.
      constexpr int RD = NG == 1 ? 4 : 2;
      uint4 rc[RD];
      uint2 rs[RD][NG];
#pragma unroll
      for (int i = 0; i < RD; ++i) {
        const int u = min(i, nbk - 1);
        rc[i] = *(const uint4*)(cp + u * 16);
#pragma unroll
        for (int g = 0; g < NG; ++g) rs[i][g] = *(const uint2*)(sp + (u * NG + g) * 16);
      }
      EE_STAGE_LOAD(0);
      EE_STAGE_STORE(0);
      EE_STAGE_LOAD(min(1, nch - 1));
      __syncthreads();
      f32x4_t cg[4];
#pragma unroll
      for (int bb = 0; bb < 4; ++bb) cg[bb] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
      // one 256-column chunk: its two blocks from ring slots sl, sl + 1, which
      // are then refilled with the blocks RD / 2 chunks ahead
      auto do_chunk = [&](const int c, const int sl) {
        const uint16_t* xb = xs + (c & 1) * kWideBuf + (lane & 15) * kWideStride + (lane >> 4) * 8;
        const float* xsr = &xsum[c & 1][lane & 15][0];
#pragma unroll
        for (int ub = 0; ub < 2; ++ub) {
          const uint4 cw = rc[sl + ub];
          uint2 sv[NG];
#pragma unroll
          for (int g = 0; g < NG; ++g) sv[g] = rs[sl + ub][g];
          const int un = min(c * 2 + ub + RD, nbk - 1);  // past the end: reload (unused)
          rc[sl + ub] = *(const uint4*)(cp + un * 16);
#pragma unroll
          for (int g = 0; g < NG; ++g) rs[sl + ub][g] = *(const uint2*)(sp + (un * NG + g) * 16);
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const bf16x8_t aop = unpack8(pick(cw, j));
#pragma unroll
            for (int bb = 0; bb < 4; ++bb)
              if (bb < NBB)
                cg[bb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                    aop, as_bf16x8(*(const uint4*)(xb + bb * 16 * kWideStride + (ub * 4 + j) * 32)), cg[bb], 0, 0, 0);
            if ((j + 1) % SPG == 0) {  // end of a scale group
              const int gi = j / SPG;
              const uint2 sc = sv[gi];
              const float q0 = bf2f(sc.x & 0xffffu), q1 = bf2f(sc.x >> 16);
              const float q2 = bf2f(sc.y & 0xffffu), q3 = bf2f(sc.y >> 16);
#pragma unroll
              for (int bb = 0; bb < 4; ++bb) {
                if (bb < NBB) {
                  const float corr = 136.0f * xsr[bb * 16 * 2 * NG + ub * NG + gi];
                  acc[bb][0] = fmaf(q0, cg[bb][0] - corr, acc[bb][0]);
                  acc[bb][1] = fmaf(q1, cg[bb][1] - corr, acc[bb][1]);
                  acc[bb][2] = fmaf(q2, cg[bb][2] - corr, acc[bb][2]);
                  acc[bb][3] = fmaf(q3, cg[bb][3] - corr, acc[bb][3]);
                }
                cg[bb] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
              }
            }
            __builtin_amdgcn_sched_barrier(0);
          }
        }
        if (c + 1 < nch) EE_STAGE_STORE((c + 1) & 1);
        __syncthreads();
        EE_STAGE_LOAD(min(c + 2, nch - 1));
      };
      if constexpr (RD == 4) {
        for (int c = 0; c < nch; c += 2) {
          do_chunk(c, 0);
          if (c + 1 < nch) do_chunk(c + 1, 2);  // uniform
        }
      } else {
        for (int c = 0; c < nch; ++c) do_chunk(c, 0);
      }
    }
#undef EE_STAGE_LOAD
#undef EE_STAGE_STORE

    // lane l holds rows 16 tile + 4 (l / 16) .. +3 of batch column l % 16 of block bb
    if (a.act) {  // gate/up in one range: SwiGLU of the pair in lanes l, l ^ 32 (uniform)
#pragma unroll
      for (int bb = 0; bb < 4; ++bb) {
        float u[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) u[i] = xor_lane<32>(acc[bb][i], lane);
        const int col = bb * 16 + (lane & 15);
        if (tile < ntiles && bb < NBB && col < n && lane < 32) {
          const uint32_t o0 = f2bf(silu_mul(acc[bb][0], u[0])) | (f2bf(silu_mul(acc[bb][1], u[1])) << 16);
          const uint32_t o1 = f2bf(silu_mul(acc[bb][2], u[2])) | (f2bf(silu_mul(acc[bb][3], u[3])) << 16);
          *(uint2*)(a.act + (size_t)list[col] * a.pair + tile * 8 + 4 * (lane >> 4)) = make_uint2(o0, o1);
        }
      }
    } else if (tile < ntiles) {
#pragma unroll
      for (int bb = 0; bb < 4; ++bb) {
        const int col = bb * 16 + (lane & 15);
        if (bb < NBB && col < n) {
          float* dst = a.y + (size_t)r * a.y_cstride + (size_t)list[col] * a.y_stride + tile * 16 + 4 * (lane >> 4);
          *(float4*)dst = make_float4(acc[bb][0], acc[bb][1], acc[bb][2], acc[bb][3]);
        }
      }
    }
  };
  // bf16 weights: 4 steps (4 KB) in flight per wave, 2 when the launch has
  // more int4 rows than bf16 rows.  The int4 workgroups that share a CU with
  // bf16 workgroups wait for their loads behind the bf16 stream's; a shallower
  // bf16 ring shortens that queue.  Measured at the 8B widths, 64 rows (gate/up,
  // bf16 / int4 rows): 8 steps 42.4 / 58.9 / 73.1 us (64/0, 32/32, 8/56), 4
  // steps 40.4 / 53.6 / 67.6, 2 steps 49.6 / 56.8 / 56.8.
  const bool shallow = !i4 && *a.cnt_i4 > n;
  auto go = [&](auto nbb_c) {
    if (shallow)
      run(nbb_c, std::integral_constant<int, 2>{});
    else
      run(nbb_c, std::integral_constant<int, 4>{});
  };
  if constexpr (NG == 1) {
    switch (nbb) {
      case 1: go(std::integral_constant<int, 1>{}); break;
      case 2: go(std::integral_constant<int, 2>{}); break;
      case 3: go(std::integral_constant<int, 3>{}); break;
      default: go(std::integral_constant<int, 4>{}); break;
    }
  } else {
    go(std::integral_constant<int, 0>{});
  }
}

void launch_wide_proj(WideArgs a, hipStream_t s) {
  if (!a.cnt_bf || !a.list_bf) a.cnt_bf = a.list_bf = no_rows();
  const bool i4 = a.q4[0] != nullptr;
  if (!i4 || !a.cnt_i4 || !a.list_i4) a.cnt_i4 = a.list_i4 = no_rows();
  if (!wide_vocab_supported(a.K) || a.N < 16 || a.N % 16 || !a.wt || !a.x || (!a.y && !a.act) || a.nr < 1 ||
      a.kr % kWideCols || (long long)a.nr * a.kr < a.K || (long long)(a.nr - 1) * a.kr >= a.K)
    throw std::logic_error("wide projection: unsupported arguments");
  if ((a.pair && (a.pair % 16 || (long long)2 * a.pair != a.N)) || (a.act && (!a.pair || a.nr != 1)))
    throw std::logic_error("wide projection: unsupported gate/up pairing");
  if (i4 && (a.n0 % 16 || a.n0 <= 0 || !a.s4[0] || (a.n0 < a.N && (!a.q4[1] || !a.s4[1])) ||
             (a.pair && a.n0 != a.pair) || (a.G != 32 && a.G != 64 && a.G != 128)))
    throw std::logic_error("wide projection: unsupported int4 arguments");
  a.nrb = (a.N + 127) / 128;
  a.g_bf = a.nrb * a.nr;
  const int g = a.g_bf * (i4 ? 2 : 1);
  if (!i4 || a.G == 128)
    hipLaunchKernelGGL(wide_proj_kernel<1>, dim3(g), dim3(kProjThreads), 0, s, a);
  else if (a.G == 64)
    hipLaunchKernelGGL(wide_proj_kernel<2>, dim3(g), dim3(kProjThreads), 0, s, a);
  else
    hipLaunchKernelGGL(wide_proj_kernel<4>, dim3(g), dim3(kProjThreads), 0, s, a);
}

// ---------------------------------------------------------------------------
// Epilogues: one thread per (row of the list, output), the ranges summed in
// order with all loads in flight.
// ---------------------------------------------------------------------------
constexpr int kEpiThreads = 256;

__device__ __forceinline__ float wide_sum(const float* y, int nr, size_t cs) {
  float v[8];
#pragma unroll
  for (int r = 0; r < 8; ++r) v[r] = y[(size_t)min(r, nr - 1) * cs];
  float t = v[0];
#pragma unroll
  for (int r = 1; r < 8; ++r)
    if (r < nr) t += v[r];
  for (int r = 8; r < nr; ++r) t += y[(size_t)r * cs];
  return t;
}

__global__ void wide_qkv_kernel(const float* y, int nr, size_t cs, int ys, const int32_t* list, const int32_t* cnt,
                                const ProjArgs qa) {
  const int p = blockIdx.y;
  if (p >= min(max(*cnt, 0), kMaxBatch)) return;
  const int nout = (qa.H + 2 * qa.Hkv) * qa.hd;
  const int nn = blockIdx.x * kEpiThreads + threadIdx.x;
  if (nn >= nout) return;
  const int seq = list[p];
  const int half = qa.hd >> 1;
  const int e = nn & (qa.hd - 1);
  const int partner = e < half ? nn + half : nn - half;
  const float* yr = y + (size_t)seq * ys;
  qkv_out(qa, seq, nn, wide_sum(yr + nn, nr, cs), wide_sum(yr + partner, nr, cs));
}

__global__ void wide_swiglu_kernel(const float* y, int nr, size_t cs, int ys, const int32_t* list, const int32_t* cnt,
                                   int F, uint16_t* out) {
  const int p = blockIdx.y;
  if (p >= min(max(*cnt, 0), kMaxBatch)) return;
  const int nn = blockIdx.x * kEpiThreads + threadIdx.x;
  if (nn >= F) return;
  const int seq = list[p];
  const float* yr = y + (size_t)seq * ys + (nn >> 3) * 16 + (nn & 7);  // the pair order: gate, then up 8 later
  out[(size_t)seq * F + nn] = (uint16_t)f2bf(silu_mul(wide_sum(yr, nr, cs), wide_sum(yr + 8, nr, cs)));
}

__global__ void wide_bf16_kernel(const float* y, int nr, size_t cs, int ys, const int32_t* list, const int32_t* cnt,
                                 int N, uint16_t* out, int out_stride) {
  const int p = blockIdx.y;
  if (p >= min(max(*cnt, 0), kMaxBatch)) return;
  const int nn = blockIdx.x * kEpiThreads + threadIdx.x;
  if (nn >= N) return;
  const int seq = list[p];
  out[(size_t)seq * out_stride + nn] = (uint16_t)f2bf(wide_sum(y + (size_t)seq * ys + nn, nr, cs));
}

void launch_wide_qkv(const float* y, int nr, size_t cstride, int ystride, const int32_t* list, const int32_t* cnt,
                     int B, const ProjArgs& qa, hipStream_t s) {
  const int nout = (qa.H + 2 * qa.Hkv) * qa.hd;
  if (!y || !list || !cnt || nr < 1 || B < 1 || B > kMaxBatch || ystride < nout || qa.hd < 2 ||
      (qa.hd & (qa.hd - 1)))
    throw std::logic_error("wide QKV epilogue: bad arguments");
  hipLaunchKernelGGL(wide_qkv_kernel, dim3((nout + kEpiThreads - 1) / kEpiThreads, B), dim3(kEpiThreads), 0, s, y,
                     nr, cstride, ystride, list, cnt, qa);
}

void launch_wide_swiglu(const float* y, int nr, size_t cstride, int ystride, const int32_t* list, const int32_t* cnt,
                        int B, int F, uint16_t* out, hipStream_t s) {
  if (!y || !list || !cnt || !out || nr < 1 || B < 1 || B > kMaxBatch || ystride < 2 * F)
    throw std::logic_error("wide SwiGLU epilogue: bad arguments");
  hipLaunchKernelGGL(wide_swiglu_kernel, dim3((F + kEpiThreads - 1) / kEpiThreads, B), dim3(kEpiThreads), 0, s, y,
                     nr, cstride, ystride, list, cnt, F, out);
}

void launch_wide_bf16(const float* y, int nr, size_t cstride, int ystride, const int32_t* list, const int32_t* cnt,
                      int B, int N, uint16_t* out, int out_stride, hipStream_t s) {
  if (!y || !list || !cnt || !out || nr < 1 || B < 1 || B > kMaxBatch || ystride < N || out_stride < N)
    throw std::logic_error("wide bf16 epilogue: bad arguments");
  hipLaunchKernelGGL(wide_bf16_kernel, dim3((N + kEpiThreads - 1) / kEpiThreads, B), dim3(kEpiThreads), 0, s, y, nr,
                     cstride, ystride, list, cnt, N, out, out_stride);
}

}  // namespace ee
