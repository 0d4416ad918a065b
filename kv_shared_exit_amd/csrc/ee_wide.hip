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
//   * A workgroup (8 waves) owns 16 tiles (256 rows), two per wave.  The input
//     rows are staged in LDS 256 columns at a time, double-buffered: the next
//     columns are fetched while the current ones are multiplied.
//   * Each wave keeps 8 steps of its two tiles' E blocks in flight in a
//     register ring, refilled as they are consumed (one workgroup per CU:
//     256 registers per lane; 128 KB of E in flight per CU).
//   * Epilogue as the vector-ALU pass: per row of the batch, the workgroup's
//     (max, sum exp) of its logits, or its top-2 (lowest index on ties); the
//     logits never reach memory (except on request for diagnostics).
// Every workgroup of the grid writes its partial for every row, so the decide
// and final kernels merge the same number of partials as after the vector-ALU
// pass.
#include "ee_internal.h"
#include "ee_device.h"

#include <hip/hip_ext.h>

#include <stdexcept>

namespace ee {

namespace {

constexpr int kWideRows = 64;             // batch rows of one pass (MFMA B columns)
constexpr int kWideCols = 256;            // input columns staged per chunk
constexpr int kWideStride = kWideCols + 8;  // LDS row stride (16 bytes of padding)
constexpr int kWideBuf = kWideRows * kWideStride;
constexpr int kWideWaves = kProjThreads / 64;
constexpr int kWideTiles = 2;             // 16-row tiles per wave
constexpr int kRing = 8;                  // 32-column steps in flight per tile

__device__ __forceinline__ bf16x8_t as_bf16x8(const uint4& v) { return __builtin_bit_cast(bf16x8_t, v); }

}  // namespace

bool wide_vocab_supported(int d) { return d > 0 && d % kWideCols == 0; }

size_t wide_vocab_elems(int V, int d) { return (size_t)((V + 15) / 16) * 16 * d; }

// Et[((t * nks + k) * 64 + l) * 8 + j] = E[16 t + l % 16][32 k + 8 (l / 16) + j]
// (zero for rows >= V).  One thread per 16 bytes.
__global__ void tile_vocab_kernel(const uint16_t* __restrict__ E, int V, int d, uint16_t* __restrict__ Et,
                                  size_t pieces) {
  const size_t g = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (g >= pieces) return;
  const int nks = d / 32;
  const int lane = (int)(g & 63);
  const size_t blk = g >> 6;
  const int t = (int)(blk / nks);
  const int k = (int)(blk - (size_t)t * nks);
  const int row = t * 16 + (lane & 15);
  const int col = k * 32 + (lane >> 4) * 8;
  uint4 v = make_uint4(0, 0, 0, 0);
  if (row < V) v = *(const uint4*)(E + (size_t)row * d + col);
  *(uint4*)(Et + g * 8) = v;
}

void launch_tile_vocab(const uint16_t* E, int V, int d, uint16_t* Et, hipStream_t s) {
  if (!wide_vocab_supported(d) || V < 1) throw std::logic_error("tiled vocabulary copy: unsupported shape");
  const size_t pieces = wide_vocab_elems(V, d) / 8;
  const int threads = 256;
  hipLaunchKernelGGL(tile_vocab_kernel, dim3((unsigned)((pieces + threads - 1) / threads)), dim3(threads), 0, s,
                     E, V, d, Et, pieces);
}

// a.wb[0]: the tiled E; a.N = V; a.K = d; rows: list_bf / cnt_bf (runs only
// when the count exceeds 8: the vector-ALU pass takes smaller counts).
template <int EPI>
__global__ __launch_bounds__(kProjThreads, 2) void wide_vocab_kernel(const ProjArgs a) {
  __shared__ __attribute__((aligned(16))) uint16_t xs[2 * kWideBuf];
  __shared__ float red[kWideWaves * kWideRows * 4];
  const int n = min(max(*a.cnt_bf, 0), kWideRows);
  if (n <= 8) return;  // the vector-ALU pass has these rows
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
#pragma unroll
    for (int off = 16; off <= 32; off <<= 1) {
      if constexpr (EPI == EPI_LSE) {
        const float m2 = __shfl_xor(lm[bb], off), s2 = __shfl_xor(ls[bb], off);
        lse_merge(lm[bb], ls[bb], m2, s2);
      } else {
        const Top2 o{__shfl_xor(tp[bb].v1, off), __shfl_xor(tp[bb].i1, off), __shfl_xor(tp[bb].v2, off)};
        top2_merge(tp[bb], o);
      }
    }
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

void launch_wide_vocab(int epi, const ProjArgs& a0, int nwg, hipStream_t s, hipEvent_t ev_end) {
  ProjArgs a = a0;
  if (!a.cnt_bf || !a.list_bf) a.cnt_bf = a.list_bf = no_rows();
  if (!wide_vocab_supported(a.K) || a.N < 1 || !a.wb[0] || !a.part)
    throw std::logic_error("wide vocabulary pass: unsupported arguments");
  if (epi != EPI_LSE && epi != EPI_ARGMAX) throw std::logic_error("wide vocabulary pass: epilogue");
  const int g = std::max(1, std::min(nwg, kNwgMax));
  auto kern = epi == EPI_LSE ? wide_vocab_kernel<EPI_LSE> : wide_vocab_kernel<EPI_ARGMAX>;
  if (ev_end)
    hipExtLaunchKernelGGL(kern, dim3(g), dim3(kProjThreads), 0, s, nullptr, ev_end, 0, a);
  else
    hipLaunchKernelGGL(kern, dim3(g), dim3(kProjThreads), 0, s, a);
}

}  // namespace ee
