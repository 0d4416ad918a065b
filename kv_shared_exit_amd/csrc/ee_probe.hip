// ee_probe: launches one of the library's kernels on synthetic operands, for
// hardware-counter runs of a single kernel (rocprofv3 --pmc) outside a Python
// process, and a plain device copy of known size that calibrates the byte
// counters.
//
//   ee_probe lse V d rows reps   exit-head vocabulary GEMV (proj_kernel<EPI_LSE>)
//                                over a V x d bf16 matrix and `rows` staged rows
//   ee_probe wide V d rows reps  the same GEMV for 9..64 rows on matrix cores
//                                (wide_vocab_kernel<EPI_LSE> over the tiled copy)
//   ee_probe proj EPI N K nbf ni4 reps
//                                a decoder projection (EPI: swiglu = gate/up
//                                with its epilogue, part = O, down or a
//                                QKV-sized map with float32 partials) of N
//                                output rows over K inputs, nbf rows on the
//                                bf16 weights and ni4 on the int4 G128 copy,
//                                on the decode step's grid (512 workgroups)
//   ee_probe copy MiB            one copy kernel reading and writing MiB each
//
// Prints the mean launch time (HIP events on the launch stream).
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <vector>

#include "ee_internal.h"

using namespace ee;

#define CK(x)                                                                        \
  do {                                                                               \
    hipError_t e_ = (x);                                                             \
    if (e_ != hipSuccess) {                                                          \
      std::fprintf(stderr, "HIP error %s at line %d\n", hipGetErrorString(e_), __LINE__); \
      std::exit(1);                                                                  \
    }                                                                                \
  } while (0)

__global__ void copy_kernel(const uint4* __restrict__ src, uint4* __restrict__ dst, size_t n) {
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (size_t)gridDim.x * blockDim.x)
    dst[i] = src[i];
}

static int usage() {
  std::fprintf(stderr,
               "usage: ee_probe lse V d rows reps | ee_probe wide V d rows reps | "
               "ee_probe proj swiglu|part N K nbf ni4 reps | ee_probe copy MiB\n");
  return 2;
}

int main(int argc, char** argv) {
  if (argc < 2) return usage();
  hipStream_t s;
  CK(hipStreamCreate(&s));
  hipEvent_t e0, e1;
  CK(hipEventCreate(&e0));
  CK(hipEventCreate(&e1));
  if (!std::strcmp(argv[1], "copy")) {
    if (argc < 3) return usage();
    const size_t mib = std::strtoull(argv[2], nullptr, 10);
    if (mib == 0 || mib > 16384) return usage();
    const size_t n = mib << 16;  // uint4 elements
    uint4 *src, *dst;
    CK(hipMalloc(&src, n * 16));
    CK(hipMalloc(&dst, n * 16));
    CK(hipMemsetAsync(src, 1, n * 16, s));
    CK(hipStreamSynchronize(s));
    CK(hipEventRecord(e0, s));
    hipLaunchKernelGGL(copy_kernel, dim3(4096), dim3(256), 0, s, src, dst, n);
    CK(hipEventRecord(e1, s));
    CK(hipEventSynchronize(e1));
    float ms = 0;
    CK(hipEventElapsedTime(&ms, e0, e1));
    std::printf("copy %zu MiB: %.2f us, %.1f GB/s (read + write)\n", mib, 1e3 * ms, 2.0 * n * 16 / (ms * 1e6));
    return 0;
  }
  if (!std::strcmp(argv[1], "proj")) {
    if (argc < 8) return usage();
    const bool swiglu = !std::strcmp(argv[2], "swiglu");
    if (!swiglu && std::strcmp(argv[2], "part")) return usage();
    const int N = std::atoi(argv[3]), K = std::atoi(argv[4]), nbf = std::atoi(argv[5]), ni4 = std::atoi(argv[6]);
    const int g = 512, reps = std::atoi(argv[7]);  // the decode step's projection grid
    constexpr int G = 128;
    if (N < 16 || N % 16 || K < G || K % G || nbf < 0 || ni4 < 0 || nbf + ni4 < 1 || nbf + ni4 > 8 || g < 1 ||
        reps < 1)
      return usage();
    if (swiglu && !proj_fits(K, nbf + ni4)) return usage();
    const int P = swiglu ? 2 : 1;
    uint16_t *W, *x, *sc;
    uint32_t* codes;
    void* y;
    int32_t* lists;
    const size_t wn = (size_t)N * K, cn = (size_t)N * K / 8, sn = (size_t)N * (K / G);
    CK(hipMalloc(&W, P * wn * 2));
    CK(hipMalloc(&codes, P * cn * 4));
    CK(hipMalloc(&sc, P * sn * 2));
    CK(hipMalloc(&x, (size_t)kMaxBatch * K * 2));
    const size_t yn = swiglu ? (size_t)kMaxBatch * N * 2 : (size_t)8 * kMaxBatch * N * 4;
    CK(hipMalloc(&y, yn));
    CK(hipMalloc(&lists, 4 * kMaxBatch * 4));
    CK(hipMemsetAsync(W, 0x3c, P * wn * 2, s));  // bf16 ~0.0115
    CK(hipMemsetAsync(codes, 0x99, P * cn * 4, s));
    CK(hipMemsetAsync(sc, 0x3c, P * sn * 2, s));
    CK(hipMemsetAsync(x, 0x3c, (size_t)kMaxBatch * K * 2, s));
    // rows 0..nbf-1 on bf16, nbf..nbf+ni4-1 on int4: lists then counts
    std::vector<int32_t> hl(4 * kMaxBatch, 0);
    for (int i = 0; i < nbf; ++i) hl[i] = i;
    for (int i = 0; i < ni4; ++i) hl[kMaxBatch + i] = nbf + i;
    hl[2 * kMaxBatch] = nbf;
    hl[3 * kMaxBatch] = ni4;
    CK(hipMemcpyAsync(lists, hl.data(), hl.size() * 4, hipMemcpyHostToDevice, s));
    ProjArgs a{};
    a.N = N;
    a.K = K;
    a.G = G;
    a.nseg = 1;
    a.wb[0] = W;
    a.seg_end[0] = a.seg_end[1] = a.seg_end[2] = N;
    a.q4 = codes;
    a.s4 = sc;
    if (swiglu) {
      a.wb2 = W + wn;
      a.q4b = codes + cn;
      a.s4b = sc + sn;
    }
    a.x = x;
    a.x_stride = K;
    a.list_bf = lists;
    a.list_i4 = lists + kMaxBatch;
    a.cnt_bf = lists + 2 * kMaxBatch;
    a.cnt_i4 = lists + 3 * kMaxBatch;
    a.y = y;
    a.y_stride = N;
    a.y_cstride = kMaxBatch * N;
    const int epi = swiglu ? EPI_SWIGLU : EPI_PART;
    int nkc = 1;
    auto launch = [&] { nkc = launch_proj(epi, a, g, nbf + ni4, s); };
    launch();  // warm-up
    CK(hipStreamSynchronize(s));
    CK(hipEventRecord(e0, s));
    for (int r = 0; r < reps; ++r) launch();
    CK(hipEventRecord(e1, s));
    CK(hipEventSynchronize(e1));
    float ms = 0;
    CK(hipEventElapsedTime(&ms, e0, e1));
    const double us = 1e3 * ms / reps;
    const double bytes = (nbf ? 2.0 * P * wn : 0.0) + (ni4 ? P * (cn * 4.0 + sn * 2.0) : 0.0);
    std::printf("proj %s N=%d K=%d bf=%d i4=%d g=%d ranges=%d: %.2f us per launch, %.1f GB/s algorithmic\n", argv[2],
                N, K, nbf, ni4, g, nkc, us, bytes / us / 1e3);
    return 0;
  }
  const bool wide = !std::strcmp(argv[1], "wide");
  if (!std::strcmp(argv[1], "lse") || wide) {
    if (argc < 6) return usage();
    const int V = std::atoi(argv[2]), d = std::atoi(argv[3]), rows = std::atoi(argv[4]), reps = std::atoi(argv[5]);
    if (V < 1 || d < 32 || d % 32 || rows < 1 || reps < 1) return usage();
    if (!wide && (rows > 8 || !proj_fits(d, rows))) return usage();
    if (wide && (rows <= 8 || rows > kMaxBatch || !wide_vocab_supported(d))) return usage();
    uint16_t *E, *x;
    float* part;
    int32_t* lists;
    CK(hipMalloc(&E, (size_t)V * d * 2));
    CK(hipMalloc(&x, (size_t)kMaxBatch * d * 2));
    CK(hipMalloc(&part, (size_t)kNwgMax * kMaxBatch * 4 * 4));
    CK(hipMalloc(&lists, 2 * kMaxBatch * 4));
    CK(hipMemsetAsync(E, 0x3c, (size_t)V * d * 2, s));  // bf16 ~0.0115
    CK(hipMemsetAsync(x, 0x3c, (size_t)kMaxBatch * d * 2, s));
    std::vector<int32_t> hl(2 * kMaxBatch, 0);
    for (int i = 0; i < kMaxBatch; ++i) hl[i] = i;
    hl[kMaxBatch] = rows;
    CK(hipMemcpyAsync(lists, hl.data(), hl.size() * 4, hipMemcpyHostToDevice, s));
    ProjArgs a{};
    a.N = V;
    a.K = d;
    a.G = 128;
    a.nseg = 1;
    a.wb[0] = E;
    a.seg_end[0] = a.seg_end[1] = a.seg_end[2] = V;
    a.x = x;
    a.x_stride = d;
    a.list_bf = lists;
    a.cnt_bf = lists + kMaxBatch;
    a.part = part;
    uint16_t* Et = nullptr;
    if (wide) {
      CK(hipMalloc(&Et, wide_vocab_elems(V, d) * 2));
      launch_tile_vocab(E, V, d, Et, s);
      a.wb[0] = Et;
    }
    // the 8-row pass runs on the grid the decode step gives it: the fewest
    // workgroups that keep the full grid's rounds of 2-row wave tiles
    const int tiles = (V + 1) / 2, waves = kProjThreads / 64;
    const int rounds = (tiles + kNwgMax * waves - 1) / (kNwgMax * waves);
    const int nv = std::max(1, std::min(kNwgMax, (tiles + rounds * waves - 1) / (rounds * waves)));
    auto launch = [&] {
      if (wide)
        launch_wide_vocab(EPI_LSE, a, kNwgMax, s);
      else
        launch_proj(EPI_LSE, a, nv, rows, s);
    };
    launch();  // warm-up
    CK(hipStreamSynchronize(s));
    CK(hipEventRecord(e0, s));
    for (int r = 0; r < reps; ++r) launch();
    CK(hipEventRecord(e1, s));
    CK(hipEventSynchronize(e1));
    float ms = 0;
    CK(hipEventElapsedTime(&ms, e0, e1));
    const double us = 1e3 * ms / reps;
    const double bytes = 2.0 * V * d + 2.0 * d * rows;
    std::printf("%s V=%d d=%d rows=%d: %.2f us per launch, %.1f GB/s algorithmic\n", wide ? "wide" : "lse", V, d,
                rows, us, bytes / us / 1e3);
    return 0;
  }
  return usage();
}
