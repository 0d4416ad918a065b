// ee_probe: launches one of the library's kernels on synthetic operands, for
// hardware-counter runs of a single kernel (rocprofv3 --pmc) outside a Python
// process, and a plain device copy of known size that calibrates the byte
// counters.
//
//   ee_probe lse V d rows reps [grid]
//                                exit-head vocabulary GEMV (proj_kernel<EPI_LSE>)
//                                over a V x d bf16 matrix and `rows` staged rows
//   ee_probe wide V d rows reps [grid]
//                                the same GEMV on matrix cores as steps of more
//                                than 8 rows run it (wide_vocab_kernel<EPI_LSE>
//                                over the tiled copy, 1..64 rows); grid: the
//                                workgroups (default: the decode step's)
//   ee_probe proj EPI N K nbf ni4 reps
//                                a decoder projection (EPI: swiglu = gate/up
//                                with its epilogue, part = O, down or a
//                                QKV-sized map with float32 partials) of N
//                                output rows over K inputs, nbf rows on the
//                                bf16 weights and ni4 on the int4 G128 copy,
//                                on the decode step's grid (512 workgroups)
//   ee_probe wproj N K nbf ni4 reps [pair]
//                                a decoder projection for more than 8 rows on
//                                matrix cores (wide_proj_kernel: N output rows
//                                over K inputs, nbf rows on the tiled bf16
//                                weights and ni4 on the int4 G128 copy, float32
//                                partial sums over the column ranges the decode
//                                step uses); pair 1: gate/up as the decode step
//                                runs it (N = 2 F, gate and up rows paired per
//                                tile, SwiGLU applied by the pass when it has
//                                one column range)
//   ee_probe copy MiB            one copy kernel reading and writing MiB each
//   ee_probe read MiB reps       a read-only stream of MiB (each thread sums its
//                                16-byte loads): the streaming-read ceiling
//   ee_probe readc MiB reps      the same bytes read with one contiguous region
//                                per workgroup (512 workgroups)
//   ee_probe attn B S ctx reps   decode attention of B sequences at the 8B heads
//                                (32 q / 8 kv of 128) over ctx + 1 cached
//                                positions, cache capacity S: attn_kernel +
//                                combine, or from 256 (sequence, kv head) pairs
//                                attn_fused_kernel, as the decode step launches
//   ee_probe gemm EPI M N K reps the prefill GEMM (EPI: bf16, resid or swiglu) of
//                                M token rows (8 sequences of M / 8 positions)
//                                with N x K bf16 weights (swiglu: gate and up)
//
// Prints the mean launch time (HIP events on the launch stream).
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <vector>

#include "ee_internal.h"
#include "ee_device.h"

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

// Reads n 16-byte words (4 loads in flight per thread) and writes one word per thread.
__global__ __launch_bounds__(256) void read_kernel(const uint4* __restrict__ src, uint32_t* __restrict__ out,
                                                   size_t n) {
  const size_t stride = (size_t)gridDim.x * blockDim.x;
  uint32_t acc = 0;
  size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  for (; i + 3 * stride < n; i += 4 * stride) {
    const uint4 a = ld_stream(src + i), b = ld_stream(src + i + stride);
    const uint4 c = ld_stream(src + i + 2 * stride), d = ld_stream(src + i + 3 * stride);
    acc ^= a.x ^ a.y ^ a.z ^ a.w ^ b.x ^ b.y ^ b.z ^ b.w ^ c.x ^ c.y ^ c.z ^ c.w ^ d.x ^ d.y ^ d.z ^ d.w;
  }
  for (; i < n; i += stride) {
    const uint4 a = ld_stream(src + i);
    acc ^= a.x ^ a.y ^ a.z ^ a.w;
  }
  out[(size_t)blockIdx.x * blockDim.x + threadIdx.x] = acc;
}

// Each workgroup reads one contiguous region of n / gridDim.x words, 4 loads
// in flight per thread, and writes one word per thread.
__global__ __launch_bounds__(256) void read_region_kernel(const uint4* __restrict__ src, uint32_t* __restrict__ out,
                                                          size_t n) {
  const size_t per = n / gridDim.x;
  const uint4* base = src + (size_t)blockIdx.x * per;
  uint32_t acc = 0;
  size_t i = threadIdx.x;
  for (; i + 3 * blockDim.x < per; i += 4 * blockDim.x) {
    const uint4 a = ld_stream(base + i), b = ld_stream(base + i + blockDim.x);
    const uint4 c = ld_stream(base + i + 2 * blockDim.x), d = ld_stream(base + i + 3 * blockDim.x);
    acc ^= a.x ^ a.y ^ a.z ^ a.w ^ b.x ^ b.y ^ b.z ^ b.w ^ c.x ^ c.y ^ c.z ^ c.w ^ d.x ^ d.y ^ d.z ^ d.w;
  }
  for (; i < per; i += blockDim.x) acc ^= ld_stream(base + i).x;
  out[(size_t)blockIdx.x * blockDim.x + threadIdx.x] = acc;
}

static int usage() {
  std::fprintf(stderr,
               "usage: ee_probe lse|wide V d rows reps [grid] | "
               "ee_probe proj swiglu|part N K nbf ni4 reps | ee_probe wproj N K nbf ni4 reps [pair] | ee_probe copy MiB | "
               "ee_probe read|readc MiB reps | "
               "ee_probe attn B S ctx reps | ee_probe gemm bf16|resid|swiglu M N K reps\n");
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
  auto timed = [&](auto&& launch, int reps) {
    launch();  // warm-up
    CK(hipStreamSynchronize(s));
    CK(hipEventRecord(e0, s));
    for (int r = 0; r < reps; ++r) launch();
    CK(hipEventRecord(e1, s));
    CK(hipEventSynchronize(e1));
    float ms = 0;
    CK(hipEventElapsedTime(&ms, e0, e1));
    return 1e3 * ms / reps;  // us per launch
  };
  const bool region = !std::strcmp(argv[1], "readc");
  if (!std::strcmp(argv[1], "read") || region) {
    if (argc < 4) return usage();
    const size_t mib = std::strtoull(argv[2], nullptr, 10);
    const int reps = std::atoi(argv[3]);
    if (mib == 0 || mib > 16384 || reps < 1) return usage();
    const size_t n = mib << 16;
    uint4* src;
    uint32_t* out;
    CK(hipMalloc(&src, n * 16));
    CK(hipMalloc(&out, (size_t)4096 * 256 * 4));
    CK(hipMemsetAsync(src, 1, n * 16, s));
    const double us = timed(
        [&] {
          if (region)
            hipLaunchKernelGGL(read_region_kernel, dim3(512), dim3(256), 0, s, src, out, n);
          else
            hipLaunchKernelGGL(read_kernel, dim3(4096), dim3(256), 0, s, src, out, n);
        },
        reps);
    std::printf("%s %zu MiB: %.2f us, %.1f GB/s\n", region ? "readc" : "read", mib, us, n * 16.0 / us / 1e3);
    return 0;
  }
  if (!std::strcmp(argv[1], "attn")) {
    if (argc < 6) return usage();
    const int B = std::atoi(argv[2]), S = std::atoi(argv[3]), ctx = std::atoi(argv[4]), reps = std::atoi(argv[5]);
    const int H = 32, Hkv = 8, hd = 128;
    if (B < 1 || B > kMaxBatch || S < 2 || ctx < 0 || ctx >= S || reps < 1) return usage();
    // the decode step's split: runs of tiles so that about 2048 waves are launched
    const int tiles = (S + 63) / 64;
    int tpw = 1;
    while (tpw < tiles && (long long)B * Hkv * ((tiles + tpw - 1) / tpw) > 2048) tpw *= 2;
    const int nch = (tiles + tpw - 1) / tpw;
    uint16_t *q, *K, *V, *out;
    float* part;
    int32_t* lens;
    const size_t kvn = (size_t)B * Hkv * S * hd;
    CK(hipMalloc(&q, (size_t)B * H * hd * 2));
    CK(hipMalloc(&K, kvn * 2));
    CK(hipMalloc(&V, kvn * 2));
    CK(hipMalloc(&out, (size_t)B * H * hd * 2));
    CK(hipMalloc(&part, (size_t)B * H * nch * (hd + 2) * 4));
    CK(hipMalloc(&lens, kMaxBatch * 4));
    CK(hipMemsetAsync(q, 0x3c, (size_t)B * H * hd * 2, s));
    CK(hipMemsetAsync(K, 0x3c, kvn * 2, s));
    CK(hipMemsetAsync(V, 0x3c, kvn * 2, s));
    std::vector<int32_t> hl(kMaxBatch, ctx);
    CK(hipMemcpyAsync(lens, hl.data(), hl.size() * 4, hipMemcpyHostToDevice, s));
    AttnArgs a{};
    a.q = q;
    a.K = K;
    a.V = V;
    a.S = S;
    a.Bmax = B;
    a.lens = lens;
    a.H = H;
    a.Hkv = Hkv;
    a.hd = hd;
    a.B = B;
    a.tpw = tpw;
    a.nch = nch;
    a.scale = 0.08838834764831845f;
    a.part = part;
    a.out = out;
    a.fused = (long long)B * Hkv >= 256;  // as the decode step: one workgroup per (sequence, kv head)
    const double us = timed([&] { launch_attention(a, s); }, reps);
    const double bytes = (double)B * (ctx + 1) * Hkv * hd * 2 * 2;
    std::printf("attn B=%d S=%d ctx=%d tiles/wave=%d partials=%d: %.2f us (attention + combine), %.1f GB/s algorithmic\n",
                B, S, ctx, tpw, nch, us, bytes / us / 1e3);
    return 0;
  }
  if (!std::strcmp(argv[1], "gemm")) {
    if (argc < 7) return usage();
    const int epi = !std::strcmp(argv[2], "bf16") ? GEPI_BF16 : !std::strcmp(argv[2], "resid") ? GEPI_RESID
                    : !std::strcmp(argv[2], "swiglu") ? GEPI_SWIGLU : -1;
    const int M = std::atoi(argv[3]), N = std::atoi(argv[4]), K = std::atoi(argv[5]), reps = std::atoi(argv[6]);
    if (epi < 0 || M < 8 || M % 8 || N < 32 || N % 32 || K < 32 || K % 32 || reps < 1) return usage();
    const int nmat = epi == GEPI_SWIGLU ? 2 : 1;
    uint16_t *W, *x, *ob;
    float* of;
    int32_t* lists;
    CK(hipMalloc(&W, (size_t)nmat * N * K * 2));
    CK(hipMalloc(&x, (size_t)M * K * 2));
    CK(hipMalloc(&ob, (size_t)M * N * 2));
    CK(hipMalloc(&of, (size_t)M * N * 4));
    CK(hipMalloc(&lists, 2 * kMaxBatch * 4));
    CK(hipMemsetAsync(W, 0x3c, (size_t)nmat * N * K * 2, s));
    CK(hipMemsetAsync(x, 0x3c, (size_t)M * K * 2, s));
    CK(hipMemsetAsync(of, 0, (size_t)M * N * 4, s));
    std::vector<int32_t> hl(2 * kMaxBatch, 0);
    for (int i = 0; i < 8; ++i) hl[i] = i;
    hl[kMaxBatch] = 8;
    CK(hipMemcpyAsync(lists, hl.data(), hl.size() * 4, hipMemcpyHostToDevice, s));
    GemmArgs g{};
    g.N = N;
    g.K = K;
    g.G = 128;
    g.nseg = 1;
    g.wb[0] = W;
    g.seg_end[0] = g.seg_end[1] = g.seg_end[2] = N;
    g.wb2 = W + (size_t)N * K;
    g.x = x;
    g.ldx = K;
    g.list = lists;
    g.cnt = lists + kMaxBatch;
    g.P = M / 8;
    g.Bt = 8;
    g.ob = ob;
    g.ldo = N;
    g.of = of;
    g.src = of;
    g.ldf = N;
    const double us = timed([&] { launch_gemm(epi, false, g, M, s); }, reps);
    const double flops = 2.0 * M * (double)N * K * nmat;
    std::printf("gemm %s M=%d N=%d K=%d: %.2f us, %.1f TFLOP/s\n", argv[2], M, N, K, us, flops / us / 1e6);
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
  if (!std::strcmp(argv[1], "wproj")) {
    if (argc < 7) return usage();
    const int N = std::atoi(argv[2]), K = std::atoi(argv[3]), nbf = std::atoi(argv[4]), ni4 = std::atoi(argv[5]);
    const int reps = std::atoi(argv[6]);
    const bool pair = argc > 7 && std::atoi(argv[7]) != 0;
    constexpr int G = 128;
    if (N < 128 || N % 128 || K < 256 || K % 256 || nbf < 0 || ni4 < 0 || nbf + ni4 < 1 || nbf + ni4 > kMaxBatch ||
        reps < 1)
      return usage();
    const int n0 = N % 256 == 0 ? N / 2 : N;  // second int4 segment from N / 2 (gate/up), if even
    const size_t wn = (size_t)N * K;
    uint16_t *W, *Wt, *x, *sc;
    uint32_t* codes;
    float* y;
    int32_t* lists;
    int kr = 0;
    const int nr = wide_ranges(N, K, &kr);
    CK(hipMalloc(&W, wn * 2));
    CK(hipMalloc(&Wt, wn * 2));
    CK(hipMalloc(&codes, wn / 2));
    CK(hipMalloc(&sc, wn / G * 2));
    CK(hipMalloc(&x, (size_t)kMaxBatch * K * 2));
    CK(hipMalloc(&y, (size_t)nr * kMaxBatch * N * 4));
    CK(hipMalloc(&lists, 4 * kMaxBatch * 4));
    uint16_t* act = nullptr;
    CK(hipMalloc(&act, (size_t)kMaxBatch * N / 2 * 2));
    CK(hipMemsetAsync(W, 0x3c, wn * 2, s));  // bf16 ~0.0115
    CK(hipMemsetAsync(codes, 0x99, wn / 2, s));
    CK(hipMemsetAsync(sc, 0x3c, wn / G * 2, s));
    CK(hipMemsetAsync(x, 0x3c, (size_t)kMaxBatch * K * 2, s));
    if (pair && (N % 256 || n0 * 2 != N)) return usage();
    if (pair)
      launch_tile_pair_rows(W, W + (size_t)n0 * K, n0, K, Wt, s);
    else
      launch_tile_rows(W, N, K, Wt, s);
    std::vector<int32_t> hl(4 * kMaxBatch, 0);
    for (int i = 0; i < nbf; ++i) hl[i] = i;
    for (int i = 0; i < ni4; ++i) hl[kMaxBatch + i] = nbf + i;
    hl[2 * kMaxBatch] = nbf;
    hl[3 * kMaxBatch] = ni4;
    CK(hipMemcpyAsync(lists, hl.data(), hl.size() * 4, hipMemcpyHostToDevice, s));
    WideArgs a{};
    a.N = N;
    a.K = K;
    a.nr = nr;
    a.kr = kr;
    a.wt = Wt;
    a.q4[0] = codes;
    a.s4[0] = sc;
    a.n0 = n0;
    if (n0 < N) {
      a.q4[1] = codes + (size_t)n0 * K / 8;
      a.s4[1] = sc + (size_t)n0 * (K / G);
    }
    a.G = G;
    a.x = x;
    a.x_stride = K;
    a.list_bf = lists;
    a.list_i4 = lists + kMaxBatch;
    a.cnt_bf = lists + 2 * kMaxBatch;
    a.cnt_i4 = lists + 3 * kMaxBatch;
    a.y = y;
    a.y_stride = N;
    a.y_cstride = (size_t)kMaxBatch * N;
    if (pair) {
      a.pair = n0;
      if (nr == 1) a.act = act;
    }
    launch_wide_proj(a, s);  // warm-up
    CK(hipStreamSynchronize(s));
    CK(hipEventRecord(e0, s));
    for (int r = 0; r < reps; ++r) launch_wide_proj(a, s);
    CK(hipEventRecord(e1, s));
    CK(hipEventSynchronize(e1));
    float ms = 0;
    CK(hipEventElapsedTime(&ms, e0, e1));
    const double us = 1e3 * ms / reps;
    const double bytes = (nbf ? 2.0 * wn : 0.0) + (ni4 ? wn / 2.0 + wn / G * 2.0 : 0.0);
    const double flops = 2.0 * wn * (nbf + ni4);
    std::printf("wproj N=%d K=%d bf=%d i4=%d ranges=%d%s: %.2f us per launch, %.1f GB/s algorithmic, %.1f TFLOP/s\n",
                N, K, nbf, ni4, nr, pair ? (a.act ? " pair+swiglu" : " pair") : "", us, bytes / us / 1e3,
                flops / us / 1e6);
    return 0;
  }
  const bool wide = !std::strcmp(argv[1], "wide");
  if (!std::strcmp(argv[1], "lse") || wide) {
    if (argc < 6) return usage();
    const int V = std::atoi(argv[2]), d = std::atoi(argv[3]), rows = std::atoi(argv[4]), reps = std::atoi(argv[5]);
    if (V < 1 || d < 32 || d % 32 || rows < 1 || reps < 1) return usage();
    if (!wide && (rows > 8 || !proj_fits(d, rows))) return usage();
    if (wide && (rows > kMaxBatch || !wide_vocab_supported(d))) return usage();
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
    int nv = std::max(1, std::min(kNwgMax, (tiles + rounds * waves - 1) / (rounds * waves)));
    if (wide) nv = kNwgMax;  // as the decode step launches it
    if (argc > 6) nv = std::atoi(argv[6]);  // or the grid given
    if (nv < 1 || nv > kNwgMax) return usage();
    auto launch = [&] {
      if (wide)
        launch_wide_vocab(EPI_LSE, a, nv, s);
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
