// Internal interface between the host orchestration (ee_api.hip) and the
// gfx950 kernels (ee_kernels.hip).  Not part of the public ABI.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ee {

constexpr int kMaxBatch = 64;      // rows of one decode step
constexpr int kProjThreads = 512;  // 8 waves per projection workgroup
constexpr int kXLdsElems = 32768;  // bf16 elements of the staged GEMV input (64 KB)
constexpr int kNwgMax = 512;       // projection grid cap (size of the per-workgroup partial buffers)

// Projection epilogues: bf16 output; float32 partial sums of a column range
// (summed into the residual by the finish kernel); SwiGLU; the exit head's
// (max, sum exp) per workgroup; the LM head's top-2 per workgroup; RoPE and the
// shared-slot K/V write.
// Sampled decoding (AdaDecode's verification) adds: the exit head's pass with
// the draft's Gumbel-max and the temperature's (max, sum exp) (EPI_LSE_S), the
// LM head's pass with the final distribution's statistics (EPI_ARGMAX_S), and
// the resampling pass over relu(p_final - p_draft) (EPI_RESAMPLE).
enum Epi {
  EPI_BF16 = 0, EPI_PART = 1, EPI_SWIGLU = 2, EPI_LSE = 3, EPI_ARGMAX = 4, EPI_QKV = 5,
  EPI_LSE_S = 6, EPI_ARGMAX_S = 7, EPI_RESAMPLE = 8
};

// Streams of the counter-based draws (the counter is (v / 4, sequence,
// position, stream)); the same numbering as the oracle's.
enum SampleStream { STREAM_DRAFT = 1, STREAM_FINAL = 2, STREAM_RESAMPLE = 3, STREAM_ACCEPT = 4 };
constexpr int kPartS = 8;  // floats per (workgroup, sequence) of the sampled partials

// Device-resident state of one step.  Every value that changes from step to
// step lives here, so a captured graph replays unchanged.
struct StepState {
  int32_t tok[kMaxBatch];      // input token of the step (next input after it)
  int32_t forced[kMaxBatch];   // 0: exit head decides; 1..L: forced exit layer
  int32_t exited[kMaxBatch];
  int32_t e[kMaxBatch];        // exit layer
  int32_t act[kMaxBatch];      // rows on the backbone (bf16 weights)
  int32_t ex[kMaxBatch];       // rows on the exit copies (int4 weights)
  int32_t all[kMaxBatch];      // 0..B-1
  int32_t n_act, n_ex, n_all, pad;
  int32_t out_tok[kMaxBatch];
  float gap[kMaxBatch];
  // sampled decoding: the draft of each sequence that exited (token, its exit
  // logit, log sum exp of the exit logits / tau; draft_tok -1: no draft), the
  // final distribution's log sum exp, and the rejected sequences as (b, 64 + b)
  // row pairs for the resampling pass
  int32_t draft_tok[kMaxBatch];
  float draft_logit[kMaxBatch];
  float draft_lse[kMaxBatch];
  float lse_f[kMaxBatch];
  int32_t rej[2 * kMaxBatch];
  int32_t n_rej, pad2;
};

struct ProjArgs {
  int N, K, G;           // rows, columns (whole matrix), int4 group size
  int nkc, kc;           // column ranges of a launch (EPI_PART only; else 1, K) and their width
  int nseg;              // bf16 row segments (QKV: 3)
  int seg_end[3];        // cumulative end row of each segment
  const uint16_t* wb[3]; // bf16 segment bases, row-major [rows][K]
  const uint16_t* wb2;   // SwiGLU: the "up" matrix (gate is wb[0])
  const uint32_t* q4;    // int4 codes [N16][K/8] dwords (layout: ee_proj.hip)
  const uint16_t* s4;    // bf16 scales [N16/16][K/G][16]
  const uint32_t* q4b;   // SwiGLU "up" codes
  const uint16_t* s4b;
  const uint16_t* x;     // bf16 input rows [seq][x_stride]
  int x_stride;
  const int32_t* list_bf; const int32_t* cnt_bf;  // rows run with bf16 weights
  const int32_t* list_i4; const int32_t* cnt_i4;  // rows run with int4 weights (may be null)
  void* y; int y_stride;                          // output rows, indexed by sequence id
  int y_cstride;                                  // EPI_PART: elements between column ranges
  float* part;                                    // EPI_LSE / EPI_ARGMAX partials per workgroup
  float* logits; int logits_stride;               // EPI_ARGMAX: optional logits out
  // EPI_QKV: RoPE on q and k, q to qrot, k and v into the cache slot of the position
  const float* cosT; const float* sinT;           // [pos][hd/2]
  const int32_t* lens;                            // position of the current token
  uint16_t* qrot;                                 // [b][H*hd]
  uint16_t* Kl; uint16_t* Vl;                     // layer base [Bmax][Hkv][S][hd]
  uint8_t* occ_l;                                 // [Bmax][S] write counters, or null
  int H, Hkv, hd, S;
  int hd_log2;                                    // log2(hd)
  int nwg_r;                                      // workgroups per column range (set by launch_proj)
  // (set by launch_proj) bf16 workgroups per range when both formats have
  // rows, workgroups per range that work when only int4 rows are present,
  // and the int4 pass's waves per 16-row tile [both formats * 2 + last
  // range]: computed once on the host instead of by every wave
  int nbf_mix;
  int nwg_i4;
  int wpt4[4];
  // sampled epilogues: 1 / temperature, the generator's seed, partials by
  // sequence [nwg][kMaxBatch][kPartS], and the step state
  float itau;
  uint32_t seed;
  float* part_s;
  const StepState* st;
};

// A projection for more than 8 rows on matrix cores (ee_wide.hip): float32
// partial sums y[r][seq][n] over column ranges r, for the rows of both lists
// (bf16 rows from the tiled copy of the weights, exited rows from the int4
// copy); an epilogue kernel (or the finish kernel) sums the ranges.
struct WideArgs {
  int N, K;              // output rows (all segments), input columns (multiple of 256)
  int nr, kr;            // column ranges and their width (multiple of 256)
  int nrb;               // 128-row blocks
  int g_bf;              // workgroups of the bf16 pass (nrb * nr); the rest run the int4 pass
  const uint16_t* wt;    // bf16 weights in the tiled order (launch_tile_rows)
  const uint32_t* q4[2]; // int4 codes / scales of rows [0, n0) and [n0, N) (layout: ee_proj.hip)
  const uint16_t* s4[2];
  int n0, G;
  const uint16_t* x; int x_stride;                // bf16 input rows [seq][x_stride]
  const int32_t* list_bf; const int32_t* cnt_bf;  // rows run with bf16 weights
  const int32_t* list_i4; const int32_t* cnt_i4;  // rows run with int4 weights (may be null)
  float* y; size_t y_cstride; int y_stride;       // y[r * y_cstride + seq * y_stride + n]
  // gate/up (pair = F): tile t holds gate rows 8t..8t+7 then up rows 8t..8t+7
  // (launch_tile_pair_rows; int4: q4/s4[0] gate, [1] up); with one column
  // range and act set, the pass applies SwiGLU itself and writes bf16
  // act[seq][F] (no partial sums); otherwise y holds the pairs in tile order
  int pair;
  uint16_t* act;
};

struct AttnArgs {
  const uint16_t* q;   // rotated q [b][H*hd]
  const uint16_t* K;   // layer base of the cache: [Bmax][Hkv][S][hd]
  const uint16_t* V;
  int S, Bmax;
  const int32_t* lens; // position of the current token per sequence
  int H, Hkv, hd, B;
  int tpw, nch;        // 64-position tiles per wave; waves (partials) per (sequence, kv head)
  float scale;
  float* part;         // [B][H][nch][hd + 2]
  uint16_t* out;       // [b][H*hd]
  int fused;           // one workgroup per (sequence, kv head), merged in LDS (no partials)
};

// A prefill projection on matrix cores (ee_prefill.hip): for the sequences
// list[0..*cnt), rows r = t * n + i (n = *cnt) are position t of sequence
// list[i], physical row t * Bt + list[i] of x and of the outputs.
// out = x W^T over K columns, W [N][K] bf16 in up to 3 row segments (QKV),
// or the int4 copy (q4/s4, rows 0..N); SwiGLU: gate = wb[0] / q4, up = wb2 /
// q4b, N = F.  int4 needs the per-row group sums of x (xs [row][ldxs]).
enum GemmEpi { GEPI_BF16 = 0, GEPI_RESID = 1, GEPI_SWIGLU = 2 };
struct GemmArgs {
  int N, K, G;
  int nseg;
  int seg_end[3];
  const uint16_t* wb[3];
  const uint16_t* wb2;
  const uint32_t* q4; const uint16_t* s4;
  const uint32_t* q4b; const uint16_t* s4b;
  const uint16_t* x; int ldx;
  const float* xs; int ldxs;
  const int32_t* list; const int32_t* cnt;
  int P, Bt;
  uint16_t* ob; int ldo;                 // GEPI_BF16 / GEPI_SWIGLU: bf16 out [row][ldo]
  float* of; const float* src; int ldf;  // GEPI_RESID: of = src + x W^T (float32; src may be of)
};
// Launches a prefill projection over at most max_rows rows (grid bound; the
// device-side count decides which tiles run).
void launch_gemm(int epi, bool w4, const GemmArgs& a, int max_rows, hipStream_t s);
// xs[row][g] = sum of x[row][g G .. (g + 1) G) for the rows of the listed sequences.
void launch_group_sums(const uint16_t* x, int ldx, int K, int G, float* xs, int ldxs, const int32_t* list,
                       const int32_t* cnt, int P, int Bt, hipStream_t s);
// RoPE of q and k of every prompt row (row t * B + b: position lens[b] + t),
// q into qrot [row][H * hd], k and v into the layer's cache slots.
void launch_rope_kv(const uint16_t* qkv, int P, int B, int H, int Hkv, int hd, const float* cosT,
                    const float* sinT, const int32_t* lens, uint16_t* qrot, uint16_t* Kl, uint16_t* Vl,
                    uint8_t* occ_l, int S, hipStream_t s);
// Causal attention of every prompt row over the layer's cache (positions
// 0..lens[b] + t), out [row][H * hd] bf16.
void launch_prefill_attention(const uint16_t* q, const uint16_t* K, const uint16_t* V, int S, int P, int B, int H,
                              int Hkv, int hd, const int32_t* lens, uint16_t* out, hipStream_t s);
// Embedding rows of every prompt row into h, the first layer's RMSNorm into
// x, and the step state's row lists reset.
void launch_prefill_embed(StepState* st, const int32_t* prompt, int P, int B, int L, const uint16_t* emb, int d,
                          int V, float* h, const uint16_t* gain, float eps, uint16_t* x, hipStream_t s);

// launchers (ee_kernels.hip)
// Whether min(8, batch) input rows of width K fit the projection's LDS stage.
bool proj_fits(int K, int batch);
// Launches a projection over `batch` rows.  EPI_PART picks its column ranges
// (a.nkc, a.kc) and returns their count; the other epilogues need
// proj_fits(K, batch).
// With ev0/ev1 set, the launch records its own start and end into them.
int launch_proj(int epi, const ProjArgs& a, int nwg, int batch, hipStream_t s, hipEvent_t ev0 = nullptr,
                hipEvent_t ev1 = nullptr);
// Device address of an all-zero row list on the current device (stands in for
// an absent list); resolved on first call per device, before any capture.
const int32_t* no_rows();
// The column ranges EPI_PART uses for K columns, N rows (and their width).
int proj_ranges(int K, int N, int nwg, int batch, int* kc);
// h[b] = hsrc[b] + sum_c parts[c][b] for b < B (hsrc may be h; nparts may be
// 0); then x[b] = bf16(rmsnorm(h[b]) * gain), and when hb is set,
// hb[b] = bf16(h[b]).  With hin and sts both set, sts[b] = cos(hin[b], h[b])
// (hin may be h: each element is read before it is overwritten).
void launch_finish(float* h, const float* hsrc, const float* parts, int nparts, size_t cstride, int B, int d,
                   const uint16_t* gain, float eps, uint16_t* x, uint16_t* hb, const float* hin, float* sts,
                   hipStream_t s);
// Step setup: h[b] = embedding of the input token, x[b] = bf16(rmsnorm(h[b]) *
// gain) (the first layer's attention input), exit state and row lists reset.
void launch_init(StepState* st, const int32_t* prompt, int P, int t, int B, int L,
                 const uint16_t* emb, int d, int V, float* h, float* p_rec, const uint16_t* gain,
                 float eps, uint16_t* x, hipStream_t s);
// p[0..n) = v (32-bit words), by a kernel.
void launch_fill_u32(uint32_t* p, size_t n, uint32_t v, hipStream_t s);
void launch_attention(const AttnArgs& a, hipStream_t s);
// Vocabulary GEMVs (EPI_LSE / EPI_ARGMAX) on MFMA for steps of more than 8
// rows (ee_wide.hip): E read once for up to 64 rows from a tiled copy made by
// launch_tile_vocab (wide_vocab_elems(V, d) bf16), whatever the device-side
// row count (nothing is done when it is 0).  Writes nwg partials per row like
// launch_proj; with events set, the launch records its start and end.
bool wide_vocab_supported(int d);
size_t wide_vocab_elems(int V, int d);
void launch_tile_vocab(const uint16_t* E, int V, int d, uint16_t* Et, hipStream_t s);
void launch_wide_vocab(int epi, const ProjArgs& a, int nwg, hipStream_t s, hipEvent_t ev_start = nullptr,
                       hipEvent_t ev_end = nullptr);
// The tiled order of a bf16 matrix [N][K] (K a multiple of 256; rows padded to
// 16 with zeros): the 1 KB A operand of each 16-row tile and 32-column step
// contiguous.  Segments of a multi-part matrix (QKV, gate/up) are tiled one
// after the other (each a multiple of 16 rows): dst is the segment's first row.
void launch_tile_rows(const uint16_t* W, int N, int K, uint16_t* dst, hipStream_t s);
// gate/up [F][K] each into F / 8 tiles of 8 gate rows and the same 8 up rows
void launch_tile_pair_rows(const uint16_t* gate, const uint16_t* up, int F, int K, uint16_t* dst, hipStream_t s);
// Column ranges of a wide projection (N rows, K columns): count and width.
int wide_ranges(int N, int K, int* kr);
// Partial sums of a wide projection over a.nr ranges (set a.nr, a.kr with
// wide_ranges); int4 pass only when a.q4[0] is set.
void launch_wide_proj(WideArgs a, hipStream_t s);
// Epilogues of a wide projection over the rows of list/cnt: the sum of the
// ranges, then RoPE and the shared-slot K/V write (QKV, ProjArgs as for
// EPI_QKV), SwiGLU of the gate/up pairs (the tile order of a WideArgs pair) into
// out [seq][F], or bf16 into out.
void launch_wide_qkv(const float* y, int nr, size_t cstride, int ystride, const int32_t* list,
                     const int32_t* cnt, int B, const ProjArgs& qa, hipStream_t s);
void launch_wide_swiglu(const float* y, int nr, size_t cstride, int ystride, const int32_t* list,
                        const int32_t* cnt, int B, int F, uint16_t* out, hipStream_t s);
void launch_wide_bf16(const float* y, int nr, size_t cstride, int ystride, const int32_t* list,
                      const int32_t* cnt, int B, int N, uint16_t* out, int out_stride, hipStream_t s);
// Exit decision after layer `layer` for the rows on the backbone: from the exit
// head's nwg (max, sum exp) partials (DECIDE_HEAD), from the state transition
// similarity per sequence in sts (DECIDE_STS), or forced exits only, no
// criterion (DECIDE_FORCED, between check layers).  batch_min: the unforced
// rows leave together when the smallest of their values exceeds the threshold.
enum DecideMode { DECIDE_HEAD = 0, DECIDE_STS = 1, DECIDE_FORCED = 2 };
void launch_decide(int mode, bool batch_min, StepState* st, const float* part, int nwg, const float* gamma,
                   int layer, int L, int B, float* p_rec, const float* sts, hipStream_t s);
void launch_final(StepState* st, const float* part, int nwg, int B, int V, int32_t* lens, int advance,
                  hipStream_t s);
// Sampled decoding (ee_sample.hip).  After the decision at an exit-head layer:
// the draft of every sequence that exited at this layer (merged from the
// EPI_LSE_S partials) and its z row copied to zx [b][d].  After the LM head's
// EPI_ARGMAX_S pass: the emitted token of each sequence (the final
// distribution's draw without a draft; the draft if accepted) and the list of
// rejected ones.  After the EPI_RESAMPLE pass: their tokens; then every
// length advances.
void launch_sample_draft(StepState* st, const float* part_s, int nwg, int layer, int B, const uint16_t* z,
                         uint16_t* zx, int d, hipStream_t s);
void launch_sample_final(StepState* st, const float* part_s, int nwg, int B, int L, int V, const int32_t* lens,
                         float itau, uint32_t seed, hipStream_t s);
void launch_resample_final(StepState* st, const float* part_s, int nwg, int B, int V, int32_t* lens,
                           hipStream_t s);
void launch_advance(int32_t* lens, int B, hipStream_t s, int delta = 1);
// out[b] = min over t < P of sts[t * B + b]: each sequence's smallest
// similarity over its prompt's tokens (the prefill's sequence-level exit).
void launch_sts_min(const float* sts, int P, int B, float* out, hipStream_t s);
void launch_quantize(const uint16_t* w, int N, int K, int G, int row0, uint32_t* codes,
                     uint16_t* scales, hipStream_t s);
void launch_unpack(const uint32_t* codes, const uint16_t* scales, int K, int G, int row0, int nrows,
                   int8_t* out, uint16_t* sout, hipStream_t s);

}  // namespace ee
