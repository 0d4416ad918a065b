// Host side of libee: model and KV-cache management, the per-step launch
// schedule, argument validation and the C ABI declared in include/ee.h.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdio>
#include <cstring>
#include <exception>
#include <map>
#include <new>
#include <string>
#include <tuple>
#include <type_traits>
#include <vector>

#include "ee.h"
#include "ee_internal.h"

using namespace ee;

// Device memory of ee_decode_step_static: the step's workspaces for callers
// that cannot allocate (kScratchBytes per device, held until the process
// ends).  Host code never uses this name as an address: the per-device
// address comes from hipGetSymbolAddress (g_scratch below).
constexpr size_t kScratchBytes = (size_t)32 << 20;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

namespace {

thread_local std::string g_err;

constexpr int kMaxDevices = 64;
char* g_scratch[kMaxDevices] = {};  // device address of `scratch` per device (resolved by ee_create_model)

struct Error {
  ee_status code;
  std::string msg;
};

[[noreturn]] void fail(ee_status code, const std::string& msg) { throw Error{code, msg}; }

#define HIPCHK(expr)                                                                       \
  do {                                                                                     \
    hipError_t e_ = (expr);                                                                \
    if (e_ != hipSuccess)                                                                  \
      fail(EE_ERR_HIP, std::string(#expr) + ": " + hipGetErrorString(e_));                 \
  } while (0)

template <typename T>
T* dalloc(size_t n) {
  void* p = nullptr;
  if (n == 0) n = 1;
  if (hipMalloc(&p, n * sizeof(T)) != hipSuccess) {
    (void)hipGetLastError();
    fail(EE_ERR_OUT_OF_MEMORY, "hipMalloc of " + std::to_string(n * sizeof(T)) + " bytes failed");
  }
  return (T*)p;
}

// Device memory held for the length of one call, freed on every exit path
// (hipFree waits for the work queued on it).
template <typename T>
struct CallBuffer {
  T* p = nullptr;
  explicit CallBuffer(size_t n) : p(dalloc<T>(n)) {}
  ~CallBuffer() {
    if (p) (void)hipFree(p);
  }
  CallBuffer(const CallBuffer&) = delete;
  CallBuffer& operator=(const CallBuffer&) = delete;
};

struct Q4 {
  uint32_t* codes = nullptr;
  uint16_t* scales = nullptr;
  int N = 0, K = 0;
};

struct LayerQ {
  Q4 qkv, o, gate, up, down;
};

constexpr int kNwg = 512;  // projection workgroups (2 per CU)

// Workgroups of an 8-row vocabulary pass over V rows: the fewest that keep
// the rounds of 2-row wave tiles the full grid would take, so that every wave
// takes the same number of tiles (V = 128256: 501 workgroups, 16 tiles each).
int vocab_nwg(int V) {
  constexpr int waves = kProjThreads / 64;
  const int tiles = (V + 1) / 2;
  const int rounds = (tiles + kNwg * waves - 1) / (kNwg * waves);
  return std::max(1, std::min(kNwg, (tiles + rounds * waves - 1) / (rounds * waves)));
}

}  // namespace

struct ee_model {
  ee_model_config cfg{};
  const uint16_t *tok_emb = nullptr, *lm_head = nullptr, *final_norm = nullptr;
  std::vector<ee_layer_weights> lw;
  std::vector<LayerQ> lq;  // index l-1; layer 1 has no copy
  std::vector<float> gamma;
  float* d_gamma = nullptr;
  float *d_cos = nullptr, *d_sin = nullptr;
  // workspaces
  float* h = nullptr;      // float32 residual [b][d]
  float* parts = nullptr;  // partial sums of the column ranges of O / down [range][b][d]
  int nkc_max = 1;
  uint16_t *xn = nullptr;  // bf16 RMSNorm of the residual, the next projection's input [b][d]
  uint16_t *hb = nullptr;  // bf16(h), the exit head's input [b][d]
  uint16_t *qrot = nullptr, *attn_o = nullptr;
  uint16_t *act = nullptr, *z = nullptr;
  float* head_part = nullptr;
  float* part_s = nullptr;  // sampled decoding: partials by sequence [kNwg][64][kPartS]
  uint16_t* lm_head_t = nullptr;  // E in the wide vocabulary pass's tiled order (max_batch > 8), else null
  // projections for more than 8 rows on matrix cores: each layer's bf16
  // weights in the tiled order (QKV, O, gate then up, down, the head's T)
  struct WideW {
    uint16_t *qkv = nullptr, *o = nullptr, *gu = nullptr, *down = nullptr, *T = nullptr;
  };
  bool wide = false;
  std::vector<WideW> ww;
  float* wide_y = nullptr;  // partial sums of the wide QKV, gate/up and T projections
  float* h2 = nullptr;   // residual after attention while the layer's input is kept in h (EE_CRIT_STS) [b][d]
  float* sts = nullptr;  // state transition similarity per sequence [64]
  float* attn_part = nullptr;
  int nch_max = 0;
  StepState* st = nullptr;
  float* p_rec = nullptr;
  float* dbg_logits = nullptr;
  float* dbg_hidden = nullptr;
  int32_t* d_prompt = nullptr;
  size_t prompt_cap = 0;
  // pinned host staging
  int32_t* h_in = nullptr;   // tok[64], forced[64]
  float* h_gamma = nullptr;  // [L-1]
  int32_t* h_out = nullptr;  // out_tok[64], e[64]
  float* h_gap = nullptr;
  hipStream_t own = nullptr;
  int device = 0;  // the HIP device the model was created on
  bool broken = false;
  std::string broken_msg;
  // profiling
  bool prof = false;
  std::vector<hipEvent_t> ev_pool;
  size_t ev_used = 0;
  int64_t prof_launches = 0;
  double prof_ms = 0.0;
  int ncaches = 0;
  // decode steps captured once per (cache, batch) and replayed
  struct StepGraph {
    const ee_kv_cache* c;
    int B;
    hipGraphExec_t exec;
  };
  std::vector<StepGraph> graphs;

  std::vector<void*> allocs;

  template <typename T>
  T* alloc(size_t n) {
    T* p = dalloc<T>(n);
    allocs.push_back(p);
    return p;
  }
};

struct ee_kv_cache {
  ee_model* m = nullptr;
  int Bmax = 0, S = 0;
  uint16_t *K = nullptr, *V = nullptr;
  int32_t* lens = nullptr;      // device [Bmax]
  int32_t* next_tok = nullptr;  // device [Bmax]: each sequence's last output token, its next input
  uint8_t* occ = nullptr;
  std::vector<int32_t> hlens;
  std::vector<uint8_t> next_ok;  // whether next_tok[b] is the token after the sequence's last position
  void* owned = nullptr;
};

namespace {

template <typename F>
ee_status guard(F&& f) {
  try {
    f();
    g_err.clear();
    return EE_OK;
  } catch (const Error& e) {
    g_err = e.msg;
    return e.code;
  } catch (const std::bad_alloc&) {
    g_err = "host allocation failed";
    return EE_ERR_OUT_OF_MEMORY;
  } catch (const std::exception& e) {
    g_err = e.what();
    return EE_ERR_INVALID_ARG;
  } catch (...) {
    g_err = "unknown error";
    return EE_ERR_INVALID_ARG;
  }
}

void check_model(const ee_model* m) {
  if (!m) fail(EE_ERR_INVALID_ARG, "null model");
  if (m->broken) fail(EE_ERR_HIP, "model is unusable after an earlier HIP error: " + m->broken_msg);
}

// Runs f; a HIP failure marks the model unusable (sticky).
template <typename F>
void with_sticky(ee_model* m, F&& f) {
  try {
    f();
  } catch (const Error& e) {
    if (e.code == EE_ERR_HIP) {
      m->broken = true;
      m->broken_msg = e.msg;
    }
    throw;
  }
}

void validate_config(const ee_model_config& c) {
  auto need = [](bool ok, const char* what) {
    if (!ok) fail(EE_ERR_INVALID_ARG, what);
  };
  auto shape = [](bool ok, const char* what) {
    if (!ok) fail(EE_ERR_SHAPE, what);
  };
  need(c.n_layers >= 1, "n_layers must be >= 1");
  need(c.d_model >= 1 && c.d_ff >= 1 && c.vocab >= 1, "d_model, d_ff, vocab must be positive");
  need(c.n_heads >= 1 && c.n_kv_heads >= 1 && c.n_heads % c.n_kv_heads == 0,
       "n_heads must be a positive multiple of n_kv_heads");
  need(c.max_batch >= 1 && c.max_batch <= kMaxBatch, "max_batch must be in [1, 64]");
  need(c.max_positions >= 1, "max_positions must be >= 1");
  need(c.exit_mode == EE_EXIT_INT4 || c.exit_mode == EE_EXIT_BF16 || c.exit_mode == EE_EXIT_NONE,
       "bad exit_mode");
  need(c.criterion == EE_CRIT_HEAD || c.criterion == EE_CRIT_STS, "bad criterion");
  need(c.check_every >= 0, "check_every must be >= 0");
  need(c.exit_rule == EE_RULE_SEQUENCE || c.exit_rule == EE_RULE_BATCH_MIN, "bad exit_rule");
  need(std::isfinite(c.temperature) && c.temperature >= 0.0f, "temperature must be finite and >= 0");
  need(c.prefill_exit == 0 || c.prefill_exit == 1, "bad prefill_exit");
  if (c.prefill_exit)
    need(c.criterion == EE_CRIT_STS && c.exit_mode != EE_EXIT_NONE,
         "the prefill's sequence-level exit uses the state transition similarity and exit copies");
  if (c.temperature > 0.0f)
    need(c.exit_mode != EE_EXIT_NONE && c.criterion == EE_CRIT_HEAD && c.check_every <= 1,
         "sampled decoding drafts from the exit head evaluated after every layer");
  need(std::isfinite(c.rms_eps) && c.rms_eps > 0 && std::isfinite(c.rope_theta) && c.rope_theta > 0,
       "rms_eps and rope_theta must be positive");
  shape(c.group_size == 32 || c.group_size == 64 || c.group_size == 128, "group_size must be 32, 64 or 128");
  shape(c.head_dim == 32 || c.head_dim == 64 || c.head_dim == 128, "head_dim must be 32, 64 or 128");
  shape(c.n_heads / c.n_kv_heads <= 16, "at most 16 query heads per kv head");
  shape(c.d_model % c.group_size == 0 && c.d_ff % c.group_size == 0,
        "d_model and d_ff must be multiples of group_size");
  const int qd = c.n_heads * c.head_dim;
  shape(qd % c.group_size == 0, "n_heads * head_dim must be a multiple of group_size");
  shape(c.d_model % 8 == 0 && c.d_ff % 8 == 0, "widths must be multiples of 8");
  shape(c.d_model <= kXLdsElems / std::min(8, c.max_batch),
        "d_model too wide for the projections' staged inputs at this max_batch");
  shape(c.d_model % 32 == 0 && c.d_ff % 32 == 0, "widths must be multiples of 32");
}

hipStream_t pick_stream(ee_model* m, void* s) { return s ? (hipStream_t)s : m->own; }

// Events for the profiled launches: the launch itself records its start and
// end into them (hipExtLaunchKernel), so they time the kernel alone.
void prof_events(ee_model* m, hipEvent_t* e0, hipEvent_t* e1) {
  *e0 = *e1 = nullptr;
  if (!m->prof) return;
  if (m->ev_used + 2 > m->ev_pool.size()) {
    for (int i = 0; i < 64; ++i) {
      hipEvent_t e;
      HIPCHK(hipEventCreate(&e));
      m->ev_pool.push_back(e);
    }
  }
  *e0 = m->ev_pool[m->ev_used++];
  *e1 = m->ev_pool[m->ev_used++];
}

void prof_collect(ee_model* m) {
  if (!m->prof) return;
  for (size_t i = 0; i + 1 < m->ev_used; i += 2) {
    float ms = 0;
    HIPCHK(hipEventElapsedTime(&ms, m->ev_pool[i], m->ev_pool[i + 1]));
    m->prof_ms += ms;
    m->prof_launches += 1;
  }
  m->ev_used = 0;
}

ProjArgs base_args(const ee_model* m) {
  ProjArgs a{};
  a.G = m->cfg.group_size;
  a.nseg = 1;
  return a;
}

void set_seg1(ProjArgs& a, const void* w, int N) {
  a.nseg = 1;
  a.wb[0] = (const uint16_t*)w;
  a.wb[1] = a.wb[2] = nullptr;
  a.seg_end[0] = a.seg_end[1] = a.seg_end[2] = N;
}

// Attention work split: one wave per run of `tpw` 64-position tiles of a
// (sequence, kv head); tpw grows with the context so that the launch keeps
// about kAttnWaves waves (and its partials stay a few percent of the K/V bytes).
constexpr long long kAttnWaves = 2048;
void attn_split(int S, int B, int Hkv, int* tpw, int* nch) {
  const int tiles = (S + 63) / 64;
  int t = 1;
  while (t < tiles && (long long)B * Hkv * ((tiles + t - 1) / t) > kAttnWaves) t *= 2;
  *tpw = t;
  *nch = (tiles + t - 1) / t;
}

// Device workspaces of the step's kernels: the residual, the staged inputs
// of the projections, partial sums, attention partials, the exit heads'
// partials and the step state.  The model owns one set (allocated by
// ee_create_model); ee_decode_step_static carves one out of the static scratch
// array instead.
struct Work {
  float* h = nullptr;          // float32 residual [64][d]
  float* parts = nullptr;      // O / down partial sums [ranges][64][d]
  uint16_t* xn = nullptr;      // normalised input of the next projection [2 * 64][d]
  uint16_t* hb = nullptr;      // bf16(h), the exit head's input [64][d]
  uint16_t* qrot = nullptr;    // rotated q [64][H * hd]
  uint16_t* attn_o = nullptr;  // attention output [64][H * hd]
  uint16_t* act = nullptr;     // SwiGLU output [64][F]
  uint16_t* z = nullptr;       // exit head's bf16(T h) [64][d]
  float* head_part = nullptr;  // vocabulary partials [512][64][4]
  float* part_s = nullptr;     // sampled partials [512][64][kPartS]
  float* h2 = nullptr;         // residual after attention (similarity criterion) [64][d]
  float* sts = nullptr;        // similarity per sequence [64]
  float* attn_part = nullptr;  // attention partials [B][H][nch][hd + 2]
  StepState* st = nullptr;
  float* p_rec = nullptr;      // criterion values [L - 1][64]
  float* d_gamma = nullptr;    // thresholds [L - 1]
  float* wide_y = nullptr;     // wide projections' partial sums
  bool prof = true;            // profiled launches may record events
};

Work model_work(const ee_model* m) {
  Work w;
  w.h = m->h;
  w.parts = m->parts;
  w.xn = m->xn;
  w.hb = m->hb;
  w.qrot = m->qrot;
  w.attn_o = m->attn_o;
  w.act = m->act;
  w.z = m->z;
  w.head_part = m->head_part;
  w.part_s = m->part_s;
  w.h2 = m->h2;
  w.sts = m->sts;
  w.attn_part = m->attn_part;
  w.st = m->st;
  w.p_rec = m->p_rec;
  w.d_gamma = m->d_gamma;
  w.wide_y = m->wide_y;
  return w;
}

// Bytes of the step's workspaces for B rows over a cache of S positions (the
// sizes the model allocates for itself, attention partials for this S and B),
// each aligned to 256 bytes; with base set, w's pointers are placed from base.
size_t work_layout(const ee_model* m, int B, int S, char* base, Work* w) {
  const ee_model_config& c = m->cfg;
  const int L = c.n_layers, d = c.d_model, F = c.d_ff, qd = c.n_heads * c.head_dim, kvd = c.n_kv_heads * c.head_dim;
  size_t off = 0;
  auto take = [&](auto*& p, size_t bytes) {
    off = (off + 255) & ~(size_t)255;
    p = base ? reinterpret_cast<std::remove_reference_t<decltype(p)>>(base + off) : nullptr;
    off += std::max<size_t>(bytes, 4);
  };
  const size_t Bm = kMaxBatch;
  take(w->h, Bm * d * 4);
  take(w->parts, (size_t)m->nkc_max * Bm * d * 4);
  take(w->xn, 2 * Bm * d * 2);
  take(w->hb, Bm * d * 2);
  take(w->qrot, Bm * qd * 2);
  take(w->attn_o, Bm * qd * 2);
  take(w->act, Bm * F * 2);
  take(w->z, Bm * d * 2);
  take(w->head_part, (size_t)kNwg * Bm * 4 * 4);
  if (c.temperature > 0.0f) take(w->part_s, (size_t)kNwg * Bm * kPartS * 4);
  if (c.criterion == EE_CRIT_STS) {
    take(w->h2, Bm * d * 4);
    take(w->sts, Bm * 4);
  }
  int tpw = 0, nch = 0;
  attn_split(S, B, c.n_kv_heads, &tpw, &nch);
  take(w->attn_part, (size_t)B * c.n_heads * nch * (c.head_dim + 2) * 4);
  take(w->st, sizeof(StepState));
  take(w->p_rec, (size_t)std::max(L - 1, 1) * Bm * 4);
  take(w->d_gamma, (size_t)std::max(L - 1, 1) * 4);
  if (m->wide && B > 8) {
    const size_t yq = (size_t)wide_ranges(qd + 2 * kvd, d, nullptr) * Bm * (qd + 2 * kvd);
    const size_t yg = (size_t)wide_ranges(2 * F, d, nullptr) * Bm * 2 * F;
    const size_t yt = (size_t)wide_ranges(d, d, nullptr) * Bm * d;
    take(w->wide_y, std::max(yq, std::max(yg, yt)) * 4);
  }
  return (off + 255) & ~(size_t)255;
}

struct Debug {
  bool hidden = false, logits = false;
};

// Enqueues one decode step of all B sequences: layers 1..L, exit heads when
// heads is set, and the final head when final is set (else the lengths advance).
void enqueue_position(ee_model* m, const Work& W, ee_kv_cache* c, int B, bool heads, bool final,
                      const int32_t* prompt, int P, int t, const Debug& dbg, hipStream_t s) {
  const ee_model_config& cf = m->cfg;
  const int L = cf.n_layers, d = cf.d_model, F = cf.d_ff, H = cf.n_heads, Hkv = cf.n_kv_heads;
  const int hd = cf.head_dim, qd = H * hd, kvd = Hkv * hd, nqkv = qd + 2 * kvd;
  StepState* st = W.st;
  const bool int4 = cf.exit_mode == EE_EXIT_INT4;
  heads = heads && cf.exit_mode != EE_EXIT_NONE;  // the plain decoder evaluates no criterion
  const bool sts_crit = cf.criterion == EE_CRIT_STS;
  const int every = std::max(1, cf.check_every);
  // sampled decoding (decode steps only; the prefill's token stays greedy)
  const bool sampled = heads && cf.temperature > 0.0f;
  // vocabulary passes: batches above 8 run the wide pass (a full grid of
  // partials); otherwise the 8-row pass on a grid of equal rounds
  const bool wide_vocab = m->lm_head_t && B > 8;
  const int nv = wide_vocab ? kNwg : vocab_nwg(cf.vocab);
  const float itau = sampled ? 1.0f / cf.temperature : 0.0f;
  auto sampled_args = [&](ProjArgs& a) {
    a.part_s = W.part_s;
    a.itau = itau;
    a.seed = cf.sample_seed;
    a.lens = c->lens;
    a.st = st;
  };

  const size_t pstride = (size_t)kMaxBatch * d;  // elements between partial-sum ranges
  float* hh = W.h;        // residual [b][d]
  uint16_t* xn = W.xn;    // the next projection's normalised input [b][d]
  launch_init(st, prompt, P, t, B, L, m->tok_emb, d, cf.vocab, hh, W.p_rec,
              (const uint16_t*)m->lw[0].attn_norm, cf.rms_eps, xn, s);
  if (dbg.hidden)
    HIPCHK(hipMemcpy2DAsync(m->dbg_hidden, (size_t)(L + 1) * d * 4, hh, (size_t)d * 4,
                            (size_t)d * 4, B, hipMemcpyDeviceToDevice, s));
  // row lists: backbone rows run the bf16 weights, exited rows the int4 copy;
  // with unquantised exit copies every row runs the bf16 weights.
  const int32_t* list_bf = int4 ? st->act : st->all;
  const int32_t* cnt_bf = int4 ? &st->n_act : &st->n_all;
  // more than 8 rows: every projection on matrix cores (weights read once for
  // all rows), float32 partial sums over column ranges summed by an epilogue
  const bool wide = m->wide && B > 8;
  auto wide_args = [&](int N, int K, const uint16_t* wt, const uint16_t* x, int x_stride, float* y, int ystride) {
    WideArgs wa{};
    wa.N = N;
    wa.K = K;
    wa.nr = wide_ranges(N, K, &wa.kr);
    wa.wt = wt;
    wa.x = x;
    wa.x_stride = x_stride;
    wa.list_bf = list_bf;
    wa.cnt_bf = cnt_bf;
    wa.y = y;
    wa.y_stride = ystride;
    wa.y_cstride = (size_t)kMaxBatch * ystride;
    wa.G = cf.group_size;
    wa.n0 = N;
    return wa;
  };
  auto wide_i4 = [&](WideArgs& wa, const Q4& q0) {
    wa.q4[0] = q0.codes;
    wa.s4[0] = q0.scales;
    wa.list_i4 = st->ex;
    wa.cnt_i4 = &st->n_ex;
  };

  for (int l = 1; l <= L; ++l) {
    const ee_layer_weights& w = m->lw[l - 1];
    const LayerQ* q = (int4 && l >= 2) ? &m->lq[l - 1] : nullptr;
    const size_t kvoff = (size_t)(l - 1) * c->Bmax * Hkv * c->S * hd;

    {
      ProjArgs a = base_args(m);
      a.N = nqkv;
      a.K = d;
      a.nseg = 3;
      a.wb[0] = (const uint16_t*)w.wq;
      a.wb[1] = (const uint16_t*)w.wk;
      a.wb[2] = (const uint16_t*)w.wv;
      a.seg_end[0] = qd;
      a.seg_end[1] = qd + kvd;
      a.seg_end[2] = nqkv;
      if (q) {
        a.q4 = q->qkv.codes;
        a.s4 = q->qkv.scales;
        a.list_i4 = st->ex;
        a.cnt_i4 = &st->n_ex;
      }
      a.list_bf = list_bf;
      a.cnt_bf = cnt_bf;
      a.x = xn;  // bf16(rmsnorm(h) * attn_norm)
      a.x_stride = d;
      // epilogue: RoPE on q and k, k and v into this position's shared cache slot
      a.cosT = m->d_cos;
      a.sinT = m->d_sin;
      a.lens = c->lens;
      a.qrot = W.qrot;
      a.Kl = c->K + kvoff;
      a.Vl = c->V + kvoff;
      a.occ_l = c->occ ? c->occ + (size_t)(l - 1) * c->Bmax * c->S : nullptr;
      a.H = H;
      a.Hkv = Hkv;
      a.hd = hd;
      a.hd_log2 = __builtin_ctz(hd);
      a.S = c->S;
      if (wide) {
        WideArgs wa = wide_args(nqkv, d, m->ww[l - 1].qkv, xn, d, W.wide_y, nqkv);
        if (q) wide_i4(wa, q->qkv);
        launch_wide_proj(wa, s);
        launch_wide_qkv(W.wide_y, wa.nr, wa.y_cstride, nqkv, st->all, &st->n_all, B, a, s);
      } else {
        launch_proj(EPI_QKV, a, kNwg, B, s);
      }
    }
    {
      AttnArgs a{};
      a.q = W.qrot;
      a.K = c->K + kvoff;
      a.V = c->V + kvoff;
      a.S = c->S;
      a.Bmax = c->Bmax;
      a.lens = c->lens;
      a.H = H;
      a.Hkv = Hkv;
      a.hd = hd;
      a.B = B;
      attn_split(c->S, B, Hkv, &a.tpw, &a.nch);
      a.scale = (float)(1.0 / std::sqrt((double)hd));
      a.part = W.attn_part;
      a.out = W.attn_o;
      // one workgroup per (sequence, kv head), merged in LDS, once there are
      // enough pairs to give every CU one (measured at 64 x 8 pairs: 173
      // against 178 us with the split runs and their combine; at 8 x 8 pairs
      // the split runs are faster: 14 against 18 us)
      a.fused = (long long)B * Hkv >= 256;
      launch_attention(a, s);
    }
    {
      ProjArgs a = base_args(m);
      a.N = d;
      a.K = qd;
      set_seg1(a, w.wo, d);
      if (q) {
        a.q4 = q->o.codes;
        a.s4 = q->o.scales;
        a.list_i4 = st->ex;
        a.cnt_i4 = &st->n_ex;
      }
      a.list_bf = list_bf;
      a.cnt_bf = cnt_bf;
      a.x = W.attn_o;
      a.x_stride = qd;
      a.y = W.parts;
      a.y_stride = d;
      a.y_cstride = (int)pstride;
      int nkc;
      if (wide) {
        WideArgs wa = wide_args(d, qd, m->ww[l - 1].o, W.attn_o, qd, W.parts, d);
        if (q) wide_i4(wa, q->o);
        launch_wide_proj(wa, s);
        nkc = wa.nr;
      } else {
        nkc = launch_proj(EPI_PART, a, kNwg, B, s);
      }
      // with the similarity criterion the layer's input stays in h (the
      // residual after attention goes to h2) until the layer's end
      float* h_mid = heads && sts_crit && l < L && l % every == 0 ? W.h2 : hh;
      launch_finish(h_mid, hh, W.parts, nkc, pstride, B, d, (const uint16_t*)w.ffn_norm, cf.rms_eps, xn,
                    nullptr, nullptr, nullptr, s);
    }
    {
      ProjArgs a = base_args(m);
      a.N = F;
      a.K = d;
      set_seg1(a, w.w_gate, F);
      a.wb2 = (const uint16_t*)w.w_up;
      if (q) {
        a.q4 = q->gate.codes;
        a.s4 = q->gate.scales;
        a.q4b = q->up.codes;
        a.s4b = q->up.scales;
        a.list_i4 = st->ex;
        a.cnt_i4 = &st->n_ex;
      }
      a.list_bf = list_bf;
      a.cnt_bf = cnt_bf;
      a.x = xn;  // bf16(rmsnorm(h) * ffn_norm)
      a.x_stride = d;
      a.y = W.act;
      a.y_stride = F;
      if (wide) {  // gate and up rows paired 8 by 8 per tile (launch_tile_pair_rows)
        WideArgs wa = wide_args(2 * F, d, m->ww[l - 1].gu, xn, d, W.wide_y, 2 * F);
        wa.pair = F;
        if (q) {
          wide_i4(wa, q->gate);
          wa.q4[1] = q->up.codes;
          wa.s4[1] = q->up.scales;
          wa.n0 = F;
        }
        if (wa.nr == 1) wa.act = W.act;  // SwiGLU in the pass itself
        launch_wide_proj(wa, s);
        if (!wa.act) launch_wide_swiglu(W.wide_y, wa.nr, wa.y_cstride, 2 * F, st->all, &st->n_all, B, F, W.act, s);
      } else {
        launch_proj(EPI_SWIGLU, a, kNwg, B, s);
      }
    }
    const bool head_here = heads && l < L && l % every == 0;  // the criterion is evaluated after this layer
    const bool sts_here = head_here && sts_crit;
    {
      ProjArgs a = base_args(m);
      a.N = d;
      a.K = F;
      set_seg1(a, w.w_down, d);
      if (q) {
        a.q4 = q->down.codes;
        a.s4 = q->down.scales;
        a.list_i4 = st->ex;
        a.cnt_i4 = &st->n_ex;
      }
      a.list_bf = list_bf;
      a.cnt_bf = cnt_bf;
      a.x = W.act;
      a.x_stride = F;
      a.y = W.parts;
      a.y_stride = d;
      a.y_cstride = (int)pstride;
      int nkc;
      if (wide) {
        WideArgs wa = wide_args(d, F, m->ww[l - 1].down, W.act, F, W.parts, d);
        if (q) wide_i4(wa, q->down);
        launch_wide_proj(wa, s);
        nkc = wa.nr;
      } else {
        nkc = launch_proj(EPI_PART, a, kNwg, B, s);
      }
      // the next projection's input: the next layer's attention norm, or the
      // final norm before the LM head; bf16(h) for this layer's exit head
      const void* g_next = l < L ? m->lw[l].attn_norm : (const void*)m->final_norm;
      if (sts_here)  // h = h2 + partials; sts = cos(layer input in h, new h)
        launch_finish(hh, W.h2, W.parts, nkc, pstride, B, d, (const uint16_t*)g_next, cf.rms_eps, xn,
                      nullptr, hh, W.sts, s);
      else
        launch_finish(hh, hh, W.parts, nkc, pstride, B, d, (const uint16_t*)g_next, cf.rms_eps, xn,
                      head_here ? W.hb : nullptr, nullptr, nullptr, s);
    }
    const bool bmin = cf.exit_rule == EE_RULE_BATCH_MIN;
    if (sts_here) launch_decide(DECIDE_STS, bmin, st, nullptr, 0, W.d_gamma, l, L, B, W.p_rec, W.sts, s);
    if (heads && l < L && !head_here)  // between checks only forced exits apply
      launch_decide(DECIDE_FORCED, false, st, nullptr, 0, W.d_gamma, l, L, B, W.p_rec, nullptr, s);
    if (head_here && !sts_crit) {
      {
        ProjArgs a = base_args(m);
        a.N = d;
        a.K = d;
        set_seg1(a, w.head_T, d);
        a.list_bf = st->act;
        a.cnt_bf = &st->n_act;
        a.x = W.hb;  // bf16(h)
        a.x_stride = d;
        a.y = W.z;
        a.y_stride = d;
        if (wide && m->ww[l - 1].T) {
          WideArgs wa = wide_args(d, d, m->ww[l - 1].T, W.hb, d, W.wide_y, d);
          wa.list_bf = st->act;
          wa.cnt_bf = &st->n_act;
          launch_wide_proj(wa, s);
          launch_wide_bf16(W.wide_y, wa.nr, wa.y_cstride, d, st->act, &st->n_act, B, d, W.z, d, s);
        } else {
          launch_proj(EPI_BF16, a, kNwg, B, s);
        }
      }
      {
        ProjArgs a = base_args(m);
        a.N = cf.vocab;
        a.K = d;
        set_seg1(a, m->lm_head, cf.vocab);
        a.list_bf = st->act;
        a.cnt_bf = &st->n_act;
        a.x = W.z;
        a.x_stride = d;
        a.part = W.head_part;
        hipEvent_t e0 = nullptr, e1 = nullptr;
        if (W.prof) prof_events(m, &e0, &e1);
        // steps of more than 8 rows use the wide pass for every count of rows
        // on the backbone (one read of E for all of them; with few rows it
        // costs about what the 8-row pass does, and one launch replaces two)
        if (sampled) {  // also the draft's Gumbel-max and the tau statistics
          sampled_args(a);
          launch_proj(EPI_LSE_S, a, nv, B, s, e0, e1);
        } else if (wide_vocab) {
          a.wb[0] = m->lm_head_t;
          launch_wide_vocab(EPI_LSE, a, nv, s, e0, e1);
        } else {
          launch_proj(EPI_LSE, a, nv, B, s, e0, e1);
        }
      }
      launch_decide(DECIDE_HEAD, bmin, st, W.head_part, nv, W.d_gamma, l, L, B, W.p_rec, nullptr, s);
      if (sampled) launch_sample_draft(st, W.part_s, nv, l, B, W.z, xn + (size_t)kMaxBatch * d, d, s);
    }
    if (dbg.hidden)
      HIPCHK(hipMemcpy2DAsync(m->dbg_hidden + (size_t)l * d, (size_t)(L + 1) * d * 4, hh,
                              (size_t)d * 4, (size_t)d * 4, B, hipMemcpyDeviceToDevice, s));
  }
  if (final) {
    ProjArgs a = base_args(m);
    a.N = cf.vocab;
    a.K = d;
    set_seg1(a, m->lm_head, cf.vocab);
    a.list_bf = st->all;
    a.cnt_bf = &st->n_all;
    a.x = xn;  // bf16(rmsnorm(h) * final_norm)
    a.x_stride = d;
    a.part = W.head_part;
    a.logits = dbg.logits ? m->dbg_logits : nullptr;
    a.logits_stride = cf.vocab;
    if (sampled) {
      // the final distribution's statistics and draw, the greedy top-2 (gap),
      // the verification, then the resampling of the rejected drafts
      sampled_args(a);
      launch_proj(EPI_ARGMAX_S, a, nv, B, s);
      launch_final(st, W.head_part, nv, B, cf.vocab, c->lens, 0, s);
      launch_sample_final(st, W.part_s, nv, B, L, cf.vocab, c->lens, itau, cf.sample_seed, s);
      ProjArgs r = base_args(m);
      r.N = cf.vocab;
      r.K = d;
      set_seg1(r, m->lm_head, cf.vocab);
      r.list_bf = st->rej;  // pairs (b, 64 + b): the final input and the exit layer's z
      r.cnt_bf = &st->n_rej;
      r.x = xn;
      r.x_stride = d;
      r.part = W.head_part;
      sampled_args(r);
      launch_proj(EPI_RESAMPLE, r, nv, 2 * B, s);
      launch_resample_final(st, W.part_s, nv, B, cf.vocab, c->lens, s);
    } else {
      if (wide_vocab) {  // every row of the batch: the wide pass alone
        a.wb[0] = m->lm_head_t;
        launch_wide_vocab(EPI_ARGMAX, a, nv, s);
      } else {
        launch_proj(EPI_ARGMAX, a, nv, B, s);
      }
      launch_final(st, W.head_part, nv, B, cf.vocab, c->lens, 1, s);
    }
  } else {
    launch_advance(c->lens, B, s);
  }
  HIPCHK(hipGetLastError());
}

// The kernels of one decode step (no debug outputs) as a HIP graph, captured on
// first use for this cache and batch, then replayed: the launches' arguments
// depend only on those (every per-step value lives in device memory), so a
// replay equals the eager launches.  Profiled steps launch eagerly (the
// kernel-recorded events of the exit head are not captured into graphs).
void replay_step(ee_model* m, ee_kv_cache* c, int B, hipStream_t s) {
  if (m->prof) {
    enqueue_position(m, model_work(m), c, B, true, true, nullptr, 1, 0, Debug{}, s);
    return;
  }

  ee_model::StepGraph* g = nullptr;
  for (auto& e : m->graphs)
    if (e.c == c && e.B == B) g = &e;
  if (!g) {
    hipGraph_t graph = nullptr;
    HIPCHK(hipStreamBeginCapture(s, hipStreamCaptureModeThreadLocal));
    bool ok = true;
    try {
      enqueue_position(m, model_work(m), c, B, true, true, nullptr, 1, 0, Debug{}, s);
    } catch (const Error&) {
      ok = false;
    }
    const hipError_t ec = hipStreamEndCapture(s, &graph);
    hipGraphExec_t exec = nullptr;
    if (ok && ec == hipSuccess && graph) ok = hipGraphInstantiate(&exec, graph, nullptr, nullptr, 0) == hipSuccess;
    else ok = false;
    if (graph) (void)hipGraphDestroy(graph);
    (void)hipGetLastError();
    if (!ok) fail(EE_ERR_HIP, "capturing the decode step failed");
    m->graphs.push_back({c, B, exec});
    g = &m->graphs.back();
  }
  HIPCHK(hipGraphLaunch(g->exec, s));
}

void drop_graphs(ee_model* m, const ee_kv_cache* c) {
  for (size_t i = 0; i < m->graphs.size();) {
    if (!c || m->graphs[i].c == c) {
      (void)hipGraphExecDestroy(m->graphs[i].exec);
      m->graphs.erase(m->graphs.begin() + i);
    } else {
      ++i;
    }
  }
}

void free_model(ee_model* m) {
  if (!m) return;
  drop_graphs(m, nullptr);
  for (void* p : m->allocs) (void)hipFree(p);
  for (hipEvent_t e : m->ev_pool) (void)hipEventDestroy(e);
  if (m->h_in) (void)hipHostFree(m->h_in);
  if (m->h_gamma) (void)hipHostFree(m->h_gamma);
  if (m->h_out) (void)hipHostFree(m->h_out);
  if (m->h_gap) (void)hipHostFree(m->h_gap);
  if (m->own) (void)hipStreamDestroy(m->own);
  delete m;
}

template <typename T>
T* halloc(size_t n) {
  void* p = nullptr;
  if (hipHostMalloc(&p, std::max<size_t>(n, 1) * sizeof(T), hipHostMallocDefault) != hipSuccess) {
    (void)hipGetLastError();
    fail(EE_ERR_OUT_OF_MEMORY, "pinned host allocation failed");
  }
  return (T*)p;
}

// The prefill of P positions of sequences 0..B-1 ("River-LLM 深度解析", section
// 6.1), layer by layer over all B * P positions at once: every projection is
// one matrix-core GEMM over the rows of the sequences on the backbone (bf16
// weights) and one over the rows of the exited sequences (int4 copies; only
// with the sequence-level exit), RoPE writes each position's k and v into its
// shared slot, causal attention reads the slots.  With prefill_exit, after
// layer l < L a sequence leaves when the smallest state transition similarity
// of its prompt's tokens exceeds tau_l (River-LLM, sections 6.1 and 5.2).
// Rows are position-major (t * B + b).  The greedy token of each sequence's
// last position, and its logits when asked, go to the step state / debug
// buffer; the lengths advance by P.  Per-call buffers of B * P rows.
void run_prefill(ee_model* m, ee_kv_cache* c, int B, int P, bool want_logits, hipStream_t s) {
  const ee_model_config& cf = m->cfg;
  const int L = cf.n_layers, d = cf.d_model, F = cf.d_ff, H = cf.n_heads, Hkv = cf.n_kv_heads;
  const int hd = cf.head_dim, qd = H * hd, kvd = Hkv * hd, nqkv = qd + 2 * kvd, G = cf.group_size;
  const bool int4 = cf.exit_mode == EE_EXIT_INT4;
  const bool pexit = cf.prefill_exit && L > 1;
  const bool w4 = pexit && int4;  // exited sequences run the int4 copies
  const int R = P * B;
  const int ngr_max = std::max(d, std::max(qd, F)) / G;
  CallBuffer<float> hA((size_t)R * d), hB((size_t)R * d), aux(pexit ? (size_t)R + kMaxBatch : 1),
      xs(w4 ? (size_t)R * ngr_max : 1);
  CallBuffer<uint16_t> xn((size_t)R * d), qkv((size_t)R * nqkv), qrot((size_t)R * qd), ao((size_t)R * qd),
      act((size_t)R * F);
  StepState* st = m->st;
  launch_prefill_embed(st, m->d_prompt, P, B, L, m->tok_emb, d, cf.vocab, hA.p,
                       (const uint16_t*)m->lw[0].attn_norm, cf.rms_eps, xn.p, s);
  const int32_t* list_bf = int4 ? st->act : st->all;
  const int32_t* cnt_bf = int4 ? &st->n_act : &st->n_all;
  float *h_in = hA.p, *h_out = hB.p;
  auto gemm = [&](int epi, const GemmArgs& g0, const Q4* qa, const Q4* qb, const uint16_t* x, int K) {
    GemmArgs g = g0;
    g.K = K;
    g.G = G;
    g.x = x;
    g.ldx = K;
    g.P = P;
    g.Bt = B;
    g.list = list_bf;
    g.cnt = cnt_bf;
    launch_gemm(epi, false, g, R, s);
    if (qa) {  // the exited sequences' rows on the int4 copy
      launch_group_sums(x, K, K, G, xs.p, ngr_max, st->ex, &st->n_ex, P, B, s);
      g.q4 = qa->codes;
      g.s4 = qa->scales;
      if (qb) {
        g.q4b = qb->codes;
        g.s4b = qb->scales;
      }
      g.xs = xs.p;
      g.ldxs = ngr_max;
      g.list = st->ex;
      g.cnt = &st->n_ex;
      launch_gemm(epi, true, g, R, s);
    }
  };
  for (int l = 1; l <= L; ++l) {
    const ee_layer_weights& w = m->lw[l - 1];
    const LayerQ* q = (w4 && l >= 2) ? &m->lq[l - 1] : nullptr;
    const size_t kvoff = (size_t)(l - 1) * c->Bmax * Hkv * c->S * hd;
    uint16_t* Kl = c->K + kvoff;
    uint16_t* Vl = c->V + kvoff;
    {  // QKV into bf16(W x), then RoPE and the shared-slot K/V write
      GemmArgs g{};
      g.N = nqkv;
      g.nseg = 3;
      g.wb[0] = (const uint16_t*)w.wq;
      g.wb[1] = (const uint16_t*)w.wk;
      g.wb[2] = (const uint16_t*)w.wv;
      g.seg_end[0] = qd;
      g.seg_end[1] = qd + kvd;
      g.seg_end[2] = nqkv;
      g.ob = qkv.p;
      g.ldo = nqkv;
      gemm(GEPI_BF16, g, q ? &q->qkv : nullptr, nullptr, xn.p, d);
      launch_rope_kv(qkv.p, P, B, H, Hkv, hd, m->d_cos, m->d_sin, c->lens, qrot.p, Kl, Vl,
                     c->occ ? c->occ + (size_t)(l - 1) * c->Bmax * c->S : nullptr, c->S, s);
    }
    launch_prefill_attention(qrot.p, Kl, Vl, c->S, P, B, H, Hkv, hd, c->lens, ao.p, s);
    {  // h_out = h_in + W_o o, then the FFN's RMSNorm
      GemmArgs g{};
      g.N = d;
      g.nseg = 1;
      g.wb[0] = (const uint16_t*)w.wo;
      g.seg_end[0] = g.seg_end[1] = g.seg_end[2] = d;
      g.of = h_out;
      g.src = h_in;
      g.ldf = d;
      gemm(GEPI_RESID, g, q ? &q->o : nullptr, nullptr, ao.p, qd);
      launch_finish(h_out, h_out, nullptr, 0, 0, R, d, (const uint16_t*)w.ffn_norm, cf.rms_eps, xn.p, nullptr,
                    nullptr, nullptr, s);
    }
    {  // gate and up with SwiGLU
      GemmArgs g{};
      g.N = F;
      g.nseg = 1;
      g.wb[0] = (const uint16_t*)w.w_gate;
      g.wb2 = (const uint16_t*)w.w_up;
      g.seg_end[0] = g.seg_end[1] = g.seg_end[2] = F;
      g.ob = act.p;
      g.ldo = F;
      gemm(GEPI_SWIGLU, g, q ? &q->gate : nullptr, q ? &q->up : nullptr, xn.p, d);
    }
    {  // h_out += W_d a, then the next norm (and the layer's similarity with the exit)
      GemmArgs g{};
      g.N = d;
      g.nseg = 1;
      g.wb[0] = (const uint16_t*)w.w_down;
      g.seg_end[0] = g.seg_end[1] = g.seg_end[2] = d;
      g.of = h_out;
      g.src = h_out;
      g.ldf = d;
      gemm(GEPI_RESID, g, q ? &q->down : nullptr, nullptr, act.p, F);
      const uint16_t* g_next = (const uint16_t*)(l < L ? m->lw[l].attn_norm : (const void*)m->final_norm);
      if (pexit && l < L) {
        float* sts = aux.p;
        float* smin = aux.p + R;
        launch_finish(h_out, h_out, nullptr, 0, 0, R, d, g_next, cf.rms_eps, xn.p, nullptr, h_in, sts, s);
        launch_sts_min(sts, P, B, smin, s);
        launch_decide(DECIDE_STS, false, st, nullptr, 0, m->d_gamma, l, L, B, nullptr, smin, s);
      } else {
        launch_finish(h_out, h_out, nullptr, 0, 0, R, d, g_next, cf.rms_eps, xn.p, nullptr, nullptr, nullptr, s);
      }
    }
    std::swap(h_in, h_out);
  }
  // the final head on each sequence's last position (rows (P - 1) * B + b)
  ProjArgs a = base_args(m);
  a.N = cf.vocab;
  a.K = d;
  set_seg1(a, m->lm_head, cf.vocab);
  a.list_bf = st->all;
  a.cnt_bf = &st->n_all;
  a.x = xn.p + (size_t)(P - 1) * B * d;
  a.x_stride = d;
  a.part = m->head_part;
  a.logits = want_logits ? m->dbg_logits : nullptr;
  a.logits_stride = cf.vocab;
  const bool wide_vocab = m->lm_head_t && B > 8;
  const int nv = wide_vocab ? kNwg : vocab_nwg(cf.vocab);
  if (wide_vocab) {
    a.wb[0] = m->lm_head_t;
    launch_wide_vocab(EPI_ARGMAX, a, nv, s);
  } else {
    launch_proj(EPI_ARGMAX, a, nv, B, s);
  }
  launch_final(st, m->head_part, nv, B, cf.vocab, c->lens, 1, s);
  if (P > 1) launch_advance(c->lens, B, s, P - 1);
  // the per-call buffers are freed when this returns: finish the work first
  HIPCHK(hipStreamSynchronize(s));
}

// Host-side checks of a decode step's arguments (no state changes).
void validate_step(ee_model* m, ee_kv_cache* c, int batch, const int32_t* in_tokens_host,
                   const int32_t* forced_exit_host, const float* gamma_host, const int32_t* out_tokens_host,
                   const int32_t* out_exit_layers_host) {
  check_model(m);
  if (!c || c->m != m) fail(EE_ERR_INVALID_ARG, "cache does not belong to the model");
  if (!out_tokens_host || !out_exit_layers_host) fail(EE_ERR_INVALID_ARG, "null output");
  if (batch < 1 || batch > c->Bmax) fail(EE_ERR_INVALID_ARG, "batch out of range");
  const ee_model_config& cf = m->cfg;
  const int L = cf.n_layers;
  if (in_tokens_host)
    for (int b = 0; b < batch; ++b)
      if (in_tokens_host[b] < 0 || in_tokens_host[b] >= cf.vocab) fail(EE_ERR_INVALID_ARG, "token out of range");
  if (forced_exit_host)
    for (int b = 0; b < batch; ++b)
      if (forced_exit_host[b] < 0 || forced_exit_host[b] > L)
        fail(EE_ERR_INVALID_ARG, "forced exit layer out of range");
  if (gamma_host)
    for (int l = 0; l < L - 1; ++l)
      if (!std::isfinite(gamma_host[l])) fail(EE_ERR_INVALID_ARG, "gamma must be finite");
  if (!in_tokens_host)
    for (int b = 0; b < batch; ++b)
      if (!c->next_ok[b])
        fail(EE_ERR_INVALID_ARG, "sequence " + std::to_string(b) +
                                     " has no kept output token (none produced yet, or reset or rolled "
                                     "back since): pass in_tokens");
  for (int b = 0; b < batch; ++b)
    if (c->hlens[b] + 1 > c->S) fail(EE_ERR_CACHE_FULL, "sequence " + std::to_string(b) + " is full");
}

}  // namespace

// ===========================================================================
// C ABI
// ===========================================================================
extern "C" {

const char* ee_last_error(void) { return g_err.c_str(); }

ee_status ee_create_model(const ee_model_config* cfg, const ee_weights* w, const float* gamma,
                          ee_model** out) {
  return guard([&] {
    if (!cfg || !w || !out) fail(EE_ERR_INVALID_ARG, "null argument");
    validate_config(*cfg);
    const ee_model_config& c = *cfg;
    if (!w->tok_emb || !w->lm_head || !w->final_norm || !w->layers)
      fail(EE_ERR_INVALID_ARG, "null weight pointer");
    for (int l = 0; l < c.n_layers; ++l) {
      const ee_layer_weights& lw = w->layers[l];
      if (!lw.attn_norm || !lw.wq || !lw.wk || !lw.wv || !lw.wo || !lw.ffn_norm || !lw.w_gate ||
          !lw.w_up || !lw.w_down ||
          (l + 1 < c.n_layers && !lw.head_T && c.exit_mode != EE_EXIT_NONE && c.criterion == EE_CRIT_HEAD))
        fail(EE_ERR_INVALID_ARG, "null weight pointer in layer " + std::to_string(l + 1));
    }
    std::vector<float> gam(c.n_layers > 1 ? c.n_layers - 1 : 0, 0.75f);
    if (gamma)
      for (size_t i = 0; i < gam.size(); ++i) {
        if (!std::isfinite(gamma[i])) fail(EE_ERR_INVALID_ARG, "gamma must be finite");
        gam[i] = gamma[i];
      }
    ee_model* m = new ee_model();
    try {
      m->cfg = c;
      m->tok_emb = (const uint16_t*)w->tok_emb;
      m->lm_head = (const uint16_t*)w->lm_head;
      m->final_norm = (const uint16_t*)w->final_norm;
      m->lw.assign(w->layers, w->layers + c.n_layers);
      m->gamma = gam;
      HIPCHK(hipStreamCreateWithFlags(&m->own, hipStreamNonBlocking));
      no_rows();  // resolved on this device here, before any graph capture
      HIPCHK(hipGetDevice(&m->device));
      if (m->device < 0 || m->device >= kMaxDevices) fail(EE_ERR_UNSUPPORTED, "device index out of range");
      if (!g_scratch[m->device]) {  // once per device, with that device current
        void* p = nullptr;
        HIPCHK(hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)));
        if (!p) fail(EE_ERR_HIP, "hipGetSymbolAddress(scratch) returned null");
        g_scratch[m->device] = (char*)p;
      }
      const int L = c.n_layers, d = c.d_model, F = c.d_ff, G = c.group_size;
      const int qd = c.n_heads * c.head_dim, kvd = c.n_kv_heads * c.head_dim;
      // int4 exit copies of layers 2..L
      m->lq.resize(L);
      if (c.exit_mode == EE_EXIT_INT4) {
        auto mk = [&](int N, int K) {
          Q4 q;
          q.N = N;
          q.K = K;
          const size_t n16 = (size_t)(N + 15) / 16 * 16;
          q.codes = m->alloc<uint32_t>(n16 * (K / 8));
          q.scales = m->alloc<uint16_t>(n16 * (K / G));
          HIPCHK(hipMemsetAsync(q.codes, 0x88, n16 * (K / 8) * 4, m->own));
          HIPCHK(hipMemsetAsync(q.scales, 0, n16 * (K / G) * 2, m->own));
          return q;
        };
        for (int l = 2; l <= L; ++l) {
          LayerQ& q = m->lq[l - 1];
          const ee_layer_weights& lw = m->lw[l - 1];
          q.qkv = mk(qd + 2 * kvd, d);
          q.o = mk(d, qd);
          q.gate = mk(F, d);
          q.up = mk(F, d);
          q.down = mk(d, F);
          launch_quantize((const uint16_t*)lw.wq, qd, d, G, 0, q.qkv.codes, q.qkv.scales, m->own);
          launch_quantize((const uint16_t*)lw.wk, kvd, d, G, qd, q.qkv.codes, q.qkv.scales, m->own);
          launch_quantize((const uint16_t*)lw.wv, kvd, d, G, qd + kvd, q.qkv.codes, q.qkv.scales, m->own);
          launch_quantize((const uint16_t*)lw.wo, d, qd, G, 0, q.o.codes, q.o.scales, m->own);
          launch_quantize((const uint16_t*)lw.w_gate, F, d, G, 0, q.gate.codes, q.gate.scales, m->own);
          launch_quantize((const uint16_t*)lw.w_up, F, d, G, 0, q.up.codes, q.up.scales, m->own);
          launch_quantize((const uint16_t*)lw.w_down, d, F, G, 0, q.down.codes, q.down.scales, m->own);
          HIPCHK(hipGetLastError());
        }
      }
      // E once more in the tiled order of the wide vocabulary pass, for batches
      // of more than 8 rows (E is read once per launch for up to 64 rows)
      if (c.max_batch > 8 && wide_vocab_supported(d)) {
        m->lm_head_t = m->alloc<uint16_t>(wide_vocab_elems(c.vocab, d));
        launch_tile_vocab(m->lm_head, c.vocab, d, m->lm_head_t, m->own);
        HIPCHK(hipGetLastError());
      }
      // and the layers' bf16 weights, for the wide projections
      m->wide = c.max_batch > 8 && wide_vocab_supported(d) && wide_vocab_supported(qd) && wide_vocab_supported(F);
      if (m->wide) {
        m->ww.resize(L);
        for (int l = 1; l <= L; ++l) {
          const ee_layer_weights& lw = m->lw[l - 1];
          ee_model::WideW& t = m->ww[l - 1];
          t.qkv = m->alloc<uint16_t>((size_t)(qd + 2 * kvd) * d);
          launch_tile_rows((const uint16_t*)lw.wq, qd, d, t.qkv, m->own);
          launch_tile_rows((const uint16_t*)lw.wk, kvd, d, t.qkv + (size_t)qd * d, m->own);
          launch_tile_rows((const uint16_t*)lw.wv, kvd, d, t.qkv + (size_t)(qd + kvd) * d, m->own);
          t.o = m->alloc<uint16_t>((size_t)d * qd);
          launch_tile_rows((const uint16_t*)lw.wo, d, qd, t.o, m->own);
          t.gu = m->alloc<uint16_t>((size_t)2 * F * d);
          launch_tile_pair_rows((const uint16_t*)lw.w_gate, (const uint16_t*)lw.w_up, F, d, t.gu, m->own);
          t.down = m->alloc<uint16_t>((size_t)d * F);
          launch_tile_rows((const uint16_t*)lw.w_down, d, F, t.down, m->own);
          if (l < L && lw.head_T) {
            t.T = m->alloc<uint16_t>((size_t)d * d);
            launch_tile_rows((const uint16_t*)lw.head_T, d, d, t.T, m->own);
          }
          HIPCHK(hipGetLastError());
        }
        const size_t yq = (size_t)wide_ranges(qd + 2 * kvd, d, nullptr) * kMaxBatch * (qd + 2 * kvd);
        const size_t yg = (size_t)wide_ranges(2 * F, d, nullptr) * kMaxBatch * 2 * F;
        const size_t yt = (size_t)wide_ranges(d, d, nullptr) * kMaxBatch * d;
        m->wide_y = m->alloc<float>(std::max(yq, std::max(yg, yt)));
      }
      // RoPE table: cos/sin of pos * theta^(-2i/hd) in double, rounded to float
      const int half = c.head_dim / 2;
      std::vector<float> cs((size_t)c.max_positions * half), sn(cs.size());
      for (int p = 0; p < c.max_positions; ++p)
        for (int i = 0; i < half; ++i) {
          const double inv = std::pow((double)c.rope_theta, -(2.0 * i) / c.head_dim);
          const double ang = (double)p * inv;
          cs[(size_t)p * half + i] = (float)std::cos(ang);
          sn[(size_t)p * half + i] = (float)std::sin(ang);
        }
      m->d_cos = m->alloc<float>(cs.size());
      m->d_sin = m->alloc<float>(sn.size());
      HIPCHK(hipMemcpy(m->d_cos, cs.data(), cs.size() * 4, hipMemcpyHostToDevice));
      HIPCHK(hipMemcpy(m->d_sin, sn.data(), sn.size() * 4, hipMemcpyHostToDevice));
      const int Bm = kMaxBatch;
      m->h = m->alloc<float>((size_t)Bm * d);
      const int rows = std::min(8, c.max_batch);
      m->nkc_max = std::max(proj_ranges(qd, d, kNwg, rows, nullptr), proj_ranges(F, d, kNwg, rows, nullptr));
      if (m->wide)
        m->nkc_max = std::max(m->nkc_max, std::max(wide_ranges(d, qd, nullptr), wide_ranges(d, F, nullptr)));
      m->parts = m->alloc<float>((size_t)m->nkc_max * Bm * d);
      // rows 64.. hold each sequence's z at its exit layer (sampled decoding)
      m->xn = m->alloc<uint16_t>((size_t)2 * Bm * d);
      m->hb = m->alloc<uint16_t>((size_t)Bm * d);
      m->qrot = m->alloc<uint16_t>((size_t)Bm * qd);
      m->attn_o = m->alloc<uint16_t>((size_t)Bm * qd);
      m->act = m->alloc<uint16_t>((size_t)Bm * F);
      m->z = m->alloc<uint16_t>((size_t)Bm * d);
      m->head_part = m->alloc<float>((size_t)kNwg * kMaxBatch * 4);
      if (c.temperature > 0.0f) m->part_s = m->alloc<float>((size_t)kNwg * kMaxBatch * kPartS);
      m->h2 = m->alloc<float>((size_t)Bm * d);
      m->sts = m->alloc<float>(kMaxBatch);
      // the most partials any cache (S <= max_positions, B >= 1) can need: the
      // split is not monotone in S, so take the maximum over every tile count
      m->nch_max = 1;
      for (int tiles = 1; tiles <= (c.max_positions + 63) / 64; ++tiles) {
        int tpw = 0, nch = 0;
        attn_split(tiles * 64, 1, c.n_kv_heads, &tpw, &nch);
        m->nch_max = std::max(m->nch_max, nch);
      }
      if (m->nch_max > 2048) fail(EE_ERR_SHAPE, "too many attention partials");
      m->attn_part = m->alloc<float>((size_t)c.max_batch * c.n_heads * m->nch_max * (c.head_dim + 2));
      m->st = m->alloc<StepState>(1);
      m->p_rec = m->alloc<float>((size_t)std::max(L - 1, 1) * kMaxBatch);
      m->d_gamma = m->alloc<float>(std::max(L - 1, 1));
      HIPCHK(hipMemset(m->st, 0, sizeof(StepState)));
      if (L > 1)
        HIPCHK(hipMemcpy(m->d_gamma, gam.data(), gam.size() * 4, hipMemcpyHostToDevice));
      m->h_in = halloc<int32_t>(2 * kMaxBatch);
      m->h_gamma = halloc<float>(std::max(L - 1, 1));
      m->h_out = halloc<int32_t>(2 * kMaxBatch);
      m->h_gap = halloc<float>(kMaxBatch);
      HIPCHK(hipStreamSynchronize(m->own));
    } catch (...) {
      free_model(m);
      throw;
    }
    *out = m;
  });
}

ee_status ee_destroy_model(ee_model* m) {
  return guard([&] {
    if (!m) return;
    if (m->ncaches > 0) fail(EE_ERR_INVALID_ARG, "destroy the model's caches first");
    (void)hipStreamSynchronize(m->own);
    free_model(m);
  });
}

ee_status ee_kv_cache_bytes(const ee_model* m, int32_t max_batch, int32_t max_seq, size_t* bytes) {
  return guard([&] {
    if (!m || !bytes) fail(EE_ERR_INVALID_ARG, "null argument");
    if (max_batch < 1 || max_batch > m->cfg.max_batch) fail(EE_ERR_INVALID_ARG, "max_batch out of range");
    if (max_seq < 1 || max_seq > m->cfg.max_positions) fail(EE_ERR_INVALID_ARG, "max_seq out of range");
    const size_t kv = (size_t)m->cfg.n_layers * max_batch * m->cfg.n_kv_heads * max_seq *
                      m->cfg.head_dim * 2;
    *bytes = 2 * kv + 512;
  });
}

ee_status ee_kv_cache_create(ee_model* m, int32_t max_batch, int32_t max_seq, void* dev_buf,
                             size_t buf_bytes, uint32_t flags, ee_kv_cache** out) {
  return guard([&] {
    check_model(m);
    if (!out) fail(EE_ERR_INVALID_ARG, "null argument");
    size_t need = 0;
    ee_status st = ee_kv_cache_bytes(m, max_batch, max_seq, &need);
    if (st != EE_OK) fail(st, g_err);
    if (flags & ~EE_KV_TRACK_OCCUPANCY) fail(EE_ERR_INVALID_ARG, "unknown flags");
    if (dev_buf && buf_bytes < need) fail(EE_ERR_INVALID_ARG, "buffer too small");
    with_sticky(m, [&] {
      ee_kv_cache* c = new ee_kv_cache();
      try {
        c->m = m;
        c->Bmax = max_batch;
        c->S = max_seq;
        char* base = (char*)dev_buf;
        if (!base) {
          base = dalloc<char>(need);
          c->owned = base;
        }
        const size_t kv = (need - 512) / 2;
        c->K = (uint16_t*)base;
        c->V = (uint16_t*)(base + kv);
        c->lens = (int32_t*)(base + 2 * kv);
        c->next_tok = (int32_t*)(base + 2 * kv + 256);
        HIPCHK(hipMemsetAsync(c->lens, 0, 512, m->own));
        if (flags & EE_KV_TRACK_OCCUPANCY) {
          const size_t n = (size_t)m->cfg.n_layers * max_batch * max_seq;
          c->occ = dalloc<uint8_t>(n);
          HIPCHK(hipMemsetAsync(c->occ, 0, n, m->own));
        }
        HIPCHK(hipStreamSynchronize(m->own));
        c->hlens.assign(max_batch, 0);
        c->next_ok.assign(max_batch, 0);
      } catch (...) {
        if (c->owned) (void)hipFree(c->owned);
        if (c->occ) (void)hipFree(c->occ);
        delete c;
        throw;
      }
      m->ncaches++;
      *out = c;
    });
  });
}

ee_status ee_kv_cache_reset(ee_kv_cache* c, int32_t seq) {
  return guard([&] {
    if (!c) fail(EE_ERR_INVALID_ARG, "null cache");
    check_model(c->m);
    if (seq < -1 || seq >= c->Bmax) fail(EE_ERR_INVALID_ARG, "seq out of range");
    ee_model* m = c->m;
    with_sticky(m, [&] {
      const int lo = seq < 0 ? 0 : seq, hi = seq < 0 ? c->Bmax : seq + 1;
      for (int b = lo; b < hi; ++b) {
        c->hlens[b] = 0;
        c->next_ok[b] = 0;
      }
      HIPCHK(hipMemcpyAsync(c->lens, c->hlens.data(), c->Bmax * 4, hipMemcpyHostToDevice, m->own));
      if (c->occ)
        for (int l = 0; l < m->cfg.n_layers; ++l)
          HIPCHK(hipMemsetAsync(c->occ + ((size_t)l * c->Bmax + lo) * c->S, 0,
                                (size_t)(hi - lo) * c->S, m->own));
      HIPCHK(hipStreamSynchronize(m->own));
    });
  });
}

ee_status ee_kv_cache_rollback(ee_kv_cache* c, int32_t seq, int32_t n) {
  return guard([&] {
    if (!c) fail(EE_ERR_INVALID_ARG, "null cache");
    check_model(c->m);
    if (seq < -1 || seq >= c->Bmax) fail(EE_ERR_INVALID_ARG, "seq out of range");
    if (n < 0) fail(EE_ERR_INVALID_ARG, "n must be >= 0");
    const int lo = seq < 0 ? 0 : seq, hi = seq < 0 ? c->Bmax : seq + 1;
    for (int b = lo; b < hi; ++b)
      if (c->hlens[b] < n) fail(EE_ERR_INVALID_ARG, "rollback beyond the start of a sequence");
    if (n == 0) return;
    ee_model* m = c->m;
    with_sticky(m, [&] {
      for (int b = lo; b < hi; ++b) {
        c->hlens[b] -= n;
        c->next_ok[b] = 0;  // the token after the new last position is not kept
        if (c->occ)
          for (int l = 0; l < m->cfg.n_layers; ++l)
            HIPCHK(hipMemsetAsync(c->occ + ((size_t)l * c->Bmax + b) * c->S + c->hlens[b], 0, n, m->own));
      }
      HIPCHK(hipMemcpyAsync(c->lens, c->hlens.data(), c->Bmax * 4, hipMemcpyHostToDevice, m->own));
      HIPCHK(hipStreamSynchronize(m->own));
    });
  });
}

ee_status ee_kv_cache_lengths(const ee_kv_cache* c, int32_t* lens_host) {
  return guard([&] {
    if (!c || !lens_host) fail(EE_ERR_INVALID_ARG, "null argument");
    std::memcpy(lens_host, c->hlens.data(), c->Bmax * 4);
  });
}

ee_status ee_kv_cache_read(const ee_kv_cache* c, int32_t layer, int32_t seq, int32_t pos0, int32_t n,
                           void* k_host, void* v_host) {
  return guard([&] {
    if (!c || !k_host || !v_host) fail(EE_ERR_INVALID_ARG, "null argument");
    ee_model* m = c->m;
    check_model(m);
    const ee_model_config& cf = m->cfg;
    if (layer < 1 || layer > cf.n_layers) fail(EE_ERR_INVALID_ARG, "layer out of range");
    if (seq < 0 || seq >= c->Bmax) fail(EE_ERR_INVALID_ARG, "seq out of range");
    if (pos0 < 0 || n < 0 || pos0 + n > c->S) fail(EE_ERR_INVALID_ARG, "positions out of range");
    if (n == 0) return;
    with_sticky(m, [&] {
      if (c->occ) {
        std::vector<uint8_t> occ(n);
        HIPCHK(hipMemcpy(occ.data(), c->occ + ((size_t)(layer - 1) * c->Bmax + seq) * c->S + pos0, n,
                         hipMemcpyDeviceToHost));
        for (int i = 0; i < n; ++i)
          if (occ[i] == 0) fail(EE_ERR_NOT_WRITTEN, "KV slot never written");
      }
      const int Hkv = cf.n_kv_heads, hd = cf.head_dim;
      for (int kh = 0; kh < Hkv; ++kh) {
        const size_t off = ((((size_t)(layer - 1) * c->Bmax + seq) * Hkv + kh) * c->S + pos0) * hd;
        HIPCHK(hipMemcpy2D((uint16_t*)k_host + kh * hd, (size_t)Hkv * hd * 2, c->K + off, (size_t)hd * 2,
                           (size_t)hd * 2, n, hipMemcpyDeviceToHost));
        HIPCHK(hipMemcpy2D((uint16_t*)v_host + kh * hd, (size_t)Hkv * hd * 2, c->V + off, (size_t)hd * 2,
                           (size_t)hd * 2, n, hipMemcpyDeviceToHost));
      }
    });
  });
}

ee_status ee_kv_cache_occupancy(const ee_kv_cache* c, uint8_t* counts_host) {
  return guard([&] {
    if (!c || !counts_host) fail(EE_ERR_INVALID_ARG, "null argument");
    check_model(c->m);
    if (!c->occ) fail(EE_ERR_UNSUPPORTED, "cache created without occupancy tracking");
    with_sticky(c->m, [&] {
      HIPCHK(hipMemcpy(counts_host, c->occ, (size_t)c->m->cfg.n_layers * c->Bmax * c->S,
                       hipMemcpyDeviceToHost));
    });
  });
}

ee_status ee_kv_cache_destroy(ee_kv_cache* c) {
  return guard([&] {
    if (!c) return;
    (void)hipStreamSynchronize(c->m->own);
    drop_graphs(c->m, c);
    if (c->owned) (void)hipFree(c->owned);
    if (c->occ) (void)hipFree(c->occ);
    c->m->ncaches--;
    delete c;
  });
}

ee_status ee_prefill(ee_model* m, ee_kv_cache* c, int32_t batch, const int32_t* tokens_host, int32_t P,
                     void* hip_stream, int32_t* out_tokens_host, float* last_logits_host,
                     int32_t* exit_layers_host) {
  return guard([&] {
    check_model(m);
    if (!c || c->m != m) fail(EE_ERR_INVALID_ARG, "cache does not belong to the model");
    if (!tokens_host || !out_tokens_host) fail(EE_ERR_INVALID_ARG, "null argument");
    if (batch < 1 || batch > c->Bmax) fail(EE_ERR_INVALID_ARG, "batch out of range");
    if (P < 1) fail(EE_ERR_INVALID_ARG, "P must be >= 1");
    const int V = m->cfg.vocab;
    for (size_t i = 0; i < (size_t)batch * P; ++i)
      if (tokens_host[i] < 0 || tokens_host[i] >= V) fail(EE_ERR_INVALID_ARG, "token out of range");
    for (int b = 0; b < batch; ++b)
      if ((long long)c->hlens[b] + P > c->S) fail(EE_ERR_CACHE_FULL, "prefill exceeds max_seq");
    with_sticky(m, [&] {
      hipStream_t s = pick_stream(m, hip_stream);
      const size_t n = (size_t)batch * P;
      if (n > m->prompt_cap) {
        if (m->d_prompt) {
          (void)hipFree(m->d_prompt);
          for (auto& p : m->allocs)
            if (p == m->d_prompt) p = nullptr;
        }
        m->d_prompt = m->alloc<int32_t>(n);
        m->prompt_cap = n;
      }
      HIPCHK(hipMemcpyAsync(m->d_prompt, tokens_host, n * 4, hipMemcpyHostToDevice, s));
      for (int b = 0; b < batch; ++b) m->h_in[kMaxBatch + b] = 0;
      HIPCHK(hipMemcpyAsync(m->st->forced, m->h_in + kMaxBatch, batch * 4, hipMemcpyHostToDevice, s));
      const bool want_logits = last_logits_host != nullptr;
      if (want_logits && !m->dbg_logits) m->dbg_logits = m->alloc<float>((size_t)kMaxBatch * m->cfg.vocab);
      if (m->cfg.prefill_exit && m->gamma.size())
        HIPCHK(hipMemcpyAsync(m->d_gamma, m->gamma.data(), m->gamma.size() * 4, hipMemcpyHostToDevice, s));
      run_prefill(m, c, batch, P, want_logits, s);
      HIPCHK(hipGetLastError());
      HIPCHK(hipMemcpyAsync(c->next_tok, m->st->out_tok, batch * 4, hipMemcpyDeviceToDevice, s));
      HIPCHK(hipMemcpyAsync(m->h_out + kMaxBatch, m->st->e, batch * 4, hipMemcpyDeviceToHost, s));
      HIPCHK(hipMemcpyAsync(m->h_out, m->st->out_tok, batch * 4, hipMemcpyDeviceToHost, s));
      if (want_logits)
        HIPCHK(hipMemcpyAsync(last_logits_host, m->dbg_logits, (size_t)batch * m->cfg.vocab * 4,
                              hipMemcpyDeviceToHost, s));
      HIPCHK(hipStreamSynchronize(s));
      m->ev_used = 0;
      std::memcpy(out_tokens_host, m->h_out, batch * 4);
      if (exit_layers_host) std::memcpy(exit_layers_host, m->h_out + kMaxBatch, batch * 4);
      for (int b = 0; b < batch; ++b) {
        c->hlens[b] += P;
        c->next_ok[b] = 1;
      }
    });
  });
}

ee_status ee_decode_step(ee_model* m, ee_kv_cache* c, int32_t batch, const int32_t* in_tokens_host,
                         const int32_t* forced_exit_host, const float* gamma_host, void* hip_stream,
                         int32_t* out_tokens_host, int32_t* out_exit_layers_host, ee_step_debug* dbg) {
  return guard([&] {
    validate_step(m, c, batch, in_tokens_host, forced_exit_host, gamma_host, out_tokens_host,
                  out_exit_layers_host);
    const ee_model_config& cf = m->cfg;
    const int L = cf.n_layers;
    with_sticky(m, [&] {
      hipStream_t s = pick_stream(m, hip_stream);
      Debug dd;
      if (dbg) {
        dd.hidden = dbg->hidden != nullptr;
        dd.logits = dbg->logits != nullptr;
        if (dd.hidden && !m->dbg_hidden)
          m->dbg_hidden = m->alloc<float>((size_t)kMaxBatch * (L + 1) * cf.d_model);
        if (dd.logits && !m->dbg_logits) m->dbg_logits = m->alloc<float>((size_t)kMaxBatch * cf.vocab);
      }
      // inputs of the step
      for (int b = 0; b < batch; ++b) {
        m->h_in[b] = in_tokens_host ? in_tokens_host[b] : 0;
        m->h_in[kMaxBatch + b] = forced_exit_host ? forced_exit_host[b] : 0;
      }
      for (int l = 0; l < L - 1; ++l) m->h_gamma[l] = gamma_host ? gamma_host[l] : m->gamma[l];
      if (in_tokens_host)
        HIPCHK(hipMemcpyAsync(m->st->tok, m->h_in, batch * 4, hipMemcpyHostToDevice, s));
      else  // this cache's last outputs (the model's step state is shared by its caches)
        HIPCHK(hipMemcpyAsync(m->st->tok, c->next_tok, batch * 4, hipMemcpyDeviceToDevice, s));
      HIPCHK(hipMemcpyAsync(m->st->forced, m->h_in + kMaxBatch, batch * 4, hipMemcpyHostToDevice, s));
      if (L > 1)
        HIPCHK(hipMemcpyAsync(m->d_gamma, m->h_gamma, (L - 1) * 4, hipMemcpyHostToDevice, s));
      if (dbg) {
        enqueue_position(m, model_work(m), c, batch, true, true, nullptr, 1, 0, dd, s);
      } else {
        replay_step(m, c, batch, s);
      }
      HIPCHK(hipMemcpyAsync(c->next_tok, m->st->out_tok, batch * 4, hipMemcpyDeviceToDevice, s));
      HIPCHK(hipMemcpyAsync(m->h_out, m->st->out_tok, batch * 4, hipMemcpyDeviceToHost, s));
      HIPCHK(hipMemcpyAsync(m->h_out + kMaxBatch, m->st->e, batch * 4, hipMemcpyDeviceToHost, s));
      HIPCHK(hipMemcpyAsync(m->h_gap, m->st->gap, batch * 4, hipMemcpyDeviceToHost, s));
      std::vector<float> prec;
      if (dbg && dbg->p_top1 && L > 1) {
        prec.resize((size_t)(L - 1) * kMaxBatch);
        HIPCHK(hipMemcpyAsync(prec.data(), m->p_rec, prec.size() * 4, hipMemcpyDeviceToHost, s));
      }
      if (dd.logits)
        HIPCHK(hipMemcpyAsync(dbg->logits, m->dbg_logits, (size_t)batch * cf.vocab * 4,
                              hipMemcpyDeviceToHost, s));
      if (dd.hidden)
        HIPCHK(hipMemcpyAsync(dbg->hidden, m->dbg_hidden, (size_t)batch * (L + 1) * cf.d_model * 4,
                              hipMemcpyDeviceToHost, s));
      HIPCHK(hipStreamSynchronize(s));
      prof_collect(m);
      std::memcpy(out_tokens_host, m->h_out, batch * 4);
      std::memcpy(out_exit_layers_host, m->h_out + kMaxBatch, batch * 4);
      if (dbg && dbg->gap) std::memcpy(dbg->gap, m->h_gap, batch * 4);
      if (dbg && dbg->p_top1)
        for (int b = 0; b < batch; ++b)
          for (int l = 0; l < L - 1; ++l) dbg->p_top1[(size_t)b * (L - 1) + l] = prec[(size_t)l * kMaxBatch + b];
      for (int b = 0; b < batch; ++b) {
        c->hlens[b] += 1;
        c->next_ok[b] = 1;
      }
    });
  });
}

ee_status ee_decode_step_static(ee_model* m, ee_kv_cache* c, int32_t batch, const int32_t* in_tokens_host,
                                const int32_t* forced_exit_host, const float* gamma_host, void* hip_stream,
                                int32_t* out_tokens_host, int32_t* out_exit_layers_host) {
  return guard([&] {
    validate_step(m, c, batch, in_tokens_host, forced_exit_host, gamma_host, out_tokens_host,
                  out_exit_layers_host);
    const ee_model_config& cf = m->cfg;
    const int L = cf.n_layers;
    Work W;
    const size_t need = work_layout(m, batch, c->S, nullptr, &W);
    if (need > kScratchBytes)
      fail(EE_ERR_UNSUPPORTED, "the step's workspaces need " + std::to_string(need) +
                                   " bytes, more than the static scratch holds (" + std::to_string(kScratchBytes) +
                                   "): use ee_decode_step");
    char* base = g_scratch[m->device];
    if (!base) fail(EE_ERR_HIP, "the static scratch was not resolved on the model's device");
    work_layout(m, batch, c->S, base, &W);
    W.prof = false;  // no events are created here
    with_sticky(m, [&] {
      hipStream_t s = pick_stream(m, hip_stream);
      // the array keeps the last call's contents: the step state starts from zero
      launch_fill_u32((uint32_t*)W.st, sizeof(StepState) / 4, 0u, s);
      for (int b = 0; b < batch; ++b) {
        m->h_in[b] = in_tokens_host ? in_tokens_host[b] : 0;
        m->h_in[kMaxBatch + b] = forced_exit_host ? forced_exit_host[b] : 0;
      }
      for (int l = 0; l < L - 1; ++l) m->h_gamma[l] = gamma_host ? gamma_host[l] : m->gamma[l];
      if (in_tokens_host)
        HIPCHK(hipMemcpyAsync(W.st->tok, m->h_in, batch * 4, hipMemcpyHostToDevice, s));
      else
        HIPCHK(hipMemcpyAsync(W.st->tok, c->next_tok, batch * 4, hipMemcpyDeviceToDevice, s));
      HIPCHK(hipMemcpyAsync(W.st->forced, m->h_in + kMaxBatch, batch * 4, hipMemcpyHostToDevice, s));
      if (L > 1) HIPCHK(hipMemcpyAsync(W.d_gamma, m->h_gamma, (L - 1) * 4, hipMemcpyHostToDevice, s));
      enqueue_position(m, W, c, batch, true, true, nullptr, 1, 0, Debug{}, s);
      HIPCHK(hipMemcpyAsync(c->next_tok, W.st->out_tok, batch * 4, hipMemcpyDeviceToDevice, s));
      HIPCHK(hipMemcpyAsync(m->h_out, W.st->out_tok, batch * 4, hipMemcpyDeviceToHost, s));
      HIPCHK(hipMemcpyAsync(m->h_out + kMaxBatch, W.st->e, batch * 4, hipMemcpyDeviceToHost, s));
      HIPCHK(hipStreamSynchronize(s));
      std::memcpy(out_tokens_host, m->h_out, batch * 4);
      std::memcpy(out_exit_layers_host, m->h_out + kMaxBatch, batch * 4);
      for (int b = 0; b < batch; ++b) {
        c->hlens[b] += 1;
        c->next_ok[b] = 1;
      }
    });
  });
}

ee_status ee_exit_weights_read(const ee_model* m, int32_t layer, int32_t which, int32_t row0, int32_t nrows,
                               int8_t* codes_host, uint16_t* scales_host) {
  return guard([&] {
    check_model(m);
    if (!codes_host || !scales_host) fail(EE_ERR_INVALID_ARG, "null argument");
    const ee_model_config& cf = m->cfg;
    if (cf.exit_mode != EE_EXIT_INT4) fail(EE_ERR_UNSUPPORTED, "no int4 copies in this exit mode");
    if (layer < 2 || layer > cf.n_layers) fail(EE_ERR_INVALID_ARG, "layer must be in [2, L]");
    const LayerQ& q = m->lq[layer - 1];
    const int qd = cf.n_heads * cf.head_dim, kvd = cf.n_kv_heads * cf.head_dim;
    const Q4* src = nullptr;
    int off = 0, N = 0;
    switch (which) {
      case 0: src = &q.qkv; off = 0; N = qd; break;
      case 1: src = &q.qkv; off = qd; N = kvd; break;
      case 2: src = &q.qkv; off = qd + kvd; N = kvd; break;
      case 3: src = &q.o; N = src->N; break;
      case 4: src = &q.gate; N = src->N; break;
      case 5: src = &q.up; N = src->N; break;
      case 6: src = &q.down; N = src->N; break;
      default: fail(EE_ERR_INVALID_ARG, "which must be in [0, 6]");
    }
    if (row0 < 0 || nrows < 0 || row0 + nrows > N) fail(EE_ERR_INVALID_ARG, "rows out of range");
    if (nrows == 0) return;
    const int K = src->K, G = cf.group_size;
    ee_model* mm = const_cast<ee_model*>(m);
    with_sticky(mm, [&] {
      CallBuffer<int8_t> tmp((size_t)nrows * K);
      CallBuffer<uint16_t> stmp((size_t)nrows * (K / G));
      launch_unpack(src->codes, src->scales, K, G, off + row0, nrows, tmp.p, stmp.p, mm->own);
      HIPCHK(hipStreamSynchronize(mm->own));
      HIPCHK(hipMemcpy(codes_host, tmp.p, (size_t)nrows * K, hipMemcpyDeviceToHost));
      HIPCHK(hipMemcpy(scales_host, stmp.p, (size_t)nrows * (K / G) * 2, hipMemcpyDeviceToHost));
    });
  });
}

ee_status ee_profile_enable(ee_model* m, int32_t on) {
  return guard([&] {
    check_model(m);
    m->prof = on != 0;
    m->prof_launches = 0;
    m->prof_ms = 0;
    m->ev_used = 0;
  });
}

ee_status ee_profile_read(ee_model* m, int32_t kind, int64_t* launches, double* total_ms) {
  return guard([&] {
    check_model(m);
    if (!launches || !total_ms) fail(EE_ERR_INVALID_ARG, "null argument");
    if (kind != 0) fail(EE_ERR_INVALID_ARG, "unknown kind");
    *launches = m->prof_launches;
    *total_ms = m->prof_ms;
    m->prof_launches = 0;
    m->prof_ms = 0;
  });
}

}  // extern "C"
