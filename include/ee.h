/*
 * ee.h - C ABI of libee, the KV-shared early-exit decode step on one MI355X (gfx950).
 *
 * The method (page titles and sections of the surveyed web pages):
 *   - "River-LLM 深度解析" section 4.1-4.3: every decoder layer has an int4 (W4A16)
 *     "exit layer" copy; once a token exits, the copies run its remaining layers
 *     and write K/V into the same cache slots as the backbone layer would, so no
 *     KV entry is ever missing (section 8.2, one store per layer).
 *   - "大语言模型解码加速：自适应层并行机制解析" (AdaDecode explainer) section 2.1:
 *     the intermediate exit head of layer l is h^(l) T^(l) E^T with T^(l) a d x d
 *     matrix and E the LM-head matrix; section 2.2: a token exits when the top-1
 *     probability exceeds gamma (default 0.75).
 *   - CALM explainer section 2.2: exit decisions are per token and per layer;
 *     section 3.3: sequences of one batch exit at different layers.
 *
 * One decode step, per sequence b: embed the input token; for l = 1..L run layer
 * l with the backbone bf16 weights while b is on the backbone, else with the
 * int4 exit copy; write k, v of position pos_b into slot (l, b, pos_b); after
 * backbone layer l < L evaluate the exit head: z = bf16(T_l bf16(h)),
 * logits = E z, p = max softmax(logits); exit iff p > gamma_l (strict), or iff
 * l equals the forced exit layer when one is given.  The emitted token is the
 * greedy argmax of the final RMSNorm + LM head after layer L (lowest index on
 * ties).  The exit layer e_b is the layer after which b left the backbone; e_b =
 * L means b never exited.  Model options replace the exit head by River-LLM's
 * state transition similarity (section 5.1-5.2), let the batch minimum decide
 * (section 5.2), evaluate the criterion only every N layers (CALM explainer,
 * checking every N layers), or drop the criterion (the plain decoder).
 *
 * Precision: bf16 weights and GEMV inputs, float32 accumulation, float32
 * residual stream, bf16 K/V cache, float32 logits and softmax.  int4 codes are
 * symmetric per group of G inputs of a row with a bf16 scale
 * s = bf16(max|w| / 7), q = clamp(rint(w / s), -8, 7), w_hat = q * s.
 *
 * Conventions
 *   - Every entry point returns ee_status; EE_OK is 0, errors are negative.
 *     Output parameters are written only on EE_OK.  ee_last_error() returns a
 *     thread-local message for the last failure.  No C++ exception crosses the ABI.
 *   - Arguments are validated on the host before any launch; an invalid call
 *     changes no state.
 *   - EE_ERR_HIP is sticky for the model: destroy it and start again.
 *   - "device" pointers point to GPU memory of the current HIP device; "host"
 *     pointers to ordinary CPU memory.  A model or cache is used by one host
 *     thread at a time.
 *   - Weight matrices are bf16, row-major [out, in] (a linear map y = W x), and
 *     are borrowed: the caller keeps them alive and unchanged until
 *     ee_destroy_model.  The library owns everything it derives (int4 copies,
 *     RoPE table, workspaces).
 */
#ifndef EE_H
#define EE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef int32_t ee_status;
#define EE_OK 0
#define EE_ERR_INVALID_ARG (-1)   /* a null pointer, a value out of range, a bad shape */
#define EE_ERR_OUT_OF_MEMORY (-2) /* device or pinned host allocation failed */
#define EE_ERR_HIP (-3)           /* a HIP runtime call failed (sticky) */
#define EE_ERR_CACHE_FULL (-4)    /* a sequence would grow beyond the cache's max_seq */
#define EE_ERR_SHAPE (-5)         /* the model shape is not supported by the kernels */
#define EE_ERR_NOT_WRITTEN (-6)   /* a KV slot read back was never written (occupancy on) */
#define EE_ERR_UNSUPPORTED (-7)   /* a feature the library does not implement */

#define EE_EXIT_INT4 0 /* exit copies are the int4 group-quantised layers */
#define EE_EXIT_BF16 1 /* exit copies are the backbone layers themselves (test mode) */
#define EE_EXIT_NONE 2 /* no exit heads: the plain decoder at full depth, the baseline
                          the method is compared with (every exit layer is n_layers;
                          head_T may be NULL; forced exits and gamma are ignored) */

/* Exit criterion evaluated after layers 1..L-1 for the sequences still on the
 * backbone (not used with EE_EXIT_NONE):
 *   EE_CRIT_HEAD  the exit head's top-1 probability p = max softmax(h T_l E^T)
 *                 compared with gamma_l (AdaDecode explainer, sections 2.1-2.2);
 *   EE_CRIT_STS   River-LLM's state transition similarity: the cosine between
 *                 the sequence's hidden state entering layer l and leaving it,
 *                 compared with tau_l (River-LLM explainer, sections 5.1-5.2),
 *                 per sequence; the model's thresholds (and a step's gamma_host)
 *                 are the tau_l, the exit heads do not run and head_T may be NULL.
 * Either way a sequence exits iff its value > the layer's threshold. */
#define EE_CRIT_HEAD 0
#define EE_CRIT_STS 1

/* Who decides an exit after an evaluated layer:
 *   EE_RULE_SEQUENCE   each sequence on the backbone, from its own value;
 *   EE_RULE_BATCH_MIN  the sequences on the backbone whose exit is not forced
 *                      leave together when the smallest of their values exceeds
 *                      the layer's threshold (River-LLM explainer, section 5.2). */
#define EE_RULE_SEQUENCE 0
#define EE_RULE_BATCH_MIN 1

#define EE_KV_TRACK_OCCUPANCY 1u /* count writes per (layer, sequence, position) slot */

typedef struct ee_model ee_model;
typedef struct ee_kv_cache ee_kv_cache;

/* Model shape.  Supported (else EE_ERR_SHAPE): group_size in {32, 64, 128};
 * d_model, d_ff and n_heads * head_dim multiples of group_size and of 32;
 * head_dim in {32, 64, 128}; n_heads a multiple of n_kv_heads with at most 16
 * query heads per kv head; d_model <= 32768 / min(8, max_batch) (the vocabulary
 * GEMV stages its input rows in 64 KB of LDS).  Also n_layers >= 1, vocab >= 1,
 * 1 <= max_batch <= 64 and max_positions >= 1 (bounds every position). */
typedef struct ee_model_config {
  int32_t n_layers;
  int32_t d_model;
  int32_t n_heads;
  int32_t n_kv_heads;
  int32_t head_dim;
  int32_t d_ff;
  int32_t vocab;
  int32_t group_size;
  float rms_eps;
  float rope_theta;
  int32_t exit_mode; /* EE_EXIT_INT4, EE_EXIT_BF16 or EE_EXIT_NONE */
  int32_t max_batch;
  int32_t max_positions;
  int32_t criterion; /* EE_CRIT_HEAD or EE_CRIT_STS */
  int32_t check_every; /* evaluate the criterion only after layers that are multiples of it
                          (CALM explainer: check every N layers); 0 or 1: every layer.
                          A forced exit applies after any layer. */
  int32_t exit_rule;   /* EE_RULE_SEQUENCE or EE_RULE_BATCH_MIN */
  float temperature;   /* 0: greedy decoding.  > 0: sampled decoding with AdaDecode's
                          verification (AdaDecode explainer, section 3.1): a sequence that
                          exits at layer l drafts a token from softmax(exit-head logits / T)
                          there; after the remaining layers the draft is accepted with
                          probability min(1, p_final / p_draft) (p_final = softmax(final
                          logits / T)), otherwise the token is drawn from the normalised
                          relu(p_final - p_draft); a sequence that runs every layer draws
                          from p_final.  Draws: Gumbel-max over Philox4x64-10 noise with key
                          (sample_seed, 0) and counter (v / 4, sequence, position, stream)
                          (streams: 1 draft, 2 final, 3 resample, 4 acceptance uniform, word
                          0 of block 0); u = ((x >> 41) + 0.5) / 2^23.  Needs EE_CRIT_HEAD,
                          check_every <= 1 and exit copies (not EE_EXIT_NONE), else
                          INVALID_ARG.  Above 8 rows the sampled vocabulary passes take
                          the rows 8 at a time (E is read once per 8 rows).  The
                          prefill's token stays greedy. */
  uint32_t sample_seed;
  int32_t prefill_exit; /* 0: the prefill runs every layer on the backbone.  1: River-LLM's
                           sequence-level exit in the prefill (River-LLM explainer, sections 6.1
                           and 5.2): the prefill runs layer by layer over all positions, and after
                           layer l < L a sequence leaves when the smallest state transition
                           similarity of its prompt's tokens exceeds the model's threshold tau_l;
                           its later layers run on the exit copies for every token (and write
                           those K/V slots).  Needs EE_CRIT_STS and exit copies. */
} ee_model_config;

/* Device pointers of one layer.  Shapes: attn_norm, ffn_norm [d]; wq [H*hd, d];
 * wk, wv [Hkv*hd, d]; wo [d, H*hd]; w_gate, w_up [F, d]; w_down [d, F];
 * head_T [d, d] holds the exit head's projection with z_j = sum_i T[j, i] h_i
 * (NULL for the last layer, which has no exit head). */
typedef struct ee_layer_weights {
  const void *attn_norm, *wq, *wk, *wv, *wo;
  const void *ffn_norm, *w_gate, *w_up, *w_down;
  const void *head_T;
} ee_layer_weights;

/* tok_emb [V, d] embedding rows; lm_head [V, d] is E of both the exit heads and
 * the final head; final_norm [d].  layers is a HOST array of n_layers entries. */
typedef struct ee_weights {
  const void *tok_emb, *lm_head, *final_norm;
  const ee_layer_weights *layers;
} ee_weights;

/* Optional per-step diagnostics (host buffers; NULL members are skipped).
 * Requesting any of them runs the step without graph replay. */
typedef struct ee_step_debug {
  float *p_top1; /* [batch][L-1]: the criterion's value (exit-head top-1 probability, or
                    the state transition similarity), NaN where it was not evaluated */
  float *logits; /* [batch][V]: final LM-head logits */
  float *hidden; /* [batch][L+1][d]: residual after the embedding and after each layer */
  float *gap;    /* [batch]: top-1 minus top-2 final logit (+inf when V == 1) */
} ee_step_debug;

/* Creates a model: the backbone plus its exit layers ("River-LLM 深度解析",
 * section 4.2: each exit layer is a 4-bit copy of the original layer, about 75%
 * smaller; section 8.1: the copy is made by quantising the original layer's
 * weights with a max/7 scale, rounded and clamped to [-8, 7]), and the exit
 * heads T_l of the AdaDecode explainer, section 2.1.
 * cfg, w: host structs describing borrowed device weights.
 * gamma: host [n_layers - 1] per-layer thresholds (gamma_l, or tau_l with
 * EE_CRIT_STS), or NULL for 0.75 everywhere.
 * Builds the int4 exit copies of layers 2..L on the device (synchronously).
 * Errors: INVALID_ARG (nulls, values), SHAPE (unsupported shape),
 * OUT_OF_MEMORY, HIP. */
ee_status ee_create_model(const ee_model_config *cfg, const ee_weights *w,
                          const float *gamma, ee_model **out);

/* Destroys a model (NULL is allowed) and everything it owns (int4 copies,
 * workspaces, captured graphs).  Caches created from it must be destroyed
 * first (else INVALID_ARG, nothing is freed). */
ee_status ee_destroy_model(ee_model *m);

/* The shared KV cache ("River-LLM 深度解析", section 4.3: the backbone and the
 * exit layers read and write one cache, so an exited token still leaves K/V for
 * every layer; section 8.2: get/update/store of one (layer, position) slot).
 * Device bytes a KV cache of max_batch sequences and max_seq positions needs:
 * K and V, each [L][max_batch][Hkv][max_seq][hd] bf16, plus the per-sequence
 * lengths and last output tokens (512 bytes). */
ee_status ee_kv_cache_bytes(const ee_model *m, int32_t max_batch, int32_t max_seq,
                            size_t *bytes);

/* Creates an empty shared cache (all lengths 0; "River-LLM 深度解析", section
 * 4.3).  dev_buf: caller-owned device buffer of
 * at least ee_kv_cache_bytes bytes (kept alive until destroy), or NULL to let the
 * library allocate.  max_batch <= model max_batch, max_seq <= max_positions.
 * flags: EE_KV_TRACK_OCCUPANCY keeps a u8 write counter per slot. */
ee_status ee_kv_cache_create(ee_model *m, int32_t max_batch, int32_t max_seq,
                             void *dev_buf, size_t buf_bytes, uint32_t flags,
                             ee_kv_cache **out);

/* Sets the length of sequence seq (or of all sequences when seq == -1) to 0 and
 * clears its occupancy counters and its kept output token. */
ee_status ee_kv_cache_reset(ee_kv_cache *c, int32_t seq);

/* Discards the last n positions of sequence seq (all sequences when seq == -1):
 * the length drops by n and, with occupancy tracking, the dropped slots' write
 * counters are cleared, so the positions can be written again.  With n > 0 the
 * sequence's kept output token is dropped too (it followed the last dropped
 * position): the next ee_decode_step must pass its input token.  This is the
 * rollback of a rejected token ("大语言模型解码加速：自适应层并行机制解析",
 * section 3.1: on a failed verification the KV entries after the last valid
 * token are discarded).  INVALID_ARG if n < 0 or n exceeds a length. */
ee_status ee_kv_cache_rollback(ee_kv_cache *c, int32_t seq, int32_t n);

/* Copies the max_batch sequence lengths (positions written per sequence) to
 * lens_host [max_batch] int32.  Host-side only: no device work. */
ee_status ee_kv_cache_lengths(const ee_kv_cache *c, int32_t *lens_host);

/* Copies K and V of positions [pos0, pos0+n) of one (1-based) layer and sequence
 * to host buffers, each [n][Hkv][hd] bf16 (uint16 bit patterns).  This is the
 * cache's "get" ("River-LLM 深度解析", section 8.2: get returns nothing for a
 * (layer, position) never stored): with occupancy tracking, NOT_WRITTEN if any
 * slot in the range was never written (nothing is copied).  INVALID_ARG for a
 * layer, sequence or range outside the cache. */
ee_status ee_kv_cache_read(const ee_kv_cache *c, int32_t layer, int32_t seq, int32_t pos0,
                           int32_t n, void *k_host, void *v_host);

/* Copies the occupancy counters [L][max_batch][max_seq] (u8) to the host: the
 * number of stores into each slot ("River-LLM 深度解析", section 8.2: one store
 * per layer and position, whichever copy ran it).
 * UNSUPPORTED if the cache was created without EE_KV_TRACK_OCCUPANCY. */
ee_status ee_kv_cache_occupancy(const ee_kv_cache *c, uint8_t *counts_host);

/* Destroys a cache (NULL is allowed) after the work queued on the model's
 * stream has finished; frees the library-owned buffer, never dev_buf, and
 * releases the decode-step graphs captured for it. */
ee_status ee_kv_cache_destroy(ee_kv_cache *c);

/* Prefill, the first of the two phases of generation ("River-LLM 深度解析",
 * section 6.1: the prompt is processed as a whole, then tokens are generated
 * one at a time).  Runs sequences 0..batch-1 over P prompt tokens each (host [batch][P]
 * int32, row-major) with the backbone weights (no exit heads; with prefill_exit,
 * River-LLM's sequence-level exit as described at ee_model_config), writing KV
 * slots at positions len_b .. len_b+P-1, then returns the greedy token after the
 * last position in out_tokens_host [batch].  That token is also kept on the
 * device as the next decode input.  last_logits_host: optional host [batch][V]
 * float32 LM-head logits of the last position (NULL: not copied).
 * exit_layers_host: optional host [batch], each sequence's prefill exit layer
 * (L: no exit; always L without prefill_exit).
 * hip_stream: a hipStream_t or NULL (the library's own stream); the call
 * returns after the work has finished.
 * Errors: INVALID_ARG (token out of [0, V), batch out of range), CACHE_FULL,
 * OUT_OF_MEMORY (prefill_exit: per-position buffers of P * batch rows). */
ee_status ee_prefill(ee_model *m, ee_kv_cache *c, int32_t batch, const int32_t *tokens_host,
                     int32_t P, void *hip_stream, int32_t *out_tokens_host,
                     float *last_logits_host, int32_t *exit_layers_host);

/* One decode step, the second phase ("River-LLM 深度解析", section 6.1: each
 * generated token decides its exit by itself), for sequences 0..batch-1: the
 * per-layer exit decision of the AdaDecode explainer, sections 2.1-2.2 (or the
 * criterion the model was created with) and the exit layers of "River-LLM
 * 深度解析", sections 4.1-4.3, as described at the top of this file.
 * in_tokens_host: [batch] input tokens, or NULL to use each sequence's last
 *   output token, which this cache keeps on the device (from the last ee_prefill
 *   or ee_decode_step on this cache that included the sequence).  NULL is
 *   INVALID_ARG while some sequence b < batch has no kept token: none produced
 *   on this cache yet, or reset or rolled back since.
 * forced_exit_host: [batch] or NULL; 0 lets the criterion decide, 1..L forces
 *   the exit layer (the criterion still runs; its decision is overridden).
 * gamma_host: [L-1] thresholds for this step (gamma_l or tau_l), or NULL for
 *   the model's.
 * out_tokens_host, out_exit_layers_host: [batch] greedy tokens and exit layers.
 * dbg: optional diagnostics.  Returns after the outputs are on the host.
 * Without diagnostics and without profiling (ee_profile_enable), the step's
 * kernels are captured into a HIP graph on the first such call for this cache
 * and batch and replayed by later calls (the graph is released with the cache
 * or the model); otherwise they are launched one by one.  Both give the same
 * results bit for bit.
 * Errors: INVALID_ARG, CACHE_FULL (some len_b + 1 > max_seq; nothing runs). */
ee_status ee_decode_step(ee_model *m, ee_kv_cache *c, int32_t batch,
                         const int32_t *in_tokens_host, const int32_t *forced_exit_host,
                         const float *gamma_host, void *hip_stream, int32_t *out_tokens_host,
                         int32_t *out_exit_layers_host, ee_step_debug *dbg);

/* For callers that cannot allocate device memory (code under HIP graph capture
 * around its own work, tight serving loops, harnesses that forbid hipMalloc):
 * the same decode step as ee_decode_step (same arguments and results, bit for
 * bit), with its per-step device workspaces (residual, staged projection
 * inputs, partial sums, attention and exit-head partials, step state) taken
 * from a static device array of 32 MiB per GPU that the library holds until
 * the process ends, instead of the model's own buffers.  It calls no
 * hipMalloc, hipFree or other allocating routine; its kernels are launched
 * one by one (no graph is captured or instantiated), without diagnostics or
 * profiling.  UNSUPPORTED when the step's workspaces exceed the array (they
 * grow with the model widths: e.g. a feed-forward width of 49152 above 8
 * rows, whose partial sums need more; the 8B shape fits at any batch);
 * nothing runs then.  Every call on one GPU uses that GPU's single
 * array, which keeps the last call's contents (the step state is cleared by a
 * kernel at the start of each call): calls that overlap on one GPU, from any
 * model or thread, race and must be serialised by the caller. */
ee_status ee_decode_step_static(ee_model *m, ee_kv_cache *c, int32_t batch,
                                const int32_t *in_tokens_host, const int32_t *forced_exit_host,
                                const float *gamma_host, void *hip_stream, int32_t *out_tokens_host,
                                int32_t *out_exit_layers_host);

/* Copies the int4 exit copy of one linear map of 1-based layer (2..L) back to the
 * host as int8 codes [nrows][K] and bf16 scales [nrows][K/G] (uint16 bits).
 * which: 0 wq, 1 wk, 2 wv, 3 wo, 4 w_gate, 5 w_up, 6 w_down.
 * UNSUPPORTED in EE_EXIT_BF16 and EE_EXIT_NONE modes. */
ee_status ee_exit_weights_read(const ee_model *m, int32_t layer, int32_t which, int32_t row0,
                               int32_t nrows, int8_t *codes_host, uint16_t *scales_host);

/* Kernel timing for measurement.  When enabled, every launch of the exit-head
 * vocabulary GEMV records its own start and end into a pair of HIP events on
 * the stream it runs on (hipExtLaunchKernel), so the pair times the kernel
 * alone; ee_profile_read returns the number of such launches and their summed
 * duration in milliseconds since the last read, then clears the counters.
 * kind: 0 exit-head vocabulary GEMV. */
ee_status ee_profile_enable(ee_model *m, int32_t on);
ee_status ee_profile_read(ee_model *m, int32_t kind, int64_t *launches, double *total_ms);

/* Thread-local message describing the last error ("" if none). */
const char *ee_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* EE_H */
