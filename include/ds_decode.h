/*
 * ds_decode.h -- C ABI of the MI355X (gfx950) single-token Llama decode step.
 *
 * The library runs the autoregressive decode step of a Llama-style decoder
 * ("simple-llm / kasahare" PyPI README 0.4.0, section "Architecture": pre-norm
 * blocks of RMSNorm, Q/K/V projections without bias, RoPE, grouped-query
 * attention, Wo plus residual, RMSNorm, SwiGLU W2(silu(W1 x) * W3 x) plus
 * residual; tied embeddings) with a key/value cache ("Inside nanochat Part 4:
 * Understanding Inference", sections "KV Cache" and "Cache Architecture")
 * and greedy argmax selection ("Inside nanochat Part 4", section "Sampling
 * Strategy").  All arithmetic is fp32; matrices may be stored as bf16, which
 * is widened by a 16-bit left shift ("GOTOken: An Inference Engine in
 * QBasic", section "Loading the model and tokenizer").
 *
 * Conventions for every call
 *  - Pointers named d_* are device pointers (hipMalloc / torch CUDA tensors);
 *    pointers named h_* are host pointers.  The caller allocates every device
 *    buffer and keeps it alive until the handle that uses it is destroyed;
 *    the library never allocates or frees caller memory.  Handles (ds_model,
 *    ds_kv) are small host objects owned by the library.
 *  - `stream` is a hipStream_t passed as void*.  NULL means the default stream.
 *  - Arguments are checked on the host before any work is enqueued: a call
 *    that returns an error has enqueued nothing and changed no state.
 *  - Apart from creation calls, calls only enqueue work on `stream` and return
 *    without synchronising.
 *  - No C++ exception crosses this interface.  ds_last_error() gives a
 *    message for the last failing call on the calling thread.
 *  - A handle must not be used from two host threads at once.
 */
#ifndef DS_DECODE_H
#define DS_DECODE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    DS_OK = 0,
    DS_ERR_INVALID_ARG = -1,  /* null/inconsistent argument, slot out of range */
    DS_ERR_UNSUPPORTED = -2,  /* shape the kernels do not handle              */
    DS_ERR_ALIGNMENT = -3,    /* device pointer not 256-byte aligned           */
    DS_ERR_CONTEXT_FULL = -4, /* a sequence would pass its T positions         */
    DS_ERR_BAD_TOKEN = -5,    /* token id outside [0, vocab)                   */
    DS_ERR_WORKSPACE = -6,    /* a buffer is smaller than the size query says  */
    DS_ERR_HIP = -7,          /* a HIP runtime call failed                     */
    DS_ERR_STATE = -8,        /* call not valid in the handle's current state  */
    DS_ERR_DEVICE = -9        /* a device-side consistency check tripped       */
} ds_status;

/* Matrix storage.  DS_Q8 is block-quantised int8, the INT8 weight loading
 * that "simple-llm / kasahare" (section "Where to go from here") names as
 * its next step: a matrix [rows][cols] is int8 q[rows][cols] row-major, then,
 * from the next 256-byte boundary, fp32 s[rows][cols/32]; its element (r, c)
 * is s[r][c/32] * q[r][c].  dim, n_heads*head_dim and hidden_dim must be
 * multiples of 32.  DS_Q4 is the INT4 variant the same section names: the
 * values are packed two per byte (value c of a row in byte c/2, the low
 * nibble for even c), each a two's complement integer in [-8, 7], rows*cols/2
 * bytes row-major, then the scales as for DS_Q8.  DS_Q8 and DS_Q4 models run
 * one launch per operation at every batch size (no single-launch step, no
 * MFMA projections). */
typedef enum { DS_F32 = 0, DS_BF16 = 1, DS_Q8 = 2, DS_Q4 = 3 } ds_dtype;

/* Model shape.  The field order is part of the ABI. */
typedef struct {
    int32_t dim;             /* d: residual width                               */
    int32_t n_layers;        /* L                                               */
    int32_t n_heads;         /* H query heads                                   */
    int32_t n_kv_heads;      /* Hkv key/value heads; H % Hkv == 0               */
    int32_t head_dim;        /* D: 16, 32, 64, 128 or 256                       */
    int32_t hidden_dim;      /* F: SwiGLU width                                 */
    int32_t vocab_size;      /* V                                               */
    int32_t tied_embeddings; /* 1: logits use token_emb; 0: a separate wcls     */
    int32_t weight_dtype;    /* ds_dtype of every matrix; norm gains are fp32   */
    float rope_theta;        /* RoPE base                                       */
    float norm_eps;          /* RMSNorm epsilon                                 */
    int32_t cache_dtype;     /* DS_F32, or DS_BF16: a bf16 key/value cache      */
} ds_config;

typedef struct ds_model ds_model;
typedef struct ds_kv ds_kv;

/* ---- size and layout queries (host only, no HIP calls) ------------------ */

/* Canonical weight arena: one buffer holding, in this order and each tensor
 * starting on a 256-byte boundary, token_emb [V][d]; per layer attn_norm [d],
 * wq [H*D][d], wk [Hkv*D][d], wv [Hkv*D][d], wo [d][H*D], ffn_norm [d],
 * w1 [F][d], w3 [F][d], w2 [d][F]; output_norm [d]; and wcls [V][d] when
 * the embeddings are not tied.  This is the weight order of "simple-llm /
 * kasahare" (section "On-disk model format (.sllm)") with the untied head
 * appended.  Matrices are row-major [out][in] in weight_dtype (DS_Q8: the
 * values, then the scales, as above), gains fp32.
 * Returns 0 for an invalid config. */
size_t ds_weights_bytes(const ds_config* cfg);
/* Number of tensors in the arena (1 + 9L + 1, plus 1 when untied). */
int32_t ds_weights_count(const ds_config* cfg);
/* Byte offset of each arena tensor into h_off[0..n); n must be at least
 * ds_weights_count(cfg). */
ds_status ds_weights_offsets(const ds_config* cfg, size_t* h_off, int32_t n);
/* Device bytes of the key/value cache: a tensor of shape (L, 2, B, Hkv, T, D),
 * row-major (the (L,2,B,H,T,D) layout of "Inside nanochat Part 4", section
 * "Cache Architecture", with H = key/value heads), fp32, or bf16 when
 * cfg->cache_dtype is DS_BF16.  A bf16 cache holds every key and value row
 * rounded to bfloat16 (nearest, ties to even) when it is stored, and
 * attention reads the rounded values: the cache compression that
 * "simple-llm / kasahare" (section "Limitations (intentional)") leaves out.
 * It needs head_dim 64 or 128 and at most 4 query heads per key/value head,
 * and runs one launch per operation (no single-launch step). */
size_t ds_kv_cache_bytes(const ds_config* cfg, int32_t B, int32_t T);
/* Device scratch the library needs for a (B, T) cache. */
size_t ds_workspace_bytes(const ds_config* cfg, int32_t B, int32_t T);

/* ---- model ---------------------------------------------------------------- */

/* Binds a device weight arena (layout above, `arena_bytes` >= ds_weights_bytes)
 * to a model handle: the model load of "simple-llm / kasahare" (section
 * "Python binding": a model is loaded once from its weight file, then
 * called per token), with the weights already in device memory.  The arena
 * is read in place and must stay unchanged while the handle lives.  Checks:
 * cfg consistent (H % Hkv == 0; D one of 16, 32, 64, 128, 256; every matrix
 * row 16-byte aligned: dim, H*D and F times the weight size multiple of 16),
 * d_arena 256-byte aligned.  `stream` is unused (kept for symmetry).  *out
 * receives the handle, which the caller frees with ds_model_destroy.
 * Errors: DS_ERR_INVALID_ARG, DS_ERR_UNSUPPORTED (a shape the kernels do
 * not handle), DS_ERR_ALIGNMENT, DS_ERR_WORKSPACE (arena_bytes too small). */
ds_status ds_load_weights(const ds_config* cfg, const void* d_arena, size_t arena_bytes,
                          void* stream, ds_model** out);
void ds_model_destroy(ds_model* model);

/* ---- key/value cache ------------------------------------------------------ */

/* Binds a cache of B sequences with T positions each: the preallocated
 * (L, 2, B, H, T, D) cache of "Inside nanochat Part 4", section "Cache
 * Architecture" (H = key/value heads here), with one length per sequence
 * instead of that page's single position, because sequences of a batch may
 * hold different lengths.  d_cache: ds_kv_cache_bytes(cfg, B, T) bytes (fp32,
 * or bf16 values for a bf16 cache; the pointer type is float* either way);
 * d_lengths: int32[B], the number of cached positions per sequence;
 * d_workspace: ds_workspace_bytes(cfg, B, T) bytes.  All three are device
 * memory, 256-byte aligned, owned by the caller and kept alive until
 * ds_kv_cache_destroy.  Zeroes d_lengths, uploads the RoPE table into the
 * workspace and synchronises `stream` once.  The library never writes cache
 * rows at positions >= lengths[b]; the caller must not write d_lengths other
 * than through the calls below.  *out receives the handle.
 * Errors: DS_ERR_INVALID_ARG (NULL, B or T <= 0), DS_ERR_ALIGNMENT,
 * DS_ERR_WORKSPACE (a buffer smaller than its size query), DS_ERR_UNSUPPORTED
 * (the kernels need more LDS than the device gives), DS_ERR_HIP. */
ds_status ds_kv_cache_create(ds_model* model, int32_t B, int32_t T, float* d_cache,
                             size_t cache_bytes, int32_t* d_lengths, void* d_workspace,
                             size_t workspace_bytes, void* stream, ds_kv** out);
void ds_kv_cache_destroy(ds_kv* kv);
/* Empties sequence `seq` (or every sequence when seq == -1): lengths := 0,
 * as the cache reset of "Inside nanochat Part 4", section "KV Cache". */
ds_status ds_kv_cache_reset(ds_kv* kv, int32_t seq, void* stream);
/* Sets every lengths[b] from h_lengths[0..B) (each in [0, T]); used to rewind
 * or to resume from a saved cache. */
ds_status ds_kv_cache_set_lengths(ds_kv* kv, const int32_t* h_lengths, void* stream);
/* Cache replication ("Inside nanochat Part 4", section "Batch Prefilling
 * via Cache Replication": a batch-1 prefill copied into the rows of a
 * decode cache, for several completions of one prompt).  Copies the first
 * n = lengths[src_seq] positions of every layer's key and value rows of
 * sequence src_seq of `src` into sequences dst_first .. dst_first+count-1
 * of `dst`, and sets their lengths to n (device lengths and host mirror).
 * dst and src may be the same cache (the source slot then must not be a
 * destination).  Positions at or past n of the destinations are not
 * written.  Both caches must belong to models of equal layer count,
 * key/value heads and head dim.  Only enqueues work on `stream`.
 * Errors: DS_ERR_INVALID_ARG (shapes, slot ranges), DS_ERR_CONTEXT_FULL
 * (n > dst's T). */
ds_status ds_kv_cache_replicate(ds_kv* dst, const ds_kv* src, int32_t src_seq, int32_t dst_first, int32_t count,
                                void* stream);
/* Copies the host-side mirror of the lengths (no device access). */
ds_status ds_kv_cache_get_lengths(const ds_kv* kv, int32_t* h_lengths);
/* Synchronises `stream` and reports device-detected errors since the last
 * check, then clears them:
 *  - DS_ERR_DEVICE if a step's own consistency checks tripped: a wait of the
 *    single-launch batch-1 step gave up (every wait in it is bounded, about a
 *    second, so the launch always ends), or a launch-shape guard fired.  The
 *    steps since the last check are then not valid.
 *  - else DS_ERR_BAD_TOKEN if a decode step read a token id outside [0, V)
 *    (that sequence used row 0 instead). */
ds_status ds_kv_cache_check(ds_kv* kv, void* stream);

/* ---- the decode path ----------------------------------------------------- */

/* The prompt phase of "Inside nanochat Part 4", sections "Phase 1: Single
 * Prefill" and "Complete Generation Flow": the prompt's keys and values go
 * into the cache and the last position's logits give the first new token.
 * Feeds h_tokens[0..n) (host, each in [0, V)) to sequence `seq` at positions
 * lengths[seq] .. lengths[seq]+n-1, one position at a time through the same
 * kernels as ds_decode_step (so a prompt re-fed here reproduces decoded
 * steps bit for bit: the cached run of "GOTOken", section "About one token
 * per second"), and appends their keys and values.  A non-empty sequence is
 * extended.  After the call lengths[seq] has grown by n, d_tok_out[seq]
 * holds the greedy token of the last position and the logits of that
 * position are kept for ds_logits.  d_tok_out is device int32[B] (only entry
 * seq is written) and may be NULL.  The host tokens are read during the call.
 * Errors: DS_ERR_INVALID_ARG (seq out of range, n <= 0, NULL tokens),
 * DS_ERR_BAD_TOKEN (a token outside [0, V)), DS_ERR_CONTEXT_FULL if
 * lengths[seq] + n > T. */
ds_status ds_prefill(ds_model* model, ds_kv* kv, int32_t seq, const int32_t* h_tokens, int32_t n,
                     int32_t* d_tok_out, void* stream);

/* The same result as ds_prefill (within floating-point rounding), with the
 * prompt's positions run side by side: positions 0 .. n-2 go through the
 * layers as the items of one pass, up to 64 at a time (the projections as
 * matrix products over the positions, each position attending over the
 * cached rows up to and including its own), then the last position runs as
 * in ds_prefill and gives the token and logits.  This is the whole-prompt
 * forward pass with the query count above one of "Inside nanochat Part 4",
 * sections "Attention Mechanism Integration" and "Phase 1: Single Prefill".
 * Arguments, ownership and errors as for ds_prefill; lengths[seq] grows by n.
 * The result differs from ds_prefill's in rounding only (the projections of
 * 16 or more positions accumulate in another order).  Each pass's attention
 * covers the cached rows up to the pass's last position as the host has
 * recorded the sequence's length (the lengths ds_kv_cache_get_lengths
 * returns); should the device's lengths have moved past that record, the
 * launch-shape guard fires and the next ds_kv_cache_check returns
 * DS_ERR_DEVICE. */
ds_status ds_prefill_batched(ds_model* model, ds_kv* kv, int32_t seq, const int32_t* h_tokens, int32_t n,
                             int32_t* d_tok_out, void* stream);

/* Ragged prefill of many sequences at once: sequence b receives
 * h_counts[b] >= 0 tokens, taken in order from h_tokens (the concatenation
 * over b).  Position by position, every sequence that still has tokens is
 * advanced in one batched pass.  d_tok_out[b] is written for every b with
 * h_counts[b] > 0. */
ds_status ds_prefill_batch(ds_model* model, ds_kv* kv, const int32_t* h_tokens,
                           const int32_t* h_counts, int32_t* d_tok_out, void* stream);

/* One decode step for every sequence b in [0, B): the per-token loop of
 * "Inside nanochat Part 4", sections "Complete Generation Flow" and
 * "Greedy Decoding" (one new token per sequence, attending over the cached
 * keys and values, its own key and value appended), computed as the
 * pre-norm block of "simple-llm / kasahare", section "Architecture".  Reads
 * d_tok_in[b], runs the token at position lengths[b] through all layers,
 * appends its key and value rows to the cache at that position, writes the
 * greedy next token (the lowest index among equal maxima) to d_tok_out[b]
 * and advances lengths[b] by one.  d_tok_in and d_tok_out are device
 * int32[B]; they may be the same buffer.  The fp32 logits [B][V] of the step
 * stay in the workspace for ds_logits.  A token id outside [0, V) is
 * detected on the device: that sequence reads row 0 and the next
 * ds_kv_cache_check returns DS_ERR_BAD_TOKEN.
 * A step that the caller captures into a graph replays the launches chosen
 * for the context at capture: it stays valid while every context stays in
 * that class (batch 1: one 32-position chunk, or more, within
 * ds_kv_cache_single_launch_ctx; otherwise the fused short-context rows of
 * the capture, or split-K).  A replay outside it is reported, not computed
 * wrong in silence: the next ds_kv_cache_check returns DS_ERR_DEVICE.
 * Errors: DS_ERR_INVALID_ARG (NULL buffers, model/cache mismatch),
 * DS_ERR_ALIGNMENT, DS_ERR_CONTEXT_FULL if any lengths[b] == T, DS_ERR_HIP. */
ds_status ds_decode_step(ds_model* model, ds_kv* kv, const int32_t* d_tok_in, int32_t* d_tok_out,
                         void* stream);

/* Sampling epilogue ("Inside nanochat Part 4", section "Sampling Strategy":
 * temperature scaling and top-k filtering; "simple-llm / kasahare", section
 * "CLI flags": --top-p, read as the nucleus).  For every sequence b in
 * [0, B) it draws one token from the logits the last ds_decode_step /
 * ds_prefill left for b (rows of sequences that call did not advance hold
 * older logits) and writes it to d_tok_out[b] (device int32[B]).
 *  - The candidates: with top_k >= 1 the min(top_k, V) largest logits,
 *    largest first (equal logits: lower index first); with top_k == 0
 *    every token in index order.
 *  - Weights exp((l - l_max) / temperature); top_p < 1 (needs top_k >= 1)
 *    keeps the shortest prefix of the candidates whose weight reaches top_p
 *    times their total.
 *  - The draw is the inverse distribution function at d_uniform[b] (device
 *    fp32[B], the caller's uniform numbers in [0, 1); values outside are
 *    clamped into it): the first kept candidate whose running weight exceeds
 *    d_uniform[b] times the kept total.
 * Temperature 0 is greedy decoding, which ds_decode_step already does: pass
 * temperature > 0 here.  Only enqueues work on `stream`.
 * Errors: DS_ERR_INVALID_ARG (temperature <= 0, top_k < 0, top_p outside
 * (0, 1]), DS_ERR_UNSUPPORTED (top_k above 1024, or top_p < 1 with
 * top_k == 0), DS_ERR_ALIGNMENT. */
ds_status ds_sample(const ds_kv* kv, const float* d_uniform, float temperature, int32_t top_k, float top_p,
                    int32_t* d_tok_out, void* stream);

/* Rows of the library's own sampling scratch (ds_sample_noalloc). */
#define DS_SAMPLE_NOALLOC_MAX_ROWS 64

/* ds_sample for callers that cannot allocate device memory (code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc): the
 * same draw as ds_sample, with the same kernels and the same argument rules,
 * from caller-owned logits d_logits (device fp32 [B][V], row-major, 4-byte
 * aligned) instead of a cache's last step, into d_tok_out[b] (device
 * int32[B]), at the uniforms d_uniform[b] (device fp32[B]).  Its scratch is
 * not a workspace but a static device array inside the library,
 * DS_SAMPLE_NOALLOC_MAX_ROWS rows (2.5 MiB) that every device the library
 * runs on holds until the process ends; the call allocates nothing (no
 * hipMalloc, no library allocation).  Its device address is looked up once
 * per device: by ds_load_weights on the device current then, else by the
 * first call on that device.  Every call on one device shares that
 * device's array: calls that may overlap on one device (two streams, two
 * host threads) race and must be serialised by the caller.  No scratch
 * content carries from one call to the next.  B == 0 does nothing.
 * Errors: as ds_sample, plus DS_ERR_UNSUPPORTED for B above
 * DS_SAMPLE_NOALLOC_MAX_ROWS, DS_ERR_INVALID_ARG for B < 0 or V <= 0, and
 * DS_ERR_HIP if the scratch's device address cannot be obtained. */
ds_status ds_sample_noalloc(const float* d_logits, int32_t B, int32_t V, const float* d_uniform, float temperature,
                            int32_t top_k, float top_p, int32_t* d_tok_out, void* stream);

/* A decode step of some of the sequences: the n_rows distinct sequence ids
 * in h_rows (host int32, each in [0, B)) each read d_tok_in[row], append at
 * lengths[row], advance by one and get their greedy token in d_tok_out[row]
 * and their logits kept for ds_logits; every other sequence is left as it
 * is.  This is the per-row completion of "Inside nanochat Part 4", section
 * "Early Stopping Implementation": rows that have finished stop costing
 * work.  Always one launch per operation.  n_rows == 0 does nothing.
 * Errors: DS_ERR_INVALID_ARG (a row repeated or out of range),
 * DS_ERR_CONTEXT_FULL (a listed row already holds T positions). */
ds_status ds_decode_step_rows(ds_model* model, ds_kv* kv, const int32_t* h_rows, int32_t n_rows,
                              const int32_t* d_tok_in, int32_t* d_tok_out, void* stream);

/* Launch shape of batch-1 steps.  When B == 1 and the sequence holds at most
 * the returned number of positions after the step, ds_decode_step (and each
 * position of ds_prefill) runs as ONE persistent kernel launch that carries
 * the whole step -- every layer, the vocabulary product and the argmax --
 * with the phases of a layer handing their outputs to each other through
 * device memory instead of kernel boundaries.  Otherwise (B > 1, longer
 * contexts, shapes without a single-launch variant, a device that cannot hold
 * all 256 workgroups of the launch at once -- such as a partitioned GPU --, or
 * DS_PERSIST=0 in the environment when the cache was created) every operation
 * is its own launch.  The single launch occupies every CU while it runs; work
 * that other streams run at the same time can delay it, and if its workgroups
 * cannot all start, its bounded waits give up and the next ds_kv_cache_check
 * returns DS_ERR_DEVICE.  With DS_PERSIST_COOP=1 in the environment when the
 * cache was created, it is launched cooperatively instead (except while its
 * stream is being captured into a graph): the runtime then starts it only
 * with all its workgroups resident, at about 16 us more per step.
 * Both give the same results within floating-point rounding.  Returns 0 when
 * batch-1 steps never take the single launch.  No device access; never fails
 * for a valid handle (returns -1 for NULL). */
int32_t ds_kv_cache_single_launch_ctx(const ds_kv* kv);

/* The logits of the last position, as the per-token call of "simple-llm /
 * kasahare", section "Python binding", returns them (a (vocab,) fp32 vector
 * per call; here one row per sequence).  Copies the fp32 logits [B][V] of
 * the last prefill / decode step into d_out (device, B*V floats, row b =
 * sequence b, owned by the caller).  Rows of sequences that the last call
 * did not touch hold what they held before.  Only enqueues a device copy on
 * `stream`.  Errors: DS_ERR_INVALID_ARG (NULL), DS_ERR_HIP. */
ds_status ds_logits(const ds_kv* kv, float* d_out, void* stream);

/* Dispatch of ds_decode_step: 0 = one kernel launch per operation (eager),
 * 1 = the same launches captured once into a HIP graph per (stream, token
 * buffers) and replayed.  A step that is a single launch (batch 1 within
 * ds_kv_cache_single_launch_ctx) is launched directly in both modes.  The
 * default comes from the environment variable DS_DISPATCH ("eager" or
 * "graph"), else graph. */
ds_status ds_set_dispatch(ds_kv* kv, int32_t mode);

/* Diagnostics: enqueues `reps` back-to-back launches of one kernel of the
 * decode step -- 0 Q/K/V projection, 1 attention partials, 2 attention
 * combine, 3 Wo, 4 W1/W3, 5 W2, 6 vocabulary logits, or 7 the handoff floor
 * of the single-launch batch-1 step (its phases and handoff words with no
 * weight or cache loads, storing nothing outside its handoff words: no cache
 * row, logit, token or length changes; needs B == 1 and a next step that is
 * a single launch) -- with exactly the
 * arguments and launch shape of the last ds_decode_step on this cache (the
 * same positions are rewritten; Wo and W2 add to the residual again).
 * Launch r uses layer (layer + r) mod L, so consecutive launches stream
 * different weights and cache rows, as the step itself does.  Lets a caller
 * time one kernel with events on `stream`.
 * Errors: DS_ERR_STATE before the first ds_decode_step. */
ds_status ds_bench_kernel(ds_model* model, ds_kv* kv, int32_t which, int32_t layer, int32_t reps,
                          void* stream);

/* Diagnostics: enqueues `reps` launches of a plain streaming read of
 * `bytes` (a positive multiple of 16) from device memory d_src (16-byte
 * aligned): coalesced 16-byte loads, each byte read once per launch, and one
 * 32-bit word per block written to d_out (device, at least 2048 words, owned
 * by the caller).  Its time per launch, with events on `stream`, gives the
 * read bandwidth a kernel that does nothing else reaches: the measured peak
 * that streaming kernels are compared with.  Errors: DS_ERR_INVALID_ARG,
 * DS_ERR_ALIGNMENT, DS_ERR_HIP. */
ds_status ds_bench_stream(const void* d_src, size_t bytes, uint32_t* d_out, int32_t reps, void* stream);

/* Message for the last failing call on this thread ("" if none). */
const char* ds_last_error(void);

#ifdef __cplusplus
}
#endif
#endif
