// kernels.h -- internal interface between the C-ABI host code and the kernels.
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include <vector>

namespace ds {

constexpr int kF32 = 0;
constexpr int kBF16 = 1;
constexpr int kQ8 = 2;   // int8 rows, then an fp32 scale per 32 values of a row
constexpr int kQ4 = 3;   // 4-bit values two per byte, then an fp32 scale per 32 values of a row
constexpr int kChunk = 64;       // cache positions per split-K attention block
constexpr int kShort = 64;       // contexts up to this many positions use the fused short path
constexpr int kMaxRep = 8;       // query heads per key/value head
constexpr int kMaxD = 256;       // head_dim limit of the attention kernels
constexpr int kMaxItems = 64;    // items per k_begin launch
constexpr int kSetChunk = 128;   // lengths per k_set_lengths launch
constexpr int kMaxArgmaxBlocks = 16384;  // vocabulary blocks per item (argmax partials)
constexpr int kPChunk = 32;      // positions per attention chunk of the persistent step
constexpr int kPMaxChunks = 64;  // 32-position attention chunks the persistent step can hold per head
constexpr int kPMaxParts = kPMaxChunks / 4;  // their partials, one per four chunks
constexpr int kPKeyWords = 1024; // argmax words of the persistent step (one per wave)
constexpr int kPRep = 8;         // most replicas of a vector the persistent step publishes
constexpr int kMaxTopK = 1024;   // largest top-k of the sampling epilogue
constexpr int kSampleMaxV = 1 << 20;  // largest vocabulary of the sampling epilogue
constexpr int kMmItems = 64;     // items per MFMA launch
constexpr int kMmMin = 16;       // steps with at least this many items use the MFMA projections

// Per-layer weight pointers (device), into the caller's arena.
struct LayerW {
    const float* attn_norm = nullptr;
    const void* wq = nullptr;
    const void* wk = nullptr;
    const void* wv = nullptr;
    const void* wo = nullptr;
    const float* ffn_norm = nullptr;
    const void* w1 = nullptr;
    const void* w3 = nullptr;
    const void* w2 = nullptr;
};

struct ModelPtrs {
    const void* emb = nullptr;
    const float* out_norm = nullptr;
    const void* wcls = nullptr;
    std::vector<LayerW> layers;
};

// Everything a step's kernels read besides the per-layer weights.
struct StepArgs {
    int d, L, H, Hkv, D, F, V, wdt;
    int B, T, n_chunks;
    int short_n;         // contexts up to this many positions take the fused short path (0: never)
    int cdt;             // cache element type: kF32, or kBF16 (rows rounded when stored)
    int mm_ok;           // shapes allow the MFMA projections
    int mm_split;        // the narrow projections may take the split-K MFMA kernel
    int attn_g;          // head_dim 64 / 128 attention takes the DPP-reduced kernel
    int attn_full;       // launches with many (item, group) pairs take the one-block-per-pair attention
    int attn_pf;         // passes whose items share one sequence (batched prefill) take k_attn_pf
    int kv_stream;       // cached key/value rows loaded with the non-temporal hint (no item shares another's rows)
    int pin;             // single-launch step's product input: kBF16 (hi/lo pairs) or kF32 (widened weights)
    int pcoop;           // single-launch step launched cooperatively (all workgroups resident, or no launch)
    float eps;
    const void* emb;
    float* cache;        // (L, 2, B, Hkv, T, D), fp32 or (cdt == kBF16) uint16 bf16 bits
    int32_t* lengths;    // [B]
    // workspace
    float* x;            // [items][d]     residual stream
    float* q;            // [items][H*D]   rotated queries
    float* o;            // [items][H*D]   attention output
    float* h;            // [items][F]     silu(a)*u
    float* part_o;       // [items][H][n_chunks][D]
    float* part_ml;      // [items][H][n_chunks][2]
    float* logits;       // [B][V] by slot
    unsigned long long* keys;  // [items][kMaxArgmaxBlocks] argmax partials
    int32_t* slot;       // [items]
    int32_t* pos;        // [items]
    int32_t* flag;       // [items] 1: this item's logits and token are wanted
    int32_t* err;        // device error word
    const float* rope_cos;  // [T][D/2]
    const float* rope_sin;  // [T][D/2]
};

// Device buffers of the persistent batch-1 step (persist.hip).
struct PersistArgs {
    const LayerW* layers;   // device copy of the per-layer pointers [L]
    const float* out_norm;
    const void* wcls;
    // ll_x, ll_x2, ll_qkv and ll_h hold kPRep replicas, rstride words apart
    uint64_t* ll_x;         // [d]      residual after W2 (value, epoch words)
    uint64_t* ll_x2;        // [d]      residual after Wo
    uint64_t* ll_qkv;       // [Hkv][(rep + 2) * D] per group: rotated queries, new key, new value
    uint64_t* ll_part;      // [Hkv][kPMaxParts][H/Hkv][D+2] attention partials (m, l, o)
    uint64_t* ll_h;         // [F]      silu(a)*u
    uint64_t* ll_keys;      // [kPKeyWords] argmax words
    uint64_t* ll_late;      // one word in a line of its own: the last layer has begun
    uint32_t* epoch;        // epoch base, advanced by every step
    int rstride;            // words between two replicas of a vector
};

// Items of one k_begin launch; by_value = 0 takes tokens from d_tok_in with
// item == slot (decode), 1 takes slots/tokens from the arrays (prefill).
struct BeginList {
    int n = 0;
    int item0 = 0;
    int by_value = 0;
    int32_t slot[kMaxItems];
    int32_t tok[kMaxItems];
    int32_t last[kMaxItems];
    int32_t off[kMaxItems] = {};  // by_value: position = lengths[slot] + off (several positions of one slot)
    int last_pos = -1;  // the positions of one slot: the last of them as the host knows it (-1: not known)
};
// by_value: 0 items are the slots 0..n-1 with tokens d_tok_in[slot]; 1 slots
// and tokens from the arrays (prefill); 2 slots from the array, tokens
// d_tok_in[slot] (a decode step of some of the sequences).

// Copies rows [0, n) of every (layer, k/v, group) of slot src_slot of one
// (L, 2, Bs, Hkv, Ts, D) cache to slots dst_first .. dst_first + count - 1
// of another (L, 2, Bd, Hkv, Td, D) cache (it may be the same one).
// Diagnostic streaming read of `bytes` (a multiple of 16) from src, reps
// times; out receives kStreamBlocks words.
constexpr int kStreamBlocks = 2048;
hipError_t enqueue_stream_read(const void* src, size_t bytes, uint32_t* out, int reps, hipStream_t st);

hipError_t enqueue_replicate(float* dst, int Bd, int Td, const float* src, int Bs, int Ts, int L, int Hkv, int D,
                             int src_slot, int dst_first, int count, int n, hipStream_t st);

struct SetList {
    int first = 0;
    int n = 0;
    int32_t val[kSetChunk];
};

// Kernel ids for enqueue_kernel (diagnostics)
enum KernelId { K_QKV = 0, K_ATTN = 1, K_COMBINE = 2, K_WO = 3, K_W13 = 4, K_W2 = 5, K_LOGITS = 6, K_FLOOR = 7 };

// (item, key/value group) pairs from which attention runs as one block per
// pair (k_attn_full: no partials, no combine launch) when s.attn_full is set
constexpr int kAttnFullMinBlocks = 128;
bool attn_full(const StepArgs& s, int n_items);

hipError_t set_kernel_attributes(int max_lds_bytes);
// One decode / prefill position for n_items items.  nload > 0: every item's
// context (pos + 1) is at most nload (<= short_n), and attention runs inside
// the Wo kernel on nload staged cache rows; nload == 0: split-K attention.
// d_tok_in != NULL marks a decode step (item i is slot i).
hipError_t enqueue_step(const StepArgs& s, const ModelPtrs& m, const BeginList* lists, int n_lists,
                        const int32_t* d_tok_in, int n_items, bool need_logits, int nload,
                        int32_t* d_tok_out, hipStream_t st);
// One launch of a single step kernel with the arguments of a decode step
// over n_items items (hipErrorInvalidValue if the kernel is not part of the
// step in that mode).
hipError_t enqueue_kernel(int which, int layer, const StepArgs& s, const ModelPtrs& m, int n_items, int nload,
                          hipStream_t st);
// Rows to stage for the short path given the longest context of a step:
// the smallest power of two >= max_ctx (at least 8, at most short_n, itself
// a power of two); 0 when max_ctx > short_n (split-K path).
inline int short_rows(const StepArgs& s, int max_ctx) {
    if (max_ctx > s.short_n) return 0;
    int n = 8;
    while (n < max_ctx) n *= 2;
    return n < s.short_n ? n : s.short_n;
}
hipError_t enqueue_set_lengths(int32_t* d_lengths, const int32_t* h_vals, int first, int n,
                               hipStream_t st);
hipError_t enqueue_fill(int32_t* p, int n, int32_t v, hipStream_t st);
size_t max_lds_bytes(const StepArgs& s);
// Persistent batch-1 step (persist.hip): the longest context it takes (0: none).
int persist_max_ctx(const StepArgs& s);
size_t persist_lds();
bool persist_fits_device(const StepArgs& s);  // all workgroups of the single launch can be resident
hipError_t persist_prepare(const StepArgs& s);
// One step of sequence 0 (B == 1): the token comes from d_tok_in[0], or from
// tok_value when d_tok_in is NULL; d_tok_out may be NULL.  ctx = the step's
// context (position + 1) picks the instantiation: one chunk (attention in
// the Wo blocks) or more (attention partials); a launch whose device
// context is of the other class flags error bit 2 and does nothing.
hipError_t enqueue_persist(const StepArgs& s, const PersistArgs& p, const int32_t* d_tok_in, int tok_value,
                           int32_t* d_tok_out, int ctx, hipStream_t st);
// The handoff floor of the single launch: the same phases and handoff words
// with no weight or cache loads and nothing stored outside the handoff words
// (no cache rows, logits, token or lengths).  Diagnostic only.
hipError_t enqueue_persist_floor(const StepArgs& s, const PersistArgs& p, int ctx, hipStream_t st);
// MFMA projections (mfma.hip): which = 0 qkv, 1 wo, 2 w13, 3 w2, 4 logits.
bool mm_supported(const StepArgs& s);
int mm_logits_blocks(const StepArgs& s);
size_t mm_max_lds(const StepArgs& s);
hipError_t mm_set_attributes(int lds);
// Attention of a pass whose n_items (<= 64) items are positions of one
// sequence (slot[0]): one block per (chunk, key/value group) on the matrix
// cores, partials for the merge launch.  head_dim 64 or 128, at most 4 query
// heads per key/value head, s.attn_pf set.  Blocks cover chunks [0,
// n_chunks) (1 <= n_chunks <= s.n_chunks); a pass whose last position on
// the device lies past them sets error bit 2 (launch shape).
bool attn_pf_supported(const StepArgs& s);
size_t attn_pf_lds(int D, int cdt, int rep);
hipError_t launch_attn_pf(const StepArgs& s, int layer, int n_items, int n_chunks, hipStream_t st);
hipError_t mm_gemv(int which, const StepArgs& s, const LayerW& w, int layer, int n_items, int ident,
                   const float* out_norm, const void* wcls, hipStream_t st);
// Longest context (a power of two <= min(kShort, T)) whose short-path staging fits in
// 64 KiB of LDS; 0 if head_dim/4 is not a power of two.
int short_positions(const StepArgs& s);

// Sampling epilogue (sample.hip): temperature > 0, 0 <= top_k <= kMaxTopK
// (0: every token), 0 < top_p <= 1 (below 1 only with top_k >= 1).
struct SampleParams {
    float temperature;
    int top_k;
    float top_p;
};
// scratch: row_words 64-bit words per row (at least sample_scratch_words()
// for the two-kernel path; the argmax-key region of the workspace).
size_t sample_scratch_words();
hipError_t enqueue_sample(const float* logits, int B, int V, const float* d_uniform, SampleParams prm,
                          uint64_t* scratch, size_t row_words, int32_t* d_tok_out, hipStream_t st);

}  // namespace ds
