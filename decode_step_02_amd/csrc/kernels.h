// kernels.h -- internal interface between the C-ABI host code and the kernels.
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include <vector>

namespace ds {

constexpr int kF32 = 0;
constexpr int kBF16 = 1;
constexpr int kChunk = 64;       // cache positions per attention block
constexpr int kMaxRep = 8;       // query heads per key/value head
constexpr int kMaxD = 256;       // head_dim limit of the attention kernel
constexpr int kMaxItems = 64;    // items per k_begin launch
constexpr int kSetChunk = 128;   // lengths per k_set_lengths launch

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
    float eps;
    const void* emb;
    float* cache;        // (L, 2, B, Hkv, T, D)
    int32_t* lengths;    // [B]
    // workspace
    float* x;            // [items][d]     residual stream
    float* q;            // [items][H*D]   rotated queries
    float* o;            // [items][H*D]   attention output
    float* h;            // [items][F]     silu(a)*u
    float* part_o;       // [items][H][n_chunks][D]
    float* part_ml;      // [items][H][n_chunks][2]
    float* logits;       // [B][V] by slot
    unsigned long long* keys;  // [items] argmax keys
    int32_t* slot;       // [items]
    int32_t* pos;        // [items]
    int32_t* flag;       // [items] 1: this item's logits and token are wanted
    int32_t* err;        // device error word
    const float* rope_cos;  // [T][D/2]
    const float* rope_sin;  // [T][D/2]
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
};

struct SetList {
    int first = 0;
    int n = 0;
    int32_t val[kSetChunk];
};

size_t attn_lds_bytes();
hipError_t set_kernel_attributes(int max_lds_bytes);
hipError_t enqueue_step(const StepArgs& s, const ModelPtrs& m, const BeginList* lists, int n_lists,
                        const int32_t* d_tok_in, int n_items, bool need_logits,
                        int32_t* d_tok_out, hipStream_t st);
// One launch of a single step kernel (0 qkv, 1 attn, 2 combine, 3 wo, 4 w13,
// 5 w2, 6 logits) with the arguments of a decode step over n_items items.
hipError_t enqueue_kernel(int which, int layer, const StepArgs& s, const ModelPtrs& m, int n_items,
                          hipStream_t st);
hipError_t enqueue_set_lengths(int32_t* d_lengths, const int32_t* h_vals, int first, int n,
                               hipStream_t st);
hipError_t enqueue_fill(int32_t* p, int n, int32_t v, hipStream_t st);

}  // namespace ds
