// sample.hip -- the sampling epilogue: one token per sequence drawn from the
// logits a step left in the workspace ("Inside nanochat Part 4", section
// "Sampling Strategy": temperature scaling, top-k filtering, the two
// combined; "simple-llm / kasahare", section "CLI flags": --top-p, read as
// the nucleus of the sorted candidates).  The uniform draw of each sequence
// is an input, so the result is a function of (logits, parameters, u).
//
// Definition (the same as the oracle's orc_sample):
//  - top_k >= 1: the candidates are the top_k largest logits, largest
//    first, equal logits by lower index; top_k == 0: every token in index
//    order (top_p must be 1).
//  - Weights exp((l - l_max) / temperature), summed in draw order; top_p
//    keeps the shortest prefix whose weight reaches top_p times the total;
//    the token is the first kept candidate whose running sum exceeds u
//    times the kept total.
//
// Keys: each logit gets a 64-bit key, order-preserving float bits above the
// complemented index, so keys are distinct and larger means earlier.
//
// Two kernels spread a row over the chip:
//  - k_sample_part, one workgroup per 1024-logit slice of a row: the slice's
//    max and weight sum (top_k == 0), or its own top-k keys, found by the
//    same radix select (top_k >= 1);
//  - k_sample_merge, one workgroup per row: merges the slices and draws.  For
//    top_k >= 1 the union of the slices' top-k holds the row's top-k; an
//    MSB-first radix select (8 passes of 8 bits) over it finds the k-th key,
//    and the k keys at or above it are sorted.
// k_sample does it all in one workgroup per row, streaming the logits, for
// top-k lists too long for the merge (slices * k above kCap).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kernels.h"

namespace ds {

namespace {

constexpr int kST = 1024;           // threads of a row workgroup
constexpr int kSW = kST / 64;       // its waves
constexpr int kCap = 4096;          // LDS room for candidate keys
constexpr int kPer = 16;            // logits per thread in one batch of loads (k_sample)
constexpr int kSlice = 1024;        // logits per k_sample_part workgroup
constexpr int kPT = 256;            // its threads
constexpr int kMaxSlices = kSampleMaxV / kSlice;
static_assert(kSlice == kST, "k_sample_merge scans a slice with one logit per thread");

__device__ __forceinline__ uint64_t sample_key(float v, int i) {
    uint32_t u = __float_as_uint(v);
    u = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
    return (static_cast<uint64_t>(u) << 32) | static_cast<uint32_t>(~static_cast<uint32_t>(i));
}
__device__ __forceinline__ float key_value(uint64_t k) {
    uint32_t u = static_cast<uint32_t>(k >> 32);
    u = (u & 0x80000000u) ? (u & 0x7FFFFFFFu) : ~u;
    return __uint_as_float(u);
}
__device__ __forceinline__ int key_index(uint64_t k) {
    return static_cast<int>(~static_cast<uint32_t>(k));
}

// Block reductions and scans for NW waves (the whole workgroup calls them).
template <int NW>
__device__ float block_scan(float v, float* red, float* total) {
    const int t = threadIdx.x, lane = t & 63, w = t >> 6;
    float x = v;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const float y = __shfl_up(x, o);
        if (lane >= o) x += y;
    }
    if (lane == 63) red[w] = x;
    __syncthreads();
    float off = 0.f, all = 0.f;
    for (int i = 0; i < NW; i++) {
        if (i < w) off += red[i];
        all += red[i];
    }
    *total = all;
    __syncthreads();
    return off + x;
}

template <int NW>
__device__ float block_max(float v, float* red) {
    for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
    __syncthreads();
    float m = red[0];
    for (int i = 1; i < NW; i++) m = fmaxf(m, red[i]);
    __syncthreads();
    return m;
}

template <int NW>
__device__ int block_min_int(int v, int* red) {
    for (int o = 32; o > 0; o >>= 1) v = min(v, __shfl_xor(v, o));
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
    __syncthreads();
    int m = red[0];
    for (int i = 1; i < NW; i++) m = min(m, red[i]);
    __syncthreads();
    return m;
}

// One radix step: given hist[256] of the digits of the keys still in play
// and rem (the rank, from the top, of the wanted key among them), the
// chosen digit and the rank left within it go to *dig / *rem_out.  Wave 0
// does it alone: lane l holds digits 4l .. 4l+3 and a suffix scan over the
// lanes gives every digit its count from the top.  Starts and ends with a
// barrier.
__device__ void pick_digit(const uint32_t* hist, uint32_t rem, uint32_t* dig, uint32_t* rem_out) {
    __syncthreads();
    const int t = threadIdx.x;
    if (t < 64) {
        const uint32_t c0 = hist[4 * t], c1 = hist[4 * t + 1], c2 = hist[4 * t + 2], c3 = hist[4 * t + 3];
        const uint32_t mine = (c0 + c1) + (c2 + c3);
        uint32_t x = mine;  // sum over lanes >= t
#pragma unroll
        for (int o = 1; o < 64; o <<= 1) {
            const uint32_t y = __shfl_down(x, o);
            if (t + o < 64) x += y;
        }
        const uint32_t s3 = x - mine + c3, s2 = s3 + c2, s1 = s2 + c1, s0 = s1 + c0;  // counts from the top
        if (s3 >= rem && s3 - c3 < rem) { *dig = 4 * t + 3; *rem_out = rem - (s3 - c3); }
        if (s2 >= rem && s2 - c2 < rem) { *dig = 4 * t + 2; *rem_out = rem - (s2 - c2); }
        if (s1 >= rem && s1 - c1 < rem) { *dig = 4 * t + 1; *rem_out = rem - (s1 - c1); }
        if (s0 >= rem && s0 - c0 < rem) { *dig = 4 * t;     *rem_out = rem - (s0 - c0); }
    }
    __syncthreads();
}

// Radix select over the n keys at cand[0..n) (in LDS, NT threads): a
// threshold such that exactly k keys are >= it (1 <= k <= n; the keys are
// distinct).  That is the k-th largest key itself, unless a pass finds that
// every key left in the chosen digit's bucket is among the k: then the
// prefix so far, with the lower bits zero, already separates them, and the
// remaining passes are skipped (with distinct logits that is usually the
// case once the 32 value bits are resolved, after half the passes).
template <int NT>
__device__ uint64_t radix_kth(const uint64_t* cand, int n, int k, uint32_t* hist, uint32_t* sh_dig,
                              uint32_t* sh_rem) {
    const int t = threadIdx.x;
    uint64_t prefix = 0, mask = 0;
    uint32_t rem = static_cast<uint32_t>(k);
    for (int pass = 0; pass < 8; pass++) {
        const int shift = 56 - 8 * pass;
        for (int i = t; i < 256; i += NT) hist[i] = 0u;
        __syncthreads();
        for (int i = t; i < n; i += NT) {
            const uint64_t key = cand[i];
            if ((key & mask) == prefix) atomicAdd(&hist[(key >> shift) & 0xFF], 1u);
        }
        pick_digit(hist, rem, sh_dig, sh_rem);
        const uint32_t dig = *sh_dig;
        prefix |= static_cast<uint64_t>(dig) << shift;
        mask |= static_cast<uint64_t>(0xFF) << shift;
        rem = *sh_rem;
        const bool whole = hist[dig] == rem;  // the bucket is all in (uniform)
        __syncthreads();  // before the next pass clears hist
        if (whole) break;
    }
    return prefix;
}

// Sort list[0..n) descending (bitonic; entries n .. NP-1, NP the power of
// two >= n, are set to 0, which sorts last); NT threads.
template <int NT>
__device__ void sort_desc(uint64_t* list, int n) {
    const int t = threadIdx.x;
    const int NP = n <= 1 ? 1 : 1 << (32 - __clz(n - 1));
    for (int i = n + t; i < NP; i += NT) list[i] = 0ull;
    __syncthreads();
    for (int size = 2; size <= NP; size <<= 1) {
        for (int stride = size >> 1; stride > 0; stride >>= 1) {
            for (int i = t; i < NP; i += NT) {
                const int j = i ^ stride;
                if (j > i) {
                    const bool desc = (i & size) == 0;
                    const uint64_t a = list[i], c = list[j];
                    if (desc ? a < c : a > c) {
                        list[i] = c;
                        list[j] = a;
                    }
                }
            }
            __syncthreads();
        }
    }
}

// The draw over the k (<= kST) sorted candidate keys list[0..k): weights,
// the top-p cut, the inverse distribution function at u.  kST threads.
__device__ int draw_sorted(const uint64_t* list, int k, float inv_t, float top_p, float u, float* redf, int* redi) {
    const int t = threadIdx.x;
    const bool mine = t < k;  // one candidate per thread
    const float lmax = key_value(list[0]);
    const float w = mine ? expf((key_value(list[t]) - lmax) * inv_t) : 0.f;
    float total;
    const float incl = block_scan<kSW>(w, redf, &total);
    int cut = k - 1;
    if (top_p < 1.0f) cut = min(block_min_int<kSW>(mine && incl >= top_p * total ? t : k, redi), k - 1);
    if (t == cut) redf[0] = incl;  // the kept total
    __syncthreads();
    const float target = u * redf[0];
    __syncthreads();
    const int pick = min(block_min_int<kSW>(mine && t <= cut && incl > target ? t : k, redi), cut);
    return key_index(list[pick]);
}

// The k keys at or above the k-th largest of cand[0..n) (in LDS), sorted,
// into list.  kST threads.
__device__ void select_sorted(const uint64_t* cand, int n, int k, uint64_t* list, uint32_t* hist, uint32_t* sh_dig,
                              uint32_t* sh_rem, uint32_t* n_list) {
    const int t = threadIdx.x;
    const uint64_t kth = radix_kth<kST>(cand, n, k, hist, sh_dig, sh_rem);
    if (t == 0) *n_list = 0u;
    __syncthreads();
    for (int i = t; i < n; i += kST) {
        const uint64_t key = cand[i];
        if (key >= kth) {
            const uint32_t at = atomicAdd(n_list, 1u);  // k in all (the keys are distinct)
            if (at < static_cast<uint32_t>(kMaxTopK)) list[at] = key;
        }
    }
    __syncthreads();
    sort_desc<kST>(list, k);
}

// One tile of the logits: kPer elements per thread, all loads issued before
// any is used (one memory latency per tile), strided: base + j*kST + t.
__device__ __forceinline__ void load_tile(const float* lg, int V, int base, float (&v)[kPer]) {
#pragma unroll
    for (int j = 0; j < kPer; j++) {
        const int e = base + j * kST + static_cast<int>(threadIdx.x);
        v[j] = e < V ? lg[e] : -INFINITY;
    }
}

}  // namespace

// ---- two-kernel path ------------------------------------------------------------------------
// Scratch per row (row_words 64-bit words; the workspace's argmax-key
// region, which nothing reads between steps): kMaxSlices (max, weight sum)
// pairs, then slices * min(k, kSlice) keys.
__global__ __launch_bounds__(kPT) void k_sample_part(const float* __restrict__ logits, int V, SampleParams prm,
                                                     uint64_t* __restrict__ scratch, int row_words) {
    __shared__ uint64_t keys[kSlice];
    __shared__ uint32_t hist[256];
    __shared__ uint32_t sh_dig, sh_rem, n_out;
    __shared__ float redf[kPT / 64];
    const int s = blockIdx.x, b = blockIdx.y, t = threadIdx.x;
    const float* lg = logits + static_cast<size_t>(b) * V + static_cast<size_t>(s) * kSlice;
    const int n = min(kSlice, V - s * kSlice);
    uint64_t* row = scratch + static_cast<size_t>(b) * row_words;
    float v[kSlice / kPT];
#pragma unroll
    for (int j = 0; j < kSlice / kPT; j++) {
        const int e = j * kPT + t;
        v[j] = e < n ? lg[e] : -INFINITY;
    }
    if (prm.top_k == 0) {
        float m = -INFINITY;
#pragma unroll
        for (int j = 0; j < kSlice / kPT; j++) m = fmaxf(m, v[j]);
        m = block_max<kPT / 64>(m, redf);
        const float inv_t = 1.0f / prm.temperature;
        float w = 0.f;
#pragma unroll
        for (int j = 0; j < kSlice / kPT; j++) w += (j * kPT + t < n) ? expf((v[j] - m) * inv_t) : 0.f;
        float tot;
        block_scan<kPT / 64>(w, redf, &tot);
        if (t == 0) reinterpret_cast<float2*>(row)[s] = make_float2(m, tot);
        return;
    }
    const int kk = min(prm.top_k, kSlice);
    const int nk = min(kk, n);  // keys this slice hands on (any order)
#pragma unroll
    for (int j = 0; j < kSlice / kPT; j++) {
        const int e = j * kPT + t;
        if (e < n) keys[e] = sample_key(v[j], s * kSlice + e);
    }
    __syncthreads();
    const uint64_t kth = radix_kth<kPT>(keys, n, nk, hist, &sh_dig, &sh_rem);
    if (t == 0) n_out = 0u;
    __syncthreads();
    uint64_t* out = row + kMaxSlices + static_cast<size_t>(s) * kk;
    for (int i = t; i < n; i += kPT) {
        const uint64_t key = keys[i];
        if (key >= kth) {
            const uint32_t at = atomicAdd(&n_out, 1u);  // nk in all
            if (at < static_cast<uint32_t>(nk)) out[at] = key;
        }
    }
}

__global__ __launch_bounds__(kST) void k_sample_merge(const float* __restrict__ logits, int V,
                                                      const float* __restrict__ uni, SampleParams prm,
                                                      const uint64_t* __restrict__ scratch, int row_words,
                                                      int32_t* __restrict__ tok_out) {
    __shared__ uint64_t list[kMaxTopK];
    __shared__ uint64_t cand[kCap];
    __shared__ uint32_t hist[256];
    __shared__ uint32_t sh_dig, sh_rem, n_list;
    __shared__ float redf[kSW];
    __shared__ int redi[kSW];
    const int b = blockIdx.x, t = threadIdx.x;
    const int G = (V + kSlice - 1) / kSlice;
    const uint64_t* row = scratch + static_cast<size_t>(b) * row_words;
    const float inv_t = 1.0f / prm.temperature;
    const float u = fminf(fmaxf(uni[b], 0.f), 0x1.fffffep-1f);
    if (prm.top_k == 0) {
        // slice weights in slice order (G <= kST: one slice per thread); then the slice and the element
        const float2 ms = t < G ? reinterpret_cast<const float2*>(row)[t] : make_float2(-INFINITY, 0.f);
        const float M = block_max<kSW>(ms.x, redf);
        const float ws = t < G ? ms.y * expf((ms.x - M) * inv_t) : 0.f;
        float S;
        const float incl = block_scan<kSW>(ws, redf, &S);
        const float target = u * S;
        const int sl = min(block_min_int<kSW>(t < G && incl > target ? t : G, redi), G - 1);
        if (t == sl) redf[0] = incl - ws;  // the running sum before slice sl
        __syncthreads();
        const float before = redf[0];
        __syncthreads();
        const int e = sl * kSlice + t;  // one logit per thread
        const float w = e < V ? expf((logits[static_cast<size_t>(b) * V + e] - M) * inv_t) : 0.f;
        float tot;
        const float run = before + block_scan<kSW>(w, redf, &tot);
        const int last = min(sl * kSlice + kSlice, V) - 1;
        const int pick = min(block_min_int<kSW>(e < V && run > target ? e : V, redi), last);
        if (t == 0) tok_out[b] = pick;
        return;
    }
    const int kk = min(prm.top_k, kSlice);
    const int k = min(prm.top_k, V);
    // the union of the slices' own top-k: contiguous in the scratch row (only
    // the last slice may hold fewer keys), at most kCap, loaded in one batch
    const int n = (G - 1) * kk + min(kk, V - (G - 1) * kSlice);
    uint64_t got[kCap / kST];
#pragma unroll
    for (int r = 0; r < kCap / kST; r++) {
        const int i = t + r * kST;
        got[r] = i < n ? row[kMaxSlices + i] : 0ull;
    }
#pragma unroll
    for (int r = 0; r < kCap / kST; r++)
        if (t + r * kST < n) cand[t + r * kST] = got[r];
    __syncthreads();
    select_sorted(cand, n, k, list, hist, &sh_dig, &sh_rem, &n_list);
    const int tok = draw_sorted(list, k, inv_t, prm.top_p, u, redf, redi);
    if (t == 0) tok_out[b] = tok;
}

// ---- one-workgroup path (long top-k lists) ----------------------------------------------------
__global__ __launch_bounds__(kST) void k_sample(const float* __restrict__ logits, int V, const float* __restrict__ uni,
                                                SampleParams prm, int32_t* __restrict__ tok_out) {
    __shared__ uint64_t list[kMaxTopK];
    __shared__ uint64_t cand[kCap];
    __shared__ uint32_t whist[kSW][256];  // a histogram per wave, summed into whist[0]
    __shared__ uint32_t sh_dig, sh_rem, n_list, n_cand;
    __shared__ float redf[kSW];
    __shared__ int redi[kSW];
    const int b = blockIdx.x, t = threadIdx.x, wv = t >> 6;
    const float* lg = logits + static_cast<size_t>(b) * V;
    const float inv_t = 1.0f / prm.temperature;
    const float u = fminf(fmaxf(uni[b], 0.f), 0x1.fffffep-1f);
    constexpr int TILE = kST * kPer;
    const int k = min(prm.top_k, V);
    uint32_t* hist = whist[0];
    // pass 0 over every logit: the top byte of the k-th key (per-wave histograms)
    for (int i = t; i < kSW * 256; i += kST) (&whist[0][0])[i] = 0u;
    __syncthreads();
    for (int base = 0; base < V; base += TILE) {
        float v[kPer];
        load_tile(lg, V, base, v);
#pragma unroll
        for (int j = 0; j < kPer; j++) {
            const int e = base + j * kST + t;
            if (e < V) atomicAdd(&whist[wv][static_cast<uint32_t>(sample_key(v[j], e) >> 56)], 1u);
        }
    }
    __syncthreads();
    if (t < 256) {
        uint32_t c = 0;
        for (int w = 0; w < kSW; w++) c += whist[w][t];
        hist[t] = c;
    }
    __syncthreads();
    pick_digit(hist, static_cast<uint32_t>(k), &sh_dig, &sh_rem);
    const uint32_t d0 = sh_dig;
    uint32_t rem = sh_rem;
    // keys above that byte are in; keys with it are the candidates for the rest
    if (t == 0) {
        n_list = 0u;
        n_cand = 0u;
    }
    __syncthreads();
    for (int base = 0; base < V; base += TILE) {
        float v[kPer];
        load_tile(lg, V, base, v);
#pragma unroll
        for (int j = 0; j < kPer; j++) {
            const int e = base + j * kST + t;
            const uint64_t key = sample_key(v[j], e);
            const uint32_t top = static_cast<uint32_t>(key >> 56);
            if (e < V && top > d0) {
                const uint32_t at = atomicAdd(&n_list, 1u);
                if (at < static_cast<uint32_t>(kMaxTopK)) list[at] = key;
            } else if (e < V && top == d0) {
                const uint32_t at = atomicAdd(&n_cand, 1u);
                if (at < static_cast<uint32_t>(kCap)) cand[at] = key;
            }
        }
    }
    __syncthreads();
    const int nc = static_cast<int>(n_cand);
    const bool in_lds = nc <= kCap;  // else the remaining passes read the logits again
    uint64_t prefix = static_cast<uint64_t>(d0) << 56, mask = 0xFF00000000000000ull;
    for (int pass = 1; pass < 8; pass++) {
        const int shift = 56 - 8 * pass;
        if (t < 256) hist[t] = 0u;
        __syncthreads();
        if (in_lds) {
            for (int i = t; i < nc; i += kST) {
                const uint64_t key = cand[i];
                if ((key & mask) == prefix) atomicAdd(&hist[(key >> shift) & 0xFF], 1u);
            }
        } else {
            for (int base = 0; base < V; base += TILE) {
                float v[kPer];
                load_tile(lg, V, base, v);
#pragma unroll
                for (int j = 0; j < kPer; j++) {
                    const int e = base + j * kST + t;
                    const uint64_t key = sample_key(v[j], e);
                    if (e < V && (key & mask) == prefix) atomicAdd(&hist[(key >> shift) & 0xFF], 1u);
                }
            }
        }
        __syncthreads();
        pick_digit(hist, rem, &sh_dig, &sh_rem);
        prefix |= static_cast<uint64_t>(sh_dig) << shift;
        mask |= static_cast<uint64_t>(0xFF) << shift;
        rem = sh_rem;
        __syncthreads();
    }
    // prefix is the k-th largest key: the candidates at or above it join the list
    if (in_lds) {
        for (int i = t; i < nc; i += kST) {
            const uint64_t key = cand[i];
            if (key >= prefix) {
                const uint32_t at = atomicAdd(&n_list, 1u);  // k in all (the keys are distinct)
                if (at < static_cast<uint32_t>(kMaxTopK)) list[at] = key;
            }
        }
    } else {
        for (int base = 0; base < V; base += TILE) {
            float v[kPer];
            load_tile(lg, V, base, v);
#pragma unroll
            for (int j = 0; j < kPer; j++) {
                const int e = base + j * kST + t;
                const uint64_t key = sample_key(v[j], e);
                if (e < V && static_cast<uint32_t>(key >> 56) == d0 && key >= prefix) {
                    const uint32_t at = atomicAdd(&n_list, 1u);
                    if (at < static_cast<uint32_t>(kMaxTopK)) list[at] = key;
                }
            }
        }
    }
    __syncthreads();
    sort_desc<kST>(list, k);
    const int tok = draw_sorted(list, k, inv_t, prm.top_p, u, redf, redi);
    if (t == 0) tok_out[b] = tok;
}

size_t sample_scratch_words() { return static_cast<size_t>(kMaxSlices) + kCap; }

hipError_t enqueue_sample(const float* logits, int B, int V, const float* d_uniform, SampleParams prm,
                          uint64_t* scratch, size_t row_words, int32_t* d_tok_out, hipStream_t st) {
    const int G = (V + kSlice - 1) / kSlice;
    const long kk = prm.top_k < kSlice ? prm.top_k : kSlice;
    const bool two = row_words >= sample_scratch_words() && (prm.top_k == 0 ? G <= kST : G * kk <= kCap);
    if (two) {
        hipLaunchKernelGGL(k_sample_part, dim3(G, B), dim3(kPT), 0, st, logits, V, prm, scratch,
                           static_cast<int>(row_words));
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
        hipLaunchKernelGGL(k_sample_merge, dim3(B), dim3(kST), 0, st, logits, V, d_uniform, prm, scratch,
                           static_cast<int>(row_words), d_tok_out);
        return hipGetLastError();
    }
    if (prm.top_k == 0) return hipErrorInvalidValue;  // needs the two-kernel path
    hipLaunchKernelGGL(k_sample, dim3(B), dim3(kST), 0, st, logits, V, d_uniform, prm, d_tok_out);
    return hipGetLastError();
}

}  // namespace ds
