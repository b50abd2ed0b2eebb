// sample.hip -- the sampling epilogue: one token per sequence drawn from the
// logits a step left in the workspace ("Inside nanochat Part 4", section
// "Sampling Strategy": temperature scaling, top-k filtering, the two
// combined; "simple-llm / kasahare", section "CLI flags": --top-p, read as
// the nucleus of the sorted candidates).  The uniform draw of each sequence
// is an input, so the result is a function of (logits, parameters, u).
//
// One workgroup of 256 threads per sequence.
//  - top_k >= 1: the candidates are the top_k largest logits, largest
//    first, equal logits by lower index.  Each logit gets a 64-bit key,
//    order-preserving float bits above the complemented index, so keys are
//    distinct and larger means earlier.  An MSB-first radix select (8 passes
//    of 8 bits, histograms in LDS) finds the k-th largest key; the keys at
//    or above it are gathered and bitonic-sorted in LDS.
//  - top_k == 0: every token in index order (top_p must be 1).
// Weights exp((l - l_max) / temperature) are summed in draw order (a block
// scan); top_p keeps the shortest prefix whose weight reaches top_p times
// the total; the token is the first kept candidate whose running sum
// exceeds u times the kept total.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kernels.h"

namespace ds {

namespace {

constexpr int kST = 256;  // threads per sampling workgroup

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

// inclusive scan of one value per thread (thread order); returns this
// thread's inclusive prefix, *total gets the sum of all
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
    float off = 0.f;
    for (int i = 0; i < w; i++) off += red[i];
    *total = (red[0] + red[1]) + (red[2] + red[3]);
    __syncthreads();
    return off + x;
}

__device__ float block_max(float v, float* red) {
    for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
    __syncthreads();
    const float m = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
    __syncthreads();
    return m;
}

__device__ int block_min_int(int v, int* red) {
    for (int o = 32; o > 0; o >>= 1) v = min(v, __shfl_xor(v, o));
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
    __syncthreads();
    const int m = min(min(red[0], red[1]), min(red[2], red[3]));
    __syncthreads();
    return m;
}

}  // namespace

__global__ __launch_bounds__(kST) void k_sample(const float* __restrict__ logits, int V, const float* __restrict__ uni,
                                                SampleParams prm, int32_t* __restrict__ tok_out) {
    __shared__ uint64_t list[kMaxTopK];
    __shared__ uint32_t hist[256];
    __shared__ uint32_t pick_digit, pick_rem, count;
    __shared__ float redf[4];
    __shared__ int redi[4];
    const int b = blockIdx.x, t = threadIdx.x;
    const float* lg = logits + static_cast<size_t>(b) * V;
    const float inv_t = 1.0f / prm.temperature;
    const float u = fminf(fmaxf(uni[b], 0.f), 0x1.fffffep-1f);

    if (prm.top_k == 0) {
        // every token, index order: thread t sums the contiguous chunk [t*C, t*C + C)
        const int C = (V + kST - 1) / kST;
        const int i0 = min(t * C, V), i1 = min(i0 + C, V);
        float m = -INFINITY;
        for (int i = i0; i < i1; i++) m = fmaxf(m, lg[i]);
        m = block_max(m, redf);
        float s = 0.f;
        for (int i = i0; i < i1; i++) s += expf((lg[i] - m) * inv_t);
        float total;
        const float incl = block_scan(s, redf, &total);
        const float target = u * total;
        const float excl = incl - s;
        // the chunk holding the target; the last token if rounding leaves none
        int pick = V;
        if (excl <= target && target < incl) {
            float run = excl;
            for (int i = i0; i < i1; i++) {
                run += expf((lg[i] - m) * inv_t);
                if (run > target) {
                    pick = i;
                    break;
                }
            }
            if (pick == V) pick = i1 - 1;
        }
        pick = block_min_int(pick, redi);
        if (t == 0) tok_out[b] = pick < V ? pick : V - 1;
        return;
    }

    // ---- top-k: radix select of the k-th largest key --------------------------------------------
    const int k = min(prm.top_k, V);
    uint64_t prefix = 0, mask = 0;
    uint32_t rem = static_cast<uint32_t>(k);
    for (int pass = 0; pass < 8; pass++) {
        const int shift = 56 - 8 * pass;
        hist[t] = 0u;
        __syncthreads();
        for (int i = t; i < V; i += kST) {
            const uint64_t key = sample_key(lg[i], i);
            if ((key & mask) == prefix) atomicAdd(&hist[(key >> shift) & 0xFF], 1u);
        }
        __syncthreads();
        // suffix sums over the digits (largest digit first), one digit per thread
        uint32_t mine = hist[t];
        __syncthreads();
        uint32_t suf = mine;
        for (int o = 1; o < 256; o <<= 1) {
            hist[t] = suf;
            __syncthreads();
            if (t + o < 256) suf += hist[t + o];
            __syncthreads();
        }
        if (suf >= rem && suf - mine < rem) {
            pick_digit = static_cast<uint32_t>(t);
            pick_rem = rem - (suf - mine);
        }
        __syncthreads();
        prefix |= static_cast<uint64_t>(pick_digit) << shift;
        mask |= static_cast<uint64_t>(0xFF) << shift;
        rem = pick_rem;
        __syncthreads();
    }
    // prefix is the k-th largest key: gather the k keys at or above it
    if (t == 0) count = 0u;
    const int NP = k <= 1 ? 1 : 1 << (32 - __clz(k - 1));  // power of two >= k
    for (int i = t; i < NP; i += kST) list[i] = 0ull;      // padding sorts last
    __syncthreads();
    for (int i = t; i < V; i += kST) {
        const uint64_t key = sample_key(lg[i], i);
        if (key >= prefix) {
            const uint32_t at = atomicAdd(&count, 1u);  // exactly k (the keys are distinct)
            if (at < static_cast<uint32_t>(kMaxTopK)) list[at] = key;
        }
    }
    __syncthreads();
    // bitonic sort, descending
    for (int size = 2; size <= NP; size <<= 1) {
        for (int stride = size >> 1; stride > 0; stride >>= 1) {
            for (int i = t; i < NP; i += kST) {
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
    // weights in sorted order: thread t holds the consecutive candidates [t*E, t*E + E)
    const int E = (k + kST - 1) / kST;
    const int j0 = min(t * E, k), j1 = min(j0 + E, k);
    const float lmax = key_value(list[0]);
    float s = 0.f;
    for (int j = j0; j < j1; j++) s += expf((key_value(list[j]) - lmax) * inv_t);
    float total;
    const float incl = block_scan(s, redf, &total);
    // top-p: the first candidate whose running sum reaches top_p * total
    int cut = k - 1;
    if (prm.top_p < 1.0f) {
        const float need = prm.top_p * total;
        int c = k;
        float run = incl - s;
        for (int j = j0; j < j1; j++) {
            run += expf((key_value(list[j]) - lmax) * inv_t);
            if (run >= need) {
                c = j;
                break;
            }
        }
        cut = min(block_min_int(c, redi), k - 1);
    }
    // the kept total: the running sum at the cut
    float kept = 0.f;
    {
        float run = incl - s;
        int have = 0;
        for (int j = j0; j < j1; j++) {
            run += expf((key_value(list[j]) - lmax) * inv_t);
            if (j == cut) {
                kept = run;
                have = 1;
            }
        }
        if (have) redf[0] = kept;
        __syncthreads();
        kept = redf[0];
        __syncthreads();
    }
    const float target = u * kept;
    int pick = k;
    {
        float run = incl - s;
        for (int j = j0; j < min(j1, cut + 1); j++) {
            run += expf((key_value(list[j]) - lmax) * inv_t);
            if (run > target) {
                pick = j;
                break;
            }
        }
    }
    pick = min(block_min_int(pick, redi), cut);
    if (t == 0) tok_out[b] = key_index(list[pick]);
}

hipError_t enqueue_sample(const float* logits, int B, int V, const float* d_uniform, SampleParams prm,
                          int32_t* d_tok_out, hipStream_t st) {
    hipLaunchKernelGGL(k_sample, dim3(B), dim3(kST), 0, st, logits, V, d_uniform, prm, d_tok_out);
    return hipGetLastError();
}

}  // namespace ds
