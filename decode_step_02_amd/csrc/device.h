// device.h -- device helpers shared by the VALU and MFMA kernels.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kernels.h"

namespace ds {

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
    return v;
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
    return v;
}

__device__ __forceinline__ size_t cache_row(const StepArgs& s, int layer, int kv, int slot, int g, int t) {
    size_t i = static_cast<size_t>(layer);
    i = i * 2 + kv;
    i = i * s.B + slot;
    i = i * s.Hkv + g;
    i = i * s.T + t;
    return i * s.D;
}

// Argmax key: the float's order-preserving 32-bit image in the high word and
// (2^32 - 1 - index) in the low word, so the largest key is the largest
// logit and, among equal logits, the lowest index ("Inside nanochat Part 4",
// section "Sampling Strategy": greedy decoding is argmax), whatever order
// the blocks run in.  Every block writes its own key; k_finalize reduces.
__device__ __forceinline__ unsigned long long argmax_key(float v, int idx) {
    uint32_t u = __float_as_uint(v);
    u = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
    return (static_cast<unsigned long long>(u) << 32) | static_cast<uint32_t>(0xFFFFFFFFu - idx);
}

__device__ __forceinline__ unsigned long long wave_max_u64(unsigned long long k) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
        const unsigned long long other = __shfl_xor(k, o);
        k = other > k ? other : k;
    }
    return k;
}

}  // namespace ds
