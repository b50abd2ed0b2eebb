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

// Stores one key or value element: fp32, or rounded to bf16 (nearest, ties
// to even; finite values) in a bf16 cache.
__device__ __forceinline__ void cache_put(const StepArgs& s, size_t idx, float v) {
    if (s.cdt == kBF16) {
        const uint32_t u = __float_as_uint(v);
        reinterpret_cast<uint16_t*>(s.cache)[idx] = static_cast<uint16_t>((u + 0x7FFFu + ((u >> 16) & 1u)) >> 16);
    } else {
        s.cache[idx] = v;
    }
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


// ---- cross-lane reductions in the VALU -----------------------------------------------------------
// __shfl_xor goes through the LDS unit (ds_bpermute) and a chain of them
// waits for each round trip.  Within a 16-lane row, DPP does the same in one
// VALU instruction (quad_perm for lane ^ 1 and lane ^ 2, the half-row and row
// mirrors once values are uniform over quads / half rows, row_ror:8 for
// lane ^ 8); gfx950's permlane16/32 swaps exchange lane ^ 16 and lane ^ 32.
// Both outputs of a swap of v with itself hold v[l] and v[l ^ 16] (or 32), so
// their sum or max is the pair's result, in the same order on both lanes.
// All of these need the whole wave active.

template <int CTRL>
__device__ __forceinline__ float dpp_mov(float v) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}

struct OpSum {
    __device__ __forceinline__ float operator()(float a, float b) const { return a + b; }
};
// One v_max_f32, without the quieting of signalling NaNs that fmaxf puts in
// front of operands that come from lane moves (no NaNs are reduced here).
struct OpMax {
    __device__ __forceinline__ float operator()(float a, float b) const {
        float r;
        asm("v_max_f32 %0, %1, %2" : "=v"(r) : "v"(a), "v"(b));
        return r;
    }
};

// op(v, v[lane ^ O]) for O in {1, 2, 4, 8, 16, 32}: true exchanges, valid for any values.
template <int O, typename Op>
__device__ __forceinline__ float xor_op(float v, Op op) {
    static_assert(O == 1 || O == 2 || O == 4 || O == 8 || O == 16 || O == 32, "lane distance");
    if constexpr (O == 1) {
        return op(v, dpp_mov<0xB1>(v));   // quad_perm [1,0,3,2]
    } else if constexpr (O == 2) {
        return op(v, dpp_mov<0x4E>(v));   // quad_perm [2,3,0,1]
    } else if constexpr (O == 4) {
        return op(v, __shfl_xor(v, 4));
    } else if constexpr (O == 8) {
        return op(v, dpp_mov<0x128>(v));  // row_ror:8
    } else if constexpr (O == 16) {
        const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
        return op(__uint_as_float(r[0]), __uint_as_float(r[1]));
    } else {
        const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
        return op(__uint_as_float(r[0]), __uint_as_float(r[1]));
    }
}

// All-reduce over aligned groups of N lanes (N a power of two <= 64); every
// lane of a group ends with the same bits.  Levels 4 and 8 use the mirrors,
// which are exchanges of whole quads / half rows once those are uniform.
// FROM > 1 takes values that are already uniform over aligned groups of
// FROM lanes and combines those groups.
template <int N, typename Op, int FROM = 1>
__device__ __forceinline__ float group_reduce(float v, Op op) {
    if constexpr (N >= 2 && FROM <= 1) v = xor_op<1>(v, op);
    if constexpr (N >= 4 && FROM <= 2) v = xor_op<2>(v, op);
    if constexpr (N >= 8 && FROM <= 4) v = op(v, dpp_mov<0x141>(v));   // row_half_mirror
    if constexpr (N >= 16 && FROM <= 8) v = op(v, dpp_mov<0x140>(v));  // row_mirror
    if constexpr (N >= 32 && FROM <= 16) v = xor_op<16>(v, op);
    if constexpr (N >= 64) v = xor_op<32>(v, op);
    return v;
}

// group_reduce of K independent values, level by level: the K exchanges of a
// level are independent, so no exchange waits on the result just computed.
template <int N, typename Op, int FROM = 1, int K>
__device__ __forceinline__ void group_reduce_n(float (&v)[K], Op op) {
#pragma unroll
    for (int k = 0; k < K; k++)
        if constexpr (N >= 2 && FROM <= 1) v[k] = xor_op<1>(v[k], op);
#pragma unroll
    for (int k = 0; k < K; k++)
        if constexpr (N >= 4 && FROM <= 2) v[k] = xor_op<2>(v[k], op);
#pragma unroll
    for (int k = 0; k < K; k++)
        if constexpr (N >= 8 && FROM <= 4) v[k] = op(v[k], dpp_mov<0x141>(v[k]));
#pragma unroll
    for (int k = 0; k < K; k++)
        if constexpr (N >= 16 && FROM <= 8) v[k] = op(v[k], dpp_mov<0x140>(v[k]));
#pragma unroll
    for (int k = 0; k < K; k++)
        if constexpr (N >= 32 && FROM <= 16) v[k] = xor_op<16>(v[k], op);
#pragma unroll
    for (int k = 0; k < K; k++)
        if constexpr (N >= 64) v[k] = xor_op<32>(v[k], op);
}

// Reduce over the lanes lane ^ k, k a multiple of LO (LO a power of two):
// combines the groups of LO lanes position by position.
template <int LO, typename Op>
__device__ __forceinline__ float stride_reduce(float v, Op op) {
    if constexpr (LO <= 1) v = xor_op<1>(v, op);
    if constexpr (LO <= 2) v = xor_op<2>(v, op);
    if constexpr (LO <= 4) v = xor_op<4>(v, op);
    if constexpr (LO <= 8) v = xor_op<8>(v, op);
    if constexpr (LO <= 16) v = xor_op<16>(v, op);
    if constexpr (LO <= 32) v = xor_op<32>(v, op);
    return v;
}

template <int N>
__device__ __forceinline__ float group_sum(float v) { return group_reduce<N>(v, OpSum{}); }
template <int N>
__device__ __forceinline__ float group_max(float v) { return group_reduce<N>(v, OpMax{}); }

}  // namespace ds
