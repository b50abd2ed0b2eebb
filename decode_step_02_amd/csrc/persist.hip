// persist.hip -- the whole batch-1 decode step as one persistent kernel.
//
// At batch 1 a decode step is a chain of dependent all-to-all phases per
// layer (Q/K/V, attention, Wo, W1/W3, W2), each moving only a few MB of
// weights, so a launch per phase is dominated by the launch and its cache
// flush.  Here one launch of 256 resident blocks runs the whole step.
//
// Every block has one role for the whole step: Q/K/V rows (role 0),
// attention partials (role 1, long contexts only), Wo (role 2), W1/W3
// (role 3) or W2 (role 4), and loops over the layers in it.  As soon as a
// block has published its outputs of layer l it issues the weight loads of
// layer l+1, which then have three or four phases to land in registers.
// Blocks without a role preload vocabulary rows.
//
// Outputs reach the next phase through "LL" words: a 32-bit value and the
// 32-bit epoch of the phase that wrote it, stored together as one 8-byte
// agent-scope atomic.  The four waves of a consumer block poll the words of
// the vector they need (a quarter each) until every word carries the
// expected epoch, then share it through LDS.  Before that they poll a
// 64-word sample of the phase before, so that blocks whose turn is far off
// do not hammer the lines being written.  No counter, fence or grid barrier
// is needed.
//
// For contexts of up to 32 positions the Wo blocks recompute attention
// themselves (one wave per key/value group, its cached rows preloaded in
// registers): four handoffs per layer instead of five.
//
// Every wait is bounded: a wave that does not see its input in about a
// second sets the error word and carries on, so the grid always drains
// (ds_kv_cache_check then reports the failure).
//
// The arithmetic is that of the pre-norm Llama block ("simple-llm /
// kasahare" PyPI README 0.4.0, section "Architecture") with the
// (L, 2, B, Hkv, T, D) cache of "Inside nanochat Part 4: Understanding
// Inference", section "Cache Architecture".  The new key/value row reaches
// attention through LL words, because plain stores of the same launch are
// not guaranteed to be visible to other workgroups.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "device.h"
#include "kernels.h"

namespace ds {

constexpr int kPBlocks = 256;
constexpr int kPThreads = 256;                // 4 waves
constexpr int kPWaves = kPBlocks * kPThreads / 64;
constexpr int kPLds = 13312;                  // floats of LDS per block
constexpr int kPGains = kPLds - 1024;         // the final RMSNorm gains, loaded at the start
constexpr int kPRed = kPGains - 16;           // block-reduction slots; the roles use LDS below them
constexpr int kPNorm = 4;                     // normalised elements per thread (d <= 1024)
constexpr long kPSpin = 1 << 20;              // poll rounds before a wait gives up
constexpr int kPhases = 5;                    // epochs per layer
constexpr int kPSample = 16;                  // words a throttle wait samples (fewer loads on the hot lines)

static_assert(kPWaves == kPKeyWords, "one argmax word per wave");

__device__ __forceinline__ void ll_put(uint64_t* p, float v, uint32_t ep) {
    __hip_atomic_store(p, (static_cast<uint64_t>(ep) << 32) | __float_as_uint(v), __ATOMIC_RELAXED,
                       __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ uint64_t ll_get(const uint64_t* p) {
    return __hip_atomic_load(const_cast<uint64_t*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ bool aborted(int32_t* err) {
    return __hip_atomic_load(err, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != 0;
}

__device__ __forceinline__ bool give_up(long& spins, int32_t* err) {
    if ((++spins & 1023) == 0 && (spins > kPSpin || aborted(err))) {
        if ((threadIdx.x & 63) == 0) atomicOr(err, 4);
        return true;
    }
    return false;
}

// A run of LL words: n words from src that must carry epoch ep; values go to dst.
struct Seg {
    const uint64_t* src;
    int n;
    uint32_t ep;
    float* dst;
};

// Wait until kPSample words spread over src[0..n) carry epoch ep (ANY: until
// one of them does).  Lanes of wave 0 poll, the other waves wait at the
// barrier, so a waiting block puts a few loads on the memory system; SLEEP
// spaces the rounds.  Used as a throttle in front of a block_fetch.
// Block-uniform call.
template <int SLEEP, bool ANY = false>
__device__ void wait_sample(const uint64_t* src, int n, uint32_t ep, int32_t* err) {
    if (n <= 0) return;
    if (threadIdx.x < 64) {
        const bool act = threadIdx.x < kPSample;
        const uint64_t* q = src + (static_cast<int>(threadIdx.x) % kPSample * n) / kPSample;
        long spins = 0;
        while (true) {
            const bool ok = act && static_cast<uint32_t>(ll_get(q) >> 32) == ep;
            if (ANY ? __any(ok) : __all(ok || !act)) break;
            if (SLEEP > 0) __builtin_amdgcn_s_sleep(SLEEP);
            if (give_up(spins, err)) break;
        }
    }
    __syncthreads();
}

// Wait until the single word w carries epoch ep: one lane polls, SLEEP
// spaces the rounds, the block waits at the barrier.  Block-uniform call.
template <int SLEEP>
__device__ void wait_word(const uint64_t* w, uint32_t ep, int32_t* err) {
    if (threadIdx.x == 0) {
        long spins = 0;
        while (static_cast<uint32_t>(ll_get(w) >> 32) != ep) {
            __builtin_amdgcn_s_sleep(SLEEP);
            if (give_up(spins, err)) break;
        }
    }
    __syncthreads();
}

// Block-cooperative fetch of segment a followed by segment b: thread t polls
// the words t, t + 256, ... of the concatenation, J per round, with
// unconditional loads of clamped indices so that a round is one memory round
// trip, and stores the values to LDS once its wave has seen the round
// complete.  No barrier here.
template <int J>
__device__ void block_fetch(const Seg& a, const Seg& b, int32_t* err) {
    const int tid = threadIdx.x;
    const int total = a.n + b.n;
    for (int base = 0; base < total; base += kPThreads * J) {
        uint64_t w[J];
        long spins = 0;
        while (true) {
#pragma unroll
            for (int j = 0; j < J; j++) {
                const int i = min(base + tid + kPThreads * j, total - 1);
                w[j] = ll_get(i < a.n ? a.src + i : b.src + (i - a.n));
            }
            bool ok = true;
#pragma unroll
            for (int j = 0; j < J; j++) {
                const int i = min(base + tid + kPThreads * j, total - 1);
                ok &= static_cast<uint32_t>(w[j] >> 32) == (i < a.n ? a.ep : b.ep);
            }
            if (__all(ok)) break;
            if (give_up(spins, err)) break;
        }
#pragma unroll
        for (int j = 0; j < J; j++) {
            const int i = base + tid + kPThreads * j;
            if (i < total) {
                float* dst = i < a.n ? a.dst + i : b.dst + (i - a.n);
                *dst = __uint_as_float(static_cast<uint32_t>(w[j]));
            }
        }
    }
}

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

// Loads through the global address space: pointers read out of memory (the
// layer table) are otherwise accessed with flat instructions, which also
// count against the LDS wait counter.  16-byte loads go through a native
// vector type (the HIP vector structs copy through generic pointers).
typedef float f32x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint4 gload_u4(const void* p) {
    const u32x4 v = *(const __attribute__((address_space(1))) u32x4*)p;
    return make_uint4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ float4 gload_f4(const void* p) {
    const f32x4 v = *(const __attribute__((address_space(1))) f32x4*)p;
    return make_float4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ float gload_f(const float* p) {
    return *(const __attribute__((address_space(1))) float*)p;
}
// The same for cached key/value rows, which a step reads once: with the
// non-temporal hint (1000-token context: 350.4 -> 348.4 us per step).
__device__ __forceinline__ float4 gload_f4_stream(const void* p) {
    const f32x4 v = __builtin_nontemporal_load((const __attribute__((address_space(1))) f32x4*)p);
    return make_float4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ float gload_f_stream(const float* p) {
    return __builtin_nontemporal_load((const __attribute__((address_space(1))) float*)p);
}

// One poll round of J 16-byte loads (two LL words each) with the cache
// policy of an agent-scope atomic load (sc1), completed inside the same asm
// block so that no result is read before it has arrived.  Every 8-byte word
// is written by a single aligned 8-byte store, so a 16-byte load may see one
// word old and the other new, but never half a word.
template <int J>
__device__ __forceinline__ void poll_wide(u32x4 (&w)[J], const uint64_t* const (&p)[J]) {
    static_assert(J >= 1 && J <= 4, "poll_wide: 1..4 loads");
    if constexpr (J == 1) {
        asm volatile("global_load_dwordx4 %0, %1, off sc1\n\ts_waitcnt vmcnt(0)" : "=&v"(w[0]) : "v"(p[0]) : "memory");
    } else if constexpr (J == 2) {
        asm volatile(
            "global_load_dwordx4 %0, %2, off sc1\n\t"
            "global_load_dwordx4 %1, %3, off sc1\n\t"
            "s_waitcnt vmcnt(0)"
            : "=&v"(w[0]), "=&v"(w[1]) : "v"(p[0]), "v"(p[1]) : "memory");
    } else if constexpr (J == 3) {
        asm volatile(
            "global_load_dwordx4 %0, %3, off sc1\n\t"
            "global_load_dwordx4 %1, %4, off sc1\n\t"
            "global_load_dwordx4 %2, %5, off sc1\n\t"
            "s_waitcnt vmcnt(0)"
            : "=&v"(w[0]), "=&v"(w[1]), "=&v"(w[2]) : "v"(p[0]), "v"(p[1]), "v"(p[2]) : "memory");
    } else {
        asm volatile(
            "global_load_dwordx4 %0, %4, off sc1\n\t"
            "global_load_dwordx4 %1, %5, off sc1\n\t"
            "global_load_dwordx4 %2, %6, off sc1\n\t"
            "global_load_dwordx4 %3, %7, off sc1\n\t"
            "s_waitcnt vmcnt(0)"
            : "=&v"(w[0]), "=&v"(w[1]), "=&v"(w[2]), "=&v"(w[3])
            : "v"(p[0]), "v"(p[1]), "v"(p[2]), "v"(p[3])
            : "memory");
    }
}

// block_fetch with two words per load: thread t polls the word pairs
// (2t, 2t+1), (2t+512, 2t+513), ... of the concatenation, J pairs per round.
// Needs a.n and b.n even (a pair never straddles the segments) and 16-byte
// aligned segment starts; otherwise it falls back to block_fetch.
// sink_a(i, v0, v1) takes the pairs of segment a in place of the stores to
// a.dst (the other overload stores them).
template <int J, typename SinkA>
__device__ void block_fetch2(const Seg& a, const Seg& b, int32_t* err, SinkA sink_a) {
    const bool ok_shape = ((a.n | b.n) & 1) == 0 &&
                          ((reinterpret_cast<uintptr_t>(a.src) | reinterpret_cast<uintptr_t>(b.src)) & 15) == 0;
    if (!ok_shape) {
        block_fetch<2 * J>(a, b, err);
        __syncthreads();
        for (int i = 2 * static_cast<int>(threadIdx.x); i < a.n; i += 2 * kPThreads) sink_a(i, a.dst[i], a.dst[i + 1]);
        return;
    }
    const int tid = threadIdx.x;
    const int total = a.n + b.n;
    for (int base = 0; base < total; base += 2 * kPThreads * J) {
        u32x4 w[J];
        const uint64_t* src[J];
        uint32_t ep[J];
#pragma unroll
        for (int j = 0; j < J; j++) {
            const int i = min(base + 2 * (tid + kPThreads * j), total - 2);
            src[j] = i < a.n ? a.src + i : b.src + (i - a.n);
            ep[j] = i < a.n ? a.ep : b.ep;
        }
        long spins = 0;
        while (true) {
            poll_wide<J>(w, src);
            bool ok = true;
#pragma unroll
            for (int j = 0; j < J; j++) ok &= w[j].y == ep[j] && w[j].w == ep[j];
            if (__all(ok)) break;
            if (give_up(spins, err)) break;
        }
#pragma unroll
        for (int j = 0; j < J; j++) {
            const int i = base + 2 * (tid + kPThreads * j);
            if (i < a.n) {
                sink_a(i, __uint_as_float(w[j].x), __uint_as_float(w[j].z));
            } else if (i < total) {
                float* dst = b.dst + (i - a.n);
                dst[0] = __uint_as_float(w[j].x);
                dst[1] = __uint_as_float(w[j].z);
            }
        }
    }
}

template <int J>
__device__ __forceinline__ void block_fetch2(const Seg& a, const Seg& b, int32_t* err) {
    float* const d = a.dst;
    block_fetch2<J>(a, b, err, [d](int i, float v0, float v1) {
        d[i] = v0;
        d[i + 1] = v1;
    });
}

template <int J>
__device__ __forceinline__ void block_fetch2(const Seg& a, int32_t* err) {
    block_fetch2<J>(a, Seg{a.src, 0, a.ep, a.dst}, err);
}

// The words of a that thread t owns (own_elem order: 2t, 2t + 1, 2t + 512,
// 2t + 513), polled like block_fetch2 and kept in registers, 0 past a.n.
// Needs 2 <= a.n <= 4 * kPThreads, a.n even and a 16-byte aligned segment.
__device__ void block_fetch_own(const Seg& a, float (&x)[kPNorm], int32_t* err) {
    static_assert(kPNorm == 4, "two word pairs per thread");
    const int tid = threadIdx.x;
    const uint64_t* src[2];
#pragma unroll
    for (int j = 0; j < 2; j++) src[j] = a.src + min(2 * (tid + kPThreads * j), a.n - 2);
    u32x4 w[2];
    long spins = 0;
    while (true) {
        poll_wide<2>(w, src);
        const bool ok = w[0].y == a.ep && w[0].w == a.ep && w[1].y == a.ep && w[1].w == a.ep;
        if (__all(ok)) break;
        if (give_up(spins, err)) break;
    }
#pragma unroll
    for (int j = 0; j < 2; j++) {
        const bool in = 2 * (tid + kPThreads * j) < a.n;
        x[2 * j] = in ? __uint_as_float(w[j].x) : 0.f;
        x[2 * j + 1] = in ? __uint_as_float(w[j].z) : 0.f;
    }
}

template <int J>
__device__ __forceinline__ void block_fetch(const Seg& a, int32_t* err) {
    block_fetch<J>(a, Seg{a.src, 0, a.ep, a.dst}, err);  // an empty second segment (never null)
}

// The input vector of a row product, in LDS.  For fp32 weights it is fp32.
// For bf16 weights every element x is held as two bf16 terms, hi = RNE(x)
// and lo = RNE(x - hi) (|x - hi - lo| <= 2^-18 |x|), packed in pairs: n/2
// words of hi pairs followed by n/2 words of lo pairs.  The products then use
// v_dot2_f32_bf16 on the weight pairs as stored, with no widening.
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ void split_pair(float a, float b, uint32_t& hi, uint32_t& lo) {
    bf16x2 h, l;
    h.x = static_cast<__bf16>(a);
    h.y = static_cast<__bf16>(b);
    l.x = static_cast<__bf16>(a - static_cast<float>(h.x));
    l.y = static_cast<__bf16>(b - static_cast<float>(h.y));
    hi = __builtin_bit_cast(uint32_t, h);
    lo = __builtin_bit_cast(uint32_t, l);
}

// Store the element pair (i, i + 1) of an n-element input vector.
template <int WDT>
__device__ __forceinline__ void put_pair(float* vin, int n, int i, float a, float b) {
    if (WDT == kBF16) {
        uint32_t hi, lo;
        split_pair(a, b, hi, lo);
        uint32_t* u = reinterpret_cast<uint32_t*>(vin);
        u[i >> 1] = hi;
        u[(n >> 1) + (i >> 1)] = lo;
    } else {
        vin[i] = a;
        vin[i + 1] = b;
    }
}

// The vector elements thread t owns: 2t, 2t + 1, 2t + 512, 2t + 513 (the ones
// block_fetch2 of a single segment gives it).
__device__ __forceinline__ int own_elem(int j) {
    return 2 * static_cast<int>(threadIdx.x) + (j & 1) + 2 * kPThreads * (j >> 1);
}

// RMSNorm for the whole block of a vector of n <= 1024 elements (n even),
// each thread holding the elements it owns (x[j] = element own_elem(j), 0
// past n).  Each thread multiplies its pairs by their gains and stores them
// as the row-product input vin (fp32 or bf16 hi/lo pairs, see put_pair); the
// function returns 1 / sqrt(mean(x^2) + eps) (v_rsq_f32, within 1 ulp), by
// which the caller scales its dot products.  Ends with a barrier, after which
// vin is complete.
template <int WDT>
__device__ float block_norm_regs(const float (&x)[kPNorm], int n, const float (&gr)[kPNorm], float eps, float* sm,
                                 float* vin) {
    const int tid = threadIdx.x;
    float ss = 0.f;
#pragma unroll
    for (int jj = 0; jj < kPNorm / 2; jj++) {
        const int i = own_elem(2 * jj);  // the pair (i, i + 1)
        const float a = x[2 * jj], b = x[2 * jj + 1];
        ss = fmaf(a, a, ss);
        ss = fmaf(b, b, ss);
        if (i < n) put_pair<WDT>(vin, n, i, gr[2 * jj] * a, gr[2 * jj + 1] * b);
    }
    ss = group_sum<64>(ss);
    if ((tid & 63) == 0) sm[kPRed + (tid >> 6)] = ss;
    __syncthreads();
    const float tot = (sm[kPRed] + sm[kPRed + 1]) + (sm[kPRed + 2] + sm[kPRed + 3]);
    return __builtin_amdgcn_rsqf(tot * (1.0f / static_cast<float>(n)) + eps);
}

__device__ __forceinline__ void load_gains(float (&gr)[kPNorm], const float* __restrict__ g, int n) {
#pragma unroll
    for (int j = 0; j < kPNorm; j++) gr[j] = gload_f(g + min(own_elem(j), n - 1));
}

// The lane's share of a row product's input: the chunks sub, sub + G, ...
// (EPC elements each, clamped to the last chunk), read from LDS into
// registers in one batch so that the products wait for LDS once.  IN is the
// input's representation: kF32 (fp32 values) or kBF16 (bf16 hi/lo pairs,
// see put_pair); bf16 weights take either.

template <int WDT, int IN, int NC>
struct XRegs;

template <int NC>
struct XRegs<kF32, kF32, NC> {
    float4 v[NC];
    __device__ __forceinline__ void load(const float* vin, int n, int sub, int G) {
        const int nchunks = n / 4;
#pragma unroll
        for (int p = 0; p < NC; p++) v[p] = reinterpret_cast<const float4*>(vin)[min(sub + p * G, nchunks - 1)];
    }
};

template <int NC>
struct XRegs<kBF16, kF32, NC> {
    float4 a[NC], b[NC];  // the chunk's 8 fp32 elements
    __device__ __forceinline__ void load(const float* vin, int n, int sub, int G) {
        const int nchunks = n / 8;
        const float4* v = reinterpret_cast<const float4*>(vin);
#pragma unroll
        for (int p = 0; p < NC; p++) {
            const int c = min(sub + p * G, nchunks - 1);
            a[p] = v[2 * c];
            b[p] = v[2 * c + 1];
        }
    }
};

template <int NC>
struct XRegs<kBF16, kBF16, NC> {
    uint4 h[NC], l[NC];  // hi and lo pairs of the chunk's 8 elements
    __device__ __forceinline__ void load(const float* vin, int n, int sub, int G) {
        const int nchunks = n / 8;
        const uint4* u = reinterpret_cast<const uint4*>(vin);
#pragma unroll
        for (int p = 0; p < NC; p++) {
            const int c = min(sub + p * G, nchunks - 1);
            h[p] = u[c];
            l[p] = u[(n >> 3) + c];
        }
    }
};

// The wave's share of one weight row: G lanes per row, lane `sub` takes the
// 16-byte chunks sub, sub + G, ..., NC of them (the host picks G and NC so
// that NC * G covers the row).  start() issues their loads into registers,
// with zeros for the chunks past the row's end and for rows that are not
// valid, so that finish() needs no masks: it multiplies them with the
// matching XRegs in four running sums and reduces over the G lanes,
// touching no memory.
// NOLOAD (the handoff-floor instantiation) issues no loads: every chunk is 0.
template <int WDT, int G, int NC, bool NOLOAD = false>
struct PStream {
    static constexpr int EPC = WDT == kBF16 ? 8 : 4;
    uint4 w[NC];
    __device__ __forceinline__ void start(const void* W, int row, int K, int sub, bool valid) {
        const size_t base = static_cast<size_t>(row) * K;
        const int nchunks = valid && !NOLOAD ? K / EPC : 0;
#pragma unroll
        for (int p = 0; p < NC; p++) {
            const int c = sub + p * G;
            w[p] = make_uint4(0u, 0u, 0u, 0u);
            if (c < nchunks) {
                const size_t e = base + static_cast<size_t>(c) * EPC;
                w[p] = WDT == kBF16 ? gload_u4(static_cast<const uint16_t*>(W) + e)
                                    : gload_u4(static_cast<const float*>(W) + e);
            }
        }
    }
    __device__ __forceinline__ static float dot2(uint32_t w2, uint32_t x2, float acc) {
        return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, w2), __builtin_bit_cast(bf16x2, x2), acc,
                                                false);
    }
    // bf16 weights times fp32 inputs: each weight widened to fp32 (the
    // element at the lower address is the low half of the 32-bit word, so
    // widening is a 16-bit left shift or a mask of the high half), one fp32
    // FMA per element.
    __device__ __forceinline__ float finish(const XRegs<kBF16, kF32, NC>& x) const {
        static_assert(WDT == kBF16, "widened products need bf16 weights");
        float a[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int p = 0; p < NC; p++) {
            float& u = a[2 * (p & 1)];
            float& v = a[2 * (p & 1) + 1];
            u = fmaf(__uint_as_float(w[p].x << 16), x.a[p].x, u);
            v = fmaf(__uint_as_float(w[p].x & 0xFFFF0000u), x.a[p].y, v);
            u = fmaf(__uint_as_float(w[p].y << 16), x.a[p].z, u);
            v = fmaf(__uint_as_float(w[p].y & 0xFFFF0000u), x.a[p].w, v);
            u = fmaf(__uint_as_float(w[p].z << 16), x.b[p].x, u);
            v = fmaf(__uint_as_float(w[p].z & 0xFFFF0000u), x.b[p].y, v);
            u = fmaf(__uint_as_float(w[p].w << 16), x.b[p].z, u);
            v = fmaf(__uint_as_float(w[p].w & 0xFFFF0000u), x.b[p].w, v);
        }
        return group_sum<G>((a[0] + a[1]) + (a[2] + a[3]));
    }
    __device__ __forceinline__ float finish(const XRegs<WDT, WDT, NC>& x) const {
        float a[4] = {0.f, 0.f, 0.f, 0.f};  // bf16: hi and lo terms of even and odd chunks
#pragma unroll
        for (int p = 0; p < NC; p++) {
            float& h = a[2 * (p & 1)];
            float& l = a[2 * (p & 1) + 1];
            if constexpr (WDT == kBF16) {
                h = dot2(w[p].x, x.h[p].x, h);
                l = dot2(w[p].x, x.l[p].x, l);
                h = dot2(w[p].y, x.h[p].y, h);
                l = dot2(w[p].y, x.l[p].y, l);
                h = dot2(w[p].z, x.h[p].z, h);
                l = dot2(w[p].z, x.l[p].z, l);
                h = dot2(w[p].w, x.h[p].w, h);
                l = dot2(w[p].w, x.l[p].w, l);
            } else {
                const float4 v = x.v[p];
                h = fmaf(__uint_as_float(w[p].x), v.x, h);
                l = fmaf(__uint_as_float(w[p].y), v.y, l);
                h = fmaf(__uint_as_float(w[p].z), v.z, h);
                l = fmaf(__uint_as_float(w[p].w), v.w, l);
            }
        }
        return group_sum<G>((a[0] + a[1]) + (a[2] + a[3]));
    }
};

// Argmax word: ordered float bits (32), (2^17 - 1 - index) (17), epoch (15):
// the largest word is the largest logit, ties going to the lowest index.
__device__ __forceinline__ uint64_t key_word(float v, int idx, uint32_t ep) {
    uint32_t u = __float_as_uint(v);
    u = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
    return (static_cast<uint64_t>(u) << 32) | (static_cast<uint64_t>(0x1FFFFu - idx) << 15) | (ep & 0x7FFFu);
}

// What every role needs to know about the step.  Epochs per layer: 0 Q/K/V
// words, 1 attention partials, 2 residual after Wo, 3 silu(a)*u, 4 residual
// after W2; the argmax words use ep(L, 0).
struct PCtx {
    uint32_t base;   // epoch base of this step
    int pos, n, nch, npart, tok;  // npart: attention partials per head (four chunks each)
    bool fused;      // attention recomputed inside the Wo blocks
    int rep;         // word offset of the replica this block reads
    int32_t* err;
    __device__ __forceinline__ uint32_t ep(int l, int ph) const {
        return base + 1u + static_cast<uint32_t>(l * kPhases + ph);
    }
};

// Compile-time shape class of one instantiation: weight type, head dim,
// query heads per key/value head, and lanes per row / chunks per lane for
// rows of d (Q/K/V, W1/W3, vocabulary), H*D (Wo) and F (W2) elements.
constexpr int cmin(int a, int b) { return a < b ? a : b; }

// IN: how row-product inputs are held (kF32, or kBF16 hi/lo pairs; see
// put_pair).  FLOOR: the handoff-floor diagnostic -- the same phases and LL
// words with no weight or cache loads and no stores outside the LL words.
// LONG: contexts of more than one chunk (role 1 partials, merged in role
// 2); otherwise one chunk, attention recomputed in the Wo blocks.  Each
// instantiation holds only its own path, so neither pays the other's
// registers.
template <int WDT_, int PD_, int REP_, int GD_, int NCD_, int GH_, int NCH_, int GF_, int NCF_, int IN_ = WDT_,
          bool FLOOR_ = false, bool LONG_ = false>
struct PCfg {
    static constexpr int WDT = WDT_, PD = PD_, REP = REP_, IN = IN_;
    static constexpr bool FLOOR = FLOOR_, LONG = LONG_;
    static constexpr int GD = GD_, NCD = NCD_, GH = GH_, NCH = NCH_, GF = GF_, NCF = NCF_;
    // replicas of each published vector: lane `sub` of a row writes replica `sub`
    static constexpr int LLR = cmin(cmin(GD, GH), cmin(GF, kPRep));
};

template <int WDT>
__device__ __forceinline__ float emb_at(const StepArgs& s, int tok, int j) {
    const size_t e = static_cast<size_t>(tok) * s.d + j;
    return WDT == kBF16 ? __uint_as_float(static_cast<uint32_t>(static_cast<const uint16_t*>(s.emb)[e]) << 16)
                        : static_cast<const float*>(s.emb)[e];
}

template <int PD, int REP, bool NOLOAD = false>
struct KV {
    // keys: 4 lanes per row with PD / 4 dims (KF float4) each, 16 rows per slot
    static constexpr int KF = PD / 16;
    static constexpr int NK = kPChunk / 16;
    // values: one dim per lane (lane = rv * PD + e), RV rows per slot, NV slots
    static constexpr int RV = 64 / PD;
    static constexpr int NV = kPChunk / RV;
    // softmax weights per head in the wave's LDS scratch: position p of the
    // chunk at (p % RV) * NV + p / RV (so a lane's NV weights are contiguous),
    // the new row's weight at kPChunk, padding
    static constexpr int PWS = kPChunk + 4;
    float4 k[NK][KF];
    float v[NV];

    // the wave's cached rows of group g from position t0 on, clamped to the
    // last row an earlier step wrote (pos - 1, or 0)
    __device__ __forceinline__ void load(const StepArgs& s, int l, int g, int t0, int pos) {
        if constexpr (NOLOAD) {
#pragma unroll
            for (int sl = 0; sl < NK; sl++)
#pragma unroll
                for (int f = 0; f < KF; f++) k[sl][f] = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
            for (int ii = 0; ii < NV; ii++) v[ii] = 0.f;
            return;
        }
        const int lane = threadIdx.x & 63, rk = lane >> 2, qk = lane & 3, rv = lane / PD, ev = lane % PD;
        const int tmax = pos > 0 ? pos - 1 : 0;
#pragma unroll
        for (int sl = 0; sl < NK; sl++) {
            const float* src = s.cache + cache_row(s, l, 0, 0, g, min(t0 + sl * 16 + rk, tmax)) + qk * (PD / 4);
#pragma unroll
            for (int f = 0; f < KF; f++) k[sl][f] = gload_f4_stream(src + 4 * f);
        }
        const float* vb = s.cache + cache_row(s, l, 1, 0, g, 0) + ev;
#pragma unroll
        for (int ii = 0; ii < NV; ii++) v[ii] = gload_f_stream(vb + static_cast<size_t>(min(t0 + ii * RV + rv, tmax)) * PD);
    }

    // acc[j] = sum over the lane's value rows of weight * value for head j,
    // the first N4 float4 groups of weights (the rest are 0), plus the new
    // row's term once (row group 0), then the RV row groups added up.
    template <int N4>
    __device__ __forceinline__ void weighted_values(const float* pw, float vn, int rv, float (&acc)[REP]) const {
#pragma unroll
        for (int j = 0; j < REP; j++) {
            const float4* pj = reinterpret_cast<const float4*>(pw + j * PWS + rv * NV);
            float4 pe[N4];
#pragma unroll
            for (int c4 = 0; c4 < N4; c4++) pe[c4] = pj[c4];  // one batch of broadcast reads
            float a0 = rv == 0 ? pw[j * PWS + kPChunk] * vn : 0.f, a1 = 0.f;
#pragma unroll
            for (int c4 = 0; c4 < N4; c4++) {
                a0 = fmaf(pe[c4].x, v[4 * c4 + 0], a0);
                a1 = fmaf(pe[c4].y, v[4 * c4 + 1], a1);
                a0 = fmaf(pe[c4].z, v[4 * c4 + 2], a0);
                a1 = fmaf(pe[c4].w, v[4 * c4 + 3], a1);
            }
            acc[j] = stride_reduce<PD>(a0 + a1, OpSum{});  // none when PD == 64
        }
    }

    // Attention of the REP query heads of group g over positions t0 ..
    // min(pos, t0 + 31).
    //  - Scores use the key layout (a 4-lane reduction per row).  The new key
    //    from qkv (LDS, group-major: REP queries, key, value) is patched into
    //    the one slot that holds pos; slots wholly past pos are skipped.
    //  - The softmax weights go through the wave's LDS scratch pw[REP][PWS],
    //    the new row's weight in its own entry, so the value rows in
    //    registers are never patched: rows past pos are clamped copies of
    //    written rows and get weight 0.  At pos == 0 nothing has been written
    //    yet and the output is the new value.
    //  - Every lane accumulates one dim; with PD < 64 the RV row groups are
    //    added up at the end.
    // For every head j the lanes of the first value row get emit(j, e, max
    // score, sum of weights, weighted sum of values for dim e, the same for
    // dim e ^ 1).
    template <typename Emit>
    __device__ __forceinline__ void attend(const float* qkv, int g, int t0, int pos, float* pw, Emit emit) {
        const int lane = threadIdx.x & 63, rk = lane >> 2, qk = lane & 3, rv = lane / PD, ev = lane % PD;
        constexpr int GS = (REP + 2) * PD;
        const float scale = 1.0f / sqrtf(static_cast<float>(PD));
        float4 q[REP][KF];
#pragma unroll
        for (int j = 0; j < REP; j++) {
#pragma unroll
            for (int f = 0; f < KF; f++)
                q[j][f] = reinterpret_cast<const float4*>(qkv + g * GS + j * PD + qk * (PD / 4))[f];
        }
        const float vn = qkv[g * GS + (REP + 1) * PD + ev];
        const int cur = pos - t0;  // chunk position of the new row (>= kPChunk: not in this chunk)
#pragma unroll
        for (int sl = 0; sl < NK; sl++) {
            if (cur >= sl * 16 && cur < sl * 16 + 16) {  // uniform: the slot holding the new row
                const float4* kn = reinterpret_cast<const float4*>(qkv + g * GS + REP * PD + qk * (PD / 4));
                const bool here = rk == cur - sl * 16;
#pragma unroll
                for (int f = 0; f < KF; f++) {
                    const float4 x = kn[f];
                    k[sl][f].x = here ? x.x : k[sl][f].x;
                    k[sl][f].y = here ? x.y : k[sl][f].y;
                    k[sl][f].z = here ? x.z : k[sl][f].z;
                    k[sl][f].w = here ? x.w : k[sl][f].w;
                }
            }
        }
        float sc[REP][NK];
#pragma unroll
        for (int sl = 0; sl < NK; sl++) {
            const int tb = t0 + sl * 16;  // first position of the slot (uniform)
            if (tb <= pos) {
                float dd[REP];
#pragma unroll
                for (int j = 0; j < REP; j++) {
                    dd[j] = 0.f;
#pragma unroll
                    for (int f = 0; f < KF; f++) {
                        dd[j] = fmaf(k[sl][f].x, q[j][f].x, dd[j]);
                        dd[j] = fmaf(k[sl][f].y, q[j][f].y, dd[j]);
                        dd[j] = fmaf(k[sl][f].z, q[j][f].z, dd[j]);
                        dd[j] = fmaf(k[sl][f].w, q[j][f].w, dd[j]);
                    }
                }
                group_reduce_n<4, OpSum>(dd, OpSum{});
#pragma unroll
                for (int j = 0; j < REP; j++) sc[j][sl] = tb + rk <= pos ? dd[j] * scale : -INFINITY;
            } else {
#pragma unroll
                for (int j = 0; j < REP; j++) sc[j][sl] = -INFINITY;
            }
        }
        // softmax statistics over the 16 row groups (values uniform over each quad)
        float m[REP], ls[REP];
#pragma unroll
        for (int j = 0; j < REP; j++) {
            m[j] = sc[j][0];
#pragma unroll
            for (int sl = 1; sl < NK; sl++) m[j] = OpMax{}(m[j], sc[j][sl]);
        }
        group_reduce_n<64, OpMax, 4>(m, OpMax{});
#pragma unroll
        for (int j = 0; j < REP; j++) {
            ls[j] = 0.f;
#pragma unroll
            for (int sl = 0; sl < NK; sl++) {
                const float pe = t0 + sl * 16 <= pos ? __expf(sc[j][sl] - m[j]) : 0.f;
                ls[j] += pe;
                const int p = sl * 16 + rk;
                // every lane of the row stores (the same value); in the new row's
                // quad lane 1 stores its weight apart and the others a 0 entry
                const bool nr = p == cur;
                pw[j * PWS + (nr && qk == 1 ? kPChunk : (p % RV) * NV + p / RV)] = nr && qk != 1 ? 0.f : pe;
            }
        }
        group_reduce_n<64, OpSum, 4>(ls, OpSum{});
        if (cur >= kPChunk && lane == 0) {
#pragma unroll
            for (int j = 0; j < REP; j++) pw[j * PWS + kPChunk] = 0.f;
        }
        __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): the weights are in LDS
        __builtin_amdgcn_wave_barrier();
        float acc[REP];
        if (pos == 0) {
#pragma unroll
            for (int j = 0; j < REP; j++) acc[j] = vn;  // one position: weight 1 on the new row
        } else if (cur < 16) {
            weighted_values<NV / 8>(pw, vn, rv, acc);  // positions 16.. of the chunk have weight 0
        } else {
            weighted_values<NV / 4>(pw, vn, rv, acc);
        }
        float nb[REP];
#pragma unroll
        for (int j = 0; j < REP; j++) nb[j] = dpp_mov<0xB1>(acc[j]);  // dim e ^ 1
        if (rv == 0) {
#pragma unroll
            for (int j = 0; j < REP; j++) emit(j, ev, m[j], ls[j], acc[j], nb[j]);
        }
    }
};

// ---- role 0: Q/K/V rows, RoPE, cache append (a task of R rows per wave) ---------------------------
template <class C>
__device__ void role_qkv(const StepArgs& s, const PersistArgs& p, const PCtx& c, int bt, float* sm) {
    constexpr int G = C::GD, R = 64 / G, PD = C::PD, REP = C::REP;
    constexpr int EPC = C::WDT == kBF16 ? 8 : 4;
    const int wv = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int d = s.d, half = PD / 2, HD = s.H * PD, KVD = s.Hkv * PD;
    constexpr int GS = (REP + 2) * PD;
    const int nq = HD / R, nk = KVD / R, ntask = nq + 2 * nk;
    const int t = bt * 4 + wv, rs = lane / G, sub = lane % G;
    const bool active = t < ntask;
    const bool roped = t < nq + nk, is_q = t < nq;
    int row = 0, i = 0, second = 0, which = 2;
    if (active) {
        if (roped) {
            // rows i and i + D/2 of a head are rotated together; they sit 32 lanes apart
            const int pp = (is_q ? t : t - nq) * (R / 2) + (rs % (R / 2));
            second = rs / (R / 2);
            i = pp % half;
            row = (pp / half) * PD + i + second * half;
            which = is_q ? 0 : 1;
        } else {
            row = (t - nq - nk) * R + rs;
        }
    }
    float cs = 1.f, sn = 0.f;
    if (roped) {
        cs = s.rope_cos[static_cast<size_t>(c.pos) * half + i];
        sn = s.rope_sin[static_cast<size_t>(c.pos) * half + i];
    }
    auto wmat = [&](int l) {
        const LayerW& w = p.layers[l];
        return which == 0 ? w.wq : (which == 1 ? w.wk : w.wv);
    };
    // the lane's word in the layer-0 Q/K/V words, and its cache element (keys and values)
    const int g = row / PD, e = row % PD;
    const int qw = which == 0 ? (g / REP) * GS + (g % REP) * PD + e : g * GS + (which == 1 ? REP : REP + 1) * PD + e;
    uint64_t* const put_at = p.ll_qkv + sub * p.rstride + qw;
    float* const crow = s.cache + cache_row(s, 0, which == 2 ? 1 : 0, 0, g, c.pos) + e;
    const size_t cstride = cache_row(s, 1, 0, 0, 0, 0);  // one layer of the cache
    PStream<C::WDT, G, C::NCD, C::FLOOR> st;
    float gr[kPNorm];
    st.start(wmat(0), row, d, sub, active);
    load_gains(gr, p.layers[0].attn_norm, d);
    float* const vin = sm;  // product input (see put_pair)
    for (int l = 0; l < s.L; l++) {
        __syncthreads();  // nobody reads the previous layer's LDS any more
        float xv[kPNorm];
        if (l == 0) {
#pragma unroll
            for (int j = 0; j < kPNorm; j++) {
                const int e = own_elem(j);
                xv[j] = e < d ? emb_at<C::WDT>(s, c.tok, e) : 0.f;
            }
        } else {
            wait_sample<2, true>(p.ll_x + c.rep, d, c.ep(l - 1, 4), c.err);
            block_fetch_own(Seg{p.ll_x + c.rep, d, c.ep(l - 1, 4), nullptr}, xv, c.err);
        }
        const float rn = block_norm_regs<C::IN>(xv, d, gr, s.eps, sm, vin);
        if (active) {
            XRegs<C::WDT, C::IN, C::NCD> xr;
            xr.load(vin, d, sub, G);
            float out = rn * st.finish(xr);
            if (roped) {  // uniform over the wave
                // r[0] holds the element of the first half (lane < 32), r[1] its partner
                const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(out), __float_as_uint(out), false, false);
                const float x0 = __uint_as_float(r[0]), x1 = __uint_as_float(r[1]);
                out = second ? fmaf(x0, sn, x1 * cs) : fmaf(-x1, sn, x0 * cs);
            }
            if (sub < C::LLR) {
                // query head h = row / D sits in group h / REP at slot h % REP; then key, value
                ll_put(put_at, out, c.ep(l, 0));
                if (!C::FLOOR && sub == 0 && which != 0) crow[static_cast<size_t>(l) * cstride] = out;
            }
        }
        if (l + 1 == s.L && bt == 0 && threadIdx.x == 0) ll_put(p.ll_late, 0.f, c.ep(l, 0));
        if (l + 1 < s.L) {
            st.start(wmat(l + 1), row, d, sub, active);
            load_gains(gr, p.layers[l + 1].attn_norm, d);
        }
    }
}

// ---- role 1: attention partials, a block per (group, four 32-position chunks) --------------------
// Each wave scores one chunk; the block folds its waves' (max, sum, weighted
// values) into one partial per head in LDS, rescaling each by e^(m_w - M),
// so the Wo blocks fetch a quarter of the partials.
template <class C>
__device__ void role_attn(const StepArgs& s, const PersistArgs& p, const PCtx& c, int bt, float* sm) {
    constexpr int PD = C::PD, REP = C::REP, PS = PD + 2;
    const int wv = threadIdx.x >> 6;
    const int HD = s.H * PD, KVD = s.Hkv * PD;
    const int g = bt % s.Hkv, part = bt / s.Hkv, ck = part * 4 + wv;
    const int nw = min(4, c.nch - part * 4);  // waves with a chunk (>= 1)
    const bool active = wv < nw;
    KV<PD, REP, C::FLOOR> kv;
    if (active) kv.load(s, 0, g, ck * kPChunk, c.pos);
    float* qkv = sm;
    float* pw = sm + ((HD + 2 * KVD + 3) & ~3) + wv * REP * KV<PD, REP>::PWS;  // softmax weights of this wave
    float* cmb = sm + ((HD + 2 * KVD + 3) & ~3) + 4 * REP * KV<PD, REP>::PWS;  // [wave][head][m, l, D]
    uint64_t* dst = p.ll_part + static_cast<size_t>((g * c.npart + part) * REP) * PS;
    constexpr int GS = (REP + 2) * PD;  // the group's queries, key and value (group-major words)
    for (int l = 0; l < s.L; l++) {
        __syncthreads();
        wait_sample<2, true>(p.ll_qkv + c.rep + g * GS, GS, c.ep(l, 0), c.err);
        block_fetch2<2>(Seg{p.ll_qkv + c.rep + g * GS, GS, c.ep(l, 0), qkv + g * GS}, c.err);
        __syncthreads();
        if (active) {
            kv.attend(qkv, g, ck * kPChunk, c.pos, pw, [&](int j, int e, float m, float lsum, float acc, float) {
                float* cw = cmb + (wv * REP + j) * PS;
                cw[2 + e] = acc;
                if (e == 0) {
                    cw[0] = m;
                    cw[1] = lsum;
                }
            });
        }
        __syncthreads();
        const uint32_t e1 = c.ep(l, 1);
        for (int idx = threadIdx.x; idx < REP * PD; idx += kPThreads) {
            const int j = idx / PD, e = idx % PD;
            float2 ml[4];
            float v[4];
#pragma unroll
            for (int w = 0; w < 4; w++) {  // waves past nw repeat the last one, with weight 0
                const float* cw = cmb + (min(w, nw - 1) * REP + j) * PS;
                ml[w] = *reinterpret_cast<const float2*>(cw);
                v[w] = cw[2 + e];
            }
            const float M = OpMax{}(OpMax{}(ml[0].x, ml[1].x), OpMax{}(ml[2].x, ml[3].x));
            float A = 0.f, L = 0.f;
#pragma unroll
            for (int w = 0; w < 4; w++) {
                const float f = w < nw ? __expf(ml[w].x - M) : 0.f;  // each wave's max is finite: its chunk holds a position <= pos
                A = fmaf(f, v[w], A);
                L = fmaf(f, ml[w].y, L);
            }
            ll_put(dst + j * PS + 2 + e, A, e1);
            if (e == 0) {
                ll_put(dst + j * PS, M, e1);
                ll_put(dst + j * PS + 1, L, e1);
            }
        }
        // after the barrier above, which would otherwise wait for these loads
        if (active && l + 1 < s.L) kv.load(s, l + 1, g, ck * kPChunk, c.pos);
    }
}

// Attention output from the block partials in LDS (layout [group][part]
// [head][m, l, D], np parts): o = sum_p e^(m_p - M) o_p / sum_p e^(m_p - M) l_p
// with M = max_p m_p, four dims per thread in one pass.  NP >= np is the
// unrolled count: parts past np repeat the last one with weight 0, so every
// LDS read is issued before the first use.
template <int PD, int REP, int NP, int WDT>
__device__ __forceinline__ void merge_parts_t(const float* in, int np, int H, float* o) {
    constexpr int PS = PD + 2, cstride = REP * PS;
    const int HD = H * PD;
    for (int t = threadIdx.x; t < HD / 4; t += kPThreads) {
        const int h = 4 * t / PD, e = 4 * t % PD;
        const float* ph = in + static_cast<size_t>((h / REP) * np * REP + h % REP) * PS;
        float2 ml[NP], a[NP], b[NP];
#pragma unroll
        for (int pp = 0; pp < NP; pp++) {
            const float* q = ph + min(pp, np - 1) * cstride;
            ml[pp] = *reinterpret_cast<const float2*>(q);
            a[pp] = *reinterpret_cast<const float2*>(q + 2 + e);
            b[pp] = *reinterpret_cast<const float2*>(q + 4 + e);
        }
        float M = ml[0].x;
#pragma unroll
        for (int pp = 1; pp < NP; pp++) M = OpMax{}(M, ml[pp].x);
        float L = 0.f, a0 = 0.f, a1 = 0.f, a2 = 0.f, a3 = 0.f;
#pragma unroll
        for (int pp = 0; pp < NP; pp++) {
            const float w = pp < np ? __expf(ml[pp].x - M) : 0.f;
            L = fmaf(w, ml[pp].y, L);
            a0 = fmaf(w, a[pp].x, a0);
            a1 = fmaf(w, a[pp].y, a1);
            a2 = fmaf(w, b[pp].x, a2);
            a3 = fmaf(w, b[pp].y, a3);
        }
        const float inv = 1.0f / L;
        put_pair<WDT>(o, HD, h * PD + e, a0 * inv, a1 * inv);
        put_pair<WDT>(o, HD, h * PD + e + 2, a2 * inv, a3 * inv);
    }
}

// ---- role 2: attention output of every head, Wo, residual (4 * R rows per block) ------------------
template <class C>
__device__ void role_wo(const StepArgs& s, const PersistArgs& p, const PCtx& c, int bt, float* sm) {
    constexpr int G = C::GH, R = 64 / G, PD = C::PD, REP = C::REP;
    constexpr int EPC = C::WDT == kBF16 ? 8 : 4;
    const int wv = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int d = s.d, HD = s.H * PD, KVD = s.Hkv * PD;
    const int rs = lane / G, sub = lane % G;
    const int r0 = bt * 4 * R, nrows = min(4 * R, d - r0);
    const int row = r0 + wv * R + rs;
    const bool valid = row < d;
    const bool attn_wave = wv < s.Hkv;  // wave g handles key/value group g
    const int g = attn_wave ? wv : 0;
    // LDS: [Q/K/V words | partials] [o: H*D] [residual rows: 4R] [softmax weights: 4][REP][32]
    const int in_n = !C::LONG ? HD + 2 * KVD : c.npart * s.H * (PD + 2);
    float* in = sm;
    float* o = sm + ((in_n + 3) & ~3);
    float* xr = o + HD;
    float* pw = xr + 64 + wv * REP * KV<PD, REP>::PWS;
    PStream<C::WDT, G, C::NCH, C::FLOOR> st;
    KV<PD, REP, C::FLOOR> kv;
    st.start(p.layers[0].wo, valid ? row : 0, HD, sub, valid);
    if (!C::LONG && attn_wave) kv.load(s, 0, g, 0, c.pos);
    for (int l = 0; l < s.L; l++) {
        __syncthreads();
        Seg rows{p.ll_x, 0, 0u, xr};
        if (l == 0) {
            if (static_cast<int>(threadIdx.x) < nrows) xr[threadIdx.x] = emb_at<C::WDT>(s, c.tok, r0 + threadIdx.x);
        } else {
            rows = Seg{p.ll_x + c.rep + r0, nrows, c.ep(l - 1, 4), xr};
        }
        if constexpr (!C::LONG) {
            wait_sample<2, true>(p.ll_qkv + c.rep, in_n, c.ep(l, 0), c.err);
            block_fetch2<2>(Seg{p.ll_qkv + c.rep, in_n, c.ep(l, 0), in}, rows, c.err);
        } else {
            wait_sample<2, true>(p.ll_part, in_n, c.ep(l, 1), c.err);
            // 20 words per thread and round: the partials of a 1024-position
            // context (8 parts x H x (D + 2) words, 4752 at 135M) arrive in
            // one memory round trip instead of the three of 2048-word rounds
            block_fetch<20>(Seg{p.ll_part, in_n, c.ep(l, 1), in}, rows, c.err);
        }
        __syncthreads();
        if (attn_wave) {
            if constexpr (!C::LONG) {
                kv.attend(in, g, 0, c.pos, pw, [&](int j, int e, float, float lsum, float acc, float acc1) {
                    const float inv = __builtin_amdgcn_rcpf(lsum);  // lsum >= 1 (the max term is exp(0))
                    if ((e & 1) == 0) put_pair<C::IN>(o, HD, (g * REP + j) * PD + e, acc * inv, acc1 * inv);
                });
            }
        }
        if constexpr (C::LONG) {
            switch ((c.npart + 3) / 4) {  // partial counts unrolled in fours
                case 1: merge_parts_t<PD, REP, 4, C::IN>(in, c.npart, s.H, o); break;
                case 2: merge_parts_t<PD, REP, 8, C::IN>(in, c.npart, s.H, o); break;
                case 3: merge_parts_t<PD, REP, 12, C::IN>(in, c.npart, s.H, o); break;
                default: merge_parts_t<PD, REP, 16, C::IN>(in, c.npart, s.H, o); break;
            }
        }
        __syncthreads();
        XRegs<C::WDT, C::IN, C::NCH> ox;
        ox.load(o, HD, sub, G);
        const float y = st.finish(ox);
        if (valid && sub < C::LLR) ll_put(p.ll_x2 + sub * p.rstride + row, xr[row - r0] + y, c.ep(l, 2));
        if (l + 1 < s.L) {
            st.start(p.layers[l + 1].wo, valid ? row : 0, HD, sub, valid);
            if (!C::LONG && attn_wave) kv.load(s, l + 1, g, 0, c.pos);
        }
    }
}

// ---- role 3: RMSNorm, W1 / W3, silu(a) * u (4 * R rows per block) ---------------------------------
template <class C>
__device__ void role_w13(const StepArgs& s, const PersistArgs& p, const PCtx& c, int bt, float* sm) {
    constexpr int G = C::GD, R = 64 / G;
    constexpr int EPC = C::WDT == kBF16 ? 8 : 4;
    const int wv = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int d = s.d, F = s.F;
    const int rs = lane / G, sub = lane % G;
    const int row = bt * 4 * R + wv * R + rs;
    const bool valid = row < F;
    PStream<C::WDT, G, C::NCD, C::FLOOR> s1, s3;
    float gr[kPNorm];
    s1.start(p.layers[0].w1, valid ? row : 0, d, sub, valid);
    s3.start(p.layers[0].w3, valid ? row : 0, d, sub, valid);
    load_gains(gr, p.layers[0].ffn_norm, d);
    float* const vin = sm;  // product input (see put_pair)
    for (int l = 0; l < s.L; l++) {
        __syncthreads();
        wait_sample<2, true>(p.ll_x2 + c.rep, d, c.ep(l, 2), c.err);
        float xv[kPNorm];
        block_fetch_own(Seg{p.ll_x2 + c.rep, d, c.ep(l, 2), nullptr}, xv, c.err);
        const float rn = block_norm_regs<C::IN>(xv, d, gr, s.eps, sm, vin);
        XRegs<C::WDT, C::IN, C::NCD> xr;
        xr.load(vin, d, sub, G);
        const float a = rn * s1.finish(xr);
        const float u = rn * s3.finish(xr);
        if (valid && sub < C::LLR)
            ll_put(p.ll_h + sub * p.rstride + row, a * __builtin_amdgcn_rcpf(1.0f + __expf(-a)) * u, c.ep(l, 3));
        if (l + 1 < s.L) {
            s1.start(p.layers[l + 1].w1, valid ? row : 0, d, sub, valid);
            s3.start(p.layers[l + 1].w3, valid ? row : 0, d, sub, valid);
            load_gains(gr, p.layers[l + 1].ffn_norm, d);
        }
    }
}

// ---- role 4: W2, residual (4 * R rows per block) --------------------------------------------------
template <class C>
__device__ void role_w2(const StepArgs& s, const PersistArgs& p, const PCtx& c, int bt, float* sm) {
    constexpr int G = C::GF, R = 64 / G;
    constexpr int EPC = C::WDT == kBF16 ? 8 : 4;
    const int wv = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int d = s.d, F = s.F;
    const int rs = lane / G, sub = lane % G;
    const int r0 = bt * 4 * R, nrows = min(4 * R, d - r0);
    const int row = r0 + wv * R + rs;
    const bool valid = row < d;
    float* hs = sm;
    float* xr = sm + ((F + 3) & ~3);
    float* hv = C::IN == kBF16 ? xr + 64 : hs;  // product input (see put_pair)
    PStream<C::WDT, G, C::NCF, C::FLOOR> st;
    st.start(p.layers[0].w2, valid ? row : 0, F, sub, valid);
    for (int l = 0; l < s.L; l++) {
        __syncthreads();
        wait_sample<2, true>(p.ll_h + c.rep, F, c.ep(l, 3), c.err);
        // h goes straight into the product input (bf16 hi/lo pairs, or fp32)
        block_fetch2<4>(Seg{p.ll_h + c.rep, F, c.ep(l, 3), hs}, Seg{p.ll_x2 + c.rep + r0, nrows, c.ep(l, 2), xr},
                        c.err, [&](int i, float v0, float v1) { put_pair<C::IN>(hv, F, i, v0, v1); });
        __syncthreads();
        XRegs<C::WDT, C::IN, C::NCF> hx;
        hx.load(hv, F, sub, G);
        const float y = st.finish(hx);
        if (valid && sub < C::LLR) ll_put(p.ll_x + sub * p.rstride + row, xr[row - r0] + y, c.ep(l, 4));
        if (l + 1 < s.L) st.start(p.layers[l + 1].w2, valid ? row : 0, F, sub, valid);
    }
}

// Blocks per role for a context of nch attention chunks (role 1 is empty when
// attention is fused into Wo).
struct Roles {
    int b[5];
    __host__ __device__ Roles(int d, int H, int Hkv, int D, int F, int gd, int gh, int gf, int nch) {
        const int HD = H * D, KVD = Hkv * D;
        b[0] = ((HD + 2 * KVD) / (64 / gd) + 3) / 4;
        b[1] = nch <= 1 ? 0 : Hkv * ((nch + 3) / 4);
        b[2] = (d + 4 * (64 / gh) - 1) / (4 * (64 / gh));
        b[3] = (F + 4 * (64 / gd) - 1) / (4 * (64 / gd));
        b[4] = (d + 4 * (64 / gf) - 1) / (4 * (64 / gf));
    }
    __host__ __device__ int total() const { return b[0] + b[1] + b[2] + b[3] + b[4]; }
};

template <class C>
__global__ __launch_bounds__(kPThreads, 1) void k_persist(StepArgs s, PersistArgs p, const int32_t* __restrict__ d_tok_in,
                                                           int tok_value, int32_t* __restrict__ d_tok_out) {
    constexpr int GD = C::GD;
    constexpr int EPC = C::WDT == kBF16 ? 8 : 4;
    extern __shared__ float sm[];
    const int blk = blockIdx.x, wv = threadIdx.x >> 6, lane = threadIdx.x & 63;
    PCtx c;
    c.err = s.err;
    c.base = *p.epoch;
    c.pos = s.lengths[0];
    c.n = c.pos + 1;
    c.nch = (c.n + kPChunk - 1) / kPChunk;
    c.npart = (c.nch + 3) / 4;
    c.fused = c.nch == 1;
    if (c.fused == C::LONG) {  // launched for the other context class: flag it and do nothing (every block)
        if (threadIdx.x == 0 && blk == 0) atomicOr(c.err, 2);
        return;
    }
    c.rep = (blk % C::LLR) * p.rstride;
    c.tok = d_tok_in ? d_tok_in[0] : tok_value;
    if (c.tok < 0 || c.tok >= s.V) {
        if (threadIdx.x == 0 && blk == 0) atomicOr(c.err, 1);
        c.tok = 0;
    }
    const Roles ro(s.d, s.H, s.Hkv, C::PD, s.F, C::GD, C::GH, C::GF, c.nch);
    {
        float g[kPNorm];
        load_gains(g, p.out_norm, s.d);
#pragma unroll
        for (int j = 0; j < kPNorm; j++) sm[kPGains + min(own_elem(j), s.d - 1)] = g[j];  // read back by this thread
    }
    int bt = blk;
    if (bt < ro.b[0]) {
        role_qkv<C>(s, p, c, bt, sm);
    } else if ((bt -= ro.b[0]) < ro.b[1]) {
        if constexpr (C::LONG) role_attn<C>(s, p, c, bt, sm);  // no role 1 blocks for one chunk
    } else if ((bt -= ro.b[1]) < ro.b[2]) {
        role_wo<C>(s, p, c, bt, sm);
    } else if ((bt -= ro.b[2]) < ro.b[3]) {
        role_w13<C>(s, p, c, bt, sm);
    } else if ((bt -= ro.b[3]) < ro.b[4]) {
        role_w2<C>(s, p, c, bt, sm);
    }

    // ---- final RMSNorm, vocabulary rows, one argmax word per wave --------------------------------
    // Wave gw takes the row tasks gw, gw + 1024, ...; two tasks are in flight.
    const uint32_t epk = c.ep(s.L, 0);
    {
        constexpr int R = 64 / GD;
        const int gw = blk * 4 + wv;
        const int ntask = (s.V + R - 1) / R;
        const int rs = lane / GD, sub = lane % GD;
        PStream<C::WDT, GD, C::NCD, C::FLOOR> sa, sb;
        const int ta = gw, tb = gw + kPWaves;
        // Workgroups without a layer role load their first two tasks now.  The
        // others load theirs once x is in: a poll waits for every load before it.
        const bool idle = blk >= ro.total();
        auto start2 = [&]() {
            sa.start(p.wcls, min(ta * R + rs, s.V - 1), s.d, sub, ta * R + rs < s.V);
            sb.start(p.wcls, min(tb * R + rs, s.V - 1), s.d, sub, tb * R + rs < s.V);
        };
        if (idle) start2();
        float gr[kPNorm];
#pragma unroll
        for (int j = 0; j < kPNorm; j++) gr[j] = sm[kPGains + min(own_elem(j), s.d - 1)];  // this thread's own
        float* const vin = sm;  // product input (see put_pair)
        __syncthreads();
        if (idle) wait_word<32>(p.ll_late, c.ep(s.L - 1, 0), c.err);  // the others are past the last layer's start
        wait_sample<2, true>(p.ll_x + c.rep, s.d, c.ep(s.L - 1, 4), c.err);
        float xv[kPNorm];
        block_fetch_own(Seg{p.ll_x + c.rep, s.d, c.ep(s.L - 1, 4), nullptr}, xv, c.err);
        if (!idle) start2();
        const float rn = block_norm_regs<C::IN>(xv, s.d, gr, s.eps, sm, vin);
        XRegs<C::WDT, C::IN, C::NCD> xr;
        xr.load(vin, s.d, sub, GD);
        uint64_t key = 0ull;
        auto take = [&](const PStream<C::WDT, GD, C::NCD, C::FLOOR>& st, int t) {
            const int row = t * R + rs;
            const float y = rn * st.finish(xr);
            if (row < s.V && sub == 0) {
                if (!C::FLOOR) s.logits[row] = y;
                const uint64_t k = key_word(y, row, epk);
                key = k > key ? k : key;
            }
        };
        // the streams alternate; the one just used takes the task after the one in flight
        for (int t = ta; t < ntask; t += 2 * kPWaves) {
            take(sa, t);
            const int t2 = t + 2 * kPWaves;
            if (t2 < ntask) sa.start(p.wcls, min(t2 * R + rs, s.V - 1), s.d, sub, t2 * R + rs < s.V);
            const int u = t + kPWaves;
            if (u >= ntask) break;
            take(sb, u);
            const int u2 = u + 2 * kPWaves;
            if (u2 < ntask) sb.start(p.wcls, min(u2 * R + rs, s.V - 1), s.d, sub, u2 * R + rs < s.V);
        }
        key = wave_max_u64(key);
        if (lane == 0) {
            if (key == 0ull) key = epk & 0x7FFFu;  // a wave without rows still reports
            __hip_atomic_store(p.ll_keys + gw, key, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
    }
    // ---- one wave reduces the argmax words, writes the token and the bookkeeping ------------------
    if (blk == 0 && wv == 0) {
        constexpr int JK = kPWaves / 64;
        uint64_t wds[JK];
        long spins = 0;
        while (true) {
#pragma unroll
            for (int j = 0; j < JK; j++) wds[j] = ll_get(p.ll_keys + lane + 64 * j);
            bool ok = true;
#pragma unroll
            for (int j = 0; j < JK; j++) ok &= (wds[j] & 0x7FFFu) == (epk & 0x7FFFu);
            if (__all(ok)) break;
            if (give_up(spins, c.err)) break;
        }
        uint64_t best = 0ull;
#pragma unroll
        for (int j = 0; j < JK; j++) best = wds[j] > best ? wds[j] : best;
        best = wave_max_u64(best);
        if (lane == 0) {
            const int idx = static_cast<int>(0x1FFFFu - static_cast<uint32_t>((best >> 15) & 0x1FFFFu));
            if (!C::FLOOR) {  // the floor diagnostic leaves the token, lengths and step state alone
                if (d_tok_out) d_tok_out[0] = idx;
                s.lengths[0] = c.pos + 1;
                s.pos[0] = c.pos;
                s.slot[0] = 0;
                s.flag[0] = 1;
            }
            *p.epoch = c.base + static_cast<uint32_t>(s.L * kPhases + 2);
        }
    }
}

// ---- host side ----------------------------------------------------------------------------------

static int epc(int wdt) { return wdt == kBF16 ? 8 : 4; }
static int pnc(int K, int wdt, int g) { return (K / epc(wdt) + g - 1) / g; }

// The instantiated shape classes, each with its lanes per row (G) and
// chunks per lane (NC) for rows of d, H*D and F elements: the 135M-class
// model with bf16 weights and the small fp32 test model.  Other shapes take
// the per-operation path.
struct PKernel {
    int wdt, in, floor, long_, D, rep, gd, ncd, gh, nch, gf, ncf;
    const void* fn;
};
// The 135M class comes with both product inputs (bf16 hi/lo pairs, and fp32
// with the weights widened), and every class with its handoff-floor twin,
// each for one-chunk and for longer contexts.
template <int IN, bool FLOOR, bool LONG>
using CfgM135 = PCfg<kBF16, 64, 3, 8, 9, 8, 9, 16, 12, IN, FLOOR, LONG>;
template <bool FLOOR, bool LONG>
using CfgTiny = PCfg<kF32, 16, 2, 4, 4, 4, 4, 4, 11, kF32, FLOOR, LONG>;
template <class C>
static constexpr PKernel pk() {
    return {C::WDT, C::IN, C::FLOOR ? 1 : 0, C::LONG ? 1 : 0, C::PD, C::REP, C::GD, C::NCD, C::GH, C::NCH, C::GF,
            C::NCF, reinterpret_cast<const void*>(k_persist<C>)};
}
static const PKernel kPKernels[] = {
    pk<CfgM135<kBF16, false, false>>(), pk<CfgM135<kBF16, false, true>>(), pk<CfgM135<kF32, false, false>>(),
    pk<CfgM135<kF32, false, true>>(),   pk<CfgM135<kBF16, true, false>>(),  pk<CfgM135<kBF16, true, true>>(),
    pk<CfgM135<kF32, true, false>>(),   pk<CfgM135<kF32, true, true>>(),    pk<CfgTiny<false, false>>(),
    pk<CfgTiny<false, true>>(),         pk<CfgTiny<true, false>>(),         pk<CfgTiny<true, true>>()};

// The kernel for this shape, product input (s.pin; fp32 weights always take
// fp32 inputs), floor flag and context class (long: more than one chunk),
// or nullptr.
static const PKernel* persist_kernel(const StepArgs& s, bool floor = false, bool long_ = false) {
    if (s.Hkv <= 0 || s.H % s.Hkv) return nullptr;
    const int in = s.wdt == kBF16 ? s.pin : kF32;
    for (const PKernel& k : kPKernels) {
        if (k.wdt != s.wdt || k.in != in || k.floor != (floor ? 1 : 0) || k.long_ != (long_ ? 1 : 0) ||
            k.D != s.D || k.rep != s.H / s.Hkv)
            continue;
        // every lane's chunks must fit its registers, and every G-lane group must have work
        if (pnc(s.d, s.wdt, k.gd) > k.ncd || pnc(s.H * s.D, s.wdt, k.gh) > k.nch || pnc(s.F, s.wdt, k.gf) > k.ncf)
            continue;
        return &k;
    }
    return nullptr;
}

int persist_max_ctx(const StepArgs& s) {
    const int HD = s.H * s.D, KVD = s.Hkv * s.D;
    const PKernel* k = s.B == 1 && s.cdt == kF32 ? persist_kernel(s) : nullptr;  // fp32 cache only
    if (!k) return 0;
    // d even (word pairs), d <= 1024 (four owned elements per thread)
    if (s.d > kPThreads * kPNorm || s.d < 64 || (s.d & 1) || s.Hkv > 4 || s.V > 0x1FFFF) return 0;
    // LDS of role 2 (Q/K/V words, o, residual rows, softmax weights) and role 4 (h, residual rows)
    const int pws = 4 * (s.H / s.Hkv) * (kPChunk + 4);
    if (2 * HD + 2 * KVD + 4 + 64 + pws > kPRed || 2 * s.F + 4 + 64 > kPRed || (s.F & 1)) return 0;
    if (Roles(s.d, s.H, s.Hkv, s.D, s.F, k->gd, k->gh, k->gf, 1).total() > kPBlocks) return 0;
    // longer contexts add role 1 blocks (Q/K/V words, softmax weights, the
    // waves' partials in LDS) and keep every block partial in role 2's LDS
    const int attn_lds = ((HD + 2 * KVD + 3) & ~3) + pws + 4 * (s.H / s.Hkv) * (s.D + 2);
    int chunks = 1;
    while (chunks < kPMaxChunks) {
        const int nc = chunks + 1;
        if (Roles(s.d, s.H, s.Hkv, s.D, s.F, k->gd, k->gh, k->gf, nc).total() > kPBlocks) break;
        if ((nc + 3) / 4 * s.H * (s.D + 2) + 4 + HD + 64 + pws > kPRed || attn_lds > kPRed || s.H * 16 > pws) break;
        chunks = nc;
    }
    const int ctx = chunks * kPChunk;
    return ctx < s.T ? ctx : s.T;
}

size_t persist_lds() { return sizeof(float) * kPLds; }

// The floor twin holds no weights in registers, so by registers alone two of
// its workgroups could share a CU; asking for more than half of a CU's 160
// KiB of LDS keeps it at one workgroup per CU, as the real step runs.
constexpr int kPFloorLds = 96 * 1024;

// Every workgroup of the single launch must be resident at once (they wait
// on each other's outputs).  This check, run when a cache is created, keeps
// batch-1 steps off the single launch on a device that could never hold all
// kPBlocks workgroups (one per CU at this kernel's register use), e.g. a
// partitioned GPU, or (with s.pcoop) one without cooperative launches.  A
// cooperative launch (s.pcoop) also makes the runtime start it only with
// every workgroup resident; a plain launch relies on this check and on the
// bounded waits, which let the grid drain and flag the step if workgroups of
// another stream's work hold CUs.
bool persist_fits_device(const StepArgs& s) {
    const PKernel* k = persist_kernel(s);
    const PKernel* kl = persist_kernel(s, false, true);
    if (!k || !kl) return false;
    int dev = 0, ncu = 0, per_cu = 0, coop = 0;
    if (hipGetDevice(&dev) != hipSuccess) return false;
    if (hipDeviceGetAttribute(&ncu, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return false;
    if (s.pcoop && (hipDeviceGetAttribute(&coop, hipDeviceAttributeCooperativeLaunch, dev) != hipSuccess || !coop))
        return false;
    for (const PKernel* kk : {k, kl}) {
        if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kk->fn, kPThreads, persist_lds()) != hipSuccess)
            return false;
        if (static_cast<long>(per_cu) * ncu < kPBlocks) return false;
    }
    return true;
}

hipError_t persist_prepare(const StepArgs& s) {
    hipError_t e = hipSuccess;
    for (bool long_ : {false, true}) {
        if (e == hipSuccess)
            e = hipFuncSetAttribute(persist_kernel(s, false, long_)->fn, hipFuncAttributeMaxDynamicSharedMemorySize,
                                    static_cast<int>(persist_lds()));
        if (e == hipSuccess)
            e = hipFuncSetAttribute(persist_kernel(s, true, long_)->fn, hipFuncAttributeMaxDynamicSharedMemorySize,
                                    kPFloorLds);
    }
    return e;
}

// Cooperative when asked for (s.pcoop) and the stream is not being captured
// into a graph; else a plain launch, whose co-residency rests on
// persist_fits_device and the bounded waits alone.
static hipError_t launch_persist(const StepArgs& s, const void* fn, void** args, size_t lds, hipStream_t st) {
    hipStreamCaptureStatus cap = hipStreamCaptureStatusNone;
    hipError_t e = hipStreamIsCapturing(st, &cap);
    if (e != hipSuccess) return e;
    if (s.pcoop && cap == hipStreamCaptureStatusNone)
        return hipLaunchCooperativeKernel(fn, dim3(kPBlocks), dim3(kPThreads), args, lds, st);
    return hipLaunchKernel(fn, dim3(kPBlocks), dim3(kPThreads), args, lds, st);
}

hipError_t enqueue_persist(const StepArgs& s, const PersistArgs& p, const int32_t* d_tok_in, int tok_value,
                           int32_t* d_tok_out, int ctx, hipStream_t st) {
    void* args[] = {const_cast<StepArgs*>(&s), const_cast<PersistArgs*>(&p), &d_tok_in, &tok_value, &d_tok_out};
    return launch_persist(s, persist_kernel(s, false, ctx > kPChunk)->fn, args, persist_lds(), st);
}

hipError_t enqueue_persist_floor(const StepArgs& s, const PersistArgs& p, int ctx, hipStream_t st) {
    const int32_t* tok_in = nullptr;
    int tok_value = 0;
    int32_t* tok_out = nullptr;
    void* args[] = {const_cast<StepArgs*>(&s), const_cast<PersistArgs*>(&p), &tok_in, &tok_value, &tok_out};
    return launch_persist(s, persist_kernel(s, true, ctx > kPChunk)->fn, args, kPFloorLds, st);
}

}  // namespace ds
