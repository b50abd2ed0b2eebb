// kernels.hip -- gfx950 kernels of the single-token Llama decode step.
//
// One decode step for n_items sequences (work items) is:
//   k_begin                      embedding gather + widen, step bookkeeping
//   per layer: k_qkv             RMSNorm -> Q/K/V GEMV -> RoPE -> K/V append
//              k_attn            split-K grouped-query attention partials
//              k_attn_combine    merge of the split-K partials
//              k_wo              Wo GEMV + residual
//              k_w13             RMSNorm -> W1/W3 GEMV -> silu(a)*u
//              k_w2              W2 GEMV + residual
//   k_logits                     RMSNorm -> vocabulary GEMV -> argmax partials
//   k_finalize                   greedy token, lengths += 1
// The block structure is the pre-norm Llama block of "simple-llm / kasahare"
// (PyPI README 0.4.0), section "Architecture"; the cache is the
// (L, 2, B, Hkv, T, D) tensor of "Inside nanochat Part 4: Understanding
// Inference", section "Cache Architecture".
//
// GEMV scheme (all weight matrices, row-major [out][in]): a wave of 64 lanes
// covers R = 64/G output rows with G lanes per row.  Lane (r, sub) streams
// 16-byte chunks sub, sub+G, sub+2G, ... of its row, so the G lanes of a row
// read G*16 contiguous bytes per load and a wave issues 64 fully used 16-byte
// loads per instruction.  bf16 chunks are widened in registers by a 16-bit
// shift ("GOTOken: An Inference Engine in QBasic", section "Loading the model
// and tokenizer") and accumulated in fp32 against the activation vector,
// which the workgroup stages once in LDS.  The G partial sums of a row are
// combined with xor shuffles inside the wave; no LDS or atomics are needed
// for the reduction.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kernels.h"

namespace ds {

constexpr int kBlock = 256;  // 4 waves of 64

// ---- weight chunk loads ------------------------------------------------------

template <int WDT> struct Wt;

template <> struct Wt<kBF16> {
    static constexpr int EPC = 8;  // elements per 16-byte chunk
    __device__ static __forceinline__ void load(const void* base, size_t elem, float (&w)[8]) {
        const uint4 u = *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(base) + elem);
        w[0] = __uint_as_float(u.x << 16); w[1] = __uint_as_float(u.x & 0xFFFF0000u);
        w[2] = __uint_as_float(u.y << 16); w[3] = __uint_as_float(u.y & 0xFFFF0000u);
        w[4] = __uint_as_float(u.z << 16); w[5] = __uint_as_float(u.z & 0xFFFF0000u);
        w[6] = __uint_as_float(u.w << 16); w[7] = __uint_as_float(u.w & 0xFFFF0000u);
    }
};

template <> struct Wt<kF32> {
    static constexpr int EPC = 4;
    __device__ static __forceinline__ void load(const void* base, size_t elem, float (&w)[4]) {
        const float4 f = *reinterpret_cast<const float4*>(static_cast<const float*>(base) + elem);
        w[0] = f.x; w[1] = f.y; w[2] = f.z; w[3] = f.w;
    }
};

template <int EPC>
__device__ __forceinline__ float dot_chunk(const float (&w)[EPC], const float* xs, float acc) {
#pragma unroll
    for (int e = 0; e < EPC; e += 4) {
        const float4 xv = *reinterpret_cast<const float4*>(xs + e);
        acc = fmaf(w[e + 0], xv.x, acc);
        acc = fmaf(w[e + 1], xv.y, acc);
        acc = fmaf(w[e + 2], xv.z, acc);
        acc = fmaf(w[e + 3], xv.w, acc);
    }
    return acc;
}

template <int G>
__device__ __forceinline__ float group_sum(float v) {
#pragma unroll
    for (int o = G / 2; o > 0; o >>= 1) v += __shfl_xor(v, o);
    return v;
}

// Partial dot product of one row (lane `sub` of its G-lane group) with the
// LDS vector xs; `valid` == false makes the lane contribute 0 (masked rows).
template <int WDT, int G>
__device__ __forceinline__ float row_dot(const void* W, size_t row, int K, const float* xs,
                                         int sub, bool valid) {
    constexpr int EPC = Wt<WDT>::EPC;
    const int nch = valid ? K / EPC : 0;
    const size_t base = row * static_cast<size_t>(K);
    float a0 = 0.f, a1 = 0.f;
    int c = sub;
    for (; c + 3 * G < nch; c += 4 * G) {
        float w0[EPC], w1[EPC], w2[EPC], w3[EPC];
        Wt<WDT>::load(W, base + static_cast<size_t>(c) * EPC, w0);
        Wt<WDT>::load(W, base + static_cast<size_t>(c + G) * EPC, w1);
        Wt<WDT>::load(W, base + static_cast<size_t>(c + 2 * G) * EPC, w2);
        Wt<WDT>::load(W, base + static_cast<size_t>(c + 3 * G) * EPC, w3);
        a0 = dot_chunk<EPC>(w0, xs + c * EPC, a0);
        a1 = dot_chunk<EPC>(w1, xs + (c + G) * EPC, a1);
        a0 = dot_chunk<EPC>(w2, xs + (c + 2 * G) * EPC, a0);
        a1 = dot_chunk<EPC>(w3, xs + (c + 3 * G) * EPC, a1);
    }
    for (; c < nch; c += G) {
        float w0[EPC];
        Wt<WDT>::load(W, base + static_cast<size_t>(c) * EPC, w0);
        a0 = dot_chunk<EPC>(w0, xs + c * EPC, a0);
    }
    return group_sum<G>(a0 + a1);
}

// ---- block helpers -------------------------------------------------------------

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

// Sum over the 256 threads of a block; every thread gets the result.
__device__ __forceinline__ float block_sum(float v, float* red4) {
    v = wave_sum(v);
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    __syncthreads();
    if (lane == 0) red4[wave] = v;
    __syncthreads();
    return red4[0] + red4[1] + red4[2] + red4[3];
}

// Stage y = g * (x / sqrt(mean(x^2) + eps)) into LDS (RMSNorm, read as in
// "simple-llm / kasahare", section "Architecture": attn_norm / ffn_norm).
__device__ __forceinline__ void stage_rmsnorm(const float* __restrict__ x,
                                              const float* __restrict__ g, int n, float eps,
                                              float* xs, float* red4) {
    float ss = 0.f;
    for (int j = threadIdx.x; j < n; j += kBlock) {
        const float v = x[j];
        ss = fmaf(v, v, ss);
    }
    ss = block_sum(ss, red4);
    const float r = 1.0f / sqrtf(ss / static_cast<float>(n) + eps);
    for (int j = threadIdx.x; j < n; j += kBlock) xs[j] = g[j] * (r * x[j]);
    __syncthreads();
}

__device__ __forceinline__ void stage_copy(const float* __restrict__ x, int n, float* xs) {
    for (int j = threadIdx.x; j < n; j += kBlock) xs[j] = x[j];
    __syncthreads();
}

__device__ __forceinline__ size_t cache_row(const StepArgs& s, int layer, int kv, int slot, int g,
                                            int t) {
    size_t i = static_cast<size_t>(layer);
    i = i * 2 + kv;
    i = i * s.B + slot;
    i = i * s.Hkv + g;
    i = i * s.T + t;
    return i * s.D;
}

// ---- k_begin: embedding gather -------------------------------------------------
// x[item] = widen(token_emb[tok]); records the slot, position and flags of the
// item and clears its argmax cell.  Token ids outside [0, V) raise the error
// word and read row 0 instead.
__global__ __launch_bounds__(kBlock) void k_begin(StepArgs s, BeginList list,
                                                   const int32_t* __restrict__ d_tok_in) {
    const int li = blockIdx.x;
    if (li >= list.n) return;
    const int item = list.item0 + li;
    const int slot = list.by_value ? list.slot[li] : item;
    int tok = list.by_value ? list.tok[li] : d_tok_in[slot];
    if (tok < 0 || tok >= s.V) {
        if (threadIdx.x == 0) atomicOr(s.err, 1);
        tok = 0;
    }
    const int pos = s.lengths[slot];
    if (threadIdx.x == 0) {
        s.slot[item] = slot;
        s.pos[item] = pos;
        s.flag[item] = list.by_value ? list.last[li] : 1;
        s.keys[item] = 0ull;
    }
    float* x = s.x + static_cast<size_t>(item) * s.d;
    const size_t row = static_cast<size_t>(tok) * s.d;
    if (s.wdt == kBF16) {
        const uint16_t* e = static_cast<const uint16_t*>(s.emb) + row;
        for (int j = threadIdx.x; j < s.d; j += kBlock)
            x[j] = __uint_as_float(static_cast<uint32_t>(e[j]) << 16);
    } else {
        const float* e = static_cast<const float*>(s.emb) + row;
        for (int j = threadIdx.x; j < s.d; j += kBlock) x[j] = e[j];
    }
}

// ---- k_qkv ---------------------------------------------------------------------
// Wave tasks: q rows, then k rows, then v rows, R rows per task.  In the q
// and k sections a task holds R/2 RoPE pairs (i, i + D/2) of a head ("GOTOken",
// section "Loading the model and tokenizer": pairs j and j + head_dim/2): rows
// of the first halves in row slots 0..R/2-1, their partners R/2 rows later,
// i.e. exactly 32 lanes away, so the rotation is one xor-32 shuffle.
template <int WDT, int G>
__global__ __launch_bounds__(kBlock) void k_qkv(StepArgs s, LayerW w, int layer) {
    extern __shared__ float xs[];
    __shared__ float red4[4];
    constexpr int R = 64 / G;
    const int item = blockIdx.y;
    stage_rmsnorm(s.x + static_cast<size_t>(item) * s.d, w.attn_norm, s.d, s.eps, xs, red4);
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int task = blockIdx.x * 4 + wave;
    const int D = s.D, half_d = s.D / 2;
    const int nq = s.H * D / R, nk = s.Hkv * D / R, nv = nk;
    if (task >= nq + nk + nv) return;
    const int rs = lane / G, sub = lane % G;
    const int slot = s.slot[item], pos = s.pos[item];
    if (task < nq + nk) {
        const bool is_q = task < nq;
        const int t = is_q ? task : task - nq;
        const int p = t * (R / 2) + (rs % (R / 2));
        const int second = rs / (R / 2);
        const int head = p / half_d, i = p % half_d;
        const int row = head * D + i + second * half_d;
        const float y = row_dot<WDT, G>(is_q ? w.wq : w.wk, row, s.d, xs, sub, true);
        const float partner = __shfl_xor(y, 32);
        const float c = s.rope_cos[static_cast<size_t>(pos) * half_d + i];
        const float sn = s.rope_sin[static_cast<size_t>(pos) * half_d + i];
        // pair (a, b) -> (a c - b s, a s + b c)
        const float out = second ? fmaf(partner, sn, y * c) : fmaf(-partner, sn, y * c);
        if (sub == 0) {
            if (is_q) {
                s.q[static_cast<size_t>(item) * s.H * D + row] = out;
            } else {
                const int g = row / D, e = row % D;
                s.cache[cache_row(s, layer, 0, slot, g, pos) + e] = out;
            }
        }
    } else {
        const int row = (task - nq - nk) * R + rs;
        const float y = row_dot<WDT, G>(w.wv, row, s.d, xs, sub, true);
        if (sub == 0) {
            const int g = row / D, e = row % D;
            s.cache[cache_row(s, layer, 1, slot, g, pos) + e] = y;
        }
    }
}

// ---- k_attn: split-K grouped-query attention -------------------------------------
// Block (chunk, kv group g, item) scores positions [chunk*kChunk, ...) of the
// item's first pos+1 cached positions against the rep = H/Hkv query heads of
// group g (query head h uses key/value head h / rep, "simple-llm / kasahare",
// section "Architecture", GQA), and writes the chunk's softmax partials
// (running max m, sum l, unnormalised output o) for the combine kernel.
// Thread layout: LPR = D/4 lanes hold one 16-byte slice each of a key/value
// row, so K and V rows are read with full 16-byte coalesced loads.
__global__ __launch_bounds__(kBlock) void k_attn(StepArgs s, int layer) {
    extern __shared__ float sm[];
    const int chunk = blockIdx.x, g = blockIdx.y, item = blockIdx.z;
    const int pos = s.pos[item], slot = s.slot[item];
    const int n = pos + 1;
    const int t0 = chunk * kChunk;
    if (t0 >= n) return;
    const int nt = min(kChunk, n - t0);
    const int D = s.D, rep = s.H / s.Hkv;
    const int LPR = D / 4, NRG = kBlock / LPR;
    const int e4 = threadIdx.x % LPR, rg = threadIdx.x / LPR;
    float* qs = sm;                           // [rep][D]
    float* sc = qs + kMaxRep * kMaxD;         // [rep][kChunk]
    float* red = sc + kMaxRep * kChunk;       // [kBlock][rep*4] reduction scratch
    float* ml = red + kBlock * kMaxRep * 4;   // [rep][2]
    const float* q = s.q + static_cast<size_t>(item) * s.H * D + static_cast<size_t>(g) * rep * D;
    for (int j = threadIdx.x; j < rep * D; j += kBlock) qs[j] = q[j];
    __syncthreads();
    const float* K = s.cache + cache_row(s, layer, 0, slot, g, t0);
    const float* V = s.cache + cache_row(s, layer, 1, slot, g, t0);
    const float scale = 1.0f / sqrtf(static_cast<float>(D));
    // scores: rows rg, rg + NRG, ...; the trip count is uniform per LPR group
    for (int t = rg; t < kChunk; t += NRG) {
        const bool ok = t < nt;
        float4 kv = make_float4(0.f, 0.f, 0.f, 0.f);
        if (ok) kv = *reinterpret_cast<const float4*>(K + static_cast<size_t>(t) * D + e4 * 4);
        for (int j = 0; j < rep; j++) {
            const float4 qv = *reinterpret_cast<const float4*>(qs + j * D + e4 * 4);
            float d = kv.x * qv.x;
            d = fmaf(kv.y, qv.y, d);
            d = fmaf(kv.z, qv.z, d);
            d = fmaf(kv.w, qv.w, d);
            for (int o = LPR / 2; o > 0; o >>= 1) d += __shfl_xor(d, o);
            if (ok && e4 == 0) sc[j * kChunk + t] = d * scale;
        }
    }
    __syncthreads();
    // per head: chunk max and exp-sum (one wave per head)
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    for (int j = wave; j < rep; j += 4) {
        float m = -INFINITY;
        for (int t = lane; t < nt; t += 64) m = fmaxf(m, sc[j * kChunk + t]);
        m = wave_max(m);
        float l = 0.f;
        for (int t = lane; t < nt; t += 64) {
            const float p = __expf(sc[j * kChunk + t] - m);
            sc[j * kChunk + t] = p;
            l += p;
        }
        l = wave_sum(l);
        if (lane == 0) {
            ml[j * 2 + 0] = m;
            ml[j * 2 + 1] = l;
        }
    }
    __syncthreads();
    // o_j = sum_t p_j[t] * V[t]
    float acc[kMaxRep][4];
    for (int j = 0; j < kMaxRep; j++) acc[j][0] = acc[j][1] = acc[j][2] = acc[j][3] = 0.f;
    for (int t = rg; t < nt; t += NRG) {
        const float4 vv = *reinterpret_cast<const float4*>(V + static_cast<size_t>(t) * D + e4 * 4);
#pragma unroll
        for (int j = 0; j < kMaxRep; j++) {
            if (j < rep) {
                const float p = sc[j * kChunk + t];
                acc[j][0] = fmaf(p, vv.x, acc[j][0]);
                acc[j][1] = fmaf(p, vv.y, acc[j][1]);
                acc[j][2] = fmaf(p, vv.z, acc[j][2]);
                acc[j][3] = fmaf(p, vv.w, acc[j][3]);
            }
        }
    }
    for (int j = 0; j < rep; j++)
        for (int c = 0; c < 4; c++) red[(j * 4 + c) * kBlock + threadIdx.x] = acc[j][c];
    __syncthreads();
    // sum the NRG row groups; thread -> (j, e)
    const int S = s.n_chunks;
    for (int idx = threadIdx.x; idx < rep * D; idx += kBlock) {
        const int j = idx / D, e = idx % D;
        const int te4 = e / 4, c = e % 4;
        float v = 0.f;
        for (int r = 0; r < NRG; r++) v += red[(j * 4 + c) * kBlock + r * LPR + te4];
        const int h = g * rep + j;
        const size_t pidx = (static_cast<size_t>(item) * s.H + h) * S + chunk;
        s.part_o[pidx * D + e] = v;
        if (e == 0) {
            s.part_ml[pidx * 2 + 0] = ml[j * 2 + 0];
            s.part_ml[pidx * 2 + 1] = ml[j * 2 + 1];
        }
    }
}

// Merge the chunk partials of one (item, head): M = max m_s,
// o = sum_s e^(m_s - M) o_s / sum_s e^(m_s - M) l_s.
__global__ __launch_bounds__(64) void k_attn_combine(StepArgs s) {
    const int h = blockIdx.x, item = blockIdx.y;
    const int n = s.pos[item] + 1;
    const int ns = (n + kChunk - 1) / kChunk;
    const int S = s.n_chunks, D = s.D;
    const size_t base = (static_cast<size_t>(item) * s.H + h) * S;
    float M = -INFINITY;
    for (int c = 0; c < ns; c++) M = fmaxf(M, s.part_ml[(base + c) * 2]);
    float L = 0.f;
    for (int c = 0; c < ns; c++) L += __expf(s.part_ml[(base + c) * 2] - M) * s.part_ml[(base + c) * 2 + 1];
    const float inv = 1.0f / L;
    for (int e = threadIdx.x; e < D; e += 64) {
        float o = 0.f;
        for (int c = 0; c < ns; c++)
            o = fmaf(__expf(s.part_ml[(base + c) * 2] - M), s.part_o[(base + c) * D + e], o);
        s.o[(static_cast<size_t>(item) * s.H + h) * D + e] = o * inv;
    }
}

// ---- k_wo: x += Wo o --------------------------------------------------------------
template <int WDT, int G>
__global__ __launch_bounds__(kBlock) void k_wo(StepArgs s, LayerW w) {
    extern __shared__ float xs[];
    constexpr int R = 64 / G;
    const int item = blockIdx.y;
    const int K = s.H * s.D;
    stage_copy(s.o + static_cast<size_t>(item) * K, K, xs);
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int row = (blockIdx.x * 4 + wave) * R + lane / G, sub = lane % G;
    const bool valid = row < s.d;
    const float y = row_dot<WDT, G>(w.wo, valid ? row : 0, K, xs, sub, valid);
    if (valid && sub == 0) s.x[static_cast<size_t>(item) * s.d + row] += y;
}

// ---- k_w13: h = silu(W1 xn) * (W3 xn) -------------------------------------------
template <int WDT, int G>
__global__ __launch_bounds__(kBlock) void k_w13(StepArgs s, LayerW w) {
    extern __shared__ float xs[];
    __shared__ float red4[4];
    constexpr int R = 64 / G;
    const int item = blockIdx.y;
    stage_rmsnorm(s.x + static_cast<size_t>(item) * s.d, w.ffn_norm, s.d, s.eps, xs, red4);
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int row = (blockIdx.x * 4 + wave) * R + lane / G, sub = lane % G;
    const bool valid = row < s.F;
    const float a = row_dot<WDT, G>(w.w1, valid ? row : 0, s.d, xs, sub, valid);
    const float u = row_dot<WDT, G>(w.w3, valid ? row : 0, s.d, xs, sub, valid);
    if (valid && sub == 0) {
        const float sig = 1.0f / (1.0f + expf(-a));
        s.h[static_cast<size_t>(item) * s.F + row] = (a * sig) * u;
    }
}

// ---- k_w2: x += W2 h ----------------------------------------------------------------
template <int WDT, int G>
__global__ __launch_bounds__(kBlock) void k_w2(StepArgs s, LayerW w) {
    extern __shared__ float xs[];
    constexpr int R = 64 / G;
    const int item = blockIdx.y;
    stage_copy(s.h + static_cast<size_t>(item) * s.F, s.F, xs);
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int row = (blockIdx.x * 4 + wave) * R + lane / G, sub = lane % G;
    const bool valid = row < s.d;
    const float y = row_dot<WDT, G>(w.w2, valid ? row : 0, s.F, xs, sub, valid);
    if (valid && sub == 0) s.x[static_cast<size_t>(item) * s.d + row] += y;
}

// ---- k_logits: logits = Wcls rmsnorm(x), greedy argmax partials ----------------------
// Argmax key: the float's order-preserving 32-bit image in the high word and
// (2^32 - 1 - index) in the low word, so one 64-bit atomic max selects the
// largest logit and, among equal logits, the lowest index ("Inside nanochat
// Part 4", section "Sampling Strategy": greedy decoding is argmax), whatever
// order the blocks finish in.
__device__ __forceinline__ unsigned long long argmax_key(float v, int idx) {
    uint32_t u = __float_as_uint(v);
    u = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
    return (static_cast<unsigned long long>(u) << 32) | static_cast<uint32_t>(0xFFFFFFFFu - idx);
}

template <int WDT, int G>
__global__ __launch_bounds__(kBlock) void k_logits(StepArgs s, const float* __restrict__ out_norm,
                                                    const void* __restrict__ wcls) {
    extern __shared__ float xs[];
    __shared__ float red4[4];
    constexpr int R = 64 / G;
    const int item = blockIdx.y;
    if (!s.flag[item]) return;
    stage_rmsnorm(s.x + static_cast<size_t>(item) * s.d, out_norm, s.d, s.eps, xs, red4);
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int row = (blockIdx.x * 4 + wave) * R + lane / G, sub = lane % G;
    const bool valid = row < s.V;
    const float y = row_dot<WDT, G>(wcls, valid ? row : 0, s.d, xs, sub, valid);
    unsigned long long key = 0ull;
    if (valid && sub == 0) {
        s.logits[static_cast<size_t>(s.slot[item]) * s.V + row] = y;
        key = argmax_key(y, row);
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
        const unsigned long long other = __shfl_xor(key, o);
        key = other > key ? other : key;
    }
    if (lane == 0) atomicMax(s.keys + item, key);
}

// ---- k_finalize ------------------------------------------------------------------------
__global__ __launch_bounds__(64) void k_finalize(StepArgs s, int n_items, int32_t* d_tok_out,
                                                 int want_tok) {
    for (int item = threadIdx.x; item < n_items; item += 64) {
        const int slot = s.slot[item];
        if (want_tok && s.flag[item] && d_tok_out)
            d_tok_out[slot] = static_cast<int32_t>(0xFFFFFFFFu - static_cast<uint32_t>(s.keys[item]));
        s.lengths[slot] = s.pos[item] + 1;
    }
}

// ---- small utility kernels ----------------------------------------------------------------
__global__ void k_set_lengths(int32_t* lengths, SetList l) {
    for (int i = threadIdx.x; i < l.n; i += blockDim.x) lengths[l.first + i] = l.val[i];
}

__global__ void k_fill_i32(int32_t* p, int n, int32_t v) {
    for (int i = blockIdx.x * blockDim.x + threadIdx.x; i < n; i += gridDim.x * blockDim.x) p[i] = v;
}

// ---- launchers ---------------------------------------------------------------------------

static int pick_g(int K, int wdt) {
    const int nch = K / (wdt == kBF16 ? 8 : 4);
    if (nch <= 128) return 8;
    if (nch <= 512) return 16;
    return 32;
}

template <int WDT, int G>
static hipError_t launch_gemv_set(int which, const StepArgs& s, const LayerW& w, int layer,
                                  int n_items, hipStream_t st, const float* out_norm,
                                  const void* wcls) {
    constexpr int R = 64 / G;
    const int rows_per_block = 4 * R;
    switch (which) {
        case 0: {
            const int tasks = (s.H + 2 * s.Hkv) * s.D / R;
            hipLaunchKernelGGL((k_qkv<WDT, G>), dim3((tasks + 3) / 4, n_items), dim3(kBlock),
                               s.d * sizeof(float), st, s, w, layer);
            break;
        }
        case 1:
            hipLaunchKernelGGL((k_wo<WDT, G>), dim3((s.d + rows_per_block - 1) / rows_per_block, n_items),
                               dim3(kBlock), s.H * s.D * sizeof(float), st, s, w);
            break;
        case 2:
            hipLaunchKernelGGL((k_w13<WDT, G>), dim3((s.F + rows_per_block - 1) / rows_per_block, n_items),
                               dim3(kBlock), s.d * sizeof(float), st, s, w);
            break;
        case 3:
            hipLaunchKernelGGL((k_w2<WDT, G>), dim3((s.d + rows_per_block - 1) / rows_per_block, n_items),
                               dim3(kBlock), s.F * sizeof(float), st, s, w);
            break;
        case 4:
            hipLaunchKernelGGL((k_logits<WDT, G>), dim3((s.V + rows_per_block - 1) / rows_per_block, n_items),
                               dim3(kBlock), s.d * sizeof(float), st, s, out_norm, wcls);
            break;
    }
    return hipGetLastError();
}

template <int WDT>
static hipError_t launch_gemv(int which, int K, const StepArgs& s, const LayerW& w, int layer,
                              int n_items, hipStream_t st, const float* out_norm, const void* wcls) {
    switch (pick_g(K, WDT)) {
        case 8: return launch_gemv_set<WDT, 8>(which, s, w, layer, n_items, st, out_norm, wcls);
        case 16: return launch_gemv_set<WDT, 16>(which, s, w, layer, n_items, st, out_norm, wcls);
        default: return launch_gemv_set<WDT, 32>(which, s, w, layer, n_items, st, out_norm, wcls);
    }
}

static hipError_t gemv(int which, int K, const StepArgs& s, const LayerW& w, int layer, int n_items,
                       hipStream_t st, const float* out_norm = nullptr, const void* wcls = nullptr) {
    if (s.wdt == kBF16) return launch_gemv<kBF16>(which, K, s, w, layer, n_items, st, out_norm, wcls);
    return launch_gemv<kF32>(which, K, s, w, layer, n_items, st, out_norm, wcls);
}

size_t attn_lds_bytes() {
    return sizeof(float) * (kMaxRep * kMaxD + kMaxRep * kChunk + kBlock * kMaxRep * 4 + kMaxRep * 2);
}

hipError_t set_kernel_attributes(int max_lds_bytes) {
    hipError_t e = hipSuccess;
#define DS_ATTR(fn)                                                                                  \
    if (e == hipSuccess)                                                                             \
        e = hipFuncSetAttribute(reinterpret_cast<const void*>(fn),                                   \
                                hipFuncAttributeMaxDynamicSharedMemorySize, max_lds_bytes);
#define DS_ATTR_SET(WDT, G)                                                                          \
    DS_ATTR((k_qkv<WDT, G>)) DS_ATTR((k_wo<WDT, G>)) DS_ATTR((k_w13<WDT, G>))                        \
    DS_ATTR((k_w2<WDT, G>)) DS_ATTR((k_logits<WDT, G>))
    DS_ATTR_SET(kBF16, 8) DS_ATTR_SET(kBF16, 16) DS_ATTR_SET(kBF16, 32)
    DS_ATTR_SET(kF32, 8) DS_ATTR_SET(kF32, 16) DS_ATTR_SET(kF32, 32)
    DS_ATTR(k_attn)
#undef DS_ATTR_SET
#undef DS_ATTR
    return e;
}

hipError_t enqueue_step(const StepArgs& s, const ModelPtrs& m, const BeginList* lists, int n_lists,
                        const int32_t* d_tok_in, int n_items, bool need_logits,
                        int32_t* d_tok_out, hipStream_t st) {
    hipError_t e = hipSuccess;
    for (int i = 0; i < n_lists && e == hipSuccess; i++) {
        hipLaunchKernelGGL(k_begin, dim3(lists[i].n), dim3(kBlock), 0, st, s, lists[i], d_tok_in);
        e = hipGetLastError();
    }
    for (int l = 0; l < s.L && e == hipSuccess; l++) {
        const LayerW& w = m.layers[l];
        e = gemv(0, s.d, s, w, l, n_items, st);
        if (e != hipSuccess) break;
        hipLaunchKernelGGL(k_attn, dim3(s.n_chunks, s.Hkv, n_items), dim3(kBlock), attn_lds_bytes(),
                           st, s, l);
        hipLaunchKernelGGL(k_attn_combine, dim3(s.H, n_items), dim3(64), 0, st, s);
        e = hipGetLastError();
        if (e == hipSuccess) e = gemv(1, s.H * s.D, s, w, l, n_items, st);
        if (e == hipSuccess) e = gemv(2, s.d, s, w, l, n_items, st);
        if (e == hipSuccess) e = gemv(3, s.F, s, w, l, n_items, st);
    }
    if (e == hipSuccess && need_logits) e = gemv(4, s.d, s, LayerW{}, 0, n_items, st, m.out_norm, m.wcls);
    if (e == hipSuccess) {
        hipLaunchKernelGGL(k_finalize, dim3(1), dim3(64), 0, st, s, n_items, d_tok_out,
                           need_logits ? 1 : 0);
        e = hipGetLastError();
    }
    return e;
}

hipError_t enqueue_kernel(int which, int layer, const StepArgs& s, const ModelPtrs& m, int n_items,
                          hipStream_t st) {
    if (which == 0) return gemv(0, s.d, s, m.layers[layer], layer, n_items, st);
    if (which == 1) {
        hipLaunchKernelGGL(k_attn, dim3(s.n_chunks, s.Hkv, n_items), dim3(kBlock), attn_lds_bytes(), st, s,
                           layer);
        return hipGetLastError();
    }
    if (which == 2) {
        hipLaunchKernelGGL(k_attn_combine, dim3(s.H, n_items), dim3(64), 0, st, s);
        return hipGetLastError();
    }
    if (which == 3) return gemv(1, s.H * s.D, s, m.layers[layer], layer, n_items, st);
    if (which == 4) return gemv(2, s.d, s, m.layers[layer], layer, n_items, st);
    if (which == 5) return gemv(3, s.F, s, m.layers[layer], layer, n_items, st);
    return gemv(4, s.d, s, LayerW{}, 0, n_items, st, m.out_norm, m.wcls);
}

hipError_t enqueue_set_lengths(int32_t* d_lengths, const int32_t* h_vals, int first, int n,
                               hipStream_t st) {
    hipError_t e = hipSuccess;
    for (int o = 0; o < n && e == hipSuccess; o += kSetChunk) {
        SetList l;
        l.first = first + o;
        l.n = n - o < kSetChunk ? n - o : kSetChunk;
        for (int i = 0; i < l.n; i++) l.val[i] = h_vals[o + i];
        hipLaunchKernelGGL(k_set_lengths, dim3(1), dim3(256), 0, st, d_lengths, l);
        e = hipGetLastError();
    }
    return e;
}

hipError_t enqueue_fill(int32_t* p, int n, int32_t v, hipStream_t st) {
    if (n <= 0) return hipSuccess;
    hipLaunchKernelGGL(k_fill_i32, dim3((n + 255) / 256 < 1024 ? (n + 255) / 256 : 1024), dim3(256), 0,
                       st, p, n, v);
    return hipGetLastError();
}

}  // namespace ds
