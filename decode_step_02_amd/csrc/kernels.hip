// kernels.hip -- gfx950 kernels of the single-token Llama decode step.
//
// One decode position for n_items sequences (work items) is:
//   k_begin                      embedding gather + widen, step bookkeeping
//   per layer: k_qkv             RMSNorm -> Q/K/V GEMV -> RoPE -> K/V append
//              [long contexts]   k_attn_g / k_attn_d (split-K partials) + k_attn_combine
//              k_wo              [short contexts: attention itself] Wo GEMV + residual
//              k_w13             RMSNorm -> W1/W3 GEMV -> silu(a)*u
//              k_w2              W2 GEMV + residual
//   k_logits                     RMSNorm -> vocabulary GEMV -> per-block argmax
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
// loads per instruction.  The first 12 or 16 chunks of every lane are in
// flight while the block stages its activation vector, so the weight stream
// overlaps the RMSNorm prologue.  bf16 chunks
// are widened in registers by a 16-bit shift ("GOTOken: An Inference Engine
// in QBasic", section "Loading the model and tokenizer") and accumulated in
// fp32 against the LDS copy of the activation vector; the G partial sums of
// a row are combined with xor shuffles inside the wave.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <algorithm>

#include "kernels.h"
#include "device.h"

namespace ds {

constexpr int kPrefetch = 12;  // 16-byte chunks per lane loaded before the prologue (16 for 32-lane rows)

// ---- weight chunks ---------------------------------------------------------------

template <int WDT> struct Wt;

template <> struct Wt<kBF16> {
    static constexpr int EPC = 8;  // elements per 16-byte chunk
    __device__ static __forceinline__ uint4 load(const void* base, size_t elem) {
        return *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(base) + elem);
    }
    __device__ static __forceinline__ float dot(const uint4 u, const float* xs, float acc) {
        const float4 a = *reinterpret_cast<const float4*>(xs);
        const float4 b = *reinterpret_cast<const float4*>(xs + 4);
        acc = fmaf(__uint_as_float(u.x << 16), a.x, acc);
        acc = fmaf(__uint_as_float(u.x & 0xFFFF0000u), a.y, acc);
        acc = fmaf(__uint_as_float(u.y << 16), a.z, acc);
        acc = fmaf(__uint_as_float(u.y & 0xFFFF0000u), a.w, acc);
        acc = fmaf(__uint_as_float(u.z << 16), b.x, acc);
        acc = fmaf(__uint_as_float(u.z & 0xFFFF0000u), b.y, acc);
        acc = fmaf(__uint_as_float(u.w << 16), b.z, acc);
        acc = fmaf(__uint_as_float(u.w & 0xFFFF0000u), b.w, acc);
        return acc;
    }
};

// Block-quantised int8: 16 values per chunk (half a 32-value block); the
// dot product of one chunk, before its block's scale.
template <> struct Wt<kQ8> {
    static constexpr int EPC = 16;
    __device__ static __forceinline__ uint4 load(const void* base, size_t elem) {
        return *reinterpret_cast<const uint4*>(static_cast<const int8_t*>(base) + elem);
    }
    __device__ static __forceinline__ float dot(const uint4 u, const float* xs, float acc) {
        const uint32_t wv[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
        for (int k = 0; k < 4; k++) {
            const float4 a = *reinterpret_cast<const float4*>(xs + 4 * k);
            const int32_t v = static_cast<int32_t>(wv[k]);
            acc = fmaf(static_cast<float>((v << 24) >> 24), a.x, acc);
            acc = fmaf(static_cast<float>((v << 16) >> 24), a.y, acc);
            acc = fmaf(static_cast<float>((v << 8) >> 24), a.z, acc);
            acc = fmaf(static_cast<float>(v >> 24), a.w, acc);
        }
        return acc;
    }
};

// Block-quantised 4-bit: 32 values per chunk (one 32-value block), two per
// byte with the even index in the low nibble, so value i of a dword is its
// nibble i; two's complement.  The dot product before the block's scale.
template <> struct Wt<kQ4> {
    static constexpr int EPC = 32;
    __device__ static __forceinline__ uint4 load(const void* base, size_t elem) {
        return *reinterpret_cast<const uint4*>(static_cast<const uint8_t*>(base) + elem / 2);
    }
    __device__ static __forceinline__ float dot(const uint4 u, const float* xs, float acc) {
        const uint32_t wv[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
        for (int k = 0; k < 4; k++) {
            const float4 a = *reinterpret_cast<const float4*>(xs + 8 * k);
            const float4 b = *reinterpret_cast<const float4*>(xs + 8 * k + 4);
            const int32_t v = static_cast<int32_t>(wv[k]);
            acc = fmaf(static_cast<float>((v << 28) >> 28), a.x, acc);
            acc = fmaf(static_cast<float>((v << 24) >> 28), a.y, acc);
            acc = fmaf(static_cast<float>((v << 20) >> 28), a.z, acc);
            acc = fmaf(static_cast<float>((v << 16) >> 28), a.w, acc);
            acc = fmaf(static_cast<float>((v << 12) >> 28), b.x, acc);
            acc = fmaf(static_cast<float>((v << 8) >> 28), b.y, acc);
            acc = fmaf(static_cast<float>((v << 4) >> 28), b.z, acc);
            acc = fmaf(static_cast<float>(v >> 28), b.w, acc);
        }
        return acc;
    }
};

// Scales of a Q8 / Q4 matrix [rows][K]: they start at the first 256-byte
// boundary after its values (rows * K bytes, or half that for Q4).
template <int WDT>
__device__ __forceinline__ const float* q_scales(const void* W, size_t rows, int K) {
    const size_t vb = WDT == kQ4 ? rows * static_cast<size_t>(K) / 2 : rows * static_cast<size_t>(K);
    const size_t nb = (vb + 255) / 256 * 256;
    return reinterpret_cast<const float*>(static_cast<const uint8_t*>(W) + nb);
}

template <> struct Wt<kF32> {
    static constexpr int EPC = 4;
    __device__ static __forceinline__ uint4 load(const void* base, size_t elem) {
        return *reinterpret_cast<const uint4*>(static_cast<const float*>(base) + elem);
    }
    __device__ static __forceinline__ float dot(const uint4 u, const float* xs, float acc) {
        const float4 a = *reinterpret_cast<const float4*>(xs);
        acc = fmaf(__uint_as_float(u.x), a.x, acc);
        acc = fmaf(__uint_as_float(u.y), a.y, acc);
        acc = fmaf(__uint_as_float(u.z), a.z, acc);
        acc = fmaf(__uint_as_float(u.w), a.w, acc);
        return acc;
    }
};

// One lane's share of one row: the first PF chunks are loaded by
// start(), the rest while finish() accumulates.  finish() returns the full
// row dot product in every lane of the row's G-lane group.
// Staged activation vectors of the block-scaled types leave 4 floats of
// padding after every chunk's EPC values (a stride of 20 or 36 floats): the
// lanes of a row read chunks sub, sub + G, ... at once, and with the plain
// stride of 16 or 32 floats the 8 lanes of one LDS read cycle would all hit
// the same four banks.
template <int WDT>
constexpr int lds_pad_q() { return (WDT == kQ8 || WDT == kQ4) ? Wt<WDT>::EPC / 4 : 0; }  // float4s per padded chunk

// Floats of LDS that a staged vector of n values takes (n a multiple of the chunk).
__host__ __device__ inline int staged_floats(int wdt, int n) {
    return wdt == kQ8 ? n + n / 16 * 4 : wdt == kQ4 ? n + n / 32 * 4 : n;
}

template <int WDT, int G, int PFO = 0, bool XP = false>
struct RowStream {
    static constexpr int EPC = Wt<WDT>::EPC;
    static constexpr bool Q8 = WDT == kQ8 || WDT == kQ4;  // block scales (Q8 or Q4)
    static constexpr int XS = XP ? EPC + 4 : EPC;  // LDS floats from one chunk's values to the next's
    // chunks in flight per lane: PFO where the caller sets it; else 8 (int8)
    // or 4 (int4) for the block-scaled types, whose lanes get as many
    // weights as bf16 lanes do (pick_g) and so 2 or 4 times fewer chunks;
    // else 16 where 32 lanes share a row of bf16 or fp32 weights (rows of
    // 512 and more chunks), which is a whole 4096-long bf16 row -- one
    // memory round trip -- and those launches have few waves per SIMD to
    // hide it
    static constexpr int PF = PFO ? PFO : WDT == kQ8 ? 8 : WDT == kQ4 ? 4 : G >= 32 ? 16 : kPrefetch;
    uint4 w[PF];
    float sc[Q8 ? PF : 1];  // Q8: the block scale of each prefetched chunk
    const void* W;
    const float* S;  // Q8: the row's block scales
    size_t base;
    int nch, nall, sub;

    // Loads are unconditional (the chunk index is clamped into the row, the
    // value masked afterwards): a guarded load becomes a branch, and the
    // compiler then waits for every load before the next one.  `rows` (the
    // matrix's row count) locates the scales of a Q8 matrix.
    __device__ __forceinline__ void start(const void* W_, size_t row, int K, int sub_, bool valid, size_t rows = 0) {
        W = W_;
        base = row * static_cast<size_t>(K);
        sub = sub_;
        nch = valid ? K / EPC : 0;
        nall = K / EPC;
        const int last = K / EPC - 1;
        if constexpr (Q8) S = q_scales<WDT>(W_, rows, K) + row * static_cast<size_t>(K / 32);
#pragma unroll
        for (int p = 0; p < PF; p++) {
            const int c = sub + p * G;
            w[p] = Wt<WDT>::load(W, base + static_cast<size_t>(min(c, last)) * EPC);
            if constexpr (Q8) sc[p] = S[(min(c, last) * EPC) >> 5];
        }
#pragma unroll
        for (int p = 0; p < PF; p++) {
            const bool keep = sub + p * G < nch;
            w[p].x = keep ? w[p].x : 0u;
            w[p].y = keep ? w[p].y : 0u;
            w[p].z = keep ? w[p].z : 0u;
            w[p].w = keep ? w[p].w : 0u;
        }
    }

    // acc + the chunk's products (times its block scale for Q8)
    __device__ __forceinline__ static float chunk(uint4 u, float scale, const float* xs, float acc) {
        if constexpr (Q8) return fmaf(scale, Wt<WDT>::dot(u, xs, 0.f), acc);
        return Wt<WDT>::dot(u, xs, acc);
    }
    __device__ __forceinline__ float scale_of(int c) const {
        if constexpr (Q8) return S[(c * EPC) >> 5];
        return 1.f;
    }

    __device__ __forceinline__ float finish(const float* xs) const {
        float a0 = 0.f, a1 = 0.f;
        const int last = nch > 0 ? nch - 1 : 0;
#pragma unroll
        for (int p = 0; p < PF; p += 2) {
            // masked chunks are zero; the LDS index is clamped so it stays in range
            a0 = chunk(w[p], sc[Q8 ? p : 0], xs + min(sub + p * G, last) * XS, a0);
            if (p + 1 < PF) a1 = chunk(w[p + 1], sc[Q8 ? p + 1 : 0], xs + min(sub + (p + 1) * G, last) * XS, a1);
        }
        int c = sub + PF * G;
        for (; c + 3 * G < nch; c += 4 * G) {
            const uint4 u0 = Wt<WDT>::load(W, base + static_cast<size_t>(c) * EPC);
            const uint4 u1 = Wt<WDT>::load(W, base + static_cast<size_t>(c + G) * EPC);
            const uint4 u2 = Wt<WDT>::load(W, base + static_cast<size_t>(c + 2 * G) * EPC);
            const uint4 u3 = Wt<WDT>::load(W, base + static_cast<size_t>(c + 3 * G) * EPC);
            const float s0 = scale_of(c), s1 = scale_of(c + G), s2 = scale_of(c + 2 * G), s3 = scale_of(c + 3 * G);
            a0 = chunk(u0, s0, xs + c * XS, a0);
            a1 = chunk(u1, s1, xs + (c + G) * XS, a1);
            a0 = chunk(u2, s2, xs + (c + 2 * G) * XS, a0);
            a1 = chunk(u3, s3, xs + (c + 3 * G) * XS, a1);
        }
        for (; c < nch; c += G) a0 = chunk(Wt<WDT>::load(W, base + static_cast<size_t>(c) * EPC), scale_of(c), xs + c * XS, a0);
        return group_sum<G>(a0 + a1);
    }

    // finish() with a rolling pipeline: slot p holds chunk j0 + p of this
    // lane; once used it is refilled with chunk j0 + p + PF, so
    // PF loads stay in flight down the whole row (finish() waits for
    // each batch of four before issuing the next).  Chunks past the lane's
    // own are loaded clamped and left out of the sum; the loop count is the
    // same for every lane.  Taken by W2, the longest rows (the 8B shape's
    // 14336: 24.5 against 25.7 us per launch); the two-stream W1/W3 would
    // hold too many registers, and Wo's 4096-long rows gained nothing.
    __device__ __forceinline__ float finish_roll(const float* xs) {
        float a0 = 0.f, a1 = 0.f;
        const int ntot = nch > 0 ? nch : 1;  // masked lanes still walk (clamped, discarded)
        const int last = ntot - 1;
        const int nj = (nall + G - 1) / G;    // chunks of the group's lane 0, the most of any lane
        int j0 = 0;
        for (; j0 + PF < nj; j0 += PF) {
#pragma unroll
            for (int p = 0; p < PF; p++) {
                const int c = sub + (j0 + p) * G;
                const float* xc = xs + min(c, last) * XS;
                float& a = (p & 1) ? a1 : a0;
                const float v = chunk(w[p], sc[Q8 ? p : 0], xc, a);
                a = c < nch ? v : a;
                const int cn = min(c + PF * G, last);
                w[p] = Wt<WDT>::load(W, base + static_cast<size_t>(cn) * EPC);
                if constexpr (Q8) sc[p] = S[(cn * EPC) >> 5];
            }
        }
#pragma unroll
        for (int p = 0; p < PF; p++) {
            const int c = sub + (j0 + p) * G;
            float& a = (p & 1) ? a1 : a0;
            const float v = chunk(w[p], sc[Q8 ? p : 0], xs + min(c, last) * XS, a);
            a = c < nch ? v : a;
        }
        return group_sum<G>(a0 + a1);
    }
};

// ---- block helpers -------------------------------------------------------------------

template <int WAVES>
__device__ __forceinline__ float block_sum(float v, float* red) {
    v = wave_sum(v);
    if (WAVES == 1) return v;
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    if (lane == 0) red[wave] = v;
    __syncthreads();
    float t = 0.f;
#pragma unroll
    for (int w = 0; w < WAVES; w++) t += red[w];
    return t;
}

// Two-phase staging of an n-float activation vector (n % 4 == 0) into LDS.
// issue() starts the first round of independent 16-byte loads (and of the
// matching gains when GAIN); the caller then puts its weight loads in flight
// before complete_*() waits.  The callers issue the vector first, so that
// (loads completing in issue order) the staging need not wait for the
// weights; the compiler may still schedule some weight loads ahead of it.
// Vectors longer than U*NT float4 take further rounds inside complete_*().
// Q > 0: float4 j of the vector goes to LDS float4 j + j / Q (the padded
// layout of RowStream's XP).
template <int NT, int U, bool GAIN, int Q = 0>
struct VecStage {
    __device__ static __forceinline__ int at(int j) { return Q ? j + j / Q : j; }
    float4 xv[U];
    float4 gv[GAIN ? U : 1];
    const float4* x4;
    const float4* g4;
    int n4;

    __device__ __forceinline__ void issue(const float* x, const float* g, int n) {
        x4 = reinterpret_cast<const float4*>(x);
        g4 = reinterpret_cast<const float4*>(g);
        n4 = n >> 2;
#pragma unroll
        for (int u = 0; u < U; u++) {  // unconditional loads of a clamped index
            const int j = min(static_cast<int>(threadIdx.x) + u * NT, n4 - 1);
            xv[u] = x4[j];
            if (GAIN) gv[u] = g4[j];
        }
    }

    // xs = g * (x * r), r = 1 / sqrt(mean(x^2) + eps): the RMSNorm of
    // "simple-llm / kasahare", section "Architecture" (attn_norm / ffn_norm).
    template <int WAVES>
    __device__ __forceinline__ void complete_rms(float* xs, float* red, int n, float eps) {
        float4* s4 = reinterpret_cast<float4*>(xs);
        float ss = 0.f;
        auto put = [&](const float4 v, const float4 gg, int j, bool in) {
            float t = 0.f;
            t = fmaf(v.x, v.x, t);
            t = fmaf(v.y, v.y, t);
            t = fmaf(v.z, v.z, t);
            t = fmaf(v.w, v.w, t);
            ss += in ? t : 0.f;
            s4[at(j)] = make_float4(gg.x * v.x, gg.y * v.y, gg.z * v.z, gg.w * v.w);
        };
        // Stores past n4 go to the last element with its own value (the loads
        // were clamped the same way), so no branch: a guarded store lets the
        // compiler sink its load into the branch and wait for it there.
#pragma unroll
        for (int u = 0; u < U; u++) {
            const int j = threadIdx.x + u * NT;
            put(xv[u], gv[GAIN ? u : 0], min(j, n4 - 1), j < n4);
        }
        for (int base = threadIdx.x + U * NT; base < n4; base += U * NT) {  // as in complete_copy
            float4 t[U], tg[U];
#pragma unroll
            for (int u = 0; u < U; u++) {
                const int j = min(base + u * NT, n4 - 1);
                t[u] = x4[j];
                tg[u] = GAIN ? g4[j] : make_float4(1.f, 1.f, 1.f, 1.f);
            }
#pragma unroll
            for (int u = 0; u < U; u++) {
                const int j = base + u * NT;
                put(t[u], tg[u], min(j, n4 - 1), j < n4);
            }
        }
        ss = block_sum<WAVES>(ss, red);
        const float r = 1.0f / sqrtf(ss / static_cast<float>(n) + eps);
        for (int j = threadIdx.x; j < n4; j += NT) {
            const float4 v = s4[at(j)];
            s4[at(j)] = make_float4(v.x * r, v.y * r, v.z * r, v.w * r);
        }
        __syncthreads();
    }

    __device__ __forceinline__ void complete_copy(float* xs) {
        float4* s4 = reinterpret_cast<float4*>(xs);
#pragma unroll
        for (int u = 0; u < U; u++) s4[at(min(static_cast<int>(threadIdx.x) + u * NT, n4 - 1))] = xv[u];  // as in complete_rms
        // later rounds load into a local array, unconditionally (clamped):
        // guarded writes into xv keep it out of registers, in scratch memory,
        // with every load waited for before the next is issued
        for (int base = threadIdx.x + U * NT; base < n4; base += U * NT) {
            float4 t[U];
#pragma unroll
            for (int u = 0; u < U; u++) t[u] = x4[min(base + u * NT, n4 - 1)];
#pragma unroll
            for (int u = 0; u < U; u++) s4[at(min(base + u * NT, n4 - 1))] = t[u];
        }
        __syncthreads();
    }
};

// ---- k_begin: embedding gather -------------------------------------------------------
// x[item] = widen(token_emb[tok]); records the slot, position and flag of the
// item.  Token ids outside [0, V) raise the error word and read row 0 instead.
__global__ __launch_bounds__(256) void k_begin(StepArgs s, BeginList list, const int32_t* __restrict__ d_tok_in) {
    const int li = blockIdx.x;
    if (li >= list.n) return;
    const int item = list.item0 + li;
    const int slot = list.by_value ? list.slot[li] : item;
    int tok = list.by_value == 1 ? list.tok[li] : d_tok_in[slot];
    if (tok < 0 || tok >= s.V) {
        if (threadIdx.x == 0) atomicOr(s.err, 1);
        tok = 0;
    }
    const int pos = s.lengths[slot] + (list.by_value ? list.off[li] : 0);
    if (threadIdx.x == 0) {
        s.slot[item] = slot;
        s.pos[item] = pos;
        s.flag[item] = list.by_value == 1 ? list.last[li] : 1;
    }
    float* x = s.x + static_cast<size_t>(item) * s.d;
    const size_t row = static_cast<size_t>(tok) * s.d;
    if (s.wdt == kBF16) {
        const uint16_t* e = static_cast<const uint16_t*>(s.emb) + row;
        for (int j = threadIdx.x; j < s.d; j += 256) x[j] = __uint_as_float(static_cast<uint32_t>(e[j]) << 16);
    } else if (s.wdt == kQ8) {
        const int8_t* e = static_cast<const int8_t*>(s.emb) + row;
        const float* sc = q_scales<kQ8>(s.emb, s.V, s.d) + static_cast<size_t>(tok) * (s.d / 32);
        for (int j = threadIdx.x; j < s.d; j += 256) x[j] = sc[j >> 5] * static_cast<float>(e[j]);
    } else if (s.wdt == kQ4) {
        const uint8_t* e = static_cast<const uint8_t*>(s.emb) + row / 2;
        const float* sc = q_scales<kQ4>(s.emb, s.V, s.d) + static_cast<size_t>(tok) * (s.d / 32);
        for (int j = threadIdx.x; j < s.d; j += 256) {
            const int nib = (j & 1) ? (e[j >> 1] >> 4) : (e[j >> 1] & 15);
            x[j] = sc[j >> 5] * static_cast<float>(nib >= 8 ? nib - 16 : nib);
        }
    } else {
        const float* e = static_cast<const float*>(s.emb) + row;
        for (int j = threadIdx.x; j < s.d; j += 256) x[j] = e[j];
    }
}

// ---- k_qkv -----------------------------------------------------------------------------
// Wave tasks: q rows, then k rows, then v rows, R rows per task.  In the q
// and k sections a task holds R/2 RoPE pairs (i, i + D/2) of a head
// ("GOTOken", section "Loading the model and tokenizer": pairs j and
// j + head_dim/2): first halves in row slots 0..R/2-1, their partners R/2
// rows later, i.e. exactly 32 lanes away, so the rotation is one xor-32
// shuffle.  Rotated q goes to the workspace, rotated k and v to the cache at
// the item's position.
template <int WDT, int G, int WAVES>
__global__ __launch_bounds__(64 * WAVES) void k_qkv(StepArgs s, LayerW w, int layer, int ident) {
    extern __shared__ float xs[];
    __shared__ float red[WAVES];
    constexpr int R = 64 / G;
    const int item = blockIdx.y;
    const int pos = s.pos[item];
    const int slot = ident ? item : s.slot[item];
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int task = blockIdx.x * WAVES + wave;
    const int D = s.D, half_d = s.D / 2;
    const int nq = s.H * D / R, nk = s.Hkv * D / R, nv = nk;
    const bool valid = task < nq + nk + nv;
    const int rs = lane / G, sub = lane % G;
    const bool roped = task < nq + nk;
    const bool is_q = task < nq;
    int row, i = 0, second = 0;
    const void* W;
    if (roped) {
        const int t = is_q ? task : task - nq;
        const int p = t * (R / 2) + (rs % (R / 2));
        second = rs / (R / 2);
        i = p % half_d;
        row = (p / half_d) * D + i + second * half_d;
        W = is_q ? w.wq : w.wk;
    } else {
        row = valid ? (task - nq - nk) * R + rs : 0;
        W = w.wv;
    }
    // the vector's loads go first (see VecStage), then the weight chunks
    VecStage<64 * WAVES, 4, true, lds_pad_q<WDT>()> vs;
    vs.issue(s.x + static_cast<size_t>(item) * s.d, w.attn_norm, s.d);
    RowStream<WDT, G, 0, (lds_pad_q<WDT>() > 0)> st;
    st.start(W, row, s.d, sub, valid, static_cast<size_t>(is_q ? s.H : s.Hkv) * D);
    float c = 1.f, sn = 0.f;
    if (roped && valid) {
        c = s.rope_cos[static_cast<size_t>(pos) * half_d + i];
        sn = s.rope_sin[static_cast<size_t>(pos) * half_d + i];
    }
    vs.template complete_rms<WAVES>(xs, red, s.d, s.eps);
    if (!valid) return;
    const float y = st.finish(xs);
    if (roped) {
        const float partner = __shfl_xor(y, 32);
        // pair (a, b) -> (a c - b s, a s + b c)
        const float out = second ? fmaf(partner, sn, y * c) : fmaf(-partner, sn, y * c);
        if (sub == 0) {
            if (is_q) {
                s.q[static_cast<size_t>(item) * s.H * D + row] = out;
            } else {
                cache_put(s, cache_row(s, layer, 0, slot, row / D, pos) + row % D, out);
            }
        }
    } else if (sub == 0) {
        cache_put(s, cache_row(s, layer, 1, slot, row / D, pos) + row % D, y);
    }
}

// ---- short-context attention (inside the Wo kernel) ----------------------------------------
// For every query head h (key/value head g = h / (H/Hkv), "simple-llm /
// kasahare", section "Architecture", GQA): softmax(q_h . K_g[0..n) / sqrt(D))
// weighted sum of V_g[0..n), for n = pos + 1 <= s.short_n.  q and the n
// cached K/V rows of every group are staged into LDS with independent 16-byte
// loads (rows padded to D + 4 floats against bank conflicts); the result
// o [H*D] is left in LDS for the Wo GEMV.
template <int WAVES>
__device__ void attention_short(const StepArgs& s, int layer, int item, int slot, int n, int nload, float* o,
                                float* lds) {
    constexpr int NT = 64 * WAVES;
    const int D = s.D, H = s.H, HD = s.H * s.D, rep = s.H / s.Hkv, Hkv = s.Hkv;
    const int DP = D + 4, NS = s.short_n;
    float* qs = lds;                          // [H*D]
    float* ks = qs + HD;                      // [Hkv][NS][DP]
    float* vs = ks + Hkv * NS * DP;           // [Hkv][NS][DP]
    // staging: float4 units -- q, then per group nload rows of K, then of V
    // (nload >= n is a host-chosen bound, so the loads need not wait for pos)
    const int D4 = D >> 2, q4 = HD >> 2, rows = Hkv * nload, total = q4 + 2 * rows * D4;
    const float4* qg = reinterpret_cast<const float4*>(s.q + static_cast<size_t>(item) * HD);
    constexpr int U = 8;
    const int lg_d4 = __ffs(D4) - 1, lg_nl = __ffs(nload) - 1;  // D4 and nload are powers of two
    for (int base = threadIdx.x; base < total; base += U * NT) {
        float4 v[U];
#pragma unroll
        for (int u = 0; u < U; u++) {  // unconditional loads from clamped indices
            const int f = min(base + u * NT, total - 1);
            const int r = max(f - q4, 0) >> lg_d4, c = max(f - q4, 0) & (D4 - 1);
            const int kv = r >= rows, rr = r - kv * rows, g = rr >> lg_nl, t = rr & (nload - 1);
            const float4* src = f < q4 ? qg + f
                                       : reinterpret_cast<const float4*>(s.cache + cache_row(s, layer, kv, slot, g, t)) + c;
            v[u] = *src;
        }
#pragma unroll
        for (int u = 0; u < U; u++) {
            const int f = base + u * NT;
            if (f < q4) {
                reinterpret_cast<float4*>(qs)[f] = v[u];
            } else if (f < total) {
                const int r = (f - q4) >> lg_d4, c = (f - q4) & (D4 - 1);
                const int kv = r >= rows, rr = r - kv * rows, g = rr >> lg_nl, t = rr & (nload - 1);
                *reinterpret_cast<float4*>((kv ? vs : ks) + (g * NS + t) * DP + 4 * c) = v[u];
            }
        }
    }
    __syncthreads();
    // one wave per query head: lane t scores position t (n <= 64), the
    // softmax is a pair of wave reductions, and lane e accumulates output
    // element e with p_t broadcast from lane t
    const float scale = 1.0f / sqrtf(static_cast<float>(D));
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    for (int h = wave; h < H; h += WAVES) {
        const int g = h / rep;
        const float4* q4p = reinterpret_cast<const float4*>(qs + h * D);
        float sc_t = -INFINITY;
        if (lane < n) {
            const float4* k4 = reinterpret_cast<const float4*>(ks + (g * NS + lane) * DP);
            float a0 = 0.f, a1 = 0.f;
            for (int c = 0; c < D4; c += 2) {
                const float4 k0 = k4[c], qv0 = q4p[c];
                a0 = fmaf(k0.x, qv0.x, a0); a0 = fmaf(k0.y, qv0.y, a0);
                a0 = fmaf(k0.z, qv0.z, a0); a0 = fmaf(k0.w, qv0.w, a0);
                const float4 k1 = k4[c + 1], qv1 = q4p[c + 1];
                a1 = fmaf(k1.x, qv1.x, a1); a1 = fmaf(k1.y, qv1.y, a1);
                a1 = fmaf(k1.z, qv1.z, a1); a1 = fmaf(k1.w, qv1.w, a1);
            }
            sc_t = (a0 + a1) * scale;
        }
        const float m = wave_max(sc_t);
        const float e_t = lane < n ? __expf(sc_t - m) : 0.f;
        const float p_t = e_t / wave_sum(e_t);
        const float* vg = vs + g * NS * DP;
        const int pbits = __float_as_int(p_t);
        for (int e0 = 0; e0 < D; e0 += 64) {  // uniform loop; readlane needs every lane's p_t in place
            const int e = e0 + lane;
            const bool ok = e < D;
            float a0 = 0.f, a1 = 0.f;
            int t = 0;
            for (; t + 1 < n; t += 2) {
                const float p0 = __int_as_float(__builtin_amdgcn_readlane(pbits, t));
                const float p1 = __int_as_float(__builtin_amdgcn_readlane(pbits, t + 1));
                if (ok) {
                    a0 = fmaf(p0, vg[t * DP + e], a0);
                    a1 = fmaf(p1, vg[(t + 1) * DP + e], a1);
                }
            }
            if (t < n) {
                const float p0 = __int_as_float(__builtin_amdgcn_readlane(pbits, t));
                if (ok) a0 = fmaf(p0, vg[t * DP + e], a0);
            }
            if (ok) o[h * D + e] = a0 + a1;
        }
    }
    __syncthreads();
}

// ---- long-context attention: split-K partials + combine ------------------------------------
// Register-resident variant for head_dim D (a power of two, 16..256): every
// K and V load of the block's chunk is issued up front (one memory round
// trip), scores and the softmax stay in registers, and the row groups are
// combined with xor shuffles inside a wave and one LDS exchange across the
// four waves.  Thread (row group rg, slice e4) holds rows rg + NRG*i of the
// chunk, columns 4*e4 .. 4*e4+3.
template <int D>
__global__ __launch_bounds__(256) void k_attn_d(StepArgs s, int layer) {
    constexpr int LPR = D / 4;             // lanes per row
    constexpr int NRG = 256 / LPR;         // row groups in the block
    constexpr int RPT = (kChunk + NRG - 1) / NRG;  // rows per thread
    constexpr int GPW = 64 / LPR;          // row groups per wave
    __shared__ float wred[4][kMaxRep][2];
    __shared__ float ored[4][kMaxRep][D];
    const int chunk = blockIdx.x, g = blockIdx.y, item = blockIdx.z;
    const int pos = s.pos[item], slot = s.slot[item];
    const int n = pos + 1;
    const int t0 = chunk * kChunk;
    if (t0 >= n) return;
    const int nt = min(kChunk, n - t0);
    const int rep = s.H / s.Hkv;
    const int e4 = threadIdx.x % LPR, rg = threadIdx.x / LPR;
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const float* K = s.cache + cache_row(s, layer, 0, slot, g, t0) + e4 * 4;
    const float* V = s.cache + cache_row(s, layer, 1, slot, g, t0) + e4 * 4;
    float4 kr[RPT], vr[RPT];
#pragma unroll
    for (int i = 0; i < RPT; i++) {
        const int t = min(rg + i * NRG, nt - 1);
        kr[i] = *reinterpret_cast<const float4*>(K + static_cast<size_t>(t) * D);
        vr[i] = *reinterpret_cast<const float4*>(V + static_cast<size_t>(t) * D);
    }
    const float* q = s.q + static_cast<size_t>(item) * s.H * D + static_cast<size_t>(g) * rep * D + e4 * 4;
    float4 qr[kMaxRep];
#pragma unroll
    for (int j = 0; j < kMaxRep; j++)
        qr[j] = *reinterpret_cast<const float4*>(q + static_cast<size_t>(min(j, rep - 1)) * D);
    const float scale = 1.0f / sqrtf(static_cast<float>(D));
    float sc[kMaxRep][RPT];
#pragma unroll
    for (int j = 0; j < kMaxRep; j++) {
#pragma unroll
        for (int i = 0; i < RPT; i++) {
            float d = kr[i].x * qr[j].x;
            d = fmaf(kr[i].y, qr[j].y, d);
            d = fmaf(kr[i].z, qr[j].z, d);
            d = fmaf(kr[i].w, qr[j].w, d);
#pragma unroll
            for (int o = LPR / 2; o > 0; o >>= 1) d += __shfl_xor(d, o);
            sc[j][i] = rg + i * NRG < nt ? d * scale : -INFINITY;
        }
    }
    // chunk max and exp-sum per head: thread rows -> wave (xor over row groups) -> block
    float m[kMaxRep], l[kMaxRep];
#pragma unroll
    for (int j = 0; j < kMaxRep; j++) {
        float mm = sc[j][0];
#pragma unroll
        for (int i = 1; i < RPT; i++) mm = fmaxf(mm, sc[j][i]);
#pragma unroll
        for (int o = LPR; o < 64; o <<= 1) mm = fmaxf(mm, __shfl_xor(mm, o));
        m[j] = mm;
    }
    if (lane == 0)
        for (int j = 0; j < kMaxRep; j++) wred[wave][j][0] = m[j];
    __syncthreads();
#pragma unroll
    for (int j = 0; j < kMaxRep; j++) m[j] = fmaxf(fmaxf(wred[0][j][0], wred[1][j][0]), fmaxf(wred[2][j][0], wred[3][j][0]));
    float acc[kMaxRep][4];
#pragma unroll
    for (int j = 0; j < kMaxRep; j++) {
        float ll = 0.f;
        acc[j][0] = acc[j][1] = acc[j][2] = acc[j][3] = 0.f;
#pragma unroll
        for (int i = 0; i < RPT; i++) {
            const float p = __expf(sc[j][i] - m[j]);  // exp(-inf) = 0 for masked rows
            ll += p;
            acc[j][0] = fmaf(p, vr[i].x, acc[j][0]);
            acc[j][1] = fmaf(p, vr[i].y, acc[j][1]);
            acc[j][2] = fmaf(p, vr[i].z, acc[j][2]);
            acc[j][3] = fmaf(p, vr[i].w, acc[j][3]);
        }
#pragma unroll
        for (int o = LPR; o < 64; o <<= 1) {
            ll += __shfl_xor(ll, o);
            acc[j][0] += __shfl_xor(acc[j][0], o);
            acc[j][1] += __shfl_xor(acc[j][1], o);
            acc[j][2] += __shfl_xor(acc[j][2], o);
            acc[j][3] += __shfl_xor(acc[j][3], o);
        }
        l[j] = ll;
    }
    __syncthreads();  // wred reads above are done before it is reused
    if (lane < LPR) {
        for (int j = 0; j < rep; j++) {
            *reinterpret_cast<float4*>(&ored[wave][j][e4 * 4]) = make_float4(acc[j][0], acc[j][1], acc[j][2], acc[j][3]);
            if (lane == 0) wred[wave][j][1] = l[j];
        }
    }
    __syncthreads();
    const int S = s.n_chunks;
    for (int idx = threadIdx.x; idx < rep * D; idx += 256) {
        const int j = idx / D, e = idx % D;
        const float v = ored[0][j][e] + ored[1][j][e] + ored[2][j][e] + ored[3][j][e];
        const size_t pidx = (static_cast<size_t>(item) * s.H + g * rep + j) * S + chunk;
        s.part_o[pidx * D + e] = v;
        if (e == 0) {
            s.part_ml[pidx * 2 + 0] = m[j];
            s.part_ml[pidx * 2 + 1] = wred[0][j][1] + wred[1][j][1] + wred[2][j][1] + wred[3][j][1];
        }
    }
    (void)GPW;
}

// Split-K decode attention for head_dim 64 or 128 with REP query heads per
// key/value head: a block of four waves per 64-position chunk of one (item,
// group), wave w taking positions t0 + 16w .. t0 + 16w + 15.
//  - Keys: 8 lanes per row, lane q holding dims 32f + 4q .. 32f + 4q + 3
//    (f < D/32), so each load instruction reads whole 128-byte lines; the
//    wave's 16 rows are two slots of 8 rows, and each dot product is reduced
//    over its 8 lanes with DPP moves.
//  - Values: D/64 dims per lane, so a load instruction reads one row.
//  - The softmax weights of the chunk go through LDS; max and sum are taken
//    over the block, the weighted values summed over the four waves in LDS.
// Partials as k_attn_d: (m, l) and the weighted sum per (item, head, chunk).
// One lane's share of the keys and values of a wave's RPW rows (16 or 8),
// fp32 or bf16.  fp32 keys: lane q holds dims 32f + 4q .. +3 (f < D/32);
// bf16 keys: dims 64f + 8q .. +7 (f < D/64, one 16-byte load each): either
// way D/8 dims, read as whole 128-byte lines per row, and qdim() gives the
// query offsets that match.  The rows come in slots of 8 (one per 8 lanes).
// Values: D/64 dims per lane; bf16 ones stay packed until used.
// Loads of cached key/value rows, which a decode step reads once: with the
// non-temporal hint they pass through the caches without displacing the
// weights and activations (B = 64, 135M: 1.412 -> 1.360 ms per step).  When
// several items of a launch are positions of one sequence (a batched
// prefill pass), they share the rows and take plain loads (s.kv_stream 0).
typedef float stream_f4 __attribute__((ext_vector_type(4)));
typedef float stream_f2 __attribute__((ext_vector_type(2)));
typedef unsigned int stream_u4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ float4 ld_stream(const float4* p) {
    const stream_f4 t = __builtin_nontemporal_load(reinterpret_cast<const stream_f4*>(p));
    return make_float4(t.x, t.y, t.z, t.w);
}
__device__ __forceinline__ float2 ld_stream(const float2* p) {
    const stream_f2 t = __builtin_nontemporal_load(reinterpret_cast<const stream_f2*>(p));
    return make_float2(t.x, t.y);
}
__device__ __forceinline__ uint4 ld_stream(const uint4* p) {
    const stream_u4 t = __builtin_nontemporal_load(reinterpret_cast<const stream_u4*>(p));
    return make_uint4(t.x, t.y, t.z, t.w);
}
template <typename T>
__device__ __forceinline__ T ld_stream(const T* p) {
    return __builtin_nontemporal_load(p);
}
template <bool NT, typename T>
__device__ __forceinline__ T ld_kv(const T* p) {
    if constexpr (NT) return ld_stream(p);
    return *p;
}

template <int D, int CDT, int RPW> struct KVRows;
template <int D, int RPW> struct KVRows<D, kF32, RPW> {
    static constexpr int KF = D / 32, DPL = D / 64, NSL = RPW / 8;
    float4 k[NSL][KF];
    float v[RPW][DPL];
    __device__ static __forceinline__ int qdim(int f, int kq) { return f * 32 + kq * 4; }
    template <bool NT>
    __device__ __forceinline__ void load_t(const float* Kb, const float* Vb, const int (&rows)[NSL], int rv0, int nlast,
                                           int kq, int lane) {
#pragma unroll
        for (int sl = 0; sl < NSL; sl++) {
#pragma unroll
            for (int f = 0; f < KF; f++)
                k[sl][f] = ld_kv<NT>(reinterpret_cast<const float4*>(Kb + rows[sl] * D + f * 32 + kq * 4));
        }
#pragma unroll
        for (int i = 0; i < RPW; i++) {
            const float* vp = Vb + min(rv0 + i, nlast) * D + lane * DPL;
            if constexpr (DPL == 1) {
                v[i][0] = ld_kv<NT>(vp);
            } else {
                const float2 v2 = ld_kv<NT>(reinterpret_cast<const float2*>(vp));
                v[i][0] = v2.x;
                v[i][1] = v2.y;
            }
        }
    }

    __device__ __forceinline__ float4 key(int sl, int f) const { return k[sl][f]; }
    __device__ __forceinline__ float val(int i, int dd) const { return v[i][dd]; }
};
template <int D, int RPW> struct KVRows<D, kBF16, RPW> {
    static constexpr int KF = D / 32, DPL = D / 64, NSL = RPW / 8;
    uint4 k[NSL][D / 64];
    uint32_t v[RPW];  // the row's DPL bf16 values (D = 128: two, the lower dim in the low half)
    __device__ static __forceinline__ int qdim(int f, int kq) { return (f >> 1) * 64 + kq * 8 + (f & 1) * 4; }
    template <bool NT>
    __device__ __forceinline__ void load_t(const float* Kb, const float* Vb, const int (&rows)[NSL], int rv0, int nlast,
                                           int kq, int lane) {
        const uint16_t* K16 = reinterpret_cast<const uint16_t*>(Kb);
        const uint16_t* V16 = reinterpret_cast<const uint16_t*>(Vb);
#pragma unroll
        for (int sl = 0; sl < NSL; sl++) {
#pragma unroll
            for (int f = 0; f < D / 64; f++)
                k[sl][f] = ld_kv<NT>(reinterpret_cast<const uint4*>(K16 + rows[sl] * D + f * 64 + kq * 8));
        }
#pragma unroll
        for (int i = 0; i < RPW; i++) {
            const uint16_t* vp = V16 + min(rv0 + i, nlast) * D + lane * DPL;
            if constexpr (DPL == 1)
                v[i] = ld_kv<NT>(vp);
            else
                v[i] = ld_kv<NT>(reinterpret_cast<const uint32_t*>(vp));
        }
    }

    // key float4 number f (f < D/32) of slot sl: dims qdim(f, kq) .. +3
    __device__ __forceinline__ float4 key(int sl, int f) const {
        const uint4 u = k[sl][f >> 1];
        const uint32_t a = (f & 1) ? u.z : u.x, b = (f & 1) ? u.w : u.y;
        return make_float4(__uint_as_float(a << 16), __uint_as_float(a & 0xFFFF0000u), __uint_as_float(b << 16),
                           __uint_as_float(b & 0xFFFF0000u));
    }
    __device__ __forceinline__ float val(int i, int dd) const {
        return __uint_as_float(dd == 0 ? v[i] << 16 : v[i] & 0xFFFF0000u);
    }
};

// Split-K decode attention for head_dim 64 or 128 with REP query heads per
// key/value head: a block of NWV waves per 64-position chunk of one (item,
// group), wave w taking positions RPW w .. RPW w + RPW - 1 (RPW = 64 / NWV).
// Each dot product is reduced over its row's 8 lanes with DPP moves; the
// softmax weights of the chunk go through LDS, with max and sum over the
// block; the weighted values are summed over the waves in LDS.  Partials
// (m, l) and the weighted sum per (item, head, chunk).
// NT: the cached rows are loaded with the non-temporal hint (no two items
// of the launch share a sequence; see ld_stream).
template <int D, int REP, int CDT, int NWV, bool NT>
__global__ __launch_bounds__(64 * NWV) void k_attn_g(StepArgs s, int layer) {
    constexpr int KF = D / 32;   // key float4s per lane and row
    constexpr int DPL = D / 64;  // value dims per lane
    constexpr int RPW = kChunk / NWV, NSL = RPW / 8;
    static_assert(D == 64 || D == 128, "head_dim");
    static_assert(kChunk == 64 && (NWV == 4 || NWV == 8), "64 positions over 4 or 8 waves");
    __shared__ float pw[REP][kChunk];
    __shared__ float wred[2][NWV][REP];
    __shared__ float ored[NWV][REP][D];
    const int chunk = blockIdx.x, g = blockIdx.y, item = blockIdx.z;
    const int pos = s.pos[item], slot = s.slot[item];
    const int n = pos + 1;
    const int t0 = chunk * kChunk;
    if (t0 >= n) return;  // whole block
    const int nt = min(kChunk, n - t0);
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int kq = lane & 7, rr = lane >> 3;
    // cache_row counts elements; element e of a bf16 cache is the uint16 at ((uint16_t*)cache)[e]
    const size_t kidx = cache_row(s, layer, 0, slot, g, t0), vidx = cache_row(s, layer, 1, slot, g, t0);
    const float* Kb = CDT == kBF16 ? reinterpret_cast<const float*>(reinterpret_cast<const uint16_t*>(s.cache) + kidx)
                                   : s.cache + kidx;
    const float* Vb = CDT == kBF16 ? reinterpret_cast<const float*>(reinterpret_cast<const uint16_t*>(s.cache) + vidx)
                                   : s.cache + vidx;
    KVRows<D, CDT, RPW> kv;
    int rows[NSL];
#pragma unroll
    for (int sl = 0; sl < NSL; sl++) rows[sl] = min(wave * RPW + sl * 8 + rr, nt - 1);
    kv.template load_t<NT>(Kb, Vb, rows, wave * RPW, nt - 1, kq, lane);
    const float* qb = s.q + (static_cast<size_t>(item) * s.H + static_cast<size_t>(g) * REP) * D;
    float4 qv[REP][KF];
#pragma unroll
    for (int j = 0; j < REP; j++) {
#pragma unroll
        for (int f = 0; f < KF; f++)
            qv[j][f] = *reinterpret_cast<const float4*>(qb + j * D + KVRows<D, CDT, RPW>::qdim(f, kq));
    }
    // scores of the lane's rows for every head, reduced over the row's 8 lanes
    float sc[REP * NSL];
#pragma unroll
    for (int j = 0; j < REP; j++) {
#pragma unroll
        for (int sl = 0; sl < NSL; sl++) {
            float d = 0.f;
#pragma unroll
            for (int f = 0; f < KF; f++) {
                const float4 kk = kv.key(sl, f);
                d = fmaf(kk.x, qv[j][f].x, d);
                d = fmaf(kk.y, qv[j][f].y, d);
                d = fmaf(kk.z, qv[j][f].z, d);
                d = fmaf(kk.w, qv[j][f].w, d);
            }
            sc[j * NSL + sl] = d;
        }
    }
    group_reduce_n<8, OpSum>(sc, OpSum{});
    const float scale = 1.0f / sqrtf(static_cast<float>(D));
    float m[REP];
#pragma unroll
    for (int j = 0; j < REP; j++) {
        m[j] = -INFINITY;
#pragma unroll
        for (int sl = 0; sl < NSL; sl++) {
            sc[j * NSL + sl] = wave * RPW + sl * 8 + rr < nt ? sc[j * NSL + sl] * scale : -INFINITY;
            m[j] = OpMax{}(m[j], sc[j * NSL + sl]);
        }
    }
    group_reduce_n<64, OpMax, 8>(m, OpMax{});  // over the wave's 8-lane row groups
    if (lane == 0) {
#pragma unroll
        for (int j = 0; j < REP; j++) wred[0][wave][j] = m[j];
    }
    __syncthreads();
    float l[REP];
#pragma unroll
    for (int j = 0; j < REP; j++) {
        float mm = wred[0][0][j];
#pragma unroll
        for (int v = 1; v < NWV; v++) mm = OpMax{}(mm, wred[0][v][j]);
        m[j] = mm;
        l[j] = 0.f;
#pragma unroll
        for (int sl = 0; sl < NSL; sl++) {
            const float p = __expf(sc[j * NSL + sl] - m[j]);  // 0 for masked rows (the block max is finite)
            if (kq == 0) pw[j][wave * RPW + sl * 8 + rr] = p;
            l[j] += p;
        }
    }
    group_reduce_n<64, OpSum, 8>(l, OpSum{});
    if (lane == 0) {
#pragma unroll
        for (int j = 0; j < REP; j++) wred[1][wave][j] = l[j];
    }
    __syncthreads();
#pragma unroll
    for (int j = 0; j < REP; j++) {
        const float4* pj = reinterpret_cast<const float4*>(&pw[j][wave * RPW]);
        float4 pe[RPW / 4];
#pragma unroll
        for (int c4 = 0; c4 < RPW / 4; c4++) pe[c4] = pj[c4];
#pragma unroll
        for (int dd = 0; dd < DPL; dd++) {
            float a0 = 0.f, a1 = 0.f;
#pragma unroll
            for (int c4 = 0; c4 < RPW / 4; c4++) {
                a0 = fmaf(pe[c4].x, kv.val(4 * c4 + 0, dd), a0);
                a1 = fmaf(pe[c4].y, kv.val(4 * c4 + 1, dd), a1);
                a0 = fmaf(pe[c4].z, kv.val(4 * c4 + 2, dd), a0);
                a1 = fmaf(pe[c4].w, kv.val(4 * c4 + 3, dd), a1);
            }
            ored[wave][j][lane * DPL + dd] = a0 + a1;
        }
    }
    __syncthreads();
    const int S = s.n_chunks;
    for (int idx = threadIdx.x; idx < REP * D; idx += 64 * NWV) {
        const int j = idx / D, e = idx % D;
        float v = 0.f, lsum = 0.f;
#pragma unroll
        for (int w = 0; w < NWV; w++) {
            v += ored[w][j][e];
            lsum += wred[1][w][j];
        }
        const size_t pidx = (static_cast<size_t>(item) * s.H + g * REP + j) * S + chunk;
        s.part_o[pidx * D + e] = v;
        if (e == 0) {
            s.part_ml[pidx * 2 + 0] = m[j];
            s.part_ml[pidx * 2 + 1] = lsum;
        }
    }
}

// Decode attention of one (item, key/value group) in one block, with no
// partials and no combine launch: wave w of NWV takes the 16-position runs
// w, w + NWV, w + 2 NWV, ... of the item's pos + 1 cached positions and keeps
// an online softmax per head in registers -- running max m, sum l and
// weighted values o, rescaled by e^(m_old - m_new) when a run raises the max
// -- loading the next run's rows while it scores the current one.  The
// waves' (m, l, o) are then merged once through LDS, o = sum_w e^(m_w - M)
// o_w / sum_w e^(m_w - M) l_w, and written to s.o.  Scores and value rows use
// the layouts of k_attn_g (8 lanes per key row, D/64 value dims per lane);
// a run's weights reach the value lanes by readlane from the lanes that
// hold them.  For launches with enough (item, group) pairs to fill the chip.
template <int D, int REP, int CDT, int NWV>
__global__ __launch_bounds__(64 * NWV) void k_attn_full(StepArgs s, int layer) {
    constexpr int KF = D / 32, DPL = D / 64, RPW = 16, NSL = RPW / 8;
    static_assert(D == 64 || D == 128, "head_dim");
    __shared__ float wml[NWV][REP][2];
    __shared__ float wov[NWV][REP][D];
    const int g = blockIdx.x, item = blockIdx.y;
    const int pos = s.pos[item], slot = s.slot[item];
    const int n = pos + 1;
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int kq = lane & 7, rr = lane >> 3;
    const size_t kidx = cache_row(s, layer, 0, slot, g, 0), vidx = cache_row(s, layer, 1, slot, g, 0);
    const float* Kb = CDT == kBF16 ? reinterpret_cast<const float*>(reinterpret_cast<const uint16_t*>(s.cache) + kidx)
                                   : s.cache + kidx;
    const float* Vb = CDT == kBF16 ? reinterpret_cast<const float*>(reinterpret_cast<const uint16_t*>(s.cache) + vidx)
                                   : s.cache + vidx;
    const int nrun = (n + RPW - 1) / RPW;
    using Rows = KVRows<D, CDT, RPW>;
    auto load = [&](Rows& kv, int run) {
        int rows[NSL];
#pragma unroll
        for (int sl = 0; sl < NSL; sl++) rows[sl] = min(run * RPW + sl * 8 + rr, n - 1);
        kv.template load_t<true>(Kb, Vb, rows, run * RPW, n - 1, kq, lane);  // decode: no shared rows
    };
    Rows cur;
    load(cur, min(wave, nrun - 1));
    const float* qb = s.q + (static_cast<size_t>(item) * s.H + static_cast<size_t>(g) * REP) * D;
    float4 qv[REP][KF];
#pragma unroll
    for (int j = 0; j < REP; j++) {
#pragma unroll
        for (int f = 0; f < KF; f++) qv[j][f] = *reinterpret_cast<const float4*>(qb + j * D + Rows::qdim(f, kq));
    }
    const float scale = 1.0f / sqrtf(static_cast<float>(D));
    float m[REP], l[REP], o[REP][DPL];
#pragma unroll
    for (int j = 0; j < REP; j++) {
        m[j] = -INFINITY;
        l[j] = 0.f;
#pragma unroll
        for (int dd = 0; dd < DPL; dd++) o[j][dd] = 0.f;
    }
    // One run of rows: the online softmax update of every head.
    auto step = [&](const Rows& kv, int run) {
        float sc[REP * NSL];
#pragma unroll
        for (int j = 0; j < REP; j++) {
#pragma unroll
            for (int sl = 0; sl < NSL; sl++) {
                float d = 0.f;
#pragma unroll
                for (int f = 0; f < KF; f++) {
                    const float4 kk = kv.key(sl, f);
                    d = fmaf(kk.x, qv[j][f].x, d);
                    d = fmaf(kk.y, qv[j][f].y, d);
                    d = fmaf(kk.z, qv[j][f].z, d);
                    d = fmaf(kk.w, qv[j][f].w, d);
                }
                sc[j * NSL + sl] = d;
            }
        }
        group_reduce_n<8, OpSum>(sc, OpSum{});  // every lane of a row holds its score
        float mr[REP];
#pragma unroll
        for (int j = 0; j < REP; j++) {
            mr[j] = -INFINITY;
#pragma unroll
            for (int sl = 0; sl < NSL; sl++) {
                const int t = run * RPW + sl * 8 + rr;
                sc[j * NSL + sl] = t < n ? sc[j * NSL + sl] * scale : -INFINITY;
                mr[j] = OpMax{}(mr[j], sc[j * NSL + sl]);
            }
        }
        group_reduce_n<64, OpMax, 8>(mr, OpMax{});  // the run's max, on every lane (-inf: run past pos)
        float ps[REP * NSL], lr[REP];
#pragma unroll
        for (int j = 0; j < REP; j++) {
            // a run wholly past pos (all scores -inf) changes nothing, even
            // before the first real run (m = -inf)
            const float mn = OpMax{}(m[j], mr[j]);
            const bool none = mn == -INFINITY;
            const float alpha = none ? 1.f : __expf(m[j] - mn);  // 0 on the first real run (m = -inf)
            m[j] = mn;
            l[j] *= alpha;
#pragma unroll
            for (int dd = 0; dd < DPL; dd++) o[j][dd] *= alpha;
            lr[j] = 0.f;
#pragma unroll
            for (int sl = 0; sl < NSL; sl++) {
                ps[j * NSL + sl] = none ? 0.f : __expf(sc[j * NSL + sl] - mn);  // 0 for rows past pos
                lr[j] += ps[j * NSL + sl];
            }
        }
        group_reduce_n<64, OpSum, 8>(lr, OpSum{});  // over the run's 8-lane row groups
#pragma unroll
        for (int j = 0; j < REP; j++) {
            l[j] += lr[j];
#pragma unroll
            for (int dd = 0; dd < DPL; dd++) {
                float a0 = 0.f, a1 = 0.f;
#pragma unroll
                for (int i = 0; i < RPW; i += 2) {  // row i's weight sits in lane (i % 8) * 8, slot i / 8
                    const float p0 = __int_as_float(
                        __builtin_amdgcn_readlane(__float_as_int(ps[j * NSL + i / 8]), (i % 8) * 8));
                    const float p1 = __int_as_float(
                        __builtin_amdgcn_readlane(__float_as_int(ps[j * NSL + (i + 1) / 8]), ((i + 1) % 8) * 8));
                    a0 = fmaf(p0, kv.val(i, dd), a0);
                    a1 = fmaf(p1, kv.val(i + 1, dd), a1);
                }
                o[j][dd] += a0 + a1;
            }
        }
    };
    // Two row buffers in turn, each loaded one run ahead of its use, with no
    // branch between a load and its use (the compiler would otherwise sink
    // the loads to it): the loads are unconditional (a run past the last one
    // re-reads the last rows) and such a run is wholly masked, a no-op.
    Rows nxt;
    for (int run = wave; run < nrun; run += 2 * NWV) {  // per wave: no barrier inside
        load(nxt, min(run + NWV, nrun - 1));
        step(cur, run);
        load(cur, min(run + 2 * NWV, nrun - 1));
        step(nxt, run + NWV);
    }
#pragma unroll
    for (int j = 0; j < REP; j++) {
        if (lane == 0) {
            wml[wave][j][0] = m[j];
            wml[wave][j][1] = l[j];
        }
#pragma unroll
        for (int dd = 0; dd < DPL; dd++) wov[wave][j][lane * DPL + dd] = o[j][dd];
    }
    __syncthreads();
    for (int idx = threadIdx.x; idx < REP * D; idx += 64 * NWV) {
        const int j = idx / D, e = idx % D;
        float M = wml[0][j][0];  // wave 0 holds position 0: finite
#pragma unroll
        for (int w = 1; w < NWV; w++) M = OpMax{}(M, wml[w][j][0]);
        float L = 0.f, O = 0.f;
#pragma unroll
        for (int w = 0; w < NWV; w++) {
            const float f = __expf(wml[w][j][0] - M);  // 0 for waves without a run
            L = fmaf(f, wml[w][j][1], L);
            O = fmaf(f, wov[w][j][e], O);
        }
        s.o[(static_cast<size_t>(item) * s.H + g * REP + j) * D + e] = O / L;
    }
}

// 16 waves (4 per SIMD, at most 128 VGPRs each) where the registers fit,
// else 8: head_dim 128, and 4 query heads per group at head_dim 64.
template <int D, int CDT>
static bool launch_attn_full2(const StepArgs& s, dim3 grid, int layer, hipStream_t st) {
    constexpr int W = D == 64 ? 16 : 8;
    switch (s.H / s.Hkv) {
        case 1: hipLaunchKernelGGL((k_attn_full<D, 1, CDT, W>), grid, dim3(64 * W), 0, st, s, layer); return true;
        case 2: hipLaunchKernelGGL((k_attn_full<D, 2, CDT, W>), grid, dim3(64 * W), 0, st, s, layer); return true;
        case 3: hipLaunchKernelGGL((k_attn_full<D, 3, CDT, W>), grid, dim3(64 * W), 0, st, s, layer); return true;
        case 4: hipLaunchKernelGGL((k_attn_full<D, 4, CDT, 8>), grid, dim3(64 * 8), 0, st, s, layer); return true;
        default: return false;
    }
}

bool attn_full(const StepArgs& s, int n_items) {
    return s.attn_full && (s.D == 64 || s.D == 128) && s.Hkv > 0 && s.H % s.Hkv == 0 && s.H / s.Hkv <= 4 &&
           n_items * s.Hkv >= kAttnFullMinBlocks;
}

static hipError_t launch_attn_full(const StepArgs& s, int layer, int n_items, hipStream_t st) {
    const dim3 grid(s.Hkv, n_items);
    bool ok;
    if (s.D == 64)
        ok = s.cdt == kBF16 ? launch_attn_full2<64, kBF16>(s, grid, layer, st)
                            : launch_attn_full2<64, kF32>(s, grid, layer, st);
    else
        ok = s.cdt == kBF16 ? launch_attn_full2<128, kBF16>(s, grid, layer, st)
                            : launch_attn_full2<128, kF32>(s, grid, layer, st);
    return ok ? hipGetLastError() : hipErrorInvalidValue;
}

constexpr int kAttnWaves = 4;  // waves per 64-position chunk of k_attn_g

template <int D, int CDT, bool NT>
static bool launch_attn_g3(const StepArgs& s, dim3 grid, int layer, hipStream_t st) {
    constexpr int W = kAttnWaves;
    const dim3 blk(64 * W);
    switch (s.H / s.Hkv) {
        case 1: hipLaunchKernelGGL((k_attn_g<D, 1, CDT, W, NT>), grid, blk, 0, st, s, layer); return true;
        case 2: hipLaunchKernelGGL((k_attn_g<D, 2, CDT, W, NT>), grid, blk, 0, st, s, layer); return true;
        case 3: hipLaunchKernelGGL((k_attn_g<D, 3, CDT, W, NT>), grid, blk, 0, st, s, layer); return true;
        case 4: hipLaunchKernelGGL((k_attn_g<D, 4, CDT, W, NT>), grid, blk, 0, st, s, layer); return true;
        default: return false;
    }
}

template <int D, int CDT>
static bool launch_attn_g2(const StepArgs& s, dim3 grid, int layer, hipStream_t st) {
    return s.kv_stream ? launch_attn_g3<D, CDT, true>(s, grid, layer, st) : launch_attn_g3<D, CDT, false>(s, grid, layer, st);
}

template <int D>
static bool launch_attn_g(const StepArgs& s, dim3 grid, int layer, hipStream_t st) {
    return s.cdt == kBF16 ? launch_attn_g2<D, kBF16>(s, grid, layer, st) : launch_attn_g2<D, kF32>(s, grid, layer, st);
}

static bool attn_d_supported(int D) { return D == 16 || D == 32 || D == 64 || D == 128 || D == 256; }

static hipError_t launch_attn(const StepArgs& s, int layer, int n_items, hipStream_t st);

// Merge the chunk partials of one (item, head): M = max m_s,
// o = sum_s e^(m_s - M) o_s / sum_s e^(m_s - M) l_s.
// Block z of gridDim.z takes dims [z Dh, (z + 1) Dh), Dh = D / gridDim.z
// (the launch splits a head over 4 blocks when there are few heads to go
// round).  Thread (g, e), g < G = 256 / Dh, holds dim e of chunks g, g + G,
// ... (NC of them per batch, loaded before the statistics are known, so the
// partials arrive in one memory round trip); the block then reduces M and
// the denominator, weights its chunks and sums the G groups through LDS.
template <int NC>
__global__ __launch_bounds__(256) void k_attn_combine(StepArgs s) {
    extern __shared__ float wts[];  // [n_chunks] e^(m_s - M)
    __shared__ float red[2][4];
    __shared__ float osum[256];
    const int h = blockIdx.x, item = blockIdx.y;
    const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
    const int n = s.pos[item] + 1;
    const int ns = (n + kChunk - 1) / kChunk;
    const int S = s.n_chunks, D = s.D;
    const int Dh = D / static_cast<int>(gridDim.z), e0 = static_cast<int>(blockIdx.z) * Dh;  // this block's dims
    const int G = 256 / Dh, g = t / Dh, e = t % Dh;
    const bool eok = g < G;
    const size_t base = (static_cast<size_t>(item) * s.H + h) * S;
    const float2* ml = reinterpret_cast<const float2*>(s.part_ml) + base;
    float2 mine = t < ns ? ml[t] : make_float2(-INFINITY, 0.f);
    float acc = 0.f, L = 0.f, M = -INFINITY;
    for (int c0 = 0; c0 < ns; c0 += NC * G) {  // one batch unless ns > NC * G (uniform)
        float ov[NC];
#pragma unroll
        for (int i = 0; i < NC; i++) {
            const int c = min(c0 + g + i * G, ns - 1);
            ov[i] = eok ? s.part_o[(base + c) * D + e0 + e] : 0.f;
        }
        if (c0 == 0) {
            M = mine.x;
            for (int c = t + 256; c < ns; c += 256) M = fmaxf(M, ml[c].x);
#pragma unroll
            for (int o = 32; o > 0; o >>= 1) M = fmaxf(M, __shfl_xor(M, o));
            if (lane == 0) red[0][wave] = M;
            __syncthreads();
            M = fmaxf(fmaxf(red[0][0], red[0][1]), fmaxf(red[0][2], red[0][3]));
            for (int c = t; c < ns; c += 256) {
                const float2 v = c == t ? mine : ml[c];
                const float wv = __expf(v.x - M);
                wts[c] = wv;
                L = fmaf(wv, v.y, L);
            }
#pragma unroll
            for (int o = 32; o > 0; o >>= 1) L += __shfl_xor(L, o);
            if (lane == 0) red[1][wave] = L;
            __syncthreads();  // also publishes wts
            L = (red[1][0] + red[1][1]) + (red[1][2] + red[1][3]);
        }
#pragma unroll
        for (int i = 0; i < NC; i++) {
            const int c = c0 + g + i * G;
            if (c < ns) acc = fmaf(wts[c], ov[i], acc);
        }
    }
    osum[t] = acc;
    __syncthreads();
    if (t < Dh) {
        float o = 0.f;
        for (int gg = 0; gg < G; gg++) o += osum[gg * Dh + t];
        s.o[(static_cast<size_t>(item) * s.H + h) * D + e0 + t] = o / L;
    }
}

// The same merge for contexts of at most kMergeChunks chunks and head_dim
// 64 or 128: one wave per (item, head), lane e holding dims e and e + 64.
// Every chunk slot up to kMergeChunks is loaded without waiting for the
// item's position (slots past its chunk count hold stale values and are left
// out by selects, not arithmetic), so the merge is one memory round trip,
// with no LDS and no barrier.
constexpr int kMergeChunks = 16;
template <int D>
__global__ __launch_bounds__(64) void k_attn_merge(StepArgs s) {
    constexpr int DPL = D / 64;
    const int pair = blockIdx.x, item = pair / s.H, lane = threadIdx.x;
    const int S = s.n_chunks;
    const size_t base = static_cast<size_t>(pair) * S;  // (item * H + h) * S
    const float2* ml = reinterpret_cast<const float2*>(s.part_ml) + base;
    const float* po = s.part_o + base * D + lane;
    float2 v[kMergeChunks];
    float o[kMergeChunks][DPL];
#pragma unroll
    for (int c = 0; c < kMergeChunks; c++) {
        const int cc = min(c, S - 1);
        v[c] = ml[cc];
#pragma unroll
        for (int k = 0; k < DPL; k++) o[c][k] = po[static_cast<size_t>(cc) * D + 64 * k];
    }
    const int ns = (s.pos[item] + kChunk) / kChunk;  // chunks of this item's n = pos + 1 positions
    float M = -INFINITY;
#pragma unroll
    for (int c = 0; c < kMergeChunks; c++) M = c < ns ? fmaxf(M, v[c].x) : M;
    float L = 0.f, acc[DPL];
#pragma unroll
    for (int k = 0; k < DPL; k++) acc[k] = 0.f;
#pragma unroll
    for (int c = 0; c < kMergeChunks; c++) {
        const float wv = c < ns ? __expf(v[c].x - M) : 0.f;
        L = c < ns ? fmaf(wv, v[c].y, L) : L;
#pragma unroll
        for (int k = 0; k < DPL; k++) acc[k] = c < ns ? fmaf(wv, o[c][k], acc[k]) : acc[k];
    }
    float* out = s.o + static_cast<size_t>(pair) * D + lane;
#pragma unroll
    for (int k = 0; k < DPL; k++) out[64 * k] = acc[k] / L;
}

// The same merge for up to 2 * NCL chunks when few (item, head) pairs share
// the launch (the batch-1 decode of a long context): one wave per (pair, 32
// dims), its lanes two chunk groups of those 32 dims, lane (g, e) holding
// dim e of chunks g, g + 2, ... .  Every slot is loaded in one round without
// waiting for the item's position (slots past its chunk count are left out
// by selects); max, weights and sums then cross the two groups with one lane
// exchange each.  No LDS and no barrier.
constexpr int kMergeLongNcl = 40;
template <int D, int NCL>
__global__ __launch_bounds__(64) void k_attn_merge_long(StepArgs s) {
    constexpr int QD = D / 32;  // 32-dim blocks per head
    const int pair = blockIdx.x / QD, item = pair / s.H, lane = threadIdx.x;
    const int g = lane >> 5, e = (blockIdx.x % QD) * 32 + (lane & 31);
    const int S = s.n_chunks;
    const size_t base = static_cast<size_t>(pair) * S;  // (item * H + h) * S
    const float2* ml = reinterpret_cast<const float2*>(s.part_ml) + base;
    const float* po = s.part_o + base * D + e;
    float2 v[NCL];
    float o[NCL];
#pragma unroll
    for (int i = 0; i < NCL; i++) {
        const int c = min(g + 2 * i, S - 1);
        v[i] = ml[c];
        o[i] = po[static_cast<size_t>(c) * D];
    }
    const int ns = (s.pos[item] + kChunk) / kChunk;  // chunks of this item's n = pos + 1 positions
    float M = -INFINITY;
#pragma unroll
    for (int i = 0; i < NCL; i++) M = g + 2 * i < ns ? fmaxf(M, v[i].x) : M;
    M = fmaxf(M, __shfl_xor(M, 32));
    float L = 0.f, acc = 0.f;
#pragma unroll
    for (int i = 0; i < NCL; i++) {
        const float wv = g + 2 * i < ns ? __expf(v[i].x - M) : 0.f;
        L = g + 2 * i < ns ? fmaf(wv, v[i].y, L) : L;
        acc = g + 2 * i < ns ? fmaf(wv, o[i], acc) : acc;
    }
    L += __shfl_xor(L, 32);
    acc += __shfl_xor(acc, 32);
    if (g == 0) s.o[static_cast<size_t>(pair) * D + e] = acc / L;
}

// max_chunks: the most chunks any item of the launch has as the host knows
// it (s.n_chunks when it does not); it sizes each thread's batch of chunk
// partials, and an item with more is still merged, in further batches.
static hipError_t launch_combine(const StepArgs& s, int n_items, hipStream_t st, int max_chunks = 0) {
    if (max_chunks < 1 || max_chunks > s.n_chunks) max_chunks = s.n_chunks;
    if (s.n_chunks <= kMergeChunks && (s.D == 64 || s.D == 128)) {
        const dim3 grid(s.H * n_items);
        if (s.D == 64) hipLaunchKernelGGL(k_attn_merge<64>, grid, dim3(64), 0, st, s);
        else hipLaunchKernelGGL(k_attn_merge<128>, grid, dim3(64), 0, st, s);
        return hipGetLastError();
    }
    if (s.H * n_items < 128 && s.n_chunks <= 2 * kMergeLongNcl && (s.D == 64 || s.D == 128)) {
        const dim3 grid(s.H * n_items * (s.D / 32));
        if (s.D == 64) hipLaunchKernelGGL((k_attn_merge_long<64, kMergeLongNcl>), grid, dim3(64), 0, st, s);
        else hipLaunchKernelGGL((k_attn_merge_long<128, kMergeLongNcl>), grid, dim3(64), 0, st, s);
        return hipGetLastError();
    }
    const int split = s.H * n_items < 128 && s.D >= 128 ? 4 : 1;  // few heads: each head's dims over 4 blocks
    const int Dh = s.D / split;
    const int per = (max_chunks + 256 / Dh - 1) / (256 / Dh);  // chunks per thread, all in one batch if it fits
    const dim3 grid(s.H, n_items, split);
    const size_t lds = sizeof(float) * s.n_chunks;
    if (per <= 8)
        hipLaunchKernelGGL(k_attn_combine<8>, grid, dim3(256), lds, st, s);
    else if (per <= 16)
        hipLaunchKernelGGL(k_attn_combine<16>, grid, dim3(256), lds, st, s);
    else if (per <= 24)
        hipLaunchKernelGGL(k_attn_combine<24>, grid, dim3(256), lds, st, s);
    else if (per <= 32)
        hipLaunchKernelGGL(k_attn_combine<32>, grid, dim3(256), lds, st, s);
    else if (per <= 40)
        hipLaunchKernelGGL(k_attn_combine<40>, grid, dim3(256), lds, st, s);
    else
        hipLaunchKernelGGL(k_attn_combine<48>, grid, dim3(256), lds, st, s);
    return hipGetLastError();
}

// ---- k_wo: x += Wo o --------------------------------------------------------------------
// SHORT: the block first computes the attention output o of every head
// itself (all cached rows fit in LDS), so no attention kernel runs.
template <int WDT, int G, int WAVES, bool SHORT>
__global__ __launch_bounds__(64 * WAVES) void k_wo(StepArgs s, LayerW w, int layer, int ident, int nload) {
    extern __shared__ float xs[];
    constexpr int R = 64 / G;
    const int item = blockIdx.y;
    int n = 0, slot = 0;
    if (SHORT) {
        n = s.pos[item] + 1;
        slot = ident ? item : s.slot[item];
    }
    const int K = s.H * s.D;
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int row = (blockIdx.x * WAVES + wave) * R + lane / G, sub = lane % G;
    const bool valid = row < s.d;
    VecStage<64 * WAVES, 8, false, SHORT ? 0 : lds_pad_q<WDT>()> vs;
    if constexpr (!SHORT) vs.issue(s.o + static_cast<size_t>(item) * K, nullptr, K);  // first, as in k_qkv
    RowStream<WDT, G, 0, !SHORT && (lds_pad_q<WDT>() > 0)> st;
    st.start(w.wo, valid ? row : 0, K, sub, valid, s.d);
    float* xr = s.x + static_cast<size_t>(item) * s.d + row;
    const float x_old = (valid && sub == 0) ? *xr : 0.f;
    if constexpr (SHORT) {
        if (n > nload) {  // the host picks nload >= every context; guard anyway
            if (threadIdx.x == 0) atomicOr(s.err, 2);
            n = nload;
        }
        attention_short<WAVES>(s, layer, item, slot, n, nload, xs, xs + K);
    } else {
        vs.complete_copy(xs);
    }
    const float y = st.finish(xs);
    if (valid && sub == 0) *xr = x_old + y;
}

// ---- k_w13: h = silu(W1 xn) * (W3 xn) -------------------------------------------------------
template <int WDT, int G, int WAVES>
__global__ __launch_bounds__(64 * WAVES) void k_w13(StepArgs s, LayerW w) {
    extern __shared__ float xs[];
    __shared__ float red[WAVES];
    constexpr int R = 64 / G;
    const int item = blockIdx.y;
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int row = (blockIdx.x * WAVES + wave) * R + lane / G, sub = lane % G;
    const bool valid = row < s.F;
    VecStage<64 * WAVES, 4, true, lds_pad_q<WDT>()> vs;
    vs.issue(s.x + static_cast<size_t>(item) * s.d, w.ffn_norm, s.d);  // first, as in k_qkv
    RowStream<WDT, G, 0, (lds_pad_q<WDT>() > 0)> s1, s3;
    s1.start(w.w1, valid ? row : 0, s.d, sub, valid, s.F);
    s3.start(w.w3, valid ? row : 0, s.d, sub, valid, s.F);
    vs.template complete_rms<WAVES>(xs, red, s.d, s.eps);
    const float a = s1.finish(xs);
    const float u = s3.finish(xs);
    if (valid && sub == 0) {
        const float sig = 1.0f / (1.0f + expf(-a));
        s.h[static_cast<size_t>(item) * s.F + row] = (a * sig) * u;
    }
}

// ---- k_w2: x += W2 h ------------------------------------------------------------------------
template <int WDT, int G, int WAVES>
__global__ __launch_bounds__(64 * WAVES) void k_w2(StepArgs s, LayerW w) {
    extern __shared__ float xs[];
    constexpr int R = 64 / G;
    const int item = blockIdx.y;
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int row = (blockIdx.x * WAVES + wave) * R + lane / G, sub = lane % G;
    const bool valid = row < s.d;
    VecStage<64 * WAVES, 8, false, lds_pad_q<WDT>()> vs;
    vs.issue(s.h + static_cast<size_t>(item) * s.F, nullptr, s.F);  // first, as in k_qkv
    RowStream<WDT, G, 0, (lds_pad_q<WDT>() > 0)> st;
    st.start(w.w2, valid ? row : 0, s.F, sub, valid, s.d);
    float* xr = s.x + static_cast<size_t>(item) * s.d + row;
    const float x_old = (valid && sub == 0) ? *xr : 0.f;
    vs.complete_copy(xs);
    const float y = st.finish_roll(xs);
    if (valid && sub == 0) *xr = x_old + y;
}

// ---- k_logits: logits = Wcls rmsnorm(x) and per-block argmax ----------------------------------
template <int WDT, int G, int WAVES>
__global__ __launch_bounds__(64 * WAVES) void k_logits(StepArgs s, const float* __restrict__ out_norm,
                                                       const void* __restrict__ wcls) {
    extern __shared__ float xs[];
    __shared__ float red[WAVES];
    __shared__ unsigned long long kred[WAVES];
    constexpr int R = 64 / G;
    const int item = blockIdx.y;
    const int flag = s.flag[item];
    const int slot = s.slot[item];
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int row = (blockIdx.x * WAVES + wave) * R + lane / G, sub = lane % G;
    const bool valid = row < s.V;
    VecStage<64 * WAVES, 4, true, lds_pad_q<WDT>()> vs;
    vs.issue(s.x + static_cast<size_t>(item) * s.d, out_norm, s.d);  // first, as in k_qkv
    RowStream<WDT, G, 0, (lds_pad_q<WDT>() > 0)> st;
    st.start(wcls, valid ? row : 0, s.d, sub, valid, s.V);
    vs.template complete_rms<WAVES>(xs, red, s.d, s.eps);
    if (!flag) return;
    const float y = st.finish(xs);
    unsigned long long key = 0ull;
    if (valid && sub == 0) {
        s.logits[static_cast<size_t>(slot) * s.V + row] = y;
        key = argmax_key(y, row);
    }
    key = wave_max_u64(key);
    if (lane == 0) kred[wave] = key;
    __syncthreads();
    if (threadIdx.x == 0) {
        unsigned long long k = kred[0];
        for (int i = 1; i < WAVES; i++) k = kred[i] > k ? kred[i] : k;
        s.keys[static_cast<size_t>(item) * kMaxArgmaxBlocks + blockIdx.x] = k;
    }
}

// ---- k_finalize: reduce the argmax keys, write the token, advance lengths ------------------------
__global__ __launch_bounds__(256) void k_finalize(StepArgs s, int n_blocks, int32_t* d_tok_out, int want_tok) {
    __shared__ unsigned long long kred[4];
    const int item = blockIdx.x;
    const int slot = s.slot[item];
    if (want_tok && s.flag[item] && d_tok_out) {
        unsigned long long k = 0ull;
        const unsigned long long* keys = s.keys + static_cast<size_t>(item) * kMaxArgmaxBlocks;
        for (int i = threadIdx.x; i < n_blocks; i += 256) k = keys[i] > k ? keys[i] : k;
        k = wave_max_u64(k);
        if ((threadIdx.x & 63) == 0) kred[threadIdx.x >> 6] = k;
        __syncthreads();
        if (threadIdx.x == 0) {
            for (int i = 1; i < 4; i++) k = kred[i] > k ? kred[i] : k;
            k = kred[0] > k ? kred[0] : k;
            d_tok_out[slot] = static_cast<int32_t>(0xFFFFFFFFu - static_cast<uint32_t>(k));
        }
    }
    // items of one slot (consecutive positions of a prompt) leave the largest
    if (threadIdx.x == 0) atomicMax(s.lengths + slot, s.pos[item] + 1);
}

// ---- small utility kernels ------------------------------------------------------------------------
// One (layer, k/v, group) and destination slot per block: rows [0, n) of the
// source slot, n * D contiguous floats on both sides.
__global__ void k_replicate(float* __restrict__ dst, int Bd, int Td, const float* __restrict__ src, int Bs, int Ts,
                            int Hkv, int D, int src_slot, int dst_first, int n) {
    const int lkg = blockIdx.x, c = blockIdx.y;
    const int g = lkg % Hkv, lk = lkg / Hkv;  // lk = layer * 2 + k/v
    const size_t so = ((static_cast<size_t>(lk) * Bs + src_slot) * Hkv + g) * static_cast<size_t>(Ts) * D;
    const size_t dof = ((static_cast<size_t>(lk) * Bd + dst_first + c) * Hkv + g) * static_cast<size_t>(Td) * D;
    const size_t m = static_cast<size_t>(n) * D;
    if ((D & 3) == 0) {  // rows start on 16-byte boundaries
        const float4* s4 = reinterpret_cast<const float4*>(src + so);
        float4* d4 = reinterpret_cast<float4*>(dst + dof);
        for (size_t i = threadIdx.x; i < m / 4; i += blockDim.x) d4[i] = s4[i];
    } else {
        for (size_t i = threadIdx.x; i < m; i += blockDim.x) dst[dof + i] = src[so + i];
    }
}

__global__ void k_set_lengths(int32_t* lengths, SetList l) {
    for (int i = threadIdx.x; i < l.n; i += blockDim.x) lengths[l.first + i] = l.val[i];
}

__global__ void k_fill_i32(int32_t* p, int n, int32_t v) {
    for (int i = blockIdx.x * blockDim.x + threadIdx.x; i < n; i += gridDim.x * blockDim.x) p[i] = v;
}

// ---- launch configuration ------------------------------------------------------------------------

// Lanes per row: more for longer rows; and two rows per wave instead of four
// when the launch would otherwise hold fewer than 2048 waves (rows = weight
// rows x items), so that every CU has the loads of several waves in flight.
// Lanes per row from the row's length in bf16-sized chunks (8 values; the
// block-scaled types count their values the same way, since a lane's work
// is one convert and one FMA per value) or fp32 chunks, and the row count.
static int pick_g(int K, int wdt, int rows = 1 << 30) {
    const int nch = K / (wdt == kF32 ? 4 : 8);
    if (nch <= 128) return 8;
    if (nch <= 512) return rows >= 4 * 2048 ? 16 : 32;
    return 32;
}

// one-wave blocks while the staged vector is small, 4-wave blocks (sharing it) beyond 2048 floats
static int pick_waves(int K) { return K <= 2048 ? 1 : 4; }

size_t short_lds(const StepArgs& s, int short_n) {
    const size_t HD = static_cast<size_t>(s.H) * s.D;
    return sizeof(float) * (2 * HD + 2 * static_cast<size_t>(s.Hkv) * short_n * (s.D + 4));
}

int short_positions(const StepArgs& s) {
    const int d4 = s.D / 4;
    if (d4 <= 0 || (d4 & (d4 - 1)) != 0) return 0;  // the staging indexes rows with shifts
    for (int n = kShort; n >= 1; n /= 2)
        if (n <= s.T && short_lds(s, n) <= 64 * 1024) return n;
    return 0;
}

size_t max_lds_bytes(const StepArgs& s) {
    return sizeof(float) * static_cast<size_t>(staged_floats(s.wdt, std::max(std::max(s.d, s.H * s.D), s.F)));
}

enum Gemv { G_QKV, G_WO_SHORT, G_WO_LONG, G_W13, G_W2, G_LOGITS };

struct Launch {
    int ident = 0;  // item i is slot i (decode steps)
    int nload = 0;  // cached rows staged by the short-context attention
};

template <int WDT, int G, int WAVES>
static hipError_t launch3(Gemv which, const StepArgs& s, const LayerW& w, int layer, int n_items,
                          hipStream_t st, const float* out_norm, const void* wcls, Launch lc) {
    constexpr int R = 64 / G;
    constexpr int RB = WAVES * R;  // rows per block
    const dim3 blk(64 * WAVES);
    switch (which) {
        case G_QKV: {
            const int tasks = (s.H + 2 * s.Hkv) * s.D / R;
            hipLaunchKernelGGL((k_qkv<WDT, G, WAVES>), dim3((tasks + WAVES - 1) / WAVES, n_items), blk,
                               sizeof(float) * staged_floats(WDT, s.d), st, s, w, layer, lc.ident);
            break;
        }
        case G_WO_SHORT:
            hipLaunchKernelGGL((k_wo<WDT, G, WAVES, true>), dim3((s.d + RB - 1) / RB, n_items), blk,
                               short_lds(s, s.short_n), st, s, w, layer, lc.ident, lc.nload);
            break;
        case G_WO_LONG:
            hipLaunchKernelGGL((k_wo<WDT, G, WAVES, false>), dim3((s.d + RB - 1) / RB, n_items), blk,
                               sizeof(float) * staged_floats(WDT, s.H * s.D), st, s, w, layer, lc.ident, 0);
            break;
        case G_W13:
            hipLaunchKernelGGL((k_w13<WDT, G, WAVES>), dim3((s.F + RB - 1) / RB, n_items), blk,
                               sizeof(float) * staged_floats(WDT, s.d), st, s, w);
            break;
        case G_W2:
            hipLaunchKernelGGL((k_w2<WDT, G, WAVES>), dim3((s.d + RB - 1) / RB, n_items), blk,
                               sizeof(float) * staged_floats(WDT, s.F), st, s, w);
            break;
        case G_LOGITS:
            hipLaunchKernelGGL((k_logits<WDT, G, WAVES>), dim3((s.V + RB - 1) / RB, n_items), blk,
                               sizeof(float) * staged_floats(WDT, s.d), st, s, out_norm, wcls);
            break;
    }
    return hipGetLastError();
}

template <int WDT, int G>
static hipError_t launch2(Gemv which, int waves, const StepArgs& s, const LayerW& w, int layer, int n_items,
                          hipStream_t st, const float* out_norm, const void* wcls, Launch lc) {
    if (waves == 1) return launch3<WDT, G, 1>(which, s, w, layer, n_items, st, out_norm, wcls, lc);
    if (waves == 8) {  // W2 over long rows only (pick in gemv)
        if (which != G_W2) return hipErrorInvalidValue;
        constexpr int RB = 8 * (64 / G);
        hipLaunchKernelGGL((k_w2<WDT, G, 8>), dim3((s.d + RB - 1) / RB, n_items), dim3(512),
                           sizeof(float) * staged_floats(WDT, s.F), st, s, w);
        return hipGetLastError();
    }
    return launch3<WDT, G, 4>(which, s, w, layer, n_items, st, out_norm, wcls, lc);
}

template <int WDT>
static hipError_t launch1(Gemv which, int K, int waves, const StepArgs& s, const LayerW& w, int layer,
                          int n_items, hipStream_t st, const float* out_norm, const void* wcls, Launch lc) {
    int N = s.d;  // Wo, W2
    if (which == G_QKV) N = (s.H + 2 * s.Hkv) * s.D;
    if (which == G_W13) N = s.F;
    // the logits keep the row-independent choice (their argmax partial count is fixed per shape)
    const int rows = which == G_LOGITS ? 1 << 30 : N * n_items;
    switch (pick_g(K, WDT, rows)) {
        case 8: return launch2<WDT, 8>(which, waves, s, w, layer, n_items, st, out_norm, wcls, lc);
        case 16: return launch2<WDT, 16>(which, waves, s, w, layer, n_items, st, out_norm, wcls, lc);
        default: return launch2<WDT, 32>(which, waves, s, w, layer, n_items, st, out_norm, wcls, lc);
    }
}

// logits always use 4-wave blocks (fewer argmax partials per item)
static int logits_blocks(const StepArgs& s) {
    const int R = 64 / pick_g(s.d, s.wdt);
    return (s.V + 4 * R - 1) / (4 * R);
}

static hipError_t gemv(Gemv which, const StepArgs& s, const LayerW& w, int layer, int n_items, hipStream_t st,
                       Launch lc, const float* out_norm = nullptr, const void* wcls = nullptr) {
    int K = s.d;
    if (which == G_WO_SHORT || which == G_WO_LONG) K = s.H * s.D;
    if (which == G_W2) K = s.F;
    int waves = pick_waves(K);
    if (which == G_LOGITS || which == G_WO_SHORT) waves = 4;
    // W2 rows longer than 8192: 8-wave blocks, so half as many blocks stage
    // the whole h (22 us against 26.6 per launch at the 8B shape; 8 waves for
    // the other long-row products measured slower)
    if (which == G_W2 && K > 8192) waves = 8;
    if (s.wdt == kBF16) return launch1<kBF16>(which, K, waves, s, w, layer, n_items, st, out_norm, wcls, lc);
    if (s.wdt == kQ8) return launch1<kQ8>(which, K, waves, s, w, layer, n_items, st, out_norm, wcls, lc);
    if (s.wdt == kQ4) return launch1<kQ4>(which, K, waves, s, w, layer, n_items, st, out_norm, wcls, lc);
    return launch1<kF32>(which, K, waves, s, w, layer, n_items, st, out_norm, wcls, lc);
}

template <int WDT, int G, int WAVES>
static hipError_t set_attrs3(int lds) {
    hipError_t e = hipSuccess;
    auto one = [&](const void* fn) {
        if (e == hipSuccess) e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, lds);
    };
    one(reinterpret_cast<const void*>(k_qkv<WDT, G, WAVES>));
    one(reinterpret_cast<const void*>(k_wo<WDT, G, WAVES, true>));
    one(reinterpret_cast<const void*>(k_wo<WDT, G, WAVES, false>));
    one(reinterpret_cast<const void*>(k_w13<WDT, G, WAVES>));
    one(reinterpret_cast<const void*>(k_w2<WDT, G, WAVES>));
    one(reinterpret_cast<const void*>(k_logits<WDT, G, WAVES>));
    return e;
}

template <int WDT>
static hipError_t set_attrs1(int lds) {
    hipError_t e = set_attrs3<WDT, 8, 1>(lds);
    if (e == hipSuccess) e = set_attrs3<WDT, 8, 4>(lds);
    if (e == hipSuccess) e = set_attrs3<WDT, 16, 1>(lds);
    if (e == hipSuccess) e = set_attrs3<WDT, 16, 4>(lds);
    if (e == hipSuccess) e = set_attrs3<WDT, 32, 1>(lds);
    if (e == hipSuccess) e = set_attrs3<WDT, 32, 4>(lds);
    for (const void* fn : {reinterpret_cast<const void*>(k_w2<WDT, 8, 8>), reinterpret_cast<const void*>(k_w2<WDT, 16, 8>),
                           reinterpret_cast<const void*>(k_w2<WDT, 32, 8>)})
        if (e == hipSuccess) e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, lds);
    return e;
}

hipError_t set_kernel_attributes(int lds) {
    hipError_t e = set_attrs1<kBF16>(lds);
    if (e == hipSuccess) e = set_attrs1<kF32>(lds);
    if (e == hipSuccess) e = set_attrs1<kQ8>(lds);
    if (e == hipSuccess) e = set_attrs1<kQ4>(lds);
    return e;
}

// ---- step enqueue ---------------------------------------------------------------------------------

// Workgroups go to the 8 XCDs round-robin by flattened index, chunk +
// gridDim.x * (group + Hkv * item).  With gridDim.x a multiple of 8, chunk c
// of every (item, group) lands on XCD c mod 8: at 16 chunks and ragged
// contexts XCD 0 takes chunks 0 and 8, always or often in use, and XCD 7
// chunks 7 and 15, often empty, so the busiest XCD streams about 1.4 times
// the mean.  A grid width of 1 mod 8 shifts each pair's chunks by one XCD
// from the previous pair's.  The added chunk indices start at or past T, so
// their blocks return at once (t0 >= n).
static int attn_grid_x(int n_chunks) { return n_chunks < 8 ? n_chunks : n_chunks + (9 - n_chunks % 8) % 8; }

static hipError_t launch_attn(const StepArgs& s, int layer, int n_items, hipStream_t st) {
    const dim3 grid(attn_grid_x(s.n_chunks), s.Hkv, n_items);
    if (s.attn_g && s.D == 64 && launch_attn_g<64>(s, grid, layer, st)) return hipGetLastError();
    if (s.attn_g && s.D == 128 && launch_attn_g<128>(s, grid, layer, st)) return hipGetLastError();
    switch (s.D) {
        case 16: hipLaunchKernelGGL(k_attn_d<16>, grid, dim3(256), 0, st, s, layer); break;
        case 32: hipLaunchKernelGGL(k_attn_d<32>, grid, dim3(256), 0, st, s, layer); break;
        case 64: hipLaunchKernelGGL(k_attn_d<64>, grid, dim3(256), 0, st, s, layer); break;
        case 128: hipLaunchKernelGGL(k_attn_d<128>, grid, dim3(256), 0, st, s, layer); break;
        case 256: hipLaunchKernelGGL(k_attn_d<256>, grid, dim3(256), 0, st, s, layer); break;
        default: return hipErrorInvalidValue;  // check_config admits only the head sizes above
    }
    return hipGetLastError();
}

static bool use_mm(const StepArgs& s, int n_items) { return s.mm_ok && n_items >= kMmMin; }

// ---- diagnostic: a plain streaming read --------------------------------------------------------
// Reads n16 16-byte words once: block b streams its own contiguous segment,
// each round 256 threads x 8 coalesced 16-byte loads (32 KiB) issued before
// any is used; then one xor of everything it read per block goes to out (so
// the loads are live).  Its rate is the read bandwidth the chip gives a
// kernel that does nothing else.
__global__ __launch_bounds__(256) void k_stream_read(const uint4* __restrict__ src, size_t n16,
                                                     uint32_t* __restrict__ out) {
    constexpr int U = 8;
    __shared__ uint32_t red[4];
    const size_t seg = (n16 + gridDim.x - 1) / gridDim.x;
    const size_t lo = static_cast<size_t>(blockIdx.x) * seg;
    const size_t hi = lo + seg < n16 ? lo + seg : n16;
    uint32_t acc = 0;
    size_t i = lo + threadIdx.x;
    for (; i + (U - 1) * 256 < hi; i += U * 256) {
        uint4 v[U];
#pragma unroll
        for (int u = 0; u < U; u++) v[u] = src[i + u * 256];
#pragma unroll
        for (int u = 0; u < U; u++) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
    }
    for (; i < hi; i += 256) {
        const uint4 a = src[i];
        acc ^= a.x ^ a.y ^ a.z ^ a.w;
    }
    for (int o = 32; o > 0; o >>= 1) acc ^= static_cast<uint32_t>(__shfl_xor(static_cast<int>(acc), o));
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = acc;
    __syncthreads();
    if (threadIdx.x == 0) out[blockIdx.x] = red[0] ^ red[1] ^ red[2] ^ red[3];
}

hipError_t enqueue_stream_read(const void* src, size_t bytes, uint32_t* out, int reps, hipStream_t st) {
    for (int r = 0; r < reps; r++) {
        hipLaunchKernelGGL(k_stream_read, dim3(kStreamBlocks), dim3(256), 0, st, static_cast<const uint4*>(src),
                           bytes / 16, out);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

hipError_t enqueue_replicate(float* dst, int Bd, int Td, const float* src, int Bs, int Ts, int L, int Hkv, int D,
                             int src_slot, int dst_first, int count, int n, hipStream_t st) {
    if (count <= 0 || n <= 0) return hipSuccess;
    hipLaunchKernelGGL(k_replicate, dim3(L * 2 * Hkv, count), dim3(256), 0, st, dst, Bd, Td, src, Bs, Ts, Hkv, D,
                       src_slot, dst_first, n);
    return hipGetLastError();
}

hipError_t enqueue_step(const StepArgs& s0, const ModelPtrs& m, const BeginList* lists, int n_lists,
                        const int32_t* d_tok_in, int n_items, bool need_logits, int nload,
                        int32_t* d_tok_out, hipStream_t st) {
    // positions of one sequence in one pass (offsets past its length) share
    // its cached rows: the attention then loads them through the caches
    StepArgs s = s0;
    s.kv_stream = 1;
    for (int i = 0; i < n_lists; i++)
        for (int j = 0; j < lists[i].n; j++)
            if (lists[i].by_value && lists[i].off[j] != 0) s.kv_stream = 0;
    // the items are positions of one sequence (a batched prefill pass): they
    // share its cached rows, and attention can read them once per chunk.  A
    // pass of one position keeps the decode kernels, so that ds_prefill
    // reproduces decode steps bit for bit.
    bool one_seq = n_lists == 1 && lists[0].by_value == 1 && lists[0].n == n_items && n_items >= 2 &&
                   n_items <= kMaxItems;
    for (int j = 1; one_seq && j < lists[0].n; j++) one_seq = lists[0].slot[j] == lists[0].slot[0];
    const bool pf = one_seq && s.mm_ok && attn_pf_supported(s);
    // its attention blocks: the chunks up to the pass's last position when
    // the host knows it, else every chunk slot of the cache
    const int pf_chunks = pf && lists[0].last_pos >= 0 ? std::min(s.n_chunks, lists[0].last_pos / kChunk + 1)
                                                       : s.n_chunks;
    Launch lc;
    lc.ident = d_tok_in != nullptr && lists[0].by_value == 0;  // item == slot
    const bool mm = use_mm(s, n_items);
    lc.nload = mm ? 0 : nload;  // the MFMA path always takes the split-K attention
    hipError_t e = hipSuccess;
    for (int i = 0; i < n_lists && e == hipSuccess; i++) {
        hipLaunchKernelGGL(k_begin, dim3(lists[i].n), dim3(256), 0, st, s, lists[i], d_tok_in);
        e = hipGetLastError();
    }
    for (int l = 0; l < s.L && e == hipSuccess; l++) {
        const LayerW& w = m.layers[l];
        e = mm ? mm_gemv(0, s, w, l, n_items, lc.ident, nullptr, nullptr, st) : gemv(G_QKV, s, w, l, n_items, st, lc);
        if (e != hipSuccess) break;
        if (lc.nload > 0) {
            e = gemv(G_WO_SHORT, s, w, l, n_items, st, lc);
        } else {
            if (attn_full(s, n_items)) {
                e = launch_attn_full(s, l, n_items, st);
            } else if (pf) {
                e = launch_attn_pf(s, l, n_items, pf_chunks, st);
                if (e == hipSuccess) e = launch_combine(s, n_items, st, pf_chunks);
            } else {
                e = launch_attn(s, l, n_items, st);
                if (e == hipSuccess) e = launch_combine(s, n_items, st);
            }
            if (e == hipSuccess)
                e = mm ? mm_gemv(1, s, w, l, n_items, lc.ident, nullptr, nullptr, st) : gemv(G_WO_LONG, s, w, l, n_items, st, lc);
        }
        if (e == hipSuccess)
            e = mm ? mm_gemv(2, s, w, l, n_items, lc.ident, nullptr, nullptr, st) : gemv(G_W13, s, w, l, n_items, st, lc);
        if (e == hipSuccess)
            e = mm ? mm_gemv(3, s, w, l, n_items, lc.ident, nullptr, nullptr, st) : gemv(G_W2, s, w, l, n_items, st, lc);
    }
    if (e == hipSuccess && need_logits)
        e = mm ? mm_gemv(4, s, LayerW{}, 0, n_items, lc.ident, m.out_norm, m.wcls, st)
               : gemv(G_LOGITS, s, LayerW{}, 0, n_items, st, lc, m.out_norm, m.wcls);
    if (e == hipSuccess) {
        hipLaunchKernelGGL(k_finalize, dim3(n_items), dim3(256), 0, st, s, mm ? mm_logits_blocks(s) : logits_blocks(s),
                           d_tok_out, need_logits ? 1 : 0);
        e = hipGetLastError();
    }
    return e;
}

hipError_t enqueue_kernel(int which, int layer, const StepArgs& s, const ModelPtrs& m, int n_items, int nload,
                          hipStream_t st) {
    const LayerW& w = m.layers[layer];
    const bool mm = use_mm(s, n_items);
    Launch lc;
    lc.ident = 1;
    lc.nload = mm ? 0 : nload;
    switch (which) {
        case K_QKV: return mm ? mm_gemv(0, s, w, layer, n_items, 1, nullptr, nullptr, st) : gemv(G_QKV, s, w, layer, n_items, st, lc);
        case K_ATTN:
            if (lc.nload > 0) return hipErrorInvalidValue;
            return attn_full(s, n_items) ? launch_attn_full(s, layer, n_items, st) : launch_attn(s, layer, n_items, st);
        case K_COMBINE:
            if (lc.nload > 0 || attn_full(s, n_items)) return hipErrorInvalidValue;
            return launch_combine(s, n_items, st);
        case K_WO:
            if (mm) return mm_gemv(1, s, w, layer, n_items, 1, nullptr, nullptr, st);
            return gemv(lc.nload > 0 ? G_WO_SHORT : G_WO_LONG, s, w, layer, n_items, st, lc);
        case K_W13: return mm ? mm_gemv(2, s, w, layer, n_items, 1, nullptr, nullptr, st) : gemv(G_W13, s, w, layer, n_items, st, lc);
        case K_W2: return mm ? mm_gemv(3, s, w, layer, n_items, 1, nullptr, nullptr, st) : gemv(G_W2, s, w, layer, n_items, st, lc);
        default:
            return mm ? mm_gemv(4, s, LayerW{}, 0, n_items, 1, m.out_norm, m.wcls, st)
                      : gemv(G_LOGITS, s, LayerW{}, 0, n_items, st, lc, m.out_norm, m.wcls);
    }
}

hipError_t enqueue_set_lengths(int32_t* d_lengths, const int32_t* h_vals, int first, int n, hipStream_t st) {
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
    const int blocks = (n + 255) / 256 < 1024 ? (n + 255) / 256 : 1024;
    hipLaunchKernelGGL(k_fill_i32, dim3(blocks), dim3(256), 0, st, p, n, v);
    return hipGetLastError();
}

}  // namespace ds
