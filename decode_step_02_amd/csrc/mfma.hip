// mfma.hip -- batched decode projections on the gfx950 matrix cores.
//
// With many sequences per step the projections become Y[m][n] = sum_k
// W[n][k] X[m][k] with M = batch items (up to 64 per launch), N = weight rows
// and K = input width.  The weights are exactly bf16, so they feed the bf16
// MFMA unchanged.  The fp32 activations are split into two bf16 terms,
// x = hi + lo + r with |r| <= 2^-18 |x| (hi = bf16(x), lo = bf16(x - hi),
// both rounded to nearest even), and every k-step runs two MFMAs with fp32
// accumulation, keeping the products within fp32-level accuracy of the
// plain matvec ("GOTOken: An Inference Engine in QBasic", section "About one
// token per second": every projection is one row-major matvec).
//
// Wave tile: 16 weight rows x 16*NG items, v_mfma_f32_16x16x32_bf16 with
//   A (16 x 32): lane l holds W[row l%16][k0 + (l/16)*8 .. +8]  (one 16-byte load)
//   B (32 x 16): lane l holds X[item l%16][k0 + (l/16)*8 .. +8] (one 16-byte LDS read)
//   C (16 x 16): lane l holds rows (l/16)*4 + r, r < 4, of item l%16.
// A block of 4 waves shares the activation tile staged in LDS (64 items x
// 64 k as bf16 hi and lo).  RMSNorm is applied per item after the product:
// W (g * x * r) = r * (W (g * x)), with r from the sum of squares gathered
// while staging.  Epilogues match the VALU kernels: RoPE pairs sit in tile
// rows i and i + 8 (lanes l and l ^ 32), residual adds, silu(a) * u, and the
// per-block argmax keys of the vocabulary product.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <algorithm>
#include <atomic>
#include <type_traits>

#include "device.h"
#include "kernels.h"

namespace ds {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));


enum MMKind { MM_QKV, MM_WO, MM_W13, MM_W2, MM_LOGITS };

typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// x = hi + lo in bf16, both rounded to nearest even, for two values at once:
// the pair's hi terms packed in one word (element 0 in the low half), and
// their lo terms in another.  The conversion is gfx950's v_cvt_pk_bf16_f32,
// one instruction per pair, whose round to nearest even gives the same bits
// as the integer rounding (u + 0x7FFF + bit 16 of u) >> 16 for finite values.
__device__ __forceinline__ void split2(float a, float b, uint32_t& hi, uint32_t& lo) {
    hi = __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{a, b}, bf16x2));
    lo = __builtin_bit_cast(uint32_t, __builtin_convertvector(
                                          f32x2{a - __uint_as_float(hi << 16), b - __uint_as_float(hi & 0xFFFF0000u)},
                                          bf16x2));
}

// 8 values into two A/B operands (hi terms, lo terms)
__device__ __forceinline__ void split8(const float4 a, const float4 b, uint4& hi, uint4& lo) {
    split2(a.x, a.y, hi.x, lo.x);
    split2(a.z, a.w, hi.y, lo.y);
    split2(b.x, b.y, hi.z, lo.z);
    split2(b.z, b.w, hi.w, lo.w);
}

__device__ __forceinline__ f32x4 mfma(const uint4 a, const uint4 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), c, 0,
                                                   0, 0);
}

template <int KIND, int NG, int KT>
__global__ __launch_bounds__(256) void k_mm(StepArgs s, LayerW w, int layer, int m0, int n_items, int ident,
                                             const float* __restrict__ out_norm, const void* __restrict__ wcls) {
    constexpr bool NORM = KIND == MM_QKV || KIND == MM_W13 || KIND == MM_LOGITS;
    constexpr int LDK = KT + 8;       // LDS row stride in bf16 (16-byte multiple)
    constexpr int KS = KT / 32;       // MFMA k-steps per tile
    constexpr int SV = KT / 16;       // float4 staged per thread per tile (4 threads per item)
    extern __shared__ __attribute__((aligned(16))) unsigned char lds[];
    uint16_t* xh = reinterpret_cast<uint16_t*>(lds);
    uint16_t* xl = xh + kMmItems * LDK;
    float* gs = reinterpret_cast<float*>(xl + kMmItems * LDK);  // gains [K] (NORM kinds)
    __shared__ float rn[kMmItems];
    __shared__ unsigned long long kred[4][kMmItems];
    // blockIdx.y picks this block's group of 16 * NG items
    m0 += static_cast<int>(blockIdx.y) * 16 * NG;
    n_items = min(n_items - static_cast<int>(blockIdx.y) * 16 * NG, 16 * NG);
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int tile = blockIdx.x * 4 + wave;
    const int ti = lane & 15, kq = lane >> 4;

    int K = s.d, N = 0;
    const void* W = nullptr;
    const void* W3 = nullptr;
    const float* gain = nullptr;
    const float* src = s.x;
    if (KIND == MM_QKV) { N = (s.H + 2 * s.Hkv) * s.D; gain = w.attn_norm; }
    if (KIND == MM_WO) { K = s.H * s.D; N = s.d; W = w.wo; src = s.o; }
    if (KIND == MM_W13) { N = s.F; W = w.w1; W3 = w.w3; gain = w.ffn_norm; }
    if (KIND == MM_W2) { K = s.F; N = s.d; W = w.w2; src = s.h; }
    if (KIND == MM_LOGITS) { N = s.V; W = wcls; gain = out_norm; }

    // the weight row this lane feeds to the A operand (tile row ti)
    const int D = s.D, half_d = s.D / 2;
    const int nq_t = s.H * D / 16, nk_t = s.Hkv * D / 16;
    int row = 0;
    bool roped = false, is_q = false, tile_ok = tile * 16 < N;
    if (KIND == MM_QKV) {
        roped = tile < nq_t + nk_t;
        is_q = tile < nq_t;
        if (roped) {
            const int p = (is_q ? tile : tile - nq_t) * 8 + (ti & 7);
            row = (p / half_d) * D + p % half_d + (ti >> 3) * half_d;
            W = is_q ? w.wq : w.wk;
        } else {
            row = tile_ok ? (tile - nq_t - nk_t) * 16 + ti : 0;
            W = w.wv;
        }
    } else {
        row = min(tile * 16 + ti, N - 1);
    }
    const uint16_t* Wrow = static_cast<const uint16_t*>(W) + static_cast<size_t>(row) * K + kq * 8;
    const uint16_t* W3row = KIND == MM_W13 ? static_cast<const uint16_t*>(W3) + static_cast<size_t>(row) * K + kq * 8
                                           : Wrow;

    // staging role of this thread: item sm, columns sk .. sk + KT/4 - 1 of each tile
    const int sm = threadIdx.x >> 2, sk = (threadIdx.x & 3) * (KT / 4);
    const bool s_ok = sm < n_items;
    const float* srow = src + static_cast<size_t>(m0 + min(sm, n_items - 1)) * K + sk;

    // issue the first tile's loads, then stage the gains while they fly
    float4 xv[SV];
    uint4 wa[KS], wb[KS];
#pragma unroll
    for (int q = 0; q < SV; q++) xv[q] = *reinterpret_cast<const float4*>(srow + q * 4);
#pragma unroll
    for (int k = 0; k < KS; k++) {
        wa[k] = *reinterpret_cast<const uint4*>(Wrow + k * 32);
        wb[k] = KIND == MM_W13 ? *reinterpret_cast<const uint4*>(W3row + k * 32) : wa[k];
    }
    if (NORM)
        for (int j = threadIdx.x; j < (K >> 2); j += 256)
            reinterpret_cast<float4*>(gs)[j] = reinterpret_cast<const float4*>(gain)[j];

    f32x4 acc[NG], acc3[NG];
#pragma unroll
    for (int g = 0; g < NG; g++) {
        acc[g] = f32x4{0.f, 0.f, 0.f, 0.f};
        acc3[g] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
    float ss = 0.f;
    for (int k0 = 0; k0 < K; k0 += KT) {
        __syncthreads();  // the previous tile's LDS reads are done (and the gains are staged)
        // fp32 -> bf16 hi + lo into LDS, gains applied
#pragma unroll
        for (int q = 0; q < SV; q += 2) {
            const float xs[8] = {xv[q].x, xv[q].y, xv[q].z, xv[q].w, xv[q + 1].x, xv[q + 1].y, xv[q + 1].z, xv[q + 1].w};
            float val[8];
#pragma unroll
            for (int c = 0; c < 8; c++) {
                const float x = s_ok ? xs[c] : 0.f;
                ss = fmaf(x, x, ss);
                val[c] = NORM ? gs[k0 + sk + q * 4 + c] * x : x;
            }
            uint4 hi, lo;
            split8(make_float4(val[0], val[1], val[2], val[3]), make_float4(val[4], val[5], val[6], val[7]), hi, lo);
            *reinterpret_cast<uint4*>(xh + sm * LDK + sk + q * 4) = hi;
            *reinterpret_cast<uint4*>(xl + sm * LDK + sk + q * 4) = lo;
        }
        __syncthreads();
        // the next tile's loads fly while this tile's MFMAs run
        uint4 na[KS], nb[KS];
        const int k1 = k0 + KT < K ? k0 + KT : k0;
#pragma unroll
        for (int q = 0; q < SV; q++) xv[q] = *reinterpret_cast<const float4*>(srow + k1 + q * 4);
#pragma unroll
        for (int k = 0; k < KS; k++) {
            na[k] = *reinterpret_cast<const uint4*>(Wrow + k1 + k * 32);
            nb[k] = KIND == MM_W13 ? *reinterpret_cast<const uint4*>(W3row + k1 + k * 32) : na[k];
        }
#pragma unroll
        for (int k = 0; k < KS; k++) {
#pragma unroll
            for (int g = 0; g < NG; g++) {
                const int off = (g * 16 + ti) * LDK + k * 32 + kq * 8;
                const uint4 bh = *reinterpret_cast<const uint4*>(xh + off);
                const uint4 bl = *reinterpret_cast<const uint4*>(xl + off);
                acc[g] = mfma(wa[k], bh, acc[g]);
                acc[g] = mfma(wa[k], bl, acc[g]);
                if (KIND == MM_W13) {
                    acc3[g] = mfma(wb[k], bh, acc3[g]);
                    acc3[g] = mfma(wb[k], bl, acc3[g]);
                }
            }
        }
#pragma unroll
        for (int k = 0; k < KS; k++) {
            wa[k] = na[k];
            wb[k] = nb[k];
        }
    }
    if (NORM) {
        ss += __shfl_xor(ss, 1);
        ss += __shfl_xor(ss, 2);
        if ((threadIdx.x & 3) == 0) rn[sm] = 1.0f / sqrtf(ss / static_cast<float>(K) + s.eps);
        __syncthreads();
    }

    // ---- epilogue: lane holds rows kq*4 + r of items g*16 + ti -------------------------------
    unsigned long long key[NG];
#pragma unroll
    for (int g = 0; g < NG; g++) {
        const int m = g * 16 + ti;
        const bool m_ok = m < n_items;
        const int item = m0 + min(m, n_items - 1);
        const float r_m = NORM ? rn[min(m, n_items - 1)] : 1.f;
        key[g] = 0ull;
        if (KIND == MM_QKV) {
            const int pos = s.pos[item];
            const int slot = ident ? item : s.slot[item];
#pragma unroll
            for (int r = 0; r < 4; r++) {
                const int i = kq * 4 + r;
                const float y = acc[g][r] * r_m;
                const float partner = __shfl_xor(y, 32);
                if (!tile_ok || !m_ok) continue;
                if (roped) {
                    const int p = (is_q ? tile : tile - nq_t) * 8 + (i & 7);
                    const int ii = p % half_d, second = i >> 3;
                    const int orow = (p / half_d) * D + ii + second * half_d;
                    const float c = s.rope_cos[static_cast<size_t>(pos) * half_d + ii];
                    const float sn = s.rope_sin[static_cast<size_t>(pos) * half_d + ii];
                    const float out = second ? fmaf(partner, sn, y * c) : fmaf(-partner, sn, y * c);
                    if (is_q)
                        s.q[static_cast<size_t>(item) * s.H * D + orow] = out;
                    else
                        cache_put(s, cache_row(s, layer, 0, slot, orow / D, pos) + orow % D, out);
                } else {
                    const int orow = (tile - nq_t - nk_t) * 16 + i;
                    cache_put(s, cache_row(s, layer, 1, slot, orow / D, pos) + orow % D, y);
                }
            }
        } else if (KIND == MM_WO || KIND == MM_W2) {
#pragma unroll
            for (int r = 0; r < 4; r++) {
                const int orow = tile * 16 + kq * 4 + r;
                if (m_ok && orow < N) s.x[static_cast<size_t>(item) * s.d + orow] += acc[g][r];
            }
        } else if (KIND == MM_W13) {
#pragma unroll
            for (int r = 0; r < 4; r++) {
                const int orow = tile * 16 + kq * 4 + r;
                const float a = acc[g][r] * r_m, u = acc3[g][r] * r_m;
                if (m_ok && orow < N) s.h[static_cast<size_t>(item) * s.F + orow] = (a / (1.0f + expf(-a))) * u;
            }
        } else {  // MM_LOGITS
            const int slot = ident ? item : s.slot[item];
            const bool want = m_ok && s.flag[item];
#pragma unroll
            for (int r = 0; r < 4; r++) {
                const int orow = tile * 16 + kq * 4 + r;
                const float y = acc[g][r] * r_m;
                if (orow < N) {
                    if (want) s.logits[static_cast<size_t>(slot) * s.V + orow] = y;
                    const unsigned long long kk = argmax_key(y, orow);
                    key[g] = kk > key[g] ? kk : key[g];
                }
            }
        }
    }
    if (KIND == MM_LOGITS) {
#pragma unroll
        for (int g = 0; g < NG; g++) {
            unsigned long long k = key[g];
            unsigned long long o = __shfl_xor(k, 16);
            k = o > k ? o : k;
            o = __shfl_xor(k, 32);
            k = o > k ? o : k;
            if (kq == 0) kred[wave][g * 16 + ti] = k;
        }
        __syncthreads();
        for (int m = threadIdx.x; m < n_items; m += 256) {
            unsigned long long k = kred[0][m];
            for (int v = 1; v < 4; v++) k = kred[v][m] > k ? kred[v][m] : k;
            s.keys[static_cast<size_t>(m0 + m) * kMaxArgmaxBlocks + blockIdx.x] = k;
        }
    }
}

// ---- split-K variant for the narrow projections ------------------------------------------------
// Q/K/V, Wo, W1/W3 and W2 of a small model have few weight rows (576..1536),
// so the tiled kernel above puts only a few dozen blocks on the chip and each
// wave walks K in dependent tiles.  Here a block is one tile of 16 weight rows
// x 16 items; its NW waves (4, 8 or 16) take every NW-th 32-wide k-step, issue
// their weight, activation and gain loads at once (the activations straight
// from global memory into the B-operand layout, split into bf16 hi + lo in
// registers; rows too long for the registers in batches, the next batch in
// flight), run their MFMAs and add their partial tiles (and the items'
// partial sums of squares) through LDS.  Waves w < 4 then finish row r = w of
// each lane's four (tile rows kq*4 + w), with the epilogues of k_mm.  The
// item groups of one row tile are 8 block indices apart, so they run on the
// same XCD and share its L2 copy of the weight tile.  With RT > 1 a block
// takes RT row tiles and each wave multiplies every activation operand it
// loads (and splits) by all of them.
template <int KIND, int MAXS, bool LOOP, int NW = 4, int RT = 1>
__global__ __launch_bounds__(64 * NW) void k_mm_sk(StepArgs s, LayerW w, int layer, int n_items, int ident, int n_tiles,
                                                    int n_groups) {
    constexpr bool NORM = KIND == MM_QKV || KIND == MM_W13;
    constexpr bool TWO = KIND == MM_W13;
    static_assert(!(TWO && RT > 1), "W1/W3 take one row tile per block");
    constexpr int NR = TWO ? 9 : 4 * RT + 1;  // LDS rows per wave: acc of each tile (acc3), sum of squares
    __shared__ float red[NW][NR][64];
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int ti = lane & 15, kq = lane >> 4;
    const int L = blockIdx.x, span = 8 * n_groups;
    const int grp = (L % span) / 8, tg = (L / span) * 8 + L % 8;  // row tiles tg*RT .. tg*RT + RT-1
    if (tg * RT >= n_tiles) return;  // padding of the last eight tile groups (whole block)

    int K = s.d, N = 0;
    const void* W = nullptr;
    const void* W3 = nullptr;
    const float* gain = nullptr;
    const float* src = s.x;
    if (KIND == MM_QKV) { N = (s.H + 2 * s.Hkv) * s.D; gain = w.attn_norm; }
    if (KIND == MM_WO) { K = s.H * s.D; N = s.d; W = w.wo; src = s.o; }
    if (KIND == MM_W13) { N = s.F; W = w.w1; W3 = w.w3; gain = w.ffn_norm; }
    if (KIND == MM_W2) { K = s.F; N = s.d; W = w.w2; src = s.h; }

    const int D = s.D, half_d = s.D / 2;
    const int nq_t = s.H * D / 16, nk_t = s.Hkv * D / 16;
    // each of the block's row tiles: its weight rows (tiles past n_tiles are
    // loaded clamped and not stored)
    int tl[RT];
    bool roped[RT], is_q[RT];
    const uint16_t* Wrow[RT];
#pragma unroll
    for (int t = 0; t < RT; t++) {
        tl[t] = min(tg * RT + t, n_tiles - 1);
        const int tile = tl[t];
        int row = 0;
        const void* Wt = W;
        roped[t] = is_q[t] = false;
        if (KIND == MM_QKV) {
            roped[t] = tile < nq_t + nk_t;
            is_q[t] = tile < nq_t;
            if (roped[t]) {
                const int p = (is_q[t] ? tile : tile - nq_t) * 8 + (ti & 7);
                row = (p / half_d) * D + p % half_d + (ti >> 3) * half_d;
                Wt = is_q[t] ? w.wq : w.wk;
            } else {
                row = (tile - nq_t - nk_t) * 16 + ti;
                Wt = w.wv;
            }
        } else {
            row = min(tile * 16 + ti, N - 1);
        }
        Wrow[t] = static_cast<const uint16_t*>(Wt) + static_cast<size_t>(row) * K + kq * 8;
    }
    const int item = grp * 16 + ti;
    const bool m_ok = item < n_items;
    const uint16_t* W3row = TWO ? static_cast<const uint16_t*>(W3) +
                                      static_cast<size_t>(min(tl[0] * 16 + ti, N - 1)) * K + kq * 8
                                : Wrow[0];
    const float* xrow = src + static_cast<size_t>(min(item, n_items - 1)) * K + kq * 8;
    const float* grow = NORM ? gain + kq * 8 : nullptr;

    // the epilogue's own loads go first: the residual row (Wo, W2) or the
    // position, slot and RoPE angle (Q/K/V) of the row this lane finishes
    const int ri = kq * 4 + wave;  // tile row this lane finishes (r = wave)
    const int item_c = min(item, n_items - 1);
    float xres[RT], rc[RT], rsn[RT];
    int pos = 0, slot = 0;
    if (KIND == MM_QKV) {
        pos = s.pos[item_c];
        slot = ident ? item_c : s.slot[item_c];
    }
#pragma unroll
    for (int t = 0; t < RT; t++) {
        xres[t] = 0.f;
        rc[t] = 1.f;
        rsn[t] = 0.f;
        if (KIND == MM_WO || KIND == MM_W2) xres[t] = s.x[static_cast<size_t>(item_c) * s.d + min(tl[t] * 16 + ri, N - 1)];
        if (KIND == MM_QKV && roped[t]) {
            const int ii = ((is_q[t] ? tl[t] : tl[t] - nq_t) * 8 + (ri & 7)) % half_d;
            rc[t] = s.rope_cos[static_cast<size_t>(pos) * half_d + ii];
            rsn[t] = s.rope_sin[static_cast<size_t>(pos) * half_d + ii];
        }
    }
    // The wave's k-steps are wave + NW i.  Without LOOP all of them (at most
    // MAXS) are loaded at once; with LOOP they go in batches of MAXS, the
    // next batch's loads issued before this batch's products (long rows).
    // Each activation operand serves the RT row tiles.
    const int nks = K / 32;
    struct Batch {
        uint4 wa[RT][MAXS], wb[MAXS];
        float4 xa[MAXS], xb[MAXS], ga[MAXS], gb[MAXS];
    };
    auto load = [&](Batch& bt, int i0) {
#pragma unroll
        for (int i = 0; i < MAXS; i++) {
            const int ks = wave + NW * (i0 + i);
            if (ks < nks) {
                const int k0 = ks * 32;
#pragma unroll
                for (int t = 0; t < RT; t++) bt.wa[t][i] = *reinterpret_cast<const uint4*>(Wrow[t] + k0);
                if (TWO) bt.wb[i] = *reinterpret_cast<const uint4*>(W3row + k0);
                bt.xa[i] = *reinterpret_cast<const float4*>(xrow + k0);
                bt.xb[i] = *reinterpret_cast<const float4*>(xrow + k0 + 4);
                if (NORM) {
                    bt.ga[i] = *reinterpret_cast<const float4*>(grow + k0);
                    bt.gb[i] = *reinterpret_cast<const float4*>(grow + k0 + 4);
                }
            }
        }
    };
    f32x4 acc[RT], acc3 = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int t = 0; t < RT; t++) acc[t] = f32x4{0.f, 0.f, 0.f, 0.f};
    float ss = 0.f;
    auto products = [&](const Batch& bt, int i0) {
#pragma unroll
        for (int i = 0; i < MAXS; i++) {
            if (wave + NW * (i0 + i) < nks) {
                const float xs[8] = {bt.xa[i].x, bt.xa[i].y, bt.xa[i].z, bt.xa[i].w,
                                     bt.xb[i].x, bt.xb[i].y, bt.xb[i].z, bt.xb[i].w};
                float gv[8] = {1.f, 1.f, 1.f, 1.f, 1.f, 1.f, 1.f, 1.f};
                if constexpr (NORM) {
                    gv[0] = bt.ga[i].x; gv[1] = bt.ga[i].y; gv[2] = bt.ga[i].z; gv[3] = bt.ga[i].w;
                    gv[4] = bt.gb[i].x; gv[5] = bt.gb[i].y; gv[6] = bt.gb[i].z; gv[7] = bt.gb[i].w;
                }
                float val[8];
#pragma unroll
                for (int c = 0; c < 8; c++) {
                    const float x = m_ok ? xs[c] : 0.f;
                    ss = fmaf(x, x, ss);
                    val[c] = NORM ? gv[c] * x : x;
                }
                uint4 bh, bl;
                split8(make_float4(val[0], val[1], val[2], val[3]), make_float4(val[4], val[5], val[6], val[7]), bh,
                       bl);
#pragma unroll
                for (int t = 0; t < RT; t++) {
                    acc[t] = mfma(bt.wa[t][i], bh, acc[t]);
                    acc[t] = mfma(bt.wa[t][i], bl, acc[t]);
                }
                if (TWO) {
                    acc3 = mfma(bt.wb[i], bh, acc3);
                    acc3 = mfma(bt.wb[i], bl, acc3);
                }
            }
        }
    };
    Batch cur;
    load(cur, 0);
    if constexpr (LOOP) {
        for (int i0 = 0; wave + NW * i0 < nks; i0 += MAXS) {  // the wave's own batch count
            Batch nxt;
            const bool more = wave + NW * (i0 + MAXS) < nks;
            if (more) load(nxt, i0 + MAXS);
            products(cur, i0);
            if (more) cur = nxt;
        }
    } else {
        products(cur, 0);
    }
    if (NORM) {  // the item's sum over the wave's k-steps: lanes ti, ti + 16, ti + 32, ti + 48
        ss += __shfl_xor(ss, 16);
        ss += __shfl_xor(ss, 32);
    }
#pragma unroll
    for (int r = 0; r < 4; r++) {
#pragma unroll
        for (int t = 0; t < RT; t++) red[wave][4 * t + r][lane] = acc[t][r];
        if (TWO) red[wave][4 + r][lane] = acc3[r];
    }
    if (NORM) red[wave][NR - 1][lane] = ss;
    __syncthreads();
    if (wave >= 4) return;  // waves 0..3 finish the tiles' rows
    const int r = wave;  // this wave finishes tile row kq * 4 + r (= ri) of every tile
    float sq = 0.f;
    if (NORM) {
#pragma unroll
        for (int v = 0; v < NW; v++) sq += red[v][NR - 1][lane];
    }
    float r_m = 1.f;
    if (NORM) r_m = 1.0f / sqrtf(sq / static_cast<float>(K) + s.eps);
    const int i = ri;
#pragma unroll
    for (int t = 0; t < RT; t++) {
        const int tile = tl[t];
        const bool t_ok = tg * RT + t < n_tiles;
        float y = 0.f, y3 = 0.f;
#pragma unroll
        for (int v = 0; v < NW; v++) {
            y += red[v][4 * t + r][lane];
            if (TWO) y3 += red[v][4 + r][lane];
        }
        if (KIND == MM_QKV) {
            y *= r_m;
            const float partner = __shfl_xor(y, 32);  // tile rows i and i ^ 8 of the same item
            if (!m_ok || !t_ok || tile * 16 >= N) continue;
            if (roped[t]) {
                const int p = (is_q[t] ? tile : tile - nq_t) * 8 + (i & 7);
                const int ii = p % half_d, second = i >> 3;
                const int orow = (p / half_d) * D + ii + second * half_d;
                const float c = rc[t], sn = rsn[t];
                const float out = second ? fmaf(partner, sn, y * c) : fmaf(-partner, sn, y * c);
                if (is_q[t])
                    s.q[static_cast<size_t>(item) * s.H * D + orow] = out;
                else
                    cache_put(s, cache_row(s, layer, 0, slot, orow / D, pos) + orow % D, out);
            } else {
                const int orow = (tile - nq_t - nk_t) * 16 + i;
                cache_put(s, cache_row(s, layer, 1, slot, orow / D, pos) + orow % D, y);
            }
        } else if (KIND == MM_WO || KIND == MM_W2) {
            const int orow = tile * 16 + i;
            if (m_ok && t_ok && orow < N) s.x[static_cast<size_t>(item) * s.d + orow] = xres[t] + y;
        } else {  // MM_W13
            const int orow = tile * 16 + i;
            const float a = y * r_m, u = y3 * r_m;
            if (m_ok && t_ok && orow < N) s.h[static_cast<size_t>(item) * s.F + orow] = (a / (1.0f + expf(-a))) * u;
        }
    }
}

// ---- launch ----------------------------------------------------------------------------------

bool mm_supported(const StepArgs& s) {
    return s.wdt == kBF16 && s.d % 64 == 0 && (s.H * s.D) % 64 == 0 && s.F % 64 == 0 && s.D % 16 == 0 &&
           ((s.H + 2 * s.Hkv) * s.D) % 16 == 0;
}

int mm_logits_blocks(const StepArgs& s) { return (s.V + 63) / 64; }

static int pick_kt(int K) {
    if (K % 256 == 0) return 256;
    if (K % 192 == 0) return 192;
    if (K % 128 == 0) return 128;
    return 64;
}

static size_t mm_lds(int KT, bool norm, int K) {
    return sizeof(uint16_t) * 2 * kMmItems * (KT + 8) + (norm ? sizeof(float) * K : 0);
}

template <int KIND, int NG, int KT>
static void launch_one(dim3 grid, size_t lds, const StepArgs& s, const LayerW& w, int layer, int m0, int n, int ident,
                       const float* out_norm, const void* wcls, hipStream_t st) {
    hipLaunchKernelGGL((k_mm<KIND, NG, KT>), grid, dim3(256), lds, st, s, w, layer, m0, n, ident, out_norm, wcls);
}

template <int KIND, int KT>
static void launch_ng(int ng, dim3 grid, size_t lds, const StepArgs& s, const LayerW& w, int layer, int m0, int n,
                      int ident, const float* out_norm, const void* wcls, hipStream_t st) {
    switch (ng) {
        case 1: launch_one<KIND, 1, KT>(grid, lds, s, w, layer, m0, n, ident, out_norm, wcls, st); break;
        case 2: launch_one<KIND, 2, KT>(grid, lds, s, w, layer, m0, n, ident, out_norm, wcls, st); break;
        case 3: launch_one<KIND, 3, KT>(grid, lds, s, w, layer, m0, n, ident, out_norm, wcls, st); break;
        default: launch_one<KIND, 4, KT>(grid, lds, s, w, layer, m0, n, ident, out_norm, wcls, st); break;
    }
}

template <int KIND>
static hipError_t launch_kind(const StepArgs& s, const LayerW& w, int layer, int m0, int n, int ident,
                              const float* out_norm, const void* wcls, hipStream_t st) {
    int N = 0, K = s.d;
    if (KIND == MM_QKV) N = (s.H + 2 * s.Hkv) * s.D;
    if (KIND == MM_WO) { N = s.d; K = s.H * s.D; }
    if (KIND == MM_W2) { N = s.d; K = s.F; }
    if (KIND == MM_W13) N = s.F;
    if (KIND == MM_LOGITS) N = s.V;
    constexpr bool norm = KIND == MM_QKV || KIND == MM_W13 || KIND == MM_LOGITS;
    // Few row blocks (every matrix but the vocabulary one): one block per 16
    // items as well, which fills more CUs at the price of reading each
    // weight tile once per item group.
    const int nbx = (N + 63) / 64;
    const int ng = nbx < 128 ? 1 : (n + 15) / 16;
    const dim3 grid(nbx, (n + 16 * ng - 1) / (16 * ng));
    // The vocabulary product takes 64-wide k-tiles: a third of the LDS per
    // block, so more of its blocks share a CU (B = 64, 135M: 28.5 against
    // 45.5 us per launch with 192-wide tiles).
    // W1/W3 over rows of 2048 or more takes 128-wide k-tiles (8B batched
    // prefill: 733.5 -> 718.0 ms; 256-wide tiles, or 32 or 16 items per block
    // with twice or four times the blocks, were slower).
    const int kt = KIND == MM_LOGITS                ? 64
                   : KIND == MM_W13 && K >= 2048 ? (K % 128 == 0 ? 128 : 64)
                                                    : pick_kt(K);
    const size_t lds = mm_lds(kt, norm, K);
    switch (kt) {
        case 256: launch_ng<KIND, 256>(ng, grid, lds, s, w, layer, m0, n, ident, out_norm, wcls, st); break;
        case 192: launch_ng<KIND, 192>(ng, grid, lds, s, w, layer, m0, n, ident, out_norm, wcls, st); break;
        case 128: launch_ng<KIND, 128>(ng, grid, lds, s, w, layer, m0, n, ident, out_norm, wcls, st); break;
        default: launch_ng<KIND, 64>(ng, grid, lds, s, w, layer, m0, n, ident, out_norm, wcls, st); break;
    }
    return hipGetLastError();
}


// ---- causal attention over one sequence's positions (batched prefill) ----------------------------
// In a batched-prefill pass the items are positions of one sequence, so they
// read the same cached rows.  One block per (64-position chunk, key/value
// group) stages the chunk's keys (row-major) and values (transposed) in LDS
// once, as bf16 hi and lo terms, and serves every item of the pass and every
// query head of the group: wave w takes items 16 (w % 4) .. + 15 of head
// w / 4 and computes
//   S = Q K^T   (16 items x 64 positions, D-long products),
//   the chunk's softmax statistics per item, m = max_p S*scale and
//   l = sum_p e^(S*scale - m), over the positions up to the item's own,
//   O = P V     (16 items x D dims, 64-long products, P through LDS),
// on the matrix cores, every product as hi*hi + hi*lo + lo*hi + lo*lo with
// fp32 accumulation (the lo terms of a bf16 cache are zero and skipped).
// The partials (m, l, O) per (item, head, chunk) are those of k_attn_g and go
// to the same merge launch.  The rows, the queries and the positions are all
// loaded before the first barrier; rows past the pass's last position are
// masked out of the scores and zeroed as values; chunks past it exit.
// n_items <= 64.
//   A (16 x 32): lane l holds Q[item l%16][d0 + (l/16)*8 .. +8], or P rows
//   B (32 x 16): lane l holds K[pos l%16][d0 + (l/16)*8 .. +8], or V^T rows
//   C (16 x 16): lane l holds rows (l/16)*4 + r of column l%16
constexpr int kPfKP(int D) { return D + 8; }   // key row stride in LDS (bf16): 16-byte rows, fewer conflicts
constexpr int kPfVP = kChunk + 8;              // transposed value row stride (bf16)
constexpr int kPfPP = kChunk + 4;              // probability row stride (floats)

size_t attn_pf_lds(int D, int cdt, int rep) {
    const size_t terms = cdt == kBF16 ? 1 : 2;
    return sizeof(uint16_t) * terms * (static_cast<size_t>(kChunk) * kPfKP(D) + static_cast<size_t>(D) * kPfVP) +
           sizeof(float) * 4 * rep * 16 * kPfPP;
}


template <int D, int REP, int CDT>
__global__ __launch_bounds__(256 * REP) void k_attn_pf(StepArgs s, int layer, int n_items) {
    constexpr bool LO = CDT != kBF16;
    constexpr int NT = 256 * REP;
    constexpr int KP = kPfKP(D), VP = kPfVP, PP = kPfPP;
    constexpr int KS = D / 32, DT = D / 16, G8 = D / 8;
    constexpr int NG = kChunk * G8;           // 8-value groups of a chunk's rows
    constexpr int PER = (NG + NT - 1) / NT;   // per thread
    using Raw = typename std::conditional<LO, float4, uint4>::type;
    constexpr int RW = LO ? 2 : 1;            // raw loads per 8 values
    extern __shared__ __attribute__((aligned(16))) unsigned char lds[];
    uint16_t* kh = reinterpret_cast<uint16_t*>(lds);  // [kChunk][KP]
    uint16_t* kl = kh + kChunk * KP;                  // LO only
    uint16_t* vh = kh + (LO ? 2 : 1) * kChunk * KP;   // [D][VP]
    uint16_t* vl = vh + D * VP;                       // LO only
    float* pw = reinterpret_cast<float*>(vh + (LO ? 2 : 1) * D * VP);  // [4 REP waves][16][PP]
    __shared__ int smax;
    const int chunk = blockIdx.x, g = blockIdx.y;
    const int t0 = chunk * kChunk;
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int ig = wave & 3, head = g * REP + (wave >> 2);
    // (1) everything that does not depend on the pass's last position
    const int slot = s.slot[0];
    const size_t kidx = cache_row(s, layer, 0, slot, g, 0), vidx = cache_row(s, layer, 1, slot, g, 0);
    Raw kraw[PER][RW], vraw[PER][RW];
#pragma unroll
    for (int i = 0; i < PER; i++) {  // rows clamped into the sequence's T rows; replaced below where past the last position
        const int q = min(static_cast<int>(threadIdx.x) + i * NT, NG - 1);
        const size_t off = static_cast<size_t>(min(t0 + q / G8, s.T - 1)) * D + (q % G8) * 8;
#pragma unroll
        for (int h = 0; h < RW; h++) {
            if constexpr (LO) {
                kraw[i][h] = *reinterpret_cast<const float4*>(s.cache + kidx + off + 4 * h);
                vraw[i][h] = *reinterpret_cast<const float4*>(s.cache + vidx + off + 4 * h);
            } else {
                const uint16_t* c16 = reinterpret_cast<const uint16_t*>(s.cache);
                kraw[i][h] = *reinterpret_cast<const uint4*>(c16 + kidx + off);
                vraw[i][h] = *reinterpret_cast<const uint4*>(c16 + vidx + off);
            }
        }
    }
    const int ia = min(16 * ig + (lane & 15), n_items - 1);  // this lane's A row (item)
    const float* qrow = s.q + (static_cast<size_t>(ia) * s.H + head) * D + (lane >> 4) * 8;
    float4 qv[KS][2];
#pragma unroll
    for (int k = 0; k < KS; k++) {
        qv[k][0] = *reinterpret_cast<const float4*>(qrow + 32 * k);
        qv[k][1] = *reinterpret_cast<const float4*>(qrow + 32 * k + 4);
    }
    int pc[4];
    bool vc[4];
#pragma unroll
    for (int r = 0; r < 4; r++) {  // the C rows' items
        const int it = 16 * ig + (lane >> 4) * 4 + r;
        vc[r] = it < n_items;
        pc[r] = s.pos[min(it, n_items - 1)];
    }
    if (wave == 0) {  // the pass's last position
        int p = lane < n_items ? s.pos[lane] : -1;
#pragma unroll
        for (int o = 32; o > 0; o >>= 1) p = max(p, __shfl_xor(p, o));
        if (lane == 0) smax = p;
    }
    __syncthreads();
    const int maxpos = smax;
    // the host sized the grid from its record of the sequence's length; a
    // pass that reaches past the grid's chunks (the device's lengths moved
    // on without the host, e.g. replayed captured steps) misses rows: flag it
    if (maxpos >= kChunk * static_cast<int>(gridDim.x) && chunk == 0 && g == 0 && threadIdx.x == 0)
        atomicOr(s.err, 2);
    if (t0 > maxpos) return;  // whole block
    const int rlast = min(kChunk - 1, maxpos - t0);
    // (2) the staged rows: keys as loaded (rows past rlast never pass the
    // mask), values of rows past rlast as zeros (their weight is 0)
#pragma unroll
    for (int i = 0; i < PER; i++) {
        const int q = threadIdx.x + i * NT;
        if (q < NG) {
            const int r = q / G8, d0 = (q % G8) * 8;
            uint4 khi, klo, vhi, vlo;
            if constexpr (LO) {
                split8(kraw[i][0], kraw[i][1], khi, klo);
                split8(vraw[i][0], vraw[i][1], vhi, vlo);
            } else {
                khi = kraw[i][0];
                vhi = vraw[i][0];
                klo = vlo = make_uint4(0u, 0u, 0u, 0u);
            }
            if (r > rlast) vhi = vlo = make_uint4(0u, 0u, 0u, 0u);
            *reinterpret_cast<uint4*>(kh + r * KP + d0) = khi;
            if constexpr (LO) *reinterpret_cast<uint4*>(kl + r * KP + d0) = klo;
            const uint32_t vw[4] = {vhi.x, vhi.y, vhi.z, vhi.w}, vlw[4] = {vlo.x, vlo.y, vlo.z, vlo.w};
#pragma unroll
            for (int e = 0; e < 8; e++) {
                vh[(d0 + e) * VP + r] = static_cast<uint16_t>(vw[e >> 1] >> (16 * (e & 1)));
                if constexpr (LO) vl[(d0 + e) * VP + r] = static_cast<uint16_t>(vlw[e >> 1] >> (16 * (e & 1)));
            }
        }
    }
    __syncthreads();

    // (3) S = Q K^T for this wave's 16 items and head
    f32x4 sacc[4];
#pragma unroll
    for (int pt = 0; pt < 4; pt++) sacc[pt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int k = 0; k < KS; k++) {
        uint4 ah, al;
        split8(qv[k][0], qv[k][1], ah, al);
#pragma unroll
        for (int pt = 0; pt < 4; pt++) {
            const int ko = (16 * pt + (lane & 15)) * KP + 32 * k + (lane >> 4) * 8;
            const uint4 bh = *reinterpret_cast<const uint4*>(kh + ko);
            sacc[pt] = mfma(ah, bh, sacc[pt]);
            sacc[pt] = mfma(al, bh, sacc[pt]);
            if constexpr (LO) {
                const uint4 bl = *reinterpret_cast<const uint4*>(kl + ko);
                sacc[pt] = mfma(ah, bl, sacc[pt]);
                sacc[pt] = mfma(al, bl, sacc[pt]);
            }
        }
    }
    // (4) the chunk's statistics per item row (16 lanes share a row group)
    const float scale = 1.0f / sqrtf(static_cast<float>(D));
    float* pwv = pw + wave * 16 * PP;
    float mr[4], lr[4];
#pragma unroll
    for (int r = 0; r < 4; r++) {
        float m = -INFINITY;
#pragma unroll
        for (int pt = 0; pt < 4; pt++) {
            const bool in = vc[r] && t0 + 16 * pt + (lane & 15) <= pc[r];
            sacc[pt][r] = in ? sacc[pt][r] * scale : -INFINITY;
            m = fmaxf(m, sacc[pt][r]);
        }
#pragma unroll
        for (int o = 1; o < 16; o <<= 1) m = fmaxf(m, __shfl_xor(m, o));
        mr[r] = m;
        float l = 0.f;
#pragma unroll
        for (int pt = 0; pt < 4; pt++) {
            const float p = m == -INFINITY ? 0.f : __expf(sacc[pt][r] - m);
            pwv[((lane >> 4) * 4 + r) * PP + 16 * pt + (lane & 15)] = p;
            l += p;
        }
#pragma unroll
        for (int o = 1; o < 16; o <<= 1) l += __shfl_xor(l, o);
        lr[r] = l;
    }
    __syncthreads();  // the probabilities in LDS (each wave reads only its own)
    // (5) O = P V
    f32x4 oacc[DT];
#pragma unroll
    for (int dt = 0; dt < DT; dt++) oacc[dt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kk = 0; kk < kChunk / 32; kk++) {
        const float* prow = pwv + (lane & 15) * PP + 32 * kk + (lane >> 4) * 8;
        uint4 ph, pl;
        split8(*reinterpret_cast<const float4*>(prow), *reinterpret_cast<const float4*>(prow + 4), ph, pl);
#pragma unroll
        for (int dt = 0; dt < DT; dt++) {
            const int vo = (16 * dt + (lane & 15)) * VP + 32 * kk + (lane >> 4) * 8;
            const uint4 bh = *reinterpret_cast<const uint4*>(vh + vo);
            oacc[dt] = mfma(ph, bh, oacc[dt]);
            oacc[dt] = mfma(pl, bh, oacc[dt]);
            if constexpr (LO) {
                const uint4 bl = *reinterpret_cast<const uint4*>(vl + vo);
                oacc[dt] = mfma(ph, bl, oacc[dt]);
                oacc[dt] = mfma(pl, bl, oacc[dt]);
            }
        }
    }
    // (6) the partials of the items that reach this chunk
    const int S = s.n_chunks;
#pragma unroll
    for (int r = 0; r < 4; r++) {
        const int it = 16 * ig + (lane >> 4) * 4 + r;
        if (vc[r] && pc[r] >= t0) {
            const size_t pidx = (static_cast<size_t>(it) * s.H + head) * S + chunk;
#pragma unroll
            for (int dt = 0; dt < DT; dt++) s.part_o[pidx * D + 16 * dt + (lane & 15)] = oacc[dt][r];
            if ((lane & 15) == 0) {
                s.part_ml[pidx * 2 + 0] = mr[r];
                s.part_ml[pidx * 2 + 1] = lr[r];
            }
        }
    }
}

bool attn_pf_supported(const StepArgs& s) {
    return s.attn_pf && (s.D == 64 || s.D == 128) && s.Hkv > 0 && s.H % s.Hkv == 0 && s.H / s.Hkv <= 4;
}

template <int D, int CDT>
static void launch_pf2(const StepArgs& s, int layer, int n_items, int n_chunks, hipStream_t st) {
    const dim3 grid(n_chunks, s.Hkv);
    const int rep = s.H / s.Hkv;
    const size_t lds = attn_pf_lds(D, CDT, rep);
    switch (rep) {
        case 1: hipLaunchKernelGGL((k_attn_pf<D, 1, CDT>), grid, dim3(256), lds, st, s, layer, n_items); break;
        case 2: hipLaunchKernelGGL((k_attn_pf<D, 2, CDT>), grid, dim3(512), lds, st, s, layer, n_items); break;
        case 3: hipLaunchKernelGGL((k_attn_pf<D, 3, CDT>), grid, dim3(768), lds, st, s, layer, n_items); break;
        default: hipLaunchKernelGGL((k_attn_pf<D, 4, CDT>), grid, dim3(1024), lds, st, s, layer, n_items); break;
    }
}

hipError_t launch_attn_pf(const StepArgs& s, int layer, int n_items, int n_chunks, hipStream_t st) {
    if (!attn_pf_supported(s) || n_items < 1 || n_items > 64 || n_chunks < 1 || n_chunks > s.n_chunks)
        return hipErrorInvalidValue;
    if (s.D == 64) {
        if (s.cdt == kBF16) launch_pf2<64, kBF16>(s, layer, n_items, n_chunks, st);
        else launch_pf2<64, kF32>(s, layer, n_items, n_chunks, st);
    } else {
        if (s.cdt == kBF16) launch_pf2<128, kBF16>(s, layer, n_items, n_chunks, st);
        else launch_pf2<128, kF32>(s, layer, n_items, n_chunks, st);
    }
    return hipGetLastError();
}

template <int D, int CDT>
static hipError_t attrs_pf(int lds) {
    hipError_t e = hipSuccess;
    auto one = [&](const void* fn) {
        if (e == hipSuccess) e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, lds);
    };
    one(reinterpret_cast<const void*>(k_attn_pf<D, 1, CDT>));
    one(reinterpret_cast<const void*>(k_attn_pf<D, 2, CDT>));
    one(reinterpret_cast<const void*>(k_attn_pf<D, 3, CDT>));
    one(reinterpret_cast<const void*>(k_attn_pf<D, 4, CDT>));
    return e;
}

template <int KIND, int KT>
static hipError_t attrs_ng(int lds) {
    hipError_t e = hipSuccess;
    auto one = [&](const void* fn) {
        if (e == hipSuccess) e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, lds);
    };
    one(reinterpret_cast<const void*>(k_mm<KIND, 1, KT>));
    one(reinterpret_cast<const void*>(k_mm<KIND, 2, KT>));
    one(reinterpret_cast<const void*>(k_mm<KIND, 3, KT>));
    one(reinterpret_cast<const void*>(k_mm<KIND, 4, KT>));
    return e;
}

template <int KIND>
static hipError_t attrs_kind(int lds) {
    hipError_t e = attrs_ng<KIND, 256>(lds);
    if (e == hipSuccess) e = attrs_ng<KIND, 192>(lds);
    if (e == hipSuccess) e = attrs_ng<KIND, 128>(lds);
    if (e == hipSuccess) e = attrs_ng<KIND, 64>(lds);
    return e;
}

size_t mm_max_lds(const StepArgs& s) {
    size_t m = 0;
    const int Ks[3] = {s.d, s.H * s.D, s.F};
    for (int K : Ks) m = std::max(m, mm_lds(pick_kt(K), K == s.d, K));
    if (s.D == 64 || s.D == 128) m = std::max(m, attn_pf_lds(s.D, kF32, 4));  // the batched prefill's attention
    return m;
}

hipError_t mm_set_attributes(int lds) {
    hipError_t e = attrs_kind<MM_QKV>(lds);
    if (e == hipSuccess) e = attrs_kind<MM_WO>(lds);
    if (e == hipSuccess) e = attrs_kind<MM_W13>(lds);
    if (e == hipSuccess) e = attrs_kind<MM_W2>(lds);
    if (e == hipSuccess) e = attrs_kind<MM_LOGITS>(lds);
    if (e == hipSuccess) e = attrs_pf<64, kF32>(lds);
    if (e == hipSuccess) e = attrs_pf<64, kBF16>(lds);
    if (e == hipSuccess) e = attrs_pf<128, kF32>(lds);
    if (e == hipSuccess) e = attrs_pf<128, kBF16>(lds);
    return e;
}

// ---- split-K launch -----------------------------------------------------------------------------
template <int KIND>
static void sk_dims(const StepArgs& s, int& K, int& N) {
    K = s.d;
    N = 0;
    if (KIND == MM_QKV) N = (s.H + 2 * s.Hkv) * s.D;
    if (KIND == MM_WO) { N = s.d; K = s.H * s.D; }
    if (KIND == MM_W13) N = s.F;
    if (KIND == MM_W2) { N = s.d; K = s.F; }
}

template <int KIND, int MAXS, bool LOOP = false, int NW = 4, int RT = 1>
static void launch_sk_one(const StepArgs& s, const LayerW& w, int layer, int n, int ident, int n_tiles, hipStream_t st) {
    const int n_groups = (n + 15) / 16;
    const int n_tg = (n_tiles + RT - 1) / RT;  // groups of RT row tiles
    const dim3 grid(((n_tg + 7) / 8) * 8 * n_groups);
    hipLaunchKernelGGL((k_mm_sk<KIND, MAXS, LOOP, NW, RT>), grid, dim3(64 * NW), 0, st, s, w, layer, n, ident, n_tiles,
                       n_groups);
}

// Rows of up to 8 k-steps per wave (5 for the kinds with gains, registers)
// take 8-wave blocks (W1/W3 and W2 of up to 48 k-steps: 16-wave blocks) with
// every load issued at once.  Longer rows take 4-wave blocks that loop over
// batches of kLoopMaxs k-steps, each wave multiplying every activation
// operand it loads by kLoopRt row tiles, so the activations are read from L2
// once per 64 weight rows instead of once per 16 (the 8B 4096-token batched
// prefill: 979 -> 749 ms; 2 or 8 tiles, and batches of 1 to 4 k-steps,
// measured slower) -- except W1/W3, whose tiled kernel reads each weight once
// for all 64 items.  false: the tiled kernel runs instead.
constexpr int kLoopRt = 4, kLoopMaxs = 2;

// The device's compute units (cached per device; 256 if the query fails).
static int cu_count() {
    static std::atomic<int> cached[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
    int v = cached[dev].load(std::memory_order_relaxed);
    if (v == 0) {
        if (hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || v <= 0) v = 256;
        cached[dev].store(v, std::memory_order_relaxed);
    }
    return v;
}

// Blocks of a long-row launch with rt row tiles per wave (launch_sk_one's grid).
static int loop_blocks(int nt, int n, int rt) { return ((nt + rt - 1) / rt + 7) / 8 * 8 * ((n + 15) / 16); }

// The long-row loop takes 6 row tiles per wave instead of kLoopRt when that
// leaves fewer rounds of blocks over the CUs times tiles per block (a
// block's time grows with its tiles): at the 8B shape, Q/K/V's 384 tiles at
// 64 items make 384 blocks with 4 (two rounds on 256 CUs) and 256 with 6
// (one), 692.7 -> 660.2 ms per 4096-token batched prefill (3 tiles, 512
// blocks: 675.5 ms); W2 and Wo, 256 tiles, keep 4.
static bool loop_six(int nt, int n) {
    const int cus = cu_count();
    const int r4 = (loop_blocks(nt, n, kLoopRt) + cus - 1) / cus, r6 = (loop_blocks(nt, n, 6) + cus - 1) / cus;
    return r6 * 6 < r4 * kLoopRt;
}
template <int KIND>
static bool launch_sk(const StepArgs& s, const LayerW& w, int layer, int n, int ident, hipStream_t st) {
    int K = 0, N = 0;
    sk_dims<KIND>(s, K, N);
    const int nt = N / 16;
    // W1/W3 and W2 take 16-wave blocks while a wave then has at most three
    // k-steps: twice the waves in flight and half the chain per wave (B = 64,
    // 135M: W2 launches only 160 blocks).  Measured 0.3% and 0.4% faster per
    // step each; Q/K/V and Wo were 0.7% slower that way.
    if constexpr (KIND == MM_W13 || KIND == MM_W2) {
        const int per16 = (K / 32 + 15) / 16;
        if (per16 <= 2) {
            launch_sk_one<KIND, 2, false, 16>(s, w, layer, n, ident, nt, st);
            return true;
        }
        if (per16 <= 3) {
            launch_sk_one<KIND, 3, false, 16>(s, w, layer, n, ident, nt, st);
            return true;
        }
    }
    const int per8 = (K / 32 + 7) / 8;
    constexpr int cap8 = (KIND == MM_QKV || KIND == MM_W13) ? 5 : 8;
    if (per8 <= cap8) {
        if (per8 <= 1) launch_sk_one<KIND, 1, false, 8>(s, w, layer, n, ident, nt, st);
        else if (per8 <= 2) launch_sk_one<KIND, 2, false, 8>(s, w, layer, n, ident, nt, st);
        else if (per8 <= 3) launch_sk_one<KIND, 3, false, 8>(s, w, layer, n, ident, nt, st);
        else if (per8 <= 5) launch_sk_one<KIND, 5, false, 8>(s, w, layer, n, ident, nt, st);
        else if constexpr (cap8 == 8) launch_sk_one<KIND, 8, false, 8>(s, w, layer, n, ident, nt, st);
        return true;
    }
    if constexpr (KIND == MM_W13) {
        return false;
    } else {
        if (loop_six(nt, n))
            launch_sk_one<KIND, kLoopMaxs, true, 4, 6>(s, w, layer, n, ident, nt, st);
        else
            launch_sk_one<KIND, kLoopMaxs, true, 4, kLoopRt>(s, w, layer, n, ident, nt, st);
        return true;
    }
}

// which: 0 qkv, 1 wo, 2 w13, 3 w2, 4 logits; items [0, n_items).  The narrow
// projections take the split-K kernel over every item in one launch when
// their K fits its registers; the rest run the tiled kernel in launches of
// kMmItems items.
hipError_t mm_gemv(int which, const StepArgs& s, const LayerW& w, int layer, int n_items, int ident,
                   const float* out_norm, const void* wcls, hipStream_t st) {
    if (n_items > 0 && s.mm_split) {
        bool done = false;
        switch (which) {
            case 0: done = launch_sk<MM_QKV>(s, w, layer, n_items, ident, st); break;
            case 1: done = launch_sk<MM_WO>(s, w, layer, n_items, ident, st); break;
            case 2: done = launch_sk<MM_W13>(s, w, layer, n_items, ident, st); break;
            case 3: done = launch_sk<MM_W2>(s, w, layer, n_items, ident, st); break;
            default: break;
        }
        if (done) return hipGetLastError();
    }
    hipError_t e = hipSuccess;
    for (int m0 = 0; m0 < n_items && e == hipSuccess; m0 += kMmItems) {
        const int n = n_items - m0 < kMmItems ? n_items - m0 : kMmItems;
        switch (which) {
            case 0: e = launch_kind<MM_QKV>(s, w, layer, m0, n, ident, out_norm, wcls, st); break;
            case 1: e = launch_kind<MM_WO>(s, w, layer, m0, n, ident, out_norm, wcls, st); break;
            case 2: e = launch_kind<MM_W13>(s, w, layer, m0, n, ident, out_norm, wcls, st); break;
            case 3: e = launch_kind<MM_W2>(s, w, layer, m0, n, ident, out_norm, wcls, st); break;
            default: e = launch_kind<MM_LOGITS>(s, w, layer, m0, n, ident, out_norm, wcls, st); break;
        }
    }
    return e;
}

}  // namespace ds
