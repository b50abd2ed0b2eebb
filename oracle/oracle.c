/*
 * oracle.c -- reference decoder for the single-token Llama decode step.
 *
 * TEST INFRASTRUCTURE ONLY: a plain, slow, single-threaded CPU definition of
 * what the decode step computes.  The HIP library is checked against it; it
 * never serves the product path.  Built with
 *     gcc -O2 -std=c11 -ffp-contract=off -fno-fast-math
 * so every floating-point operation below is one IEEE binary32 operation in
 * the order written (no fused multiply-add, no reassociation).
 *
 * Sources (the web pages this decoder is written from):
 *   [GOT]  "GOTOken: An Inference Engine in QBasic"
 *   [NANO] "Inside nanochat Part 4: Understanding Inference"
 *   [KAS]  "simple-llm / kasahare" (PyPI README, 0.4.0)
 */
#include "oracle.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>

/* [GOT] "Loading the model and tokenizer": bf16 keeps the top 16 bits of an
 * fp32 value, so widening is a 16-bit left shift of the bit pattern. */
float orc_widen_bf16(uint16_t h) {
    uint32_t bits = (uint32_t)h << 16;
    float f;
    memcpy(&f, &bits, sizeof f);
    return f;
}

/* Round to nearest bfloat16, ties to even: keep the top 16 bits after adding
 * half of the dropped range, less one unless the kept part is odd. */
float orc_round_bf16(float x) {
    uint32_t u;
    memcpy(&u, &x, sizeof u);
    uint32_t lsb = (u >> 16) & 1u;
    u = (u + 0x7FFFu + lsb) & 0xFFFF0000u;
    float f;
    memcpy(&f, &u, sizeof f);
    return f;
}

void orc_widen_bf16_array(const uint16_t* src, float* dst, size_t n) {
    for (size_t i = 0; i < n; i++) dst[i] = orc_widen_bf16(src[i]);
}

/* Element (r, c) of a [rows][cols] matrix.  ORC_Q8 (see oracle.h): the int8
 * value times its block's fp32 scale, one rounding; the scales start at the
 * first 256-byte boundary after the rows*cols int8 values. */
float orc_weight(const void* W, int32_t wdtype, size_t rows, size_t cols, size_t r, size_t c) {
    size_t idx = r * cols + c;
    if (wdtype == ORC_BF16) return orc_widen_bf16(((const uint16_t*)W)[idx]);
    if (wdtype == ORC_Q8) {
        const int8_t* q = (const int8_t*)W;
        size_t sbase = (rows * cols + 255u) / 256u * 256u;
        const float* sc = (const float*)((const uint8_t*)W + sbase);
        float s = sc[r * (cols / 32u) + c / 32u];
        return s * (float)q[idx];
    }
    if (wdtype == ORC_Q4) {
        const uint8_t* b = (const uint8_t*)W;
        int nib = (idx & 1u) ? (b[idx / 2u] >> 4) : (b[idx / 2u] & 15);
        int q = nib >= 8 ? nib - 16 : nib;
        size_t sbase = (rows * cols / 2u + 255u) / 256u * 256u;
        const float* sc = (const float*)(b + sbase);
        float s = sc[r * (cols / 32u) + c / 32u];
        return s * (float)q;
    }
    return ((const float*)W)[idx];
}

/* [GOT] "About one token per second", the MatMul routine: W is row-major
 * [n_out][n_in]; for every output row the accumulator starts at zero and
 * adds W[i][j]*x[j] for j ascending.  "Building it one piece at a time":
 * this sequential fp32 order (no fused multiply-add) is the one the page's
 * replay matched bit for bit. */
void orc_matvec(const void* W, int32_t wdtype, int32_t n_out, int32_t n_in, const float* x,
                float* y) {
    for (int32_t i = 0; i < n_out; i++) {
        float acc = 0.0f;
        for (int32_t j = 0; j < n_in; j++) {
            float prod = orc_weight(W, wdtype, (size_t)n_out, (size_t)n_in, (size_t)i, (size_t)j) * x[j];
            acc = acc + prod;
        }
        y[i] = acc;
    }
}

/* [KAS] "Architecture": attn_norm / ffn_norm are RMSNorm (named only).
 * Plainest reading: y = g * (x / sqrt(mean(x^2) + eps)), evaluated as
 * ss = sum x_j*x_j (j ascending); ss /= n; ss += eps; r = 1/sqrtf(ss);
 * y_j = g_j * (r * x_j). */
void orc_rmsnorm(const float* x, const float* g, int32_t n, float eps, float* y) {
    float ss = 0.0f;
    for (int32_t j = 0; j < n; j++) {
        float sq = x[j] * x[j];
        ss = ss + sq;
    }
    ss = ss / (float)n;
    ss = ss + eps;
    float r = 1.0f / sqrtf(ss);
    for (int32_t j = 0; j < n; j++) {
        float t = r * x[j];
        y[j] = g[j] * t;
    }
}

/* [GOT] "Loading the model and tokenizer": the rotation pairs element j with
 * element j + head_dim/2 of a head.  The frequency of pair i is
 * theta^(-2i/head_dim) (the page names only the pairing; this is the
 * convention of the library the page matches).  Angle, cos and sin in
 * binary64, rounded once to binary32. */
void orc_rope_angles(int32_t pos, int32_t head_dim, float theta, float* c, float* s) {
    for (int32_t i = 0; i < head_dim / 2; i++) {
        double inv_freq = pow((double)theta, -(double)(2 * i) / (double)head_dim);
        double ang = (double)pos * inv_freq;
        c[i] = (float)cos(ang);
        s[i] = (float)sin(ang);
    }
}

/* Rotate each pair (a, b) = (v[i], v[i+D/2]) by the pair's angle:
 * (a*c - b*s, a*s + b*c). */
void orc_rope_apply(float* v, int32_t head_dim, const float* c, const float* s) {
    int32_t half = head_dim / 2;
    for (int32_t i = 0; i < half; i++) {
        float a = v[i], b = v[i + half];
        float ac = a * c[i], bs = b * s[i];
        float as = a * s[i], bc = b * c[i];
        v[i] = ac - bs;
        v[i + half] = as + bc;
    }
}

/* [KAS] "Architecture": attn = softmax(q . K^T / sqrt(d_head)) . V over the
 * n cached positions (the new one included).  Each score is a sequential
 * dot product divided by sqrtf(D); the softmax subtracts the maximum score
 * (mathematically the same softmax), exponentiates in binary64 and rounds
 * once, sums sequentially and divides; the output is the t-ascending sum of
 * p_t * V[t].  K and V are [n][D] row-major.  probs (n floats) is scratch
 * that holds the normalised weights on return. */
void orc_attend(const float* q, const float* K, const float* V, int32_t n, int32_t head_dim,
                float* probs, float* out) {
    float scale = sqrtf((float)head_dim);
    for (int32_t t = 0; t < n; t++) {
        float dot = 0.0f;
        for (int32_t e = 0; e < head_dim; e++) {
            float prod = q[e] * K[(size_t)t * head_dim + e];
            dot = dot + prod;
        }
        probs[t] = dot / scale;
    }
    float m = probs[0];
    for (int32_t t = 1; t < n; t++)
        if (probs[t] > m) m = probs[t];
    float sum = 0.0f;
    for (int32_t t = 0; t < n; t++) {
        float z = probs[t] - m;
        float ez = (float)exp((double)z);
        probs[t] = ez;
        sum = sum + ez;
    }
    for (int32_t t = 0; t < n; t++) probs[t] = probs[t] / sum;
    for (int32_t e = 0; e < head_dim; e++) {
        float acc = 0.0f;
        for (int32_t t = 0; t < n; t++) {
            float prod = probs[t] * V[(size_t)t * head_dim + e];
            acc = acc + prod;
        }
        out[e] = acc;
    }
}

/* [KAS] "Architecture": silu(W1 x) * (W3 x).  silu(a) = a * sigmoid(a) with
 * sigmoid(a) = 1 / (1 + exp(-a)); exp in binary64 rounded once. */
float orc_silu_mul(float a, float u) {
    float e = (float)exp(-(double)a);
    float den = 1.0f + e;
    float sig = 1.0f / den;
    float sa = a * sig;
    return sa * u;
}

/* [NANO] "Sampling Strategy": greedy decoding is argmax over the logits;
 * among equal maxima the lowest index wins (a strict '>' scan from 0). */
int32_t orc_argmax(const float* v, int32_t n) {
    int32_t best = 0;
    for (int32_t i = 1; i < n; i++)
        if (v[i] > v[best]) best = i;
    return best;
}

/* [NANO] "Sampling Strategy" ("Temperature Sampling", "Top-K Filtering",
 * "Combined Temperature and Top-K") and [KAS] "CLI flags" (--top-p):
 * one draw from the logits.
 *  - temperature == 0: the greedy token (orc_argmax); *n_out = 1.
 *  - top_k >= 1: the candidates are the min(top_k, V) largest logits, in
 *    the order largest first (equal logits: lower index first).  Each gets
 *    the weight exp((l_j - l_0) / temperature) (binary64; l_0 is the
 *    largest, so the softmax is unchanged).  top_p < 1 keeps the shortest
 *    prefix whose weight sum reaches top_p times the sum of all candidate
 *    weights (the nucleus reading of --top-p, applied after top-k).
 *  - top_k == 0: every token, in index order, with those weights; top_p
 *    must be 1.
 * The draw is the inverse distribution function at u in [0, 1): the first
 * kept candidate j whose cumulative weight exceeds u times the kept total
 * (the last kept candidate if rounding leaves none).  cand[] gets the
 * candidates in draw order and cum[] their cumulative weights divided by
 * the kept total (both of length *n_out, the kept count).  Returns the
 * token, or -1 on a bad argument. */
static int cmp_desc(const void* a, const void* b) {
    const float* x = (const float*)a;
    const float* y = (const float*)b;
    if (x[0] > y[0]) return -1;
    if (x[0] < y[0]) return 1;
    return x[1] < y[1] ? -1 : (x[1] > y[1] ? 1 : 0);  /* lower index first */
}

int32_t orc_sample(const float* logits, int32_t V, float temperature, int32_t top_k, float top_p,
                   double u, int32_t* cand, double* cum, int32_t* n_out) {
    if (V <= 0 || !(temperature >= 0.0f) || top_k < 0 || !(top_p > 0.0f && top_p <= 1.0f) ||
        !(u >= 0.0 && u < 1.0) || (top_k == 0 && top_p < 1.0f))
        return -1;
    if (temperature == 0.0f) {
        cand[0] = orc_argmax(logits, V);
        cum[0] = 1.0;
        *n_out = 1;
        return cand[0];
    }
    int32_t n = V;
    if (top_k >= 1) {
        /* (value, index) pairs sorted; indices below 2^24 are exact as float */
        float* pr = (float*)malloc(sizeof(float) * 2 * (size_t)V);
        if (!pr) return -1;
        for (int32_t i = 0; i < V; i++) {
            pr[2 * i] = logits[i];
            pr[2 * i + 1] = (float)i;
        }
        qsort(pr, (size_t)V, 2 * sizeof(float), cmp_desc);
        n = top_k < V ? top_k : V;
        for (int32_t j = 0; j < n; j++) cand[j] = (int32_t)pr[2 * j + 1];
        free(pr);
    } else {
        for (int32_t j = 0; j < V; j++) cand[j] = j;
    }
    double lmax = logits[cand[0]];
    if (top_k == 0)
        for (int32_t j = 1; j < n; j++)
            if (logits[j] > lmax) lmax = logits[j];
    double tot = 0.0;
    for (int32_t j = 0; j < n; j++) {
        tot += exp(((double)logits[cand[j]] - lmax) / (double)temperature);
        cum[j] = tot;
    }
    int32_t kept = n;
    if (top_p < 1.0f) {
        kept = 1;
        while (kept < n && cum[kept - 1] < (double)top_p * tot) kept++;
    }
    const double total = cum[kept - 1];
    int32_t pick = kept - 1;
    for (int32_t j = 0; j < kept; j++)
        if (cum[j] > u * total) {
            pick = j;
            break;
        }
    for (int32_t j = 0; j < kept; j++) cum[j] /= total;
    *n_out = kept;
    return cand[pick];
}

/* ---- arena layout: [KAS] "On-disk model format (.sllm)" order ----------- */
enum { ORC_ALIGN = 256 };
enum { T_ATTN_NORM = 0, T_WQ, T_WK, T_WV, T_WO, T_FFN_NORM, T_W1, T_W3, T_W2, T_PER_LAYER };

int32_t orc_n_tensors(const orc_config* c) {
    return 1 + T_PER_LAYER * c->n_layers + 1 + (c->tied_embeddings ? 0 : 1);
}

static size_t mat_bytes(const orc_config* c, size_t rows, size_t cols) {
    if (c->weight_dtype == ORC_Q8) return (rows * cols + 255u) / 256u * 256u + rows * (cols / 32u) * 4u;
    if (c->weight_dtype == ORC_Q4) return (rows * cols / 2u + 255u) / 256u * 256u + rows * (cols / 32u) * 4u;
    return rows * cols * (c->weight_dtype == ORC_BF16 ? 2u : 4u);
}

/* Offsets of every tensor in the canonical arena, each rounded up to a
 * 256-byte boundary; returns the arena size. */
size_t orc_tensor_offsets(const orc_config* c, size_t* off, int32_t n) {
    size_t d = (size_t)c->dim, F = (size_t)c->hidden_dim, V = (size_t)c->vocab_size;
    size_t qr = (size_t)c->n_heads * c->head_dim, kvr = (size_t)c->n_kv_heads * c->head_dim;
    size_t pos = 0;
    int32_t k = 0;
#define PLACE(bytes)                                              \
    do {                                                          \
        if (k < n) off[k] = pos;                                  \
        k++;                                                      \
        pos = (pos + (bytes) + ORC_ALIGN - 1) / ORC_ALIGN * ORC_ALIGN; \
    } while (0)
    PLACE(mat_bytes(c, V, d));
    for (int32_t l = 0; l < c->n_layers; l++) {
        PLACE(d * 4);
        PLACE(mat_bytes(c, qr, d));
        PLACE(mat_bytes(c, kvr, d));
        PLACE(mat_bytes(c, kvr, d));
        PLACE(mat_bytes(c, d, qr));
        PLACE(d * 4);
        PLACE(mat_bytes(c, F, d));
        PLACE(mat_bytes(c, F, d));
        PLACE(mat_bytes(c, d, F));
    }
    PLACE(d * 4);
    if (!c->tied_embeddings) PLACE(mat_bytes(c, V, d));
#undef PLACE
    return pos;
}

/* [NANO] "Cache Architecture": the cache is one (L, 2, B, H, T, D) tensor,
 * where H counts key/value heads; index of element 0 of row t. */
size_t orc_cache_index(const orc_config* c, int32_t B, int32_t T, int32_t layer, int32_t kv,
                       int32_t b, int32_t g, int32_t t) {
    size_t i = (size_t)layer;
    i = i * 2 + (size_t)kv;
    i = i * (size_t)B + (size_t)b;
    i = i * (size_t)c->n_kv_heads + (size_t)g;
    i = i * (size_t)T + (size_t)t;
    return i * (size_t)c->head_dim;
}

/* ---- one position ------------------------------------------------------ */
/* [KAS] "Architecture", read as the pre-norm LLaMA-2 block:
 *   xn = attn_norm(x); q,k,v = Wq xn, Wk xn, Wv xn; RoPE(q, k, pos);
 *   o = softmax(q K^T / sqrt(D)) V per head; x = x + Wo o;
 *   xn = ffn_norm(x); x = x + W2(silu(W1 xn) * (W3 xn)).
 * (The page's listing assigns the normed value back to x_n; its "# residual"
 * comments and the LLaMA-2 label fix the pre-norm reading used here.)
 * The k and v rows of this position are stored at [l][0|1][b][g][pos]
 * ([NANO] "Dynamic Memory Allocation", insert_kv) before attention reads
 * positions 0..pos.  Query head h uses key/value head h / (H / Hkv) (grouped
 * query attention, [KAS] "Architecture").  The final norm is followed by the
 * vocabulary product with the tied embedding ([KAS] "Architecture"), or with
 * the separate head when the embeddings are not tied. */
int32_t orc_forward(const orc_config* c, const uint8_t* arena, float* cache, int32_t B,
                    int32_t T, int32_t b, int32_t pos, int32_t token, float* logits) {
    const int32_t d = c->dim, H = c->n_heads, Hkv = c->n_kv_heads, D = c->head_dim;
    const int32_t F = c->hidden_dim, V = c->vocab_size, wd = c->weight_dtype;
    if (token < 0 || token >= V || pos < 0 || pos >= T || b < 0 || b >= B) return -1;
    if (H % Hkv != 0 || D % 2 != 0) return -2;
    const int32_t group = H / Hkv;
    int32_t nt = orc_n_tensors(c);
    size_t* off = (size_t*)malloc(sizeof(size_t) * (size_t)nt);
    orc_tensor_offsets(c, off, nt);

    float* x = (float*)malloc(sizeof(float) * (size_t)d);
    float* xn = (float*)malloc(sizeof(float) * (size_t)d);
    float* tmp = (float*)malloc(sizeof(float) * (size_t)d);
    float* q = (float*)malloc(sizeof(float) * (size_t)H * D);
    float* k = (float*)malloc(sizeof(float) * (size_t)Hkv * D);
    float* v = (float*)malloc(sizeof(float) * (size_t)Hkv * D);
    float* o = (float*)malloc(sizeof(float) * (size_t)H * D);
    float* a = (float*)malloc(sizeof(float) * (size_t)F);
    float* u = (float*)malloc(sizeof(float) * (size_t)F);
    float* hb = (float*)malloc(sizeof(float) * (size_t)F);
    float* probs = (float*)malloc(sizeof(float) * (size_t)(pos + 1));
    float* cs = (float*)malloc(sizeof(float) * (size_t)(D / 2));
    float* sn = (float*)malloc(sizeof(float) * (size_t)(D / 2));

    /* embedding row, widened ([GOT] "Loading the model and tokenizer") */
    const void* emb = arena + off[0];
    for (int32_t j = 0; j < d; j++) x[j] = orc_weight(emb, wd, (size_t)V, (size_t)d, (size_t)token, (size_t)j);

    orc_rope_angles(pos, D, c->rope_theta, cs, sn);
    for (int32_t l = 0; l < c->n_layers; l++) {
        const size_t* lo = off + 1 + (size_t)l * T_PER_LAYER;
        orc_rmsnorm(x, (const float*)(arena + lo[T_ATTN_NORM]), d, c->norm_eps, xn);
        orc_matvec(arena + lo[T_WQ], wd, H * D, d, xn, q);
        orc_matvec(arena + lo[T_WK], wd, Hkv * D, d, xn, k);
        orc_matvec(arena + lo[T_WV], wd, Hkv * D, d, xn, v);
        for (int32_t h = 0; h < H; h++) orc_rope_apply(q + (size_t)h * D, D, cs, sn);
        for (int32_t g = 0; g < Hkv; g++) orc_rope_apply(k + (size_t)g * D, D, cs, sn);
        if (c->cache_dtype == ORC_BF16) {
            for (int32_t i = 0; i < Hkv * D; i++) {
                k[i] = orc_round_bf16(k[i]);
                v[i] = orc_round_bf16(v[i]);
            }
        }
        for (int32_t g = 0; g < Hkv; g++) {
            memcpy(cache + orc_cache_index(c, B, T, l, 0, b, g, pos), k + (size_t)g * D,
                   sizeof(float) * (size_t)D);
            memcpy(cache + orc_cache_index(c, B, T, l, 1, b, g, pos), v + (size_t)g * D,
                   sizeof(float) * (size_t)D);
        }
        for (int32_t h = 0; h < H; h++) {
            int32_t g = h / group;
            orc_attend(q + (size_t)h * D, cache + orc_cache_index(c, B, T, l, 0, b, g, 0),
                       cache + orc_cache_index(c, B, T, l, 1, b, g, 0), pos + 1, D, probs,
                       o + (size_t)h * D);
        }
        orc_matvec(arena + lo[T_WO], wd, d, H * D, o, tmp);
        for (int32_t j = 0; j < d; j++) x[j] = x[j] + tmp[j];
        orc_rmsnorm(x, (const float*)(arena + lo[T_FFN_NORM]), d, c->norm_eps, xn);
        orc_matvec(arena + lo[T_W1], wd, F, d, xn, a);
        orc_matvec(arena + lo[T_W3], wd, F, d, xn, u);
        for (int32_t i = 0; i < F; i++) hb[i] = orc_silu_mul(a[i], u[i]);
        orc_matvec(arena + lo[T_W2], wd, d, F, hb, tmp);
        for (int32_t j = 0; j < d; j++) x[j] = x[j] + tmp[j];
    }
    size_t out_norm = off[1 + (size_t)c->n_layers * T_PER_LAYER];
    orc_rmsnorm(x, (const float*)(arena + out_norm), d, c->norm_eps, xn);
    const void* wcls = c->tied_embeddings ? (const void*)(arena + off[0])
                                          : (const void*)(arena + off[nt - 1]);
    orc_matvec(wcls, wd, V, d, xn, logits);
    int32_t tok = orc_argmax(logits, V);

    free(off); free(x); free(xn); free(tmp); free(q); free(k); free(v); free(o);
    free(a); free(u); free(hb); free(probs); free(cs); free(sn);
    return tok;
}

int32_t orc_decode_step(const orc_config* c, const uint8_t* arena, float* cache, int32_t B,
                        int32_t T, int32_t* lengths, const int32_t* tok_in, int32_t* tok_out,
                        float* logits) {
    for (int32_t b = 0; b < B; b++) {
        int32_t r = orc_forward(c, arena, cache, B, T, b, lengths[b], tok_in[b],
                                logits + (size_t)b * c->vocab_size);
        if (r < 0) return r;
        tok_out[b] = r;
        lengths[b] += 1;
    }
    return 0;
}

static void clear_slot(const orc_config* c, float* cache, int32_t B, int32_t T, int32_t b) {
    for (int32_t l = 0; l < c->n_layers; l++)
        for (int32_t kv = 0; kv < 2; kv++)
            for (int32_t g = 0; g < c->n_kv_heads; g++)
                memset(cache + orc_cache_index(c, B, T, l, kv, b, g, 0), 0,
                       sizeof(float) * (size_t)T * c->head_dim);
}

/* [GOT] "About one token per second": with the cache, the prompt is run once
 * and then one position per new token; without it, every new token reruns
 * the prompt and all tokens generated so far.  Either way new token k is the
 * argmax at the last position of a causal forward over prompt + tokens 0..k-1;
 * the last generated token is never fed back. */
int32_t orc_generate(const orc_config* c, const uint8_t* arena, float* cache, int32_t B,
                     int32_t T, int32_t b, const int32_t* prompt, int32_t n_prompt,
                     int32_t n_new, int32_t mode, int32_t* out_tokens, float* out_logits,
                     int64_t* passes) {
    const int32_t V = c->vocab_size;
    if (n_prompt < 1 || n_new < 1 || n_prompt + n_new - 1 > T) return -1;
    float* lg = (float*)malloc(sizeof(float) * (size_t)V);
    int32_t* seq = (int32_t*)malloc(sizeof(int32_t) * (size_t)(n_prompt + n_new));
    memcpy(seq, prompt, sizeof(int32_t) * (size_t)n_prompt);
    int64_t count = 0;
    int32_t r = 0;
    if (mode == 0) {
        clear_slot(c, cache, B, T, b);
        for (int32_t t = 0; t < n_prompt + n_new - 1 && r >= 0; t++) {
            r = orc_forward(c, arena, cache, B, T, b, t, seq[t], lg);
            count++;
            if (r >= 0 && t >= n_prompt - 1) {
                int32_t k = t - (n_prompt - 1);
                out_tokens[k] = r;
                seq[t + 1] = r;
                if (out_logits) memcpy(out_logits + (size_t)k * V, lg, sizeof(float) * (size_t)V);
            }
        }
    } else {
        for (int32_t k = 0; k < n_new && r >= 0; k++) {
            clear_slot(c, cache, B, T, b);
            for (int32_t t = 0; t < n_prompt + k && r >= 0; t++) {
                r = orc_forward(c, arena, cache, B, T, b, t, seq[t], lg);
                count++;
            }
            if (r >= 0) {
                out_tokens[k] = r;
                seq[n_prompt + k] = r;
                if (out_logits) memcpy(out_logits + (size_t)k * V, lg, sizeof(float) * (size_t)V);
            }
        }
    }
    if (passes) *passes = count;
    free(lg);
    free(seq);
    return r < 0 ? r : 0;
}
