/*
 * batch.c -- the reference decoder evaluated for many positions at once.
 *
 * TEST INFRASTRUCTURE ONLY, like oracle.c.  orc_forward_items computes, for
 * a list of items (sequence b, position p, token), exactly what orc_forward
 * computes for each of them, bit for bit: every fp32 scalar goes through the
 * same operations in the same order (one binary32 rounding each, no fused
 * multiply-add: built with -ffp-contract=off, and no reassociation).  What
 * changes is only which independent scalars are computed side by side:
 *
 *   - the items advance layer by layer together, so a weight row is read
 *     once for all of them ([NANO] "Attention Mechanism Integration": a
 *     prompt's positions go through the model as one batch, each position
 *     attending only to the positions before it);
 *   - a matrix-vector product computes several output rows and several items
 *     in vector lanes, each lane its own sequential sum over the inputs in
 *     ascending order, as in orc_matvec;
 *   - attention scores several cached positions and output dims at a time,
 *     each score and each output dim its own sequential sum, as in
 *     orc_attend;
 *   - independent rows, items and heads are spread over host threads.
 *
 * The tests assert bit-identity with orc_forward (logits and cache) on the
 * tiny and 135M shapes in every weight and cache format.  The goldens of the
 * full-size workloads are written with this mode.
 *
 * Sources: as oracle.c -- [GOT] "GOTOken: An Inference Engine in QBasic",
 * [NANO] "Inside nanochat Part 4: Understanding Inference", [KAS]
 * "simple-llm / kasahare".
 */
#include "oracle.h"

#include <math.h>
#include <pthread.h>
#include <stdlib.h>
#include <string.h>

typedef float v16 __attribute__((vector_size(64)));

/* The vector width only decides how many independent sums run side by side;
 * each lane's operations and their order are the same in every clone. */
#define HOT __attribute__((target_clones("avx512f", "avx2", "default")))

/* ---- a parallel loop over tasks ---------------------------------------- */
typedef void (*task_fn)(void* ctx, int64_t task, int tid);

typedef struct {
    task_fn fn;
    void* ctx;
    int64_t n;
    int64_t next;
    int tid;
} pool_job;

typedef struct {
    pool_job* job;
    int tid;
} pool_arg;

static void* pool_worker(void* p) {
    pool_arg* a = (pool_arg*)p;
    for (;;) {
        int64_t t = __atomic_fetch_add(&a->job->next, 1, __ATOMIC_RELAXED);
        if (t >= a->job->n) break;
        a->job->fn(a->job->ctx, t, a->tid);
    }
    return NULL;
}

static void par_for(int64_t n, task_fn fn, void* ctx, int nthreads) {
    if (n <= 0) return;
    if (nthreads > n) nthreads = (int)n;
    pool_job job = {fn, ctx, n, 0, 0};
    if (nthreads <= 1) {
        for (int64_t t = 0; t < n; t++) fn(ctx, t, 0);
        return;
    }
    pthread_t th[256];
    pool_arg args[256];
    if (nthreads > 256) nthreads = 256;
    for (int i = 0; i < nthreads; i++) {
        args[i].job = &job;
        args[i].tid = i;
    }
    int started = 0;
    for (int i = 1; i < nthreads; i++) {
        if (pthread_create(&th[i], NULL, pool_worker, &args[i]) != 0) break;
        started = i;
    }
    pool_worker(&args[0]);
    for (int i = 1; i <= started; i++) pthread_join(th[i], NULL);
}

/* ---- weights as fp32, exactly as orc_weight gives them ------------------ */
/* Row r, columns [c0, c0 + n) of a [rows][cols] matrix into dst. */
static void weight_run(const void* W, int32_t wd, size_t rows, size_t cols, size_t r, size_t c0,
                       size_t n, float* dst) {
    if (wd == ORC_BF16) {
        const uint16_t* p = (const uint16_t*)W + r * cols + c0;
        for (size_t k = 0; k < n; k++) dst[k] = orc_widen_bf16(p[k]);
    } else if (wd == ORC_F32) {
        memcpy(dst, (const float*)W + r * cols + c0, n * sizeof(float));
    } else {
        for (size_t k = 0; k < n; k++) dst[k] = orc_weight(W, wd, rows, cols, r, c0 + k);
    }
}

/* ---- Y[m][i] = sum_j W[i][j] * X[m][j], per scalar as orc_matvec -------- */
enum { KB = 256,      /* columns converted per block */
       RA = 8,        /* rows per task, items in lanes (kernel A) */
       PA = 32,       /* items per register tile (two vectors) */
       IC = 256,      /* items per task (kernel A) */
       RB = 16 };     /* rows in lanes per task (kernel B) */

typedef struct {
    const void* W;
    int32_t wd, rows, cols, M;
    const float* X;   /* [M][cols] */
    float* XT;        /* [cols][Mp] (kernel A) */
    int32_t Mp;
    float* Y;         /* [M][ldy] */
    int32_t ldy;
    float* scratch;   /* per thread: KB * RB floats of weights + RA * IC partial sums */
} mm_ctx;

enum { MM_SCRATCH = KB * RB + RA * IC };

/* Kernel A: RA rows x up to IC items.  The running sum of row r and item m
 * is lane l of vector v of tile s (m = m0 + 32s + 16v + l); between column
 * blocks it waits in `part` (a store and a load of the same float). */
HOT static void mm_task_items(void* vctx, int64_t task, int tid) {
    mm_ctx* c = (mm_ctx*)vctx;
    int32_t ngroups = (c->rows + RA - 1) / RA;
    int32_t r0 = (int32_t)(task % ngroups) * RA;
    int32_t m0 = (int32_t)(task / ngroups) * IC;
    int32_t ntile = (c->Mp - m0 < IC ? c->Mp - m0 : IC) / PA;
    float* wf = c->scratch + (size_t)tid * MM_SCRATCH;
    v16* part = (v16*)(wf + KB * RB);   /* [ntile][RA][2] */
    for (int32_t k = 0; k < ntile * RA * 2; k++) part[k] = (v16){0};
    for (int32_t j0 = 0; j0 < c->cols; j0 += KB) {
        int32_t nb = c->cols - j0 < KB ? c->cols - j0 : KB;
        for (int r = 0; r < RA; r++) {
            if (r0 + r < c->rows)
                weight_run(c->W, c->wd, (size_t)c->rows, (size_t)c->cols, (size_t)(r0 + r), (size_t)j0,
                           (size_t)nb, wf + (size_t)r * KB);
            else
                memset(wf + (size_t)r * KB, 0, sizeof(float) * KB);
        }
        for (int32_t s = 0; s < ntile; s++) {
            v16 acc[RA][2];
#pragma GCC unroll 8
            for (int r = 0; r < RA; r++) {
                acc[r][0] = part[(s * RA + r) * 2];
                acc[r][1] = part[(s * RA + r) * 2 + 1];
            }
            const float* xr = c->XT + (size_t)j0 * c->Mp + m0 + (size_t)s * PA;
            for (int32_t j = 0; j < nb; j++, xr += c->Mp) {
                v16 x0, x1;
                memcpy(&x0, xr, sizeof x0);
                memcpy(&x1, xr + 16, sizeof x1);
#pragma GCC unroll 8
                for (int r = 0; r < RA; r++) {
                    float w = wf[(size_t)r * KB + j];
                    v16 p0 = x0 * w;
                    v16 p1 = x1 * w;
                    acc[r][0] = acc[r][0] + p0;
                    acc[r][1] = acc[r][1] + p1;
                }
            }
#pragma GCC unroll 8
            for (int r = 0; r < RA; r++) {
                part[(s * RA + r) * 2] = acc[r][0];
                part[(s * RA + r) * 2 + 1] = acc[r][1];
            }
        }
    }
    for (int32_t s = 0; s < ntile; s++)
        for (int r = 0; r < RA && r0 + r < c->rows; r++)
            for (int v = 0; v < 2; v++)
                for (int l = 0; l < 16; l++) {
                    int32_t m = m0 + s * PA + 16 * v + l;
                    if (m < c->M) c->Y[(size_t)m * c->ldy + r0 + r] = part[(s * RA + r) * 2 + v][l];
                }
}

/* Kernel B: RB rows in the lanes of one vector, items one after another. */
HOT static void mm_task_rows(void* vctx, int64_t task, int tid) {
    mm_ctx* c = (mm_ctx*)vctx;
    int32_t r0 = (int32_t)task * RB;
    float* wt = c->scratch + (size_t)tid * MM_SCRATCH;   /* [KB][RB], transposed */
    float row[KB];
    for (int32_t m0 = 0; m0 < c->M; m0 += 4) {
        int32_t mn = c->M - m0 < 4 ? c->M - m0 : 4;
        v16 acc[4];
        for (int k = 0; k < 4; k++) acc[k] = (v16){0};
        for (int32_t j0 = 0; j0 < c->cols; j0 += KB) {
            int32_t nb = c->cols - j0 < KB ? c->cols - j0 : KB;
            for (int r = 0; r < RB; r++) {
                if (r0 + r < c->rows)
                    weight_run(c->W, c->wd, (size_t)c->rows, (size_t)c->cols, (size_t)(r0 + r), (size_t)j0,
                               (size_t)nb, row);
                else
                    memset(row, 0, sizeof row);
                for (int32_t j = 0; j < nb; j++) wt[(size_t)j * RB + r] = row[j];
            }
            for (int32_t j = 0; j < nb; j++) {
                v16 w;
                memcpy(&w, wt + (size_t)j * RB, sizeof w);
#pragma GCC unroll 4
                for (int k = 0; k < mn; k++) {
                    v16 p = w * c->X[(size_t)(m0 + k) * c->cols + j0 + j];
                    acc[k] = acc[k] + p;
                }
            }
        }
        for (int k = 0; k < mn; k++)
            for (int r = 0; r < RB && r0 + r < c->rows; r++)
                c->Y[(size_t)(m0 + k) * c->ldy + r0 + r] = acc[k][r];
    }
}

/* X [M][cols] -> XT [cols][Mp], one task per block of 64 columns. */
static void transpose_task(void* vctx, int64_t task, int tid) {
    (void)tid;
    mm_ctx* c = (mm_ctx*)vctx;
    int32_t j0 = (int32_t)task * 64, j1 = j0 + 64 < c->cols ? j0 + 64 : c->cols;
    for (int32_t m = 0; m < c->M; m++)
        for (int32_t j = j0; j < j1; j++) c->XT[(size_t)j * c->Mp + m] = c->X[(size_t)m * c->cols + j];
}

/* Y[m][0..rows) for m < M; X [M][cols] row-major; ldy = Y's row stride. */
static void matmul_items(const void* W, int32_t wd, int32_t rows, int32_t cols, const float* X,
                         int32_t M, float* Y, int32_t ldy, int nthreads) {
    mm_ctx c = {W, wd, rows, cols, M, X, NULL, 0, Y, ldy, NULL};
    /* 64-byte aligned: the partial sums are read and written as whole vectors */
    c.scratch = (float*)aligned_alloc(64, sizeof(float) * (size_t)MM_SCRATCH * (size_t)(nthreads > 0 ? nthreads : 1));
    if (M >= 16) {
        int32_t Mp = (M + PA - 1) / PA * PA;
        c.XT = (float*)calloc((size_t)cols * Mp, sizeof(float));
        c.Mp = Mp;
        par_for((cols + 63) / 64, transpose_task, &c, nthreads);
        int64_t ngroups = (rows + RA - 1) / RA;
        par_for(ngroups * ((Mp + IC - 1) / IC), mm_task_items, &c, nthreads);
        free(c.XT);
    } else {
        par_for((rows + RB - 1) / RB, mm_task_rows, &c, nthreads);
    }
    free(c.scratch);
}

/* ---- attention of one query head, per scalar as orc_attend -------------- */
/* KT [D][ldk] holds the cached keys transposed (KT[e][t] = K[t][e]), so the
 * scores of 16 positions are 16 lanes, each its own sequential sum over e.
 * V [n][D] row-major; the output dims are lanes of the weighted sum. */
HOT static void attend_fast(const float* q, const float* KT, int32_t ldk, const float* V, int32_t n,
                            int32_t D, float* probs, float* out) {
    float scale = sqrtf((float)D);
    int32_t t = 0;
    for (; t + 16 <= n; t += 16) {
        v16 dot = (v16){0};
        for (int32_t e = 0; e < D; e++) {
            v16 k;
            memcpy(&k, KT + (size_t)e * ldk + t, sizeof k);
            v16 prod = k * q[e];
            dot = dot + prod;
        }
        v16 sc = dot / scale;
        memcpy(probs + t, &sc, sizeof sc);
    }
    for (; t < n; t++) {
        float dot = 0.0f;
        for (int32_t e = 0; e < D; e++) {
            float prod = q[e] * KT[(size_t)e * ldk + t];
            dot = dot + prod;
        }
        probs[t] = dot / scale;
    }
    float m = probs[0];
    for (t = 1; t < n; t++)
        if (probs[t] > m) m = probs[t];
    float sum = 0.0f;
    for (t = 0; t < n; t++) {
        float z = probs[t] - m;
        float ez = (float)exp((double)z);
        probs[t] = ez;
        sum = sum + ez;
    }
    for (t = 0; t < n; t++) probs[t] = probs[t] / sum;
    int32_t e0 = 0;
    for (; e0 + 64 <= D; e0 += 64) {
        v16 acc[4] = {{0}, {0}, {0}, {0}};
        for (t = 0; t < n; t++) {
            const float* vr = V + (size_t)t * D + e0;
            float p = probs[t];
#pragma GCC unroll 4
            for (int k = 0; k < 4; k++) {
                v16 vv;
                memcpy(&vv, vr + 16 * k, sizeof vv);
                v16 prod = vv * p;
                acc[k] = acc[k] + prod;
            }
        }
        memcpy(out + e0, acc, sizeof acc);
    }
    for (; e0 + 16 <= D; e0 += 16) {
        v16 acc = (v16){0};
        for (t = 0; t < n; t++) {
            v16 vv;
            memcpy(&vv, V + (size_t)t * D + e0, sizeof vv);
            v16 prod = vv * probs[t];
            acc = acc + prod;
        }
        memcpy(out + e0, &acc, sizeof acc);
    }
    for (; e0 < D; e0++) {
        float acc = 0.0f;
        for (t = 0; t < n; t++) {
            float prod = probs[t] * V[(size_t)t * D + e0];
            acc = acc + prod;
        }
        out[e0] = acc;
    }
}

/* ---- the items, layer by layer ------------------------------------------ */
enum { T_ATTN_NORM = 0, T_WQ, T_WK, T_WV, T_WO, T_FFN_NORM, T_W1, T_W3, T_W2, T_PER_LAYER };

typedef struct {
    const orc_config* c;
    float* cache;
    int32_t B, T, n, layer;
    const int32_t *seq, *pos;
    int32_t nseq;           /* distinct sequences among the items */
    const int32_t* seqs;    /* [nseq] their slots */
    const int32_t* slot_of; /* [n] item -> index into seqs */
    const int32_t* npos;    /* [nseq] positions 0..npos-1 read by that sequence's items */
    float* KT;              /* [nseq][Hkv][D][T] transposed keys of this layer */
    const float* Q;         /* [n][H*D] */
    float* O;               /* [n][H*D] */
    float* scratch;         /* per thread: T floats of weights */
} attn_ctx;

static float* kt_of(attn_ctx* a, int32_t s, int32_t g) {
    return a->KT + ((size_t)s * a->c->n_kv_heads + (size_t)g) * (size_t)a->c->head_dim * (size_t)a->T;
}

/* One (sequence, key/value head): its cached keys of this layer, transposed. */
static void kt_task(void* vctx, int64_t task, int tid) {
    (void)tid;
    attn_ctx* a = (attn_ctx*)vctx;
    const orc_config* c = a->c;
    int32_t s = (int32_t)(task / c->n_kv_heads), g = (int32_t)(task % c->n_kv_heads), D = c->head_dim;
    const float* K = a->cache + orc_cache_index(c, a->B, a->T, a->layer, 0, a->seqs[s], g, 0);
    float* kt = kt_of(a, s, g);
    for (int32_t t = 0; t < a->npos[s]; t++)
        for (int32_t e = 0; e < D; e++) kt[(size_t)e * a->T + t] = K[(size_t)t * D + e];
}

static void attn_task(void* vctx, int64_t task, int tid) {
    attn_ctx* a = (attn_ctx*)vctx;
    const orc_config* c = a->c;
    int32_t H = c->n_heads, D = c->head_dim, group = c->n_heads / c->n_kv_heads;
    int32_t i = (int32_t)(task / H), h = (int32_t)(task % H), g = h / group;
    float* probs = a->scratch + (size_t)tid * (size_t)a->T;
    const float* Vv = a->cache + orc_cache_index(c, a->B, a->T, a->layer, 1, a->seq[i], g, 0);
    attend_fast(a->Q + (size_t)i * H * D + (size_t)h * D, kt_of(a, a->slot_of[i], g), a->T, Vv,
                a->pos[i] + 1, D, probs, a->O + (size_t)i * H * D + (size_t)h * D);
}

/* Elementwise work spread over the items. */
typedef struct {
    float *A, *U, *X, *TMP;
    int32_t F, d;
} ew_ctx;

static void silu_task(void* vctx, int64_t i, int tid) {
    (void)tid;
    ew_ctx* e = (ew_ctx*)vctx;
    float* a = e->A + (size_t)i * e->F;
    const float* u = e->U + (size_t)i * e->F;
    for (int32_t k = 0; k < e->F; k++) a[k] = orc_silu_mul(a[k], u[k]);
}

static int cmp_i64(const void* x, const void* y) {
    int64_t a = *(const int64_t*)x, b = *(const int64_t*)y;
    return a < b ? -1 : (a > b ? 1 : 0);
}

int32_t orc_forward_items(const orc_config* c, const uint8_t* arena, float* cache, int32_t B,
                          int32_t T, int32_t n, const int32_t* seq, const int32_t* pos,
                          const int32_t* tok, const int32_t* want, float* logits, int32_t* tok_out,
                          int32_t nthreads) {
    const int32_t d = c->dim, H = c->n_heads, Hkv = c->n_kv_heads, D = c->head_dim;
    const int32_t F = c->hidden_dim, V = c->vocab_size, wd = c->weight_dtype;
    if (n < 0 || nthreads < 1) return -1;
    if (H % Hkv != 0 || D % 2 != 0) return -2;
    int64_t* keys = (int64_t*)malloc(sizeof(int64_t) * (size_t)(n > 0 ? n : 1));
    for (int32_t i = 0; i < n; i++) {
        if (tok[i] < 0 || tok[i] >= V || pos[i] < 0 || pos[i] >= T || seq[i] < 0 || seq[i] >= B) {
            free(keys);
            return -1;
        }
        keys[i] = (int64_t)seq[i] * T + pos[i];
    }
    qsort(keys, (size_t)n, sizeof(int64_t), cmp_i64);
    for (int32_t i = 1; i < n; i++)
        if (keys[i] == keys[i - 1]) {
            free(keys);
            return -3; /* one (sequence, position) twice */
        }
    free(keys);
    if (n == 0) return 0;

    int32_t nt = orc_n_tensors(c);
    size_t* off = (size_t*)malloc(sizeof(size_t) * (size_t)nt);
    orc_tensor_offsets(c, off, nt);
    const size_t qd = (size_t)H * D, kd = (size_t)Hkv * D;
    float* X = (float*)malloc(sizeof(float) * (size_t)n * d);
    float* XN = (float*)malloc(sizeof(float) * (size_t)n * d);
    float* TMP = (float*)malloc(sizeof(float) * (size_t)n * d);
    float* Q = (float*)malloc(sizeof(float) * (size_t)n * qd);
    float* Kn = (float*)malloc(sizeof(float) * (size_t)n * kd);
    float* Vn = (float*)malloc(sizeof(float) * (size_t)n * kd);
    float* O = (float*)malloc(sizeof(float) * (size_t)n * qd);
    float* A = (float*)malloc(sizeof(float) * (size_t)n * F);
    float* U = (float*)malloc(sizeof(float) * (size_t)n * F);
    float* cs = (float*)malloc(sizeof(float) * (size_t)(D / 2));
    float* sn = (float*)malloc(sizeof(float) * (size_t)(D / 2));
    /* the distinct sequences and how far back their items read */
    int32_t* seqs = (int32_t*)malloc(sizeof(int32_t) * (size_t)n);
    int32_t* slot_of = (int32_t*)malloc(sizeof(int32_t) * (size_t)n);
    int32_t* npos = (int32_t*)malloc(sizeof(int32_t) * (size_t)n);
    int32_t nseq = 0;
    for (int32_t i = 0; i < n; i++) {
        int32_t s = 0;
        while (s < nseq && seqs[s] != seq[i]) s++;
        if (s == nseq) {
            seqs[nseq] = seq[i];
            npos[nseq] = 0;
            nseq++;
        }
        slot_of[i] = s;
        if (pos[i] + 1 > npos[s]) npos[s] = pos[i] + 1;
    }
    attn_ctx ac = {c, cache, B, T, n, 0, seq, pos, nseq, seqs, slot_of, npos, NULL, Q, O, NULL};
    ac.scratch = (float*)malloc(sizeof(float) * (size_t)T * (size_t)nthreads);
    ac.KT = (float*)malloc(sizeof(float) * (size_t)nseq * Hkv * D * T);
    ew_ctx ew = {A, U, X, TMP, F, d};

    /* embedding rows, widened ([GOT] "Loading the model and tokenizer") */
    const void* emb = arena + off[0];
    for (int32_t i = 0; i < n; i++)
        for (int32_t j = 0; j < d; j++)
            X[(size_t)i * d + j] = orc_weight(emb, wd, (size_t)V, (size_t)d, (size_t)tok[i], (size_t)j);

    for (int32_t l = 0; l < c->n_layers; l++) {
        const size_t* lo = off + 1 + (size_t)l * T_PER_LAYER;
        const float* g_att = (const float*)(arena + lo[T_ATTN_NORM]);
        for (int32_t i = 0; i < n; i++) orc_rmsnorm(X + (size_t)i * d, g_att, d, c->norm_eps, XN + (size_t)i * d);
        matmul_items(arena + lo[T_WQ], wd, H * D, d, XN, n, Q, (int32_t)qd, nthreads);
        matmul_items(arena + lo[T_WK], wd, Hkv * D, d, XN, n, Kn, (int32_t)kd, nthreads);
        matmul_items(arena + lo[T_WV], wd, Hkv * D, d, XN, n, Vn, (int32_t)kd, nthreads);
        for (int32_t i = 0; i < n; i++) {
            orc_rope_angles(pos[i], D, c->rope_theta, cs, sn);
            for (int32_t h = 0; h < H; h++) orc_rope_apply(Q + (size_t)i * qd + (size_t)h * D, D, cs, sn);
            float* k = Kn + (size_t)i * kd;
            float* v = Vn + (size_t)i * kd;
            for (int32_t g = 0; g < Hkv; g++) orc_rope_apply(k + (size_t)g * D, D, cs, sn);
            if (c->cache_dtype == ORC_BF16)
                for (size_t e = 0; e < kd; e++) {
                    k[e] = orc_round_bf16(k[e]);
                    v[e] = orc_round_bf16(v[e]);
                }
            for (int32_t g = 0; g < Hkv; g++) {
                memcpy(cache + orc_cache_index(c, B, T, l, 0, seq[i], g, pos[i]), k + (size_t)g * D,
                       sizeof(float) * (size_t)D);
                memcpy(cache + orc_cache_index(c, B, T, l, 1, seq[i], g, pos[i]), v + (size_t)g * D,
                       sizeof(float) * (size_t)D);
            }
        }
        ac.layer = l;
        par_for((int64_t)nseq * Hkv, kt_task, &ac, nthreads);
        par_for((int64_t)n * H, attn_task, &ac, nthreads);
        matmul_items(arena + lo[T_WO], wd, d, H * D, O, n, TMP, d, nthreads);
        for (size_t e = 0; e < (size_t)n * d; e++) X[e] = X[e] + TMP[e];
        const float* g_ffn = (const float*)(arena + lo[T_FFN_NORM]);
        for (int32_t i = 0; i < n; i++) orc_rmsnorm(X + (size_t)i * d, g_ffn, d, c->norm_eps, XN + (size_t)i * d);
        matmul_items(arena + lo[T_W1], wd, F, d, XN, n, A, F, nthreads);
        matmul_items(arena + lo[T_W3], wd, F, d, XN, n, U, F, nthreads);
        par_for(n, silu_task, &ew, nthreads);
        matmul_items(arena + lo[T_W2], wd, d, F, A, n, TMP, d, nthreads);
        for (size_t e = 0; e < (size_t)n * d; e++) X[e] = X[e] + TMP[e];
    }

    /* final norm and vocabulary product for the wanted items only */
    int32_t nw = 0;
    for (int32_t i = 0; i < n; i++) {
        tok_out[i] = -1;
        if (want[i]) {
            const float* g_out = (const float*)(arena + off[1 + (size_t)c->n_layers * T_PER_LAYER]);
            orc_rmsnorm(X + (size_t)i * d, g_out, d, c->norm_eps, XN + (size_t)nw * d);
            nw++;
        }
    }
    if (nw > 0) {
        const void* wcls = c->tied_embeddings ? (const void*)(arena + off[0]) : (const void*)(arena + off[nt - 1]);
        matmul_items(wcls, wd, V, d, XN, nw, logits, V, nthreads);
        for (int32_t i = 0, k = 0; i < n; i++)
            if (want[i]) {
                tok_out[i] = orc_argmax(logits + (size_t)k * V, V);
                k++;
            }
    }
    free(off); free(X); free(XN); free(TMP); free(Q); free(Kn); free(Vn); free(O);
    free(A); free(U); free(cs); free(sn); free(ac.scratch); free(ac.KT);
    free(seqs); free(slot_of); free(npos);
    return 0;
}
