/*
 * oracle.h -- reference decoder for the single-token Llama decode step.
 *
 * TEST INFRASTRUCTURE ONLY.  This is the plain, slow CPU definition that the
 * HIP library is checked against.  Only the tests, the smoke check and the
 * benchmark's CPU-baseline leg may load it; the product path never does.  It
 * shares no code, header or table with the HIP library.
 *
 * All arithmetic is IEEE binary32, one rounding per operation, in the order
 * the functions below state, with no fused multiply-add (build with
 * -ffp-contract=off).  exp, sin, cos and pow are evaluated in binary64 and
 * rounded once to binary32.
 */
#ifndef DS_ORACLE_H
#define DS_ORACLE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Matrix storage.  ORC_Q8 is the block-quantised int8 reading of "simple-llm
 * / kasahare" (section "Where to go from here": INT8 weight loading,
 * block-quantised as in GGUF): a matrix [rows][cols] is int8 q[rows][cols]
 * row-major, then, from the next 256-byte boundary of the tensor, fp32
 * s[rows][cols/32]; element (r, c) is the fp32 product s[r][c/32] * q[r][c].
 * cols is a multiple of 32.  ORC_Q4 is the 4-bit variant the same section
 * names: the values are packed two per byte (value c of a row in byte c/2,
 * the low nibble for even c), each a two's complement integer in [-8, 7],
 * rows*cols/2 bytes row-major, then the scales as for ORC_Q8. */
enum { ORC_F32 = 0, ORC_BF16 = 1, ORC_Q8 = 2, ORC_Q4 = 3 };

typedef struct {
    int32_t dim, n_layers, n_heads, n_kv_heads, head_dim, hidden_dim, vocab_size;
    int32_t tied_embeddings;
    int32_t weight_dtype; /* ORC_F32, ORC_BF16, ORC_Q8 or ORC_Q4 for matrices; gains are fp32 */
    float rope_theta, norm_eps;
    /* ORC_F32, or ORC_BF16: every key and value row is rounded to bfloat16
     * (nearest, ties to even) when it is stored, and attention reads the
     * rounded values (the bf16 cache that "simple-llm / kasahare", section
     * "Limitations (intentional)", lists among the cache compressions it
     * leaves out).  The host cache array stays fp32 and holds those values. */
    int32_t cache_dtype;
} orc_config;

/* ---- primitives ------------------------------------------------------- */
float orc_widen_bf16(uint16_t h);
/* x rounded to the nearest bfloat16 (ties to even), as fp32; x finite. */
float orc_round_bf16(float x);
void orc_widen_bf16_array(const uint16_t* src, float* dst, size_t n);
void orc_matvec(const void* W, int32_t wdtype, int32_t n_out, int32_t n_in,
                const float* x, float* y);
/* Element (r, c) of a [rows][cols] matrix stored as wdtype, as fp32. */
float orc_weight(const void* W, int32_t wdtype, size_t rows, size_t cols, size_t r, size_t c);
void orc_rmsnorm(const float* x, const float* g, int32_t n, float eps, float* y);
void orc_rope_angles(int32_t pos, int32_t head_dim, float theta, float* c, float* s);
void orc_rope_apply(float* v, int32_t head_dim, const float* c, const float* s);
void orc_attend(const float* q, const float* K, const float* V, int32_t n, int32_t head_dim,
                float* probs, float* out);
float orc_silu_mul(float a, float u);
int32_t orc_argmax(const float* v, int32_t n);
/* One sampled token (temperature, top-k, top-p, the uniform draw u); the
 * kept candidates in draw order and their normalised cumulative weights go
 * to cand / cum (room for V entries each). */
int32_t orc_sample(const float* logits, int32_t V, float temperature, int32_t top_k, float top_p,
                   double u, int32_t* cand, double* cum, int32_t* n_out);

/* ---- arena and cache layout ------------------------------------------ */
int32_t orc_n_tensors(const orc_config* c);
size_t orc_tensor_offsets(const orc_config* c, size_t* off, int32_t n);
size_t orc_cache_index(const orc_config* c, int32_t B, int32_t T, int32_t layer, int32_t kv,
                       int32_t b, int32_t g, int32_t t);

/* ---- the model -------------------------------------------------------- */
/* One position of sequence b: reads token, writes K/V rows at pos into the
 * (L,2,B,Hkv,T,D) fp32 cache, writes V logits, returns the greedy token, or
 * a negative value on a bad argument. */
int32_t orc_forward(const orc_config* c, const uint8_t* arena, float* cache, int32_t B,
                    int32_t T, int32_t b, int32_t pos, int32_t token, float* logits);

/* Advance every sequence by one position: lengths[b] is the position that
 * tok_in[b] is fed at; on return lengths[b] is one larger. */
int32_t orc_decode_step(const orc_config* c, const uint8_t* arena, float* cache, int32_t B,
                        int32_t T, int32_t* lengths, const int32_t* tok_in, int32_t* tok_out,
                        float* logits);

/* Greedy generation for sequence b from an empty slot.  mode 0 = cached
 * (prompt once, then one position per new token); mode 1 = uncached (the
 * slot is cleared and every position recomputed for every new token).
 * out_logits (n_new x V) may be NULL.  *passes counts forward positions. */
int32_t orc_generate(const orc_config* c, const uint8_t* arena, float* cache, int32_t B,
                     int32_t T, int32_t b, const int32_t* prompt, int32_t n_prompt,
                     int32_t n_new, int32_t mode, int32_t* out_tokens, float* out_logits,
                     int64_t* passes);

/* The same computation as orc_forward for n items (sequence seq[i],
 * position pos[i], token tok[i]), bit for bit, evaluated layer by layer for
 * all items together and spread over nthreads host threads (batch.c).  No
 * (sequence, position) may appear twice; every item's earlier positions must
 * already be in the cache (or among the items).  For the items with want[i]
 * != 0, in item order, the logits go to consecutive rows of logits [.][V]
 * and tok_out[i] gets the greedy token; tok_out[i] = -1 for the others.
 * Returns 0, or a negative value on a bad argument (nothing is written). */
int32_t orc_forward_items(const orc_config* c, const uint8_t* arena, float* cache, int32_t B,
                          int32_t T, int32_t n, const int32_t* seq, const int32_t* pos,
                          const int32_t* tok, const int32_t* want, float* logits, int32_t* tok_out,
                          int32_t nthreads);

#ifdef __cplusplus
}
#endif
#endif
