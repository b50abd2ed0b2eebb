// api.hip -- the C ABI declared in include/ds_decode.h: argument checks on the
// host, the host mirror of the cache lengths, workspace layout, the RoPE
// table, and dispatch of the step kernels (eager or HIP-graph replay).
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <cstdlib>
#include <mutex>
#include <new>
#include <string>
#include <utility>
#include <vector>

#include "ds_decode.h"
#include "kernels.h"

namespace {

thread_local std::string g_err;

ds_status fail(ds_status st, const char* fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    g_err = buf;
    return st;
}

ds_status ok() {
    g_err.clear();
    return DS_OK;
}

ds_status hip_fail(hipError_t e, const char* what) {
    return fail(DS_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

// The current device's copy of ds_sample_noalloc's static scratch (defined
// with it below), or nullptr with the reason in g_err.
uint64_t* device_scratch();

constexpr size_t kAlign = 256;

size_t round_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

size_t wsize(const ds_config* c) { return c->weight_dtype == DS_BF16 ? 2 : (c->weight_dtype == DS_Q8 || c->weight_dtype == DS_Q4) ? 1 : 4; }

// Bytes of one [rows][cols] matrix; DS_Q8: the int8 values, then from the
// next 256-byte boundary one fp32 scale per 32 values of a row.
size_t mat_bytes(const ds_config* c, size_t rows, size_t cols) {
    if (c->weight_dtype == DS_Q8) return round_up(rows * cols, kAlign) + 4 * rows * (cols / 32);
    if (c->weight_dtype == DS_Q4) return round_up(rows * cols / 2, kAlign) + 4 * rows * (cols / 32);
    return rows * cols * wsize(c);
}

// Shape checks shared by every entry point.  Returns DS_OK or an error with
// the reason in g_err.
ds_status check_config(const ds_config* c) {
    if (!c) return fail(DS_ERR_INVALID_ARG, "config is NULL");
    if (c->dim <= 0 || c->n_layers <= 0 || c->n_heads <= 0 || c->n_kv_heads <= 0 ||
        c->head_dim <= 0 || c->hidden_dim <= 0 || c->vocab_size <= 0)
        return fail(DS_ERR_INVALID_ARG, "every dimension must be positive");
    if (c->weight_dtype != DS_F32 && c->weight_dtype != DS_BF16 && c->weight_dtype != DS_Q8 &&
        c->weight_dtype != DS_Q4)
        return fail(DS_ERR_INVALID_ARG, "weight_dtype must be DS_F32, DS_BF16, DS_Q8 or DS_Q4");
    if ((c->weight_dtype == DS_Q8 || c->weight_dtype == DS_Q4) &&
        (c->dim % 32 || (static_cast<int64_t>(c->n_heads) * c->head_dim) % 32 || c->hidden_dim % 32))
        return fail(DS_ERR_UNSUPPORTED, "DS_Q8 and DS_Q4 need dim, n_heads*head_dim and hidden_dim multiples of 32");
    if (c->cache_dtype != DS_F32 && c->cache_dtype != DS_BF16)
        return fail(DS_ERR_INVALID_ARG, "cache_dtype must be DS_F32 or DS_BF16");
    if (c->cache_dtype == DS_BF16 && !((c->head_dim == 64 || c->head_dim == 128) && c->n_kv_heads > 0 &&
                                      c->n_heads % c->n_kv_heads == 0 && c->n_heads / c->n_kv_heads <= 4))
        return fail(DS_ERR_UNSUPPORTED, "a bf16 cache needs head_dim 64 or 128 and at most 4 query heads per key/value head");
    if (c->n_heads % c->n_kv_heads != 0)
        return fail(DS_ERR_INVALID_ARG, "n_heads (%d) is not a multiple of n_kv_heads (%d)", c->n_heads,
                    c->n_kv_heads);
    if (c->head_dim % 2 != 0) return fail(DS_ERR_INVALID_ARG, "head_dim must be even");
    if (!(c->norm_eps > 0.f) || !(c->rope_theta > 0.f))
        return fail(DS_ERR_INVALID_ARG, "norm_eps and rope_theta must be positive");
    if (c->head_dim != 16 && c->head_dim != 32 && c->head_dim != 64 && c->head_dim != 128 && c->head_dim != 256)
        return fail(DS_ERR_UNSUPPORTED, "head_dim %d: the attention kernels are built for 16, 32, 64, 128 and 256",
                    c->head_dim);
    if (c->n_heads / c->n_kv_heads > ds::kMaxRep)
        return fail(DS_ERR_UNSUPPORTED, "at most %d query heads per key/value head", ds::kMaxRep);
    const size_t ws = wsize(c);
    if ((c->dim * ws) % 16 || (static_cast<size_t>(c->n_heads) * c->head_dim * ws) % 16 ||
        (c->hidden_dim * ws) % 16)
        return fail(DS_ERR_UNSUPPORTED, "matrix rows must be whole 16-byte chunks");
    const size_t lds = sizeof(float) * std::max(std::max(c->dim, c->n_heads * c->head_dim), c->hidden_dim);
    if (lds > 160 * 1024) return fail(DS_ERR_UNSUPPORTED, "activation vector exceeds 160 KiB of LDS");
    // vocabulary blocks of 4 waves, 64/G rows per wave (G <= 32): at least 8 rows per block
    if ((static_cast<int64_t>(c->vocab_size) + 7) / 8 > ds::kMaxArgmaxBlocks)
        return fail(DS_ERR_UNSUPPORTED, "vocab_size above %d", 8 * ds::kMaxArgmaxBlocks);
    return DS_OK;
}

int n_tensors(const ds_config* c) { return 1 + 9 * c->n_layers + 1 + (c->tied_embeddings ? 0 : 1); }

// Canonical arena offsets (weight order of "simple-llm / kasahare", section
// "On-disk model format (.sllm)", 256-byte aligned, untied head last).
size_t layout(const ds_config* c, std::vector<size_t>* off) {
    const size_t d = c->dim, F = c->hidden_dim, V = c->vocab_size;
    const size_t qr = static_cast<size_t>(c->n_heads) * c->head_dim;
    const size_t kvr = static_cast<size_t>(c->n_kv_heads) * c->head_dim;
    size_t p = 0;
    auto put = [&](size_t bytes) {
        if (off) off->push_back(p);
        p = round_up(p + bytes, kAlign);
    };
    put(mat_bytes(c, V, d));
    for (int l = 0; l < c->n_layers; l++) {
        put(d * 4);
        put(mat_bytes(c, qr, d));
        put(mat_bytes(c, kvr, d));
        put(mat_bytes(c, kvr, d));
        put(mat_bytes(c, d, qr));
        put(d * 4);
        put(mat_bytes(c, F, d));
        put(mat_bytes(c, F, d));
        put(mat_bytes(c, d, F));
    }
    put(d * 4);
    if (!c->tied_embeddings) put(mat_bytes(c, V, d));
    return p;
}

// Workspace carve-up for a (B, T) cache.
struct WsLayout {
    size_t x, q, o, h, part_o, part_ml, logits, keys, slot, pos, flag, err, rope_cos, rope_sin;
    size_t ll_x, ll_x2, ll_qkv, ll_part, ll_h, ll_keys, ll_late, epoch, layers, ll_end, total, rstride;
};

WsLayout ws_layout(const ds_config* c, int B, int T) {
    WsLayout w{};
    const size_t S = (static_cast<size_t>(T) + ds::kChunk - 1) / ds::kChunk;
    const size_t HD = static_cast<size_t>(c->n_heads) * c->head_dim;
    size_t p = 0;
    auto take = [&](size_t bytes) {
        size_t at = p;
        p = round_up(p + bytes, kAlign);
        return at;
    };
    // per-item rows: B for a decode step, up to kMaxItems positions for a batched prefill
    const size_t BI = std::max(B, ds::kMaxItems);
    w.x = take(sizeof(float) * BI * c->dim);
    w.q = take(sizeof(float) * BI * HD);
    w.o = take(sizeof(float) * BI * HD);
    w.h = take(sizeof(float) * BI * c->hidden_dim);
    w.part_o = take(sizeof(float) * BI * c->n_heads * S * c->head_dim);
    w.part_ml = take(sizeof(float) * BI * c->n_heads * S * 2);
    w.logits = take(sizeof(float) * B * static_cast<size_t>(c->vocab_size));  // by slot
    w.keys = take(sizeof(unsigned long long) * B * static_cast<size_t>(ds::kMaxArgmaxBlocks));
    w.slot = take(sizeof(int32_t) * BI);
    w.pos = take(sizeof(int32_t) * BI);
    w.flag = take(sizeof(int32_t) * BI);
    w.err = take(sizeof(int32_t));
    w.rope_cos = take(sizeof(float) * T * (c->head_dim / 2));
    w.rope_sin = take(sizeof(float) * T * (c->head_dim / 2));
    // persistent batch-1 step: LL words (zeroed at creation), epoch, layer table
    const size_t kvd = static_cast<size_t>(c->n_kv_heads) * c->head_dim;
    // ll_x, ll_x2, ll_qkv and ll_h: kPRep replicas each, 4 KiB apart, so that
    // the blocks that poll a vector spread over several memory channels
    const size_t nmax = std::max({static_cast<size_t>(c->dim), HD + 2 * kvd, static_cast<size_t>(c->hidden_dim)});
    w.rstride = round_up(nmax, 512);
    const size_t rbytes = 8 * ds::kPRep * w.rstride;
    w.ll_x = take(rbytes);
    w.ll_x2 = take(rbytes);
    w.ll_qkv = take(rbytes);
    w.ll_part = take(8 * static_cast<size_t>(c->n_heads) * ds::kPMaxParts * (c->head_dim + 2));
    w.ll_h = take(rbytes);
    w.ll_keys = take(8 * static_cast<size_t>(ds::kPKeyWords));
    w.ll_late = take(8);
    w.epoch = take(sizeof(uint32_t));
    w.ll_end = p;
    w.layers = take(sizeof(ds::LayerW) * static_cast<size_t>(c->n_layers));
    w.total = p;
    return w;
}

}  // namespace

struct ds_model {
    ds_config cfg;
    const void* arena;
    std::vector<size_t> off;
    ds::ModelPtrs ptrs;
};

struct GraphEntry {
    int nload;
    hipStream_t stream;
    const int32_t* tok_in;
    int32_t* tok_out;
    hipGraph_t graph;
    hipGraphExec_t exec;
};

struct ds_kv {
    ds_model* model;
    int B, T;
    float* cache;
    int32_t* lengths;
    uint8_t* ws;
    WsLayout lay;
    ds::StepArgs s;
    std::vector<int32_t> mirror;  // host copy of lengths, updated at enqueue
    int dispatch;                 // 0 eager, 1 graph
    bool stepped = false;         // a decode step has filled the per-item state
    int last_nload = 0;           // short-path rows of the last decode step (0: split-K path)
    std::vector<GraphEntry> graphs;
    ds::PersistArgs pa{};
    int persist_ctx = 0;          // longest context of the persistent step (0: off)
};

extern "C" {

const char* ds_last_error(void) { return g_err.c_str(); }

size_t ds_weights_bytes(const ds_config* cfg) {
    if (check_config(cfg) != DS_OK) return 0;
    return layout(cfg, nullptr);
}

int32_t ds_weights_count(const ds_config* cfg) {
    if (check_config(cfg) != DS_OK) return 0;
    return n_tensors(cfg);
}

ds_status ds_weights_offsets(const ds_config* cfg, size_t* h_off, int32_t n) {
    ds_status st = check_config(cfg);
    if (st != DS_OK) return st;
    if (!h_off || n < n_tensors(cfg)) return fail(DS_ERR_INVALID_ARG, "offset array too small");
    std::vector<size_t> off;
    layout(cfg, &off);
    for (size_t i = 0; i < off.size(); i++) h_off[i] = off[i];
    return ok();
}

size_t ds_kv_cache_bytes(const ds_config* cfg, int32_t B, int32_t T) {
    if (check_config(cfg) != DS_OK || B <= 0 || T <= 0) return 0;
    const size_t esz = cfg->cache_dtype == DS_BF16 ? 2 : 4;
    return esz * static_cast<size_t>(cfg->n_layers) * 2 * B * cfg->n_kv_heads * T * cfg->head_dim;
}

size_t ds_workspace_bytes(const ds_config* cfg, int32_t B, int32_t T) {
    if (check_config(cfg) != DS_OK || B <= 0 || T <= 0) return 0;
    return ws_layout(cfg, B, T).total;
}

ds_status ds_load_weights(const ds_config* cfg, const void* d_arena, size_t arena_bytes, void* stream,
                          ds_model** out) {
    (void)stream;
    ds_status st = check_config(cfg);
    if (st != DS_OK) return st;
    if (!out) return fail(DS_ERR_INVALID_ARG, "out is NULL");
    if (!d_arena) return fail(DS_ERR_INVALID_ARG, "d_arena is NULL");
    if (!aligned(d_arena, kAlign)) return fail(DS_ERR_ALIGNMENT, "d_arena is not 256-byte aligned");
    const size_t need = layout(cfg, nullptr);
    if (arena_bytes < need)
        return fail(DS_ERR_WORKSPACE, "arena has %zu bytes, the layout needs %zu", arena_bytes, need);
    ds_model* m = new (std::nothrow) ds_model();
    if (!m) return fail(DS_ERR_INVALID_ARG, "out of host memory");
    // set-up of ds_sample_noalloc on this device: its scratch's address, so
    // that a first call under graph capture need not look it up (a failure
    // here is reported by that call instead)
    (void)device_scratch();
    m->cfg = *cfg;
    m->arena = d_arena;
    layout(cfg, &m->off);
    const uint8_t* a = static_cast<const uint8_t*>(d_arena);
    m->ptrs.emb = a + m->off[0];
    m->ptrs.layers.resize(cfg->n_layers);
    for (int l = 0; l < cfg->n_layers; l++) {
        const size_t* o = m->off.data() + 1 + 9 * l;
        ds::LayerW& w = m->ptrs.layers[l];
        w.attn_norm = reinterpret_cast<const float*>(a + o[0]);
        w.wq = a + o[1];
        w.wk = a + o[2];
        w.wv = a + o[3];
        w.wo = a + o[4];
        w.ffn_norm = reinterpret_cast<const float*>(a + o[5]);
        w.w1 = a + o[6];
        w.w3 = a + o[7];
        w.w2 = a + o[8];
    }
    m->ptrs.out_norm = reinterpret_cast<const float*>(a + m->off[1 + 9 * cfg->n_layers]);
    m->ptrs.wcls = cfg->tied_embeddings ? m->ptrs.emb : a + m->off.back();
    *out = m;
    return ok();
}

void ds_model_destroy(ds_model* model) { delete model; }

ds_status ds_kv_cache_create(ds_model* model, int32_t B, int32_t T, float* d_cache, size_t cache_bytes,
                             int32_t* d_lengths, void* d_workspace, size_t workspace_bytes, void* stream,
                             ds_kv** out) {
    if (!model || !out) return fail(DS_ERR_INVALID_ARG, "model or out is NULL");
    const ds_config* c = &model->cfg;
    if (B <= 0 || T <= 0) return fail(DS_ERR_INVALID_ARG, "B and T must be positive");
    if (!d_cache || !d_lengths || !d_workspace) return fail(DS_ERR_INVALID_ARG, "NULL device buffer");
    if (!aligned(d_cache, kAlign) || !aligned(d_lengths, kAlign) || !aligned(d_workspace, kAlign))
        return fail(DS_ERR_ALIGNMENT, "cache, lengths and workspace must be 256-byte aligned");
    if (cache_bytes < ds_kv_cache_bytes(c, B, T))
        return fail(DS_ERR_WORKSPACE, "cache has %zu bytes, needs %zu", cache_bytes, ds_kv_cache_bytes(c, B, T));
    const WsLayout lay = ws_layout(c, B, T);
    if (workspace_bytes < lay.total)
        return fail(DS_ERR_WORKSPACE, "workspace has %zu bytes, needs %zu", workspace_bytes, lay.total);
    hipStream_t st = static_cast<hipStream_t>(stream);

    // Dynamic LDS above 64 KiB needs the per-kernel opt-in, up to the device's
    // per-block limit; the need is computed from the shape below.
    ds::StepArgs probe{};
    probe.d = c->dim;
    probe.H = c->n_heads;
    probe.Hkv = c->n_kv_heads;
    probe.D = c->head_dim;
    probe.F = c->hidden_dim;
    probe.wdt = c->weight_dtype;
    const int need_lds = static_cast<int>(ds::max_lds_bytes(probe));
    const int need_mm = ds::mm_supported(probe) ? static_cast<int>(ds::mm_max_lds(probe)) : 0;
    // Function attributes belong to a device: the levels already set are
    // kept per device, under a lock (caches may be created from several
    // threads and for several devices).
    if (need_lds > 64 * 1024 || need_mm > 64 * 1024) {
        static std::mutex attr_mu;
        static std::vector<std::pair<int, int>> attr_set;  // per device: (lds, mm) levels set
        std::lock_guard<std::mutex> lock(attr_mu);
        int dev = 0, optin = 0;
        hipError_t e = hipGetDevice(&dev);
        if (e == hipSuccess) e = hipDeviceGetAttribute(&optin, hipDeviceAttributeSharedMemPerBlockOptin, dev);
        if (e != hipSuccess) return hip_fail(e, "hipDeviceGetAttribute");
        if (std::max(need_lds, need_mm) > optin - 4096)
            return fail(DS_ERR_UNSUPPORTED, "kernels need %d bytes of LDS, the device allows %d",
                        std::max(need_lds, need_mm), optin);
        if (static_cast<int>(attr_set.size()) <= dev) attr_set.resize(dev + 1, {64 * 1024, 64 * 1024});
        std::pair<int, int>& lv = attr_set[dev];
        if (need_lds > lv.first) {
            e = ds::set_kernel_attributes(need_lds);
            if (e != hipSuccess) return hip_fail(e, "hipFuncSetAttribute");
            lv.first = need_lds;
        }
        if (need_mm > lv.second) {
            e = ds::mm_set_attributes(need_mm);
            if (e != hipSuccess) return hip_fail(e, "hipFuncSetAttribute");
            lv.second = need_mm;
        }
    }

    // RoPE table: pair i of position p turns by p * theta^(-2i/D) ("GOTOken",
    // section "Loading the model and tokenizer", pairs (j, j + head_dim/2));
    // angle, cos and sin in double, rounded once to float.
    const int half = c->head_dim / 2;
    std::vector<float> cs(static_cast<size_t>(T) * half), sn(static_cast<size_t>(T) * half);
    for (int p = 0; p < T; p++)
        for (int i = 0; i < half; i++) {
            const double inv = std::pow(static_cast<double>(c->rope_theta),
                                        -static_cast<double>(2 * i) / static_cast<double>(c->head_dim));
            const double ang = static_cast<double>(p) * inv;
            cs[static_cast<size_t>(p) * half + i] = static_cast<float>(std::cos(ang));
            sn[static_cast<size_t>(p) * half + i] = static_cast<float>(std::sin(ang));
        }
    uint8_t* ws = static_cast<uint8_t*>(d_workspace);
    hipError_t e = hipMemcpyAsync(ws + lay.rope_cos, cs.data(), cs.size() * sizeof(float),
                                  hipMemcpyHostToDevice, st);
    if (e == hipSuccess)
        e = hipMemcpyAsync(ws + lay.rope_sin, sn.data(), sn.size() * sizeof(float), hipMemcpyHostToDevice, st);
    if (e == hipSuccess) e = ds::enqueue_fill(d_lengths, B, 0, st);
    if (e == hipSuccess) e = ds::enqueue_fill(reinterpret_cast<int32_t*>(ws + lay.err), 1, 0, st);
    if (e == hipSuccess)
        e = ds::enqueue_fill(reinterpret_cast<int32_t*>(ws + lay.ll_x), static_cast<int>((lay.ll_end - lay.ll_x) / 4), 0,
                             st);
    if (e == hipSuccess)
        e = hipMemcpyAsync(ws + lay.layers, model->ptrs.layers.data(), sizeof(ds::LayerW) * model->ptrs.layers.size(),
                           hipMemcpyHostToDevice, st);
    if (e == hipSuccess) e = hipStreamSynchronize(st);
    if (e != hipSuccess) return hip_fail(e, "cache setup");

    ds_kv* kv = new (std::nothrow) ds_kv();
    if (!kv) return fail(DS_ERR_INVALID_ARG, "out of host memory");
    kv->model = model;
    kv->B = B;
    kv->T = T;
    kv->cache = d_cache;
    kv->lengths = d_lengths;
    kv->ws = ws;
    kv->lay = lay;
    kv->mirror.assign(B, 0);
    const char* env = std::getenv("DS_DISPATCH");
    kv->dispatch = (env && std::strcmp(env, "eager") == 0) ? 0 : 1;
    ds::StepArgs& s = kv->s;
    s.d = c->dim;
    s.L = c->n_layers;
    s.H = c->n_heads;
    s.Hkv = c->n_kv_heads;
    s.D = c->head_dim;
    s.F = c->hidden_dim;
    s.V = c->vocab_size;
    s.wdt = c->weight_dtype;
    s.B = B;
    s.T = T;
    s.n_chunks = (T + ds::kChunk - 1) / ds::kChunk;
    s.cdt = c->cache_dtype;
    s.short_n = s.cdt == DS_BF16 ? 0 : ds::short_positions(s);  // the fused short path reads an fp32 cache
    s.mm_ok = ds::mm_supported(s) ? 1 : 0;
    const char* mmenv = std::getenv("DS_MFMA");  // "0" keeps the VALU projections for every batch size
    if (mmenv && std::strcmp(mmenv, "0") == 0) s.mm_ok = 0;
    s.mm_split = 1;
    const char* skenv = std::getenv("DS_MM_SPLIT");  // "0" keeps the tiled MFMA kernel for every projection
    if (skenv && std::strcmp(skenv, "0") == 0) s.mm_split = 0;
    s.attn_g = 1;
    const char* agenv = std::getenv("DS_ATTN_G");  // "0" keeps the shuffle-reduced attention kernel
    if (agenv && std::strcmp(agenv, "0") == 0 && s.cdt != DS_BF16) s.attn_g = 0;  // the only bf16-cache reader
    // the single-launch step's products: bf16 weights times the input as bf16
    // hi/lo pairs (default), or DS_PERSIST_IN=f32: weights widened to fp32
    s.pin = ds::kBF16;
    const char* pin = std::getenv("DS_PERSIST_IN");
    if (pin && std::strcmp(pin, "f32") == 0) s.pin = ds::kF32;
    // DS_PERSIST_COOP=1 launches the single launch cooperatively: it then
    // starts with every workgroup resident or not at all.  Off by default: it
    // measured 16 us (6.6%) slower per 135M step than a plain launch, whose
    // co-residency rests on the occupancy check below and the bounded waits.
    s.pcoop = 0;
    const char* pco = std::getenv("DS_PERSIST_COOP");
    if (pco && std::strcmp(pco, "1") == 0) s.pcoop = 1;
    s.kv_stream = 1;  // enqueue_step sets it per pass
    // DS_ATTN_FULL=1: launches with at least kAttnFullMinBlocks (sequence,
    // group) pairs run attention as one block per pair (k_attn_full), with no
    // partials or combine launch.  Off by default: at B = 64 (135M) it
    // measured the same step time as split-K plus its combine (1.444 against
    // 1.450 ms), its longest sequences' blocks setting the pace.
    s.attn_full = 0;
    const char* afenv = std::getenv("DS_ATTN_FULL");
    if (afenv && std::strcmp(afenv, "1") == 0) s.attn_full = 1;
    // batched-prefill passes (positions of one sequence) take the attention
    // that reads each chunk once for all positions; DS_ATTN_PF=0 keeps the
    // split-K attention per position
    s.attn_pf = 1;
    const char* pfenv = std::getenv("DS_ATTN_PF");
    if (pfenv && std::strcmp(pfenv, "0") == 0) s.attn_pf = 0;
    const char* sa = std::getenv("DS_SHORT_ATTN");  // "0" turns the fused short-context path off
    if (sa && std::strcmp(sa, "0") == 0) s.short_n = 0;
    ds::PersistArgs& pa = kv->pa;
    pa.layers = reinterpret_cast<const ds::LayerW*>(ws + lay.layers);
    pa.out_norm = model->ptrs.out_norm;
    pa.wcls = model->ptrs.wcls;
    pa.ll_x = reinterpret_cast<uint64_t*>(ws + lay.ll_x);
    pa.ll_x2 = reinterpret_cast<uint64_t*>(ws + lay.ll_x2);
    pa.ll_qkv = reinterpret_cast<uint64_t*>(ws + lay.ll_qkv);
    pa.ll_part = reinterpret_cast<uint64_t*>(ws + lay.ll_part);
    pa.ll_h = reinterpret_cast<uint64_t*>(ws + lay.ll_h);
    pa.ll_keys = reinterpret_cast<uint64_t*>(ws + lay.ll_keys);
    pa.ll_late = reinterpret_cast<uint64_t*>(ws + lay.ll_late);
    pa.epoch = reinterpret_cast<uint32_t*>(ws + lay.epoch);
    pa.rstride = static_cast<int>(lay.rstride);
    kv->persist_ctx = ds::persist_max_ctx(s);
    const char* pe = std::getenv("DS_PERSIST");  // "0" keeps batch-1 steps on one launch per operation
    if (pe && std::strcmp(pe, "0") == 0) kv->persist_ctx = 0;
    if (kv->persist_ctx > 0) {
        hipError_t ee = ds::persist_prepare(s);
        if (ee == hipSuccess && !ds::persist_fits_device(s)) kv->persist_ctx = 0;  // e.g. a partitioned GPU
        if (ee != hipSuccess) {
            delete kv;
            return hip_fail(ee, "persistent step attributes");
        }
    }
    s.eps = c->norm_eps;
    s.emb = model->ptrs.emb;
    s.cache = d_cache;
    s.lengths = d_lengths;
    s.x = reinterpret_cast<float*>(ws + lay.x);
    s.q = reinterpret_cast<float*>(ws + lay.q);
    s.o = reinterpret_cast<float*>(ws + lay.o);
    s.h = reinterpret_cast<float*>(ws + lay.h);
    s.part_o = reinterpret_cast<float*>(ws + lay.part_o);
    s.part_ml = reinterpret_cast<float*>(ws + lay.part_ml);
    s.logits = reinterpret_cast<float*>(ws + lay.logits);
    s.keys = reinterpret_cast<unsigned long long*>(ws + lay.keys);
    s.slot = reinterpret_cast<int32_t*>(ws + lay.slot);
    s.pos = reinterpret_cast<int32_t*>(ws + lay.pos);
    s.flag = reinterpret_cast<int32_t*>(ws + lay.flag);
    s.err = reinterpret_cast<int32_t*>(ws + lay.err);
    s.rope_cos = reinterpret_cast<const float*>(ws + lay.rope_cos);
    s.rope_sin = reinterpret_cast<const float*>(ws + lay.rope_sin);
    *out = kv;
    return ok();
}

void ds_kv_cache_destroy(ds_kv* kv) {
    if (!kv) return;
    for (GraphEntry& g : kv->graphs) {
        (void)hipGraphExecDestroy(g.exec);
        (void)hipGraphDestroy(g.graph);
    }
    delete kv;
}

ds_status ds_kv_cache_reset(ds_kv* kv, int32_t seq, void* stream) {
    if (!kv) return fail(DS_ERR_INVALID_ARG, "kv is NULL");
    if (seq < -1 || seq >= kv->B) return fail(DS_ERR_INVALID_ARG, "seq %d outside [-1, %d)", seq, kv->B);
    hipStream_t st = static_cast<hipStream_t>(stream);
    hipError_t e = seq < 0 ? ds::enqueue_fill(kv->lengths, kv->B, 0, st)
                           : ds::enqueue_fill(kv->lengths + seq, 1, 0, st);
    if (e != hipSuccess) return hip_fail(e, "reset");
    if (seq < 0)
        std::fill(kv->mirror.begin(), kv->mirror.end(), 0);
    else
        kv->mirror[seq] = 0;
    return ok();
}

ds_status ds_kv_cache_set_lengths(ds_kv* kv, const int32_t* h_lengths, void* stream) {
    if (!kv || !h_lengths) return fail(DS_ERR_INVALID_ARG, "NULL argument");
    for (int b = 0; b < kv->B; b++)
        if (h_lengths[b] < 0 || h_lengths[b] > kv->T)
            return fail(DS_ERR_INVALID_ARG, "lengths[%d] = %d outside [0, %d]", b, h_lengths[b], kv->T);
    hipError_t e = ds::enqueue_set_lengths(kv->lengths, h_lengths, 0, kv->B, static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return hip_fail(e, "set_lengths");
    kv->mirror.assign(h_lengths, h_lengths + kv->B);
    return ok();
}

ds_status ds_kv_cache_replicate(ds_kv* dst, const ds_kv* src, int32_t src_seq, int32_t dst_first, int32_t count,
                                void* stream) {
    if (!dst || !src) return fail(DS_ERR_INVALID_ARG, "NULL cache");
    const ds_config& a = dst->model->cfg;
    const ds_config& b = src->model->cfg;
    if (a.n_layers != b.n_layers || a.n_kv_heads != b.n_kv_heads || a.head_dim != b.head_dim ||
        a.cache_dtype != b.cache_dtype)
        return fail(DS_ERR_INVALID_ARG, "caches of different layer / key-value head / head shapes or element types");
    if (src_seq < 0 || src_seq >= src->B) return fail(DS_ERR_INVALID_ARG, "src_seq %d outside [0, %d)", src_seq, src->B);
    if (count < 0 || dst_first < 0 || dst_first + static_cast<int64_t>(count) > dst->B)
        return fail(DS_ERR_INVALID_ARG, "slots [%d, %d + %d) outside [0, %d)", dst_first, dst_first, count, dst->B);
    if (dst == src && src_seq >= dst_first && src_seq < dst_first + count)
        return fail(DS_ERR_INVALID_ARG, "the source slot %d is among the destinations", src_seq);
    const int n = src->mirror[src_seq];
    if (n > dst->T) return fail(DS_ERR_CONTEXT_FULL, "%d positions do not fit a cache of %d", n, dst->T);
    if (count == 0) return ok();
    hipStream_t st = static_cast<hipStream_t>(stream);
    // a bf16 row of D values is copied as D/2 four-byte words
    const int wpr = a.cache_dtype == DS_BF16 ? a.head_dim / 2 : a.head_dim;
    hipError_t e = ds::enqueue_replicate(dst->cache, dst->B, dst->T, src->cache, src->B, src->T, a.n_layers,
                                         a.n_kv_heads, wpr, src_seq, dst_first, count, n, st);
    std::vector<int32_t> len(static_cast<size_t>(count), n);
    if (e == hipSuccess) e = ds::enqueue_set_lengths(dst->lengths, len.data(), dst_first, count, st);
    if (e != hipSuccess) return hip_fail(e, "replicate");
    for (int i = 0; i < count; i++) dst->mirror[dst_first + i] = n;
    return ok();
}

ds_status ds_decode_step_rows(ds_model* model, ds_kv* kv, const int32_t* h_rows, int32_t n_rows,
                              const int32_t* d_tok_in, int32_t* d_tok_out, void* stream) {
    if (!model || !kv || kv->model != model) return fail(DS_ERR_INVALID_ARG, "model/kv mismatch");
    if (!d_tok_in || !d_tok_out || (n_rows > 0 && !h_rows)) return fail(DS_ERR_INVALID_ARG, "NULL argument");
    if (!aligned(d_tok_in, 4) || !aligned(d_tok_out, 4)) return fail(DS_ERR_ALIGNMENT, "token buffers");
    if (n_rows < 0 || n_rows > kv->B) return fail(DS_ERR_INVALID_ARG, "n_rows %d outside [0, %d]", n_rows, kv->B);
    std::vector<char> seen(static_cast<size_t>(kv->B), 0);
    int max_ctx = 0;
    for (int i = 0; i < n_rows; i++) {
        const int r = h_rows[i];
        if (r < 0 || r >= kv->B || seen[r]) return fail(DS_ERR_INVALID_ARG, "row %d repeated or outside [0, %d)", r, kv->B);
        seen[r] = 1;
        if (kv->mirror[r] >= kv->T)
            return fail(DS_ERR_CONTEXT_FULL, "sequence %d already holds all %d positions", r, kv->T);
        max_ctx = std::max(max_ctx, kv->mirror[r] + 1);
    }
    if (n_rows == 0) return ok();
    hipStream_t st = static_cast<hipStream_t>(stream);
    std::vector<ds::BeginList> lists;
    for (int i = 0; i < n_rows; i++) {
        if (lists.empty() || lists.back().n == ds::kMaxItems) {
            lists.emplace_back();
            lists.back().item0 = i;
            lists.back().by_value = 2;
        }
        ds::BeginList& l = lists.back();
        l.slot[l.n] = h_rows[i];
        l.tok[l.n] = 0;
        l.last[l.n] = 1;
        l.n++;
    }
    hipError_t e = ds::enqueue_step(kv->s, model->ptrs, lists.data(), static_cast<int>(lists.size()), d_tok_in, n_rows,
                                    true, ds::short_rows(kv->s, max_ctx), d_tok_out, st);
    if (e != hipSuccess) return hip_fail(e, "decode_step_rows");
    for (int i = 0; i < n_rows; i++) kv->mirror[h_rows[i]] += 1;
    return ok();
}

ds_status ds_kv_cache_get_lengths(const ds_kv* kv, int32_t* h_lengths) {
    if (!kv || !h_lengths) return fail(DS_ERR_INVALID_ARG, "NULL argument");
    std::memcpy(h_lengths, kv->mirror.data(), sizeof(int32_t) * kv->B);
    return ok();
}

ds_status ds_kv_cache_check(ds_kv* kv, void* stream) {
    if (!kv) return fail(DS_ERR_INVALID_ARG, "kv is NULL");
    hipStream_t st = static_cast<hipStream_t>(stream);
    int32_t err = 0;
    hipError_t e = hipStreamSynchronize(st);
    if (e == hipSuccess) e = hipMemcpy(&err, kv->s.err, sizeof err, hipMemcpyDeviceToHost);
    if (e == hipSuccess && err) e = hipMemset(kv->s.err, 0, sizeof(int32_t));
    if (e != hipSuccess) return hip_fail(e, "check");
    if (err & ~1)
        return fail(DS_ERR_DEVICE, "device-side check failed (flags 0x%x: 2 = launch-shape guard, "
                    "4 = a wait of the single-launch step gave up)%s", err & ~1,
                    (err & 1) ? "; a token id was also out of range" : "");
    if (err) return fail(DS_ERR_BAD_TOKEN, "a decode step read a token id outside [0, %d)", kv->s.V);
    return ok();
}

ds_status ds_prefill(ds_model* model, ds_kv* kv, int32_t seq, const int32_t* h_tokens, int32_t n,
                     int32_t* d_tok_out, void* stream) {
    if (!model || !kv || kv->model != model) return fail(DS_ERR_INVALID_ARG, "model/kv mismatch");
    if (seq < 0 || seq >= kv->B) return fail(DS_ERR_INVALID_ARG, "seq %d outside [0, %d)", seq, kv->B);
    if (n <= 0 || !h_tokens) return fail(DS_ERR_INVALID_ARG, "need n > 0 host tokens");
    if (kv->mirror[seq] + static_cast<int64_t>(n) > kv->T)
        return fail(DS_ERR_CONTEXT_FULL, "sequence %d has %d of %d positions; %d more do not fit", seq,
                    kv->mirror[seq], kv->T, n);
    for (int j = 0; j < n; j++)
        if (h_tokens[j] < 0 || h_tokens[j] >= kv->s.V)
            return fail(DS_ERR_BAD_TOKEN, "token %d at %d outside [0, %d)", h_tokens[j], j, kv->s.V);
    hipStream_t st = static_cast<hipStream_t>(stream);
    ds::BeginList list;
    list.n = 1;
    list.item0 = 0;
    list.by_value = 1;
    list.slot[0] = seq;
    for (int j = 0; j < n; j++) {
        list.tok[0] = h_tokens[j];
        list.last[0] = j == n - 1;
        const int ctx = kv->mirror[seq] + j + 1;
        hipError_t e;
        if (kv->B == 1 && ctx <= kv->persist_ctx) {
            // the same kernel as a batch-1 decode step at this position, so a
            // prompt re-fed through prefill reproduces decoded steps bit for bit
            e = ds::enqueue_persist(kv->s, kv->pa, nullptr, h_tokens[j], j == n - 1 ? d_tok_out : nullptr, ctx, st);
        } else {
            const int nload = ds::short_rows(kv->s, ctx);
            e = ds::enqueue_step(kv->s, model->ptrs, &list, 1, nullptr, 1, j == n - 1, nload, d_tok_out, st);
        }
        if (e != hipSuccess) {
            kv->mirror[seq] += j;  // the positions already enqueued advance the device lengths
            return hip_fail(e, "prefill");
        }
    }
    kv->mirror[seq] += n;
    return ok();
}

ds_status ds_prefill_batched(ds_model* model, ds_kv* kv, int32_t seq, const int32_t* h_tokens, int32_t n,
                             int32_t* d_tok_out, void* stream) {
    if (!model || !kv || kv->model != model) return fail(DS_ERR_INVALID_ARG, "model/kv mismatch");
    if (seq < 0 || seq >= kv->B) return fail(DS_ERR_INVALID_ARG, "seq %d outside [0, %d)", seq, kv->B);
    if (n <= 0 || !h_tokens) return fail(DS_ERR_INVALID_ARG, "need n > 0 host tokens");
    if (kv->mirror[seq] + static_cast<int64_t>(n) > kv->T)
        return fail(DS_ERR_CONTEXT_FULL, "sequence %d has %d of %d positions; %d more do not fit", seq,
                    kv->mirror[seq], kv->T, n);
    for (int j = 0; j < n; j++)
        if (h_tokens[j] < 0 || h_tokens[j] >= kv->s.V)
            return fail(DS_ERR_BAD_TOKEN, "token %d at %d outside [0, %d)", h_tokens[j], j, kv->s.V);
    hipStream_t st = static_cast<hipStream_t>(stream);
    // positions 0 .. n-2: up to kMaxItems at a time as the items of one step
    // (projections as GEMMs over the positions, each item attending over the
    // rows up to its own position), no logits
    for (int done = 0; done < n - 1;) {
        const int m = std::min(n - 1 - done, ds::kMaxItems);
        ds::BeginList list;
        list.n = m;
        list.item0 = 0;
        list.by_value = 1;
        for (int i = 0; i < m; i++) {
            list.slot[i] = seq;
            list.tok[i] = h_tokens[done + i];
            list.last[i] = 0;
            list.off[i] = i;
        }
        list.last_pos = kv->mirror[seq] + m - 1;  // sizes the attention launch to the chunks in use
        hipError_t e = ds::enqueue_step(kv->s, model->ptrs, &list, 1, nullptr, m, false, 0, nullptr, st);
        if (e != hipSuccess) return hip_fail(e, "batched prefill");
        kv->mirror[seq] += m;
        done += m;
    }
    // the last position as in ds_prefill: its logits and token
    return ds_prefill(model, kv, seq, h_tokens + (n - 1), 1, d_tok_out, stream);
}

ds_status ds_prefill_batch(ds_model* model, ds_kv* kv, const int32_t* h_tokens, const int32_t* h_counts,
                           int32_t* d_tok_out, void* stream) {
    if (!model || !kv || kv->model != model) return fail(DS_ERR_INVALID_ARG, "model/kv mismatch");
    if (!h_counts) return fail(DS_ERR_INVALID_ARG, "h_counts is NULL");
    if (kv->B == 1) return h_counts[0] > 0 ? ds_prefill(model, kv, 0, h_tokens, h_counts[0], d_tok_out, stream) : ok();
    const int B = kv->B;
    std::vector<int64_t> start(B + 1, 0);
    int max_n = 0;
    for (int b = 0; b < B; b++) {
        if (h_counts[b] < 0) return fail(DS_ERR_INVALID_ARG, "h_counts[%d] < 0", b);
        if (kv->mirror[b] + static_cast<int64_t>(h_counts[b]) > kv->T)
            return fail(DS_ERR_CONTEXT_FULL, "sequence %d: %d + %d positions exceed %d", b, kv->mirror[b],
                        h_counts[b], kv->T);
        start[b + 1] = start[b] + h_counts[b];
        max_n = std::max(max_n, h_counts[b]);
    }
    if (start[B] > 0 && !h_tokens) return fail(DS_ERR_INVALID_ARG, "h_tokens is NULL");
    for (int64_t i = 0; i < start[B]; i++)
        if (h_tokens[i] < 0 || h_tokens[i] >= kv->s.V)
            return fail(DS_ERR_BAD_TOKEN, "token %d at %lld outside [0, %d)", h_tokens[i],
                        static_cast<long long>(i), kv->s.V);
    hipStream_t st = static_cast<hipStream_t>(stream);
    std::vector<ds::BeginList> lists;
    for (int j = 0; j < max_n; j++) {
        lists.clear();
        int items = 0;
        bool any_last = false;
        int max_ctx = 0;
        for (int b = 0; b < B; b++) {
            if (h_counts[b] <= j) continue;
            if (lists.empty() || lists.back().n == ds::kMaxItems) {
                lists.emplace_back();
                lists.back().item0 = items;
                lists.back().by_value = 1;
            }
            ds::BeginList& l = lists.back();
            l.slot[l.n] = b;
            l.tok[l.n] = h_tokens[start[b] + j];
            l.last[l.n] = (j == h_counts[b] - 1);
            any_last |= l.last[l.n] != 0;
            max_ctx = std::max(max_ctx, kv->mirror[b] + j + 1);
            l.n++;
            items++;
        }
        hipError_t e = ds::enqueue_step(kv->s, model->ptrs, lists.data(), static_cast<int>(lists.size()),
                                        nullptr, items, any_last, ds::short_rows(kv->s, max_ctx), d_tok_out,
                                        st);
        if (e != hipSuccess) {
            // the passes already enqueued advance the device lengths
            for (int b = 0; b < B; b++) kv->mirror[b] += std::min(h_counts[b], j);
            return hip_fail(e, "prefill_batch");
        }
    }
    for (int b = 0; b < B; b++) kv->mirror[b] += h_counts[b];
    return ok();
}

ds_status ds_decode_step(ds_model* model, ds_kv* kv, const int32_t* d_tok_in, int32_t* d_tok_out,
                         void* stream) {
    if (!model || !kv || kv->model != model) return fail(DS_ERR_INVALID_ARG, "model/kv mismatch");
    if (!d_tok_in || !d_tok_out) return fail(DS_ERR_INVALID_ARG, "token buffers are NULL");
    if (!aligned(d_tok_in, 4) || !aligned(d_tok_out, 4)) return fail(DS_ERR_ALIGNMENT, "token buffers");
    for (int b = 0; b < kv->B; b++)
        if (kv->mirror[b] >= kv->T)
            return fail(DS_ERR_CONTEXT_FULL, "sequence %d already holds all %d positions", b, kv->T);
    hipStream_t st = static_cast<hipStream_t>(stream);
    ds::BeginList list;
    list.n = kv->B;
    list.item0 = 0;
    list.by_value = 0;
    int max_ctx = 0;
    for (int b = 0; b < kv->B; b++) max_ctx = std::max(max_ctx, kv->mirror[b] + 1);
    const bool persist = kv->B == 1 && max_ctx <= kv->persist_ctx;
    const int nload = persist ? -1 : ds::short_rows(kv->s, max_ctx);  // -1 marks the persistent step
    auto enqueue = [&]() -> hipError_t {
        if (persist) return ds::enqueue_persist(kv->s, kv->pa, d_tok_in, 0, d_tok_out, max_ctx, st);
        return ds::enqueue_step(kv->s, model->ptrs, &list, 1, d_tok_in, kv->B, true, nload, d_tok_out, st);
    };
    hipError_t e = hipSuccess;
    // the single-launch step goes straight to the stream: replaying a one-node
    // graph only adds to it (about 6 us per step measured)
    if (kv->dispatch == 1 && st != nullptr && !persist) {
        GraphEntry* ge = nullptr;
        for (GraphEntry& g : kv->graphs)
            if (g.nload == nload && g.stream == st && g.tok_in == d_tok_in && g.tok_out == d_tok_out) ge = &g;
        if (!ge) {
            GraphEntry g{nload, st, d_tok_in, d_tok_out, nullptr, nullptr};
            e = hipStreamBeginCapture(st, hipStreamCaptureModeThreadLocal);
            if (e != hipSuccess) return hip_fail(e, "hipStreamBeginCapture");
            hipError_t ee = enqueue();
            e = hipStreamEndCapture(st, &g.graph);
            if (ee != hipSuccess) return hip_fail(ee, "capture decode step");
            if (e != hipSuccess) return hip_fail(e, "hipStreamEndCapture");
            e = hipGraphInstantiate(&g.exec, g.graph, nullptr, nullptr, 0);
            if (e != hipSuccess) {
                (void)hipGraphDestroy(g.graph);
                return hip_fail(e, "hipGraphInstantiate");
            }
            kv->graphs.push_back(g);
            ge = &kv->graphs.back();
        }
        e = hipGraphLaunch(ge->exec, st);
        if (e != hipSuccess) return hip_fail(e, "hipGraphLaunch");
    } else {
        e = enqueue();
        if (e != hipSuccess) return hip_fail(e, "decode step");
    }
    for (int b = 0; b < kv->B; b++) kv->mirror[b] += 1;
    kv->stepped = true;
    kv->last_nload = persist ? ds::short_rows(kv->s, max_ctx) : nload;
    return ok();
}

int32_t ds_kv_cache_single_launch_ctx(const ds_kv* kv) { return kv ? kv->persist_ctx : -1; }

ds_status ds_bench_kernel(ds_model* model, ds_kv* kv, int32_t which, int32_t layer, int32_t reps,
                          void* stream) {
    if (!model || !kv || kv->model != model) return fail(DS_ERR_INVALID_ARG, "model/kv mismatch");
    if (!kv->stepped) return fail(DS_ERR_STATE, "run ds_decode_step before ds_bench_kernel");
    if (which < 0 || which > 7) return fail(DS_ERR_INVALID_ARG, "which must be in [0, 7]");
    if (layer < 0 || layer >= kv->s.L) return fail(DS_ERR_INVALID_ARG, "layer outside [0, L)");
    if (reps < 1) return fail(DS_ERR_INVALID_ARG, "reps must be positive");
    hipStream_t st = static_cast<hipStream_t>(stream);
    if (which == ds::K_FLOOR) {
        if (kv->B != 1 || kv->mirror[0] + 1 > kv->persist_ctx)
            return fail(DS_ERR_STATE, "the handoff floor needs a batch-1 cache whose next step is a single launch");
        for (int r = 0; r < reps; r++) {
            hipError_t e = ds::enqueue_persist_floor(kv->s, kv->pa, kv->mirror[0] + 1, st);
            if (e != hipSuccess) return hip_fail(e, "bench floor");
        }
        return ok();
    }
    for (int r = 0; r < reps; r++) {
        if (kv->last_nload > 0 && !(kv->s.mm_ok && kv->B >= ds::kMmMin) &&
            (which == ds::K_ATTN || which == ds::K_COMBINE))
            return fail(DS_ERR_STATE, "kernel %d is not part of a short-context step", which);
        if (which == ds::K_COMBINE && ds::attn_full(kv->s, kv->B))
            return fail(DS_ERR_STATE, "attention runs one block per (sequence, group) here: no combine launch");
        hipError_t e = ds::enqueue_kernel(which, (layer + r) % kv->s.L, kv->s, model->ptrs, kv->B, kv->last_nload, st);
        if (e != hipSuccess) return hip_fail(e, "bench kernel");
    }
    return ok();
}

ds_status ds_bench_stream(const void* d_src, size_t bytes, uint32_t* d_out, int32_t reps, void* stream) {
    if (!d_src || !d_out) return fail(DS_ERR_INVALID_ARG, "NULL argument");
    if (!aligned(d_src, 16) || !aligned(d_out, 4)) return fail(DS_ERR_ALIGNMENT, "source must be 16-byte aligned");
    if (bytes == 0 || bytes % 16) return fail(DS_ERR_INVALID_ARG, "bytes must be a positive multiple of 16");
    if (reps < 1) return fail(DS_ERR_INVALID_ARG, "reps must be positive");
    hipError_t e = ds::enqueue_stream_read(d_src, bytes, d_out, reps, static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return hip_fail(e, "bench stream");
    return ok();
}

ds_status ds_logits(const ds_kv* kv, float* d_out, void* stream) {
    if (!kv || !d_out) return fail(DS_ERR_INVALID_ARG, "NULL argument");
    hipError_t e = hipMemcpyAsync(d_out, kv->s.logits, sizeof(float) * kv->B * static_cast<size_t>(kv->s.V),
                                  hipMemcpyDeviceToDevice, static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return hip_fail(e, "logits copy");
    return ok();
}

}  // extern "C"

namespace {

// Argument checks shared by ds_sample and ds_sample_noalloc; on success the
// effective top-k (at most V) is in *k_out.
ds_status check_sample_args(int V, const float* d_uniform, float temperature, int32_t top_k, float top_p,
                            const int32_t* d_tok_out, int* k_out) {
    if (!d_uniform || !d_tok_out) return fail(DS_ERR_INVALID_ARG, "NULL argument");
    if (!aligned(d_uniform, 4) || !aligned(d_tok_out, 4)) return fail(DS_ERR_ALIGNMENT, "uniform / token buffers");
    if (!(temperature > 0.0f) || !(temperature < INFINITY))
        return fail(DS_ERR_INVALID_ARG, "temperature %g: needs 0 < t < inf (0 is the greedy step itself)",
                    static_cast<double>(temperature));
    if (top_k < 0) return fail(DS_ERR_INVALID_ARG, "top_k %d < 0", top_k);
    if (!(top_p > 0.0f && top_p <= 1.0f))
        return fail(DS_ERR_INVALID_ARG, "top_p %g outside (0, 1]", static_cast<double>(top_p));
    const int k = std::min(top_k, V);
    if (k > ds::kMaxTopK) return fail(DS_ERR_UNSUPPORTED, "top_k %d above %d", top_k, ds::kMaxTopK);
    if (k == 0 && top_p < 1.0f) return fail(DS_ERR_UNSUPPORTED, "top_p below 1 needs top_k >= 1");
    if (V > ds::kSampleMaxV) return fail(DS_ERR_UNSUPPORTED, "vocabulary %d above %d", V, ds::kSampleMaxV);
    *k_out = k;
    return DS_OK;
}

// The sampling scratch of ds_sample_noalloc: DS_SAMPLE_NOALLOC_MAX_ROWS rows
// of the per-row words the two-kernel sampler uses (2.5 MiB), held by every
// device the library runs on until the process ends.  Host code never uses
// the array's name as an address: each device's address comes from
// hipGetSymbolAddress, once per device, with that device current.
constexpr size_t kNoAllocRowWords = static_cast<size_t>(ds::kSampleMaxV) / 1024 + 4096;
static __device__ __align__(256) uint64_t scratch[DS_SAMPLE_NOALLOC_MAX_ROWS * kNoAllocRowWords];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
uint64_t* g_scratch_ptr[kMaxDevices] = {};

// The current device's copy of `scratch`, or nullptr with the reason in g_err.
uint64_t* device_scratch() {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) {
        hip_fail(e, "hipGetDevice");
        return nullptr;
    }
    if (dev < 0 || dev >= kMaxDevices) {
        fail(DS_ERR_UNSUPPORTED, "device %d: at most %d devices", dev, kMaxDevices);
        return nullptr;
    }
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void* ptr = nullptr;
        e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
        if (e != hipSuccess || !ptr) {
            hip_fail(e != hipSuccess ? e : hipErrorInvalidSymbol, "hipGetSymbolAddress(scratch)");
            return nullptr;
        }
        g_scratch_ptr[dev] = static_cast<uint64_t*>(ptr);
    }
    return g_scratch_ptr[dev];
}

}  // namespace

extern "C" {

ds_status ds_sample(const ds_kv* kv, const float* d_uniform, float temperature, int32_t top_k, float top_p,
                    int32_t* d_tok_out, void* stream) {
    if (!kv) return fail(DS_ERR_INVALID_ARG, "NULL argument");
    int k = 0;
    ds_status cs = check_sample_args(kv->s.V, d_uniform, temperature, top_k, top_p, d_tok_out, &k);
    if (cs != DS_OK) return cs;
    const ds::SampleParams prm{temperature, k, top_p};
    // scratch: the argmax-key rows of the workspace, which nothing reads between steps
    hipError_t e = ds::enqueue_sample(kv->s.logits, kv->B, kv->s.V, d_uniform, prm,
                                      reinterpret_cast<uint64_t*>(kv->s.keys), ds::kMaxArgmaxBlocks, d_tok_out,
                                      static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return hip_fail(e, "sample");
    return ok();
}

ds_status ds_sample_noalloc(const float* d_logits, int32_t B, int32_t V, const float* d_uniform, float temperature,
                            int32_t top_k, float top_p, int32_t* d_tok_out, void* stream) {
    if (!d_logits) return fail(DS_ERR_INVALID_ARG, "NULL argument");
    if (!aligned(d_logits, 4)) return fail(DS_ERR_ALIGNMENT, "logits buffer");
    if (B < 0 || V <= 0) return fail(DS_ERR_INVALID_ARG, "B %d, V %d: need B >= 0 and V > 0", B, V);
    if (B > DS_SAMPLE_NOALLOC_MAX_ROWS)
        return fail(DS_ERR_UNSUPPORTED, "B %d above %d rows of the library's sampling scratch (use ds_sample)", B,
                    DS_SAMPLE_NOALLOC_MAX_ROWS);
    int k = 0;
    ds_status cs = check_sample_args(V, d_uniform, temperature, top_k, top_p, d_tok_out, &k);
    if (cs != DS_OK) return cs;
    if (B == 0) return ok();
    uint64_t* ptr = device_scratch();
    if (!ptr) return DS_ERR_HIP;
    static_assert(kNoAllocRowWords >= 1, "row words");
    const ds::SampleParams prm{temperature, k, top_p};
    hipError_t e = ds::enqueue_sample(d_logits, B, V, d_uniform, prm, ptr, kNoAllocRowWords, d_tok_out,
                                      static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return hip_fail(e, "sample_noalloc");
    return ok();
}

ds_status ds_set_dispatch(ds_kv* kv, int32_t mode) {
    if (!kv) return fail(DS_ERR_INVALID_ARG, "kv is NULL");
    if (mode != 0 && mode != 1) return fail(DS_ERR_INVALID_ARG, "mode must be 0 (eager) or 1 (graph)");
    kv->dispatch = mode;
    return ok();
}

}  // extern "C"
