"""Seeded synthetic inputs for the decode step: model shapes, weight arenas,
prompts and per-sequence cache lengths.

This module serves both the reference decoder under ``oracle/`` and the HIP
library, so that both read identical bytes.  It holds none of the decode
step's arithmetic: it draws random numbers, rounds them to the storage dtype,
and lays them out in the canonical arena format.

Arena format (one contiguous byte buffer, tensors in this order, each starting
on a 256-byte boundary; matrices row-major ``[out][in]``):

    token_emb [V][d]
    per layer: attn_norm [d], wq [H*D][d], wk [Hkv*D][d], wv [Hkv*D][d],
               wo [d][H*D], ffn_norm [d], w1 [F][d], w3 [F][d], w2 [d][F]
    output_norm [d]
    wcls [V][d]            (only when the embeddings are not tied)

The order and the shapes follow the weight listing of "simple-llm / kasahare"
(PyPI README 0.4.0), section "On-disk model format (.sllm)"; the untied head
is appended after ``output_norm``.  Matrices are bf16 (stored as uint16) or
fp32; norm gains are always fp32.  bf16 is the top half of an fp32 value
("GOTOken: An Inference Engine in QBasic", section "Loading the model and
tokenizer"); the generator rounds fp32 draws to bf16 to nearest-even.
"""
from __future__ import annotations

import dataclasses
import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np

ALIGN = 256
F32, BF16, Q8, Q4 = 0, 1, 2, 3
Q8_BLOCK = 32  # weights per fp32 scale of a Q8 or Q4 matrix row
_CHUNK = 1 << 22  # elements per independent random stream


@dataclasses.dataclass(frozen=True)
class ModelShape:
    dim: int
    n_layers: int
    n_heads: int
    n_kv_heads: int
    head_dim: int
    hidden_dim: int
    vocab_size: int
    tied_embeddings: int
    weight_dtype: int  # F32, BF16, Q8 or Q4
    rope_theta: float
    norm_eps: float
    cache_dtype: int = F32  # F32, or BF16: key/value rows rounded to bf16 when stored

    @property
    def q_rows(self) -> int:
        return self.n_heads * self.head_dim

    @property
    def kv_rows(self) -> int:
        return self.n_kv_heads * self.head_dim

    @property
    def wbytes(self) -> int:
        """Bytes per matrix element (Q8: the int8 value, Q4: half a byte, the scale not counted)."""
        return {BF16: 2, Q8: 1, Q4: 0.5}.get(self.weight_dtype, 4)

    def as_tuple(self):
        return dataclasses.astuple(self)


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    model: ModelShape
    model_seed: int
    batch: int
    ctx: int               # allocated cache positions T
    prompt_len: int        # per sequence (ignored when lengths_seed is set)
    prompt_seed: int
    decode_calls: int
    lengths_seed: int = -1  # ragged batch: prompt lengths drawn from this seed
    max_prompt: int = 0     # ragged batch: lengths uniform in [1, max_prompt]
    description: str = ""


TINY = ModelShape(64, 2, 4, 2, 16, 172, 256, 1, F32, 10000.0, 1e-5)
M135 = ModelShape(576, 30, 9, 3, 64, 1536, 49152, 1, BF16, 100000.0, 1e-5)
M8B = ModelShape(4096, 32, 32, 8, 128, 14336, 128256, 0, BF16, 500000.0, 1e-5)

WORKLOADS = {
    w.name: w
    for w in [
        Workload("tiny_p5", TINY, 1, 1, 128, 5, 101, 7,
                 description="tiny random Llama, fp32 weights, 5-token prompt, 8 new tokens"),
        Workload("llama135m_p5", M135, 2, 1, 1024, 5, 102, 7,
                 description="135M-shaped Llama, bf16 weights, batch 1, 5-token prompt, 8 new tokens"),
        Workload("llama135m_p1000", M135, 2, 1, 1024, 1000, 103, 23,
                 description="135M-shaped Llama, batch 1, 1000-token prompt, 23 decode steps"),
        Workload("llama135m_b64", M135, 2, 64, 1024, 0, 104, 16, lengths_seed=204, max_prompt=1008,
                 description="135M-shaped Llama, 64 sequences, prompt lengths uniform in [1,1008], 16 decode steps"),
        Workload("llama8b_p4096", M8B, 3, 1, 4160, 4096, 105, 32,
                 description="8B-shaped Llama, untied head, batch 1, 4096-token prompt, 32 decode steps"),
    ]
}


def tensor_table(m: ModelShape):
    """Canonical arena layout: list of (name, byte offset, shape, dtype code)."""
    d, F, V = m.dim, m.hidden_dim, m.vocab_size
    mats = [("token_emb", (V, d), m.weight_dtype)]
    for l in range(m.n_layers):
        mats += [
            (f"l{l}.attn_norm", (d,), F32),
            (f"l{l}.wq", (m.q_rows, d), m.weight_dtype),
            (f"l{l}.wk", (m.kv_rows, d), m.weight_dtype),
            (f"l{l}.wv", (m.kv_rows, d), m.weight_dtype),
            (f"l{l}.wo", (d, m.q_rows), m.weight_dtype),
            (f"l{l}.ffn_norm", (d,), F32),
            (f"l{l}.w1", (F, d), m.weight_dtype),
            (f"l{l}.w3", (F, d), m.weight_dtype),
            (f"l{l}.w2", (d, F), m.weight_dtype),
        ]
    mats.append(("output_norm", (d,), F32))
    if not m.tied_embeddings:
        mats.append(("wcls", (V, d), m.weight_dtype))
    out, off = [], 0
    for name, shape, dt in mats:
        out.append((name, off, shape, dt))
        n = tensor_bytes(shape, dt)
        off = (off + n + ALIGN - 1) // ALIGN * ALIGN
    return out, off


def tensor_bytes(shape, dt) -> int:
    """Bytes of one arena tensor.  Q8 [rows][cols]: int8 values, then fp32
    scales [rows][cols / 32] from the next 256-byte boundary."""
    n = int(np.prod(shape))
    if dt == Q8:
        return (n + ALIGN - 1) // ALIGN * ALIGN + 4 * (n // Q8_BLOCK)
    if dt == Q4:
        return (n // 2 + ALIGN - 1) // ALIGN * ALIGN + 4 * (n // Q8_BLOCK)
    return n * (2 if dt == BF16 else 4)


def _values_bytes(n, dt) -> int:
    """Bytes of the values of an n-element Q8 / Q4 matrix, before its scales."""
    return n if dt == Q8 else n // 2


def quantize_q4(w: np.ndarray):
    """Block-quantise fp32 weights to 4-bit values packed two per byte (even
    index in the low nibble, two's complement) and fp32 scales: s = max|w| / 7
    per 32-weight block, q = round(w / s) to nearest even, clipped to [-8, 7]."""
    b = w.reshape(-1, Q8_BLOCK).astype(np.float32)
    amax = np.abs(b).max(axis=1)
    sc = np.where(amax > 0, amax / np.float32(7.0), np.float32(1.0)).astype(np.float32)
    q = np.clip(np.rint(b / sc[:, None]), -8, 7).astype(np.int8).reshape(-1)
    return pack_q4(q), sc


def pack_q4(q: np.ndarray) -> np.ndarray:
    """Pack int values in [-8, 7] two per byte, even index in the low nibble."""
    u = (q.astype(np.int16) & 15).astype(np.uint8)
    return (u[0::2] | (u[1::2] << 4)).astype(np.uint8)


def quantize_q8(w: np.ndarray):
    """Block-quantise fp32 weights (a flat run of whole 32-weight blocks) to
    int8 values and fp32 scales: s = max|w| / 127 per block, q = round(w / s)
    to nearest even.  An all-zero block gets s = 1 and q = 0."""
    b = w.reshape(-1, Q8_BLOCK).astype(np.float32)
    amax = np.abs(b).max(axis=1)
    sc = np.where(amax > 0, amax / np.float32(127.0), np.float32(1.0)).astype(np.float32)
    q = np.clip(np.rint(b / sc[:, None]), -127, 127).astype(np.int8)
    return q.reshape(-1), sc


def arena_bytes(m: ModelShape) -> int:
    return tensor_table(m)[1]


def _round_bf16(f32: np.ndarray) -> np.ndarray:
    """Round fp32 to bf16 (nearest, ties to even); returns the uint16 bits."""
    u = f32.view(np.uint32)
    u = (u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)
    return u.astype(np.uint16)


def _fill_matrix(dst, n, dtype_code, seed, tensor_index, std, scales=None, exact=False):
    """Fill ``dst`` (flat view, n elements) with N(0, std) draws.

    Each block of ``_CHUNK`` elements has its own PCG64 stream keyed by
    (seed, tensor index, block index), so blocks can be drawn in parallel and
    the bytes do not depend on the thread count.
    """
    jobs = []
    for c0 in range(0, n, _CHUNK):
        jobs.append((c0, min(n, c0 + _CHUNK)))

    def one(job):
        c0, c1 = job
        g = np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, tensor_index, c0 // _CHUNK])))
        v = g.standard_normal(c1 - c0, dtype=np.float32)
        v *= np.float32(std)
        if exact:  # the grid k * step, |k| <= kmax: exact in bf16, and q = k with s = step in Q8 / Q4
            step, kmax = (1.0 / 512.0, 7) if exact == "q4" else (1.0 / 4096.0, 127)
            k = np.clip(np.rint(v / np.float32(step)), -kmax, kmax)
            if dtype_code == Q8:
                dst[c0:c1] = k.astype(np.int8)
                scales[c0 // Q8_BLOCK:c1 // Q8_BLOCK] = np.float32(step)
                return
            if dtype_code == Q4:
                dst[c0 // 2:c1 // 2] = pack_q4(k.astype(np.int8))
                scales[c0 // Q8_BLOCK:c1 // Q8_BLOCK] = np.float32(step)
                return
            v = (k * np.float32(step)).astype(np.float32)
        if dtype_code == BF16:
            dst[c0:c1] = _round_bf16(v)
        elif dtype_code == Q8:
            q, sc = quantize_q8(v)
            dst[c0:c1] = q
            scales[c0 // Q8_BLOCK:c1 // Q8_BLOCK] = sc
        elif dtype_code == Q4:
            q, sc = quantize_q4(v)
            dst[c0 // 2:c1 // 2] = q
            scales[c0 // Q8_BLOCK:c1 // Q8_BLOCK] = sc
        else:
            dst[c0:c1] = v
    return jobs, one


def make_arena(m: ModelShape, seed: int, std: float = 0.02, gain_sigma: float = 0.0,
               threads: int | None = None, out: np.ndarray | None = None, exact: bool | str = False) -> np.ndarray:
    """Generate the seeded weight arena as a flat uint8 array.

    Matrices ~ N(0, std) rounded to the storage dtype (Q8: block-quantised by
    quantize_q8).  Norm gains are 1.0, or 1 + N(0, gain_sigma) when
    ``gain_sigma`` > 0 (used to exercise the gain multiply in small tests).
    With ``exact`` every weight is k / 4096 for an integer |k| <= 127 (the
    N(0, std) draw rounded to that grid; with ``exact="q4"`` k / 512, |k| <= 7):
    a BF16 arena and a Q8 (Q4) arena of the same shape and seed then hold the
    same weight values.
    """
    table, total = tensor_table(m)
    arena = out if out is not None else np.zeros(total, dtype=np.uint8)
    assert arena.nbytes >= total
    threads = threads or min(16, os.cpu_count() or 1)
    all_jobs = []
    for ti, (name, off, shape, dt) in enumerate(table):
        n = int(np.prod(shape))
        if len(shape) == 1:
            g = arena[off:off + 4 * n].view(np.float32)
            if gain_sigma > 0:
                r = np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, ti, 0])))
                g[:] = np.float32(1.0) + r.standard_normal(n, dtype=np.float32) * np.float32(gain_sigma)
            else:
                g[:] = np.float32(1.0)
            continue
        scales = None
        if dt in (Q8, Q4):
            nv = _values_bytes(n, dt)
            flat = arena[off:off + nv].view(np.int8 if dt == Q8 else np.uint8)
            s0 = off + (nv + ALIGN - 1) // ALIGN * ALIGN
            scales = arena[s0:s0 + 4 * (n // Q8_BLOCK)].view(np.float32)
        else:
            esz = 2 if dt == BF16 else 4
            flat = arena[off:off + esz * n].view(np.uint16 if dt == BF16 else np.float32)
        jobs, fn = _fill_matrix(flat, n, dt, seed, ti, std, scales, exact)
        all_jobs += [(fn, j) for j in jobs]
    if threads <= 1 or len(all_jobs) <= 1:
        for fn, j in all_jobs:
            fn(j)
    else:
        with ThreadPoolExecutor(threads) as ex:
            list(ex.map(lambda p: p[0](p[1]), all_jobs))
    return arena


def views(m: ModelShape, arena: np.ndarray) -> dict:
    """Name -> numpy view (uint16 bf16 bits, or float32) into an arena."""
    table, _ = tensor_table(m)
    out = {}
    for name, off, shape, dt in table:
        n = int(np.prod(shape))
        if dt == BF16:
            out[name] = arena[off:off + 2 * n].view(np.uint16).reshape(shape)
        elif dt in (Q8, Q4):
            nv = _values_bytes(n, dt)
            s0 = off + (nv + ALIGN - 1) // ALIGN * ALIGN
            if dt == Q8:
                out[name] = arena[off:off + n].view(np.int8).reshape(shape)
            else:  # packed bytes, two values each
                out[name] = arena[off:off + nv].reshape(shape[0], shape[1] // 2)
            out[name + ".scale"] = arena[s0:s0 + 4 * (n // Q8_BLOCK)].view(np.float32).reshape(
                shape[0], shape[1] // Q8_BLOCK)
        else:
            out[name] = arena[off:off + 4 * n].view(np.float32).reshape(shape)
    return out


def prompts(w: Workload) -> list[np.ndarray]:
    """Per-sequence prompt token ids (int32), uniform over the vocabulary."""
    V = w.model.vocab_size
    if w.lengths_seed >= 0:
        lens = prompt_lengths(w)
        g = np.random.Generator(np.random.PCG64(w.prompt_seed))
        ids = g.integers(0, V, size=int(lens.sum()), dtype=np.int64).astype(np.int32)
        out, o = [], 0
        for n in lens:
            out.append(ids[o:o + n].copy())
            o += n
        return out
    g = np.random.Generator(np.random.PCG64(w.prompt_seed))
    return [g.integers(0, V, size=w.prompt_len, dtype=np.int64).astype(np.int32) for _ in range(w.batch)]


def prompt_lengths(w: Workload) -> np.ndarray:
    if w.lengths_seed >= 0:
        g = np.random.Generator(np.random.PCG64(w.lengths_seed))
        return g.integers(1, w.max_prompt + 1, size=w.batch, dtype=np.int64).astype(np.int32)
    return np.full(w.batch, w.prompt_len, dtype=np.int32)


def random_tokens(seed: int, n: int, vocab: int) -> np.ndarray:
    g = np.random.Generator(np.random.PCG64(seed))
    return g.integers(0, vocab, size=n, dtype=np.int64).astype(np.int32)


def small_shape(**kw) -> ModelShape:
    """A ModelShape derived from the tiny one with some fields replaced."""
    return dataclasses.replace(TINY, **kw)
