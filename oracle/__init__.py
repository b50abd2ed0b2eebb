"""Python access to the reference decoder in ``oracle.c``.

TEST INFRASTRUCTURE ONLY.  The tests, the smoke check and the benchmark's
CPU-baseline leg are the only callers.  The HIP library never imports this
package and this package never imports the HIP library.

The shared object is built by ``build()`` with gcc in strict IEEE mode
(``-ffp-contract=off -fno-fast-math``): every operation in ``oracle.c`` is one
binary32 rounding, in the order written there.
"""
from __future__ import annotations

import ctypes as C
import os
import subprocess

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
SRCS = [os.path.join(HERE, "oracle.c"), os.path.join(HERE, "batch.c")]
LIB = os.path.join(HERE, "liboracle.so")
STRICT_FLAGS = ["-O2", "-std=c11", "-ffp-contract=off", "-fno-fast-math", "-fPIC", "-shared", "-pthread"]


ORC_F32, ORC_BF16, ORC_Q8, ORC_Q4 = 0, 1, 2, 3


def build(out: str = LIB, extra_flags: list[str] | None = None) -> str:
    """Compile oracle.c and batch.c into a shared object (``extra_flags``
    replaces nothing, it is appended: tests use it to build a deliberately
    contracted copy)."""
    cmd = ["gcc", *STRICT_FLAGS, *(extra_flags or []), *SRCS, "-o", out + ".tmp", "-lm"]
    subprocess.run(cmd, check=True, cwd=HERE)
    os.replace(out + ".tmp", out)
    return out


class OrcConfig(C.Structure):
    _fields_ = [
        ("dim", C.c_int32), ("n_layers", C.c_int32), ("n_heads", C.c_int32),
        ("n_kv_heads", C.c_int32), ("head_dim", C.c_int32), ("hidden_dim", C.c_int32),
        ("vocab_size", C.c_int32), ("tied_embeddings", C.c_int32), ("weight_dtype", C.c_int32),
        ("rope_theta", C.c_float), ("norm_eps", C.c_float), ("cache_dtype", C.c_int32),
    ]


def config_of(shape) -> OrcConfig:
    """OrcConfig from a synth.ModelShape (same field order)."""
    return OrcConfig(*shape.as_tuple())


_F = np.ctypeslib.ndpointer(dtype=np.float32, flags="C_CONTIGUOUS")
_I = np.ctypeslib.ndpointer(dtype=np.int32, flags="C_CONTIGUOUS")
_U8 = np.ctypeslib.ndpointer(dtype=np.uint8, flags="C_CONTIGUOUS")
_U16 = np.ctypeslib.ndpointer(dtype=np.uint16, flags="C_CONTIGUOUS")


def load(path: str = LIB):
    if not os.path.exists(path):
        build(path)
    lib = C.CDLL(path)
    P = C.POINTER(OrcConfig)
    sig = {
        "orc_widen_bf16": (C.c_float, [C.c_uint16]),
        "orc_round_bf16": (C.c_float, [C.c_float]),
        "orc_widen_bf16_array": (None, [_U16, _F, C.c_size_t]),
        "orc_matvec": (None, [C.c_void_p, C.c_int32, C.c_int32, C.c_int32, _F, _F]),
        "orc_weight": (C.c_float, [C.c_void_p, C.c_int32, C.c_size_t, C.c_size_t, C.c_size_t, C.c_size_t]),
        "orc_rmsnorm": (None, [_F, _F, C.c_int32, C.c_float, _F]),
        "orc_rope_angles": (None, [C.c_int32, C.c_int32, C.c_float, _F, _F]),
        "orc_rope_apply": (None, [_F, C.c_int32, _F, _F]),
        "orc_attend": (None, [_F, _F, _F, C.c_int32, C.c_int32, _F, _F]),
        "orc_silu_mul": (C.c_float, [C.c_float, C.c_float]),
        "orc_argmax": (C.c_int32, [_F, C.c_int32]),
        "orc_sample": (C.c_int32, [_F, C.c_int32, C.c_float, C.c_int32, C.c_float, C.c_double, _I,
                                   C.POINTER(C.c_double), C.POINTER(C.c_int32)]),
        "orc_n_tensors": (C.c_int32, [P]),
        "orc_tensor_offsets": (C.c_size_t, [P, C.POINTER(C.c_size_t), C.c_int32]),
        "orc_cache_index": (C.c_size_t, [P, C.c_int32, C.c_int32, C.c_int32, C.c_int32, C.c_int32,
                                         C.c_int32, C.c_int32]),
        "orc_forward": (C.c_int32, [P, _U8, _F, C.c_int32, C.c_int32, C.c_int32, C.c_int32,
                                    C.c_int32, _F]),
        "orc_decode_step": (C.c_int32, [P, _U8, _F, C.c_int32, C.c_int32, _I, _I, _I, _F]),
        "orc_generate": (C.c_int32, [P, _U8, _F, C.c_int32, C.c_int32, C.c_int32, _I, C.c_int32,
                                     C.c_int32, C.c_int32, _I, C.c_void_p, C.POINTER(C.c_int64)]),
        "orc_forward_items": (C.c_int32, [P, _U8, _F, C.c_int32, C.c_int32, C.c_int32, _I, _I, _I, _I,
                                          C.c_void_p, _I, C.c_int32]),
    }
    for name, (res, args) in sig.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    return lib


_lib = None


def lib():
    global _lib
    if _lib is None:
        _lib = load()
    return _lib


# ---- thin numpy-level helpers ------------------------------------------------

def matvec(W: np.ndarray, x: np.ndarray) -> np.ndarray:
    """W: float32 or uint16 (bf16 bits) [n_out][n_in]; x float32 [n_in]."""
    W = np.ascontiguousarray(W)
    wd = 1 if W.dtype == np.uint16 else 0
    if wd == 0:
        W = W.astype(np.float32, copy=False)
    y = np.zeros(W.shape[0], np.float32)
    lib().orc_matvec(W.ctypes.data, wd, W.shape[0], W.shape[1],
                     np.ascontiguousarray(x, np.float32), y)
    return y


def rmsnorm(x, g, eps):
    y = np.zeros(len(x), np.float32)
    lib().orc_rmsnorm(np.ascontiguousarray(x, np.float32), np.ascontiguousarray(g, np.float32),
                      len(x), eps, y)
    return y


def rope_angles(pos, head_dim, theta):
    c = np.zeros(head_dim // 2, np.float32)
    s = np.zeros(head_dim // 2, np.float32)
    lib().orc_rope_angles(pos, head_dim, theta, c, s)
    return c, s


def rope_apply(v, pos, theta):
    v = np.array(v, np.float32)
    c, s = rope_angles(pos, len(v), theta)
    lib().orc_rope_apply(v, len(v), c, s)
    return v


def attend(q, K, V):
    K = np.ascontiguousarray(K, np.float32)
    Vv = np.ascontiguousarray(V, np.float32)
    n, D = K.shape
    probs = np.zeros(n, np.float32)
    out = np.zeros(D, np.float32)
    lib().orc_attend(np.ascontiguousarray(q, np.float32), K, Vv, n, D, probs, out)
    return out, probs


def argmax(v):
    v = np.ascontiguousarray(v, np.float32)
    return int(lib().orc_argmax(v, len(v)))


def sample(logits, temperature, top_k, top_p, u):
    """orc_sample: (token, kept candidates in draw order, their normalised
    cumulative weights)."""
    v = np.ascontiguousarray(logits, np.float32)
    cand = np.zeros(len(v), np.int32)
    cum = np.zeros(len(v), np.float64)
    n = C.c_int32(0)
    tok = lib().orc_sample(v, len(v), float(temperature), int(top_k), float(top_p), float(u), cand,
                           cum.ctypes.data_as(C.POINTER(C.c_double)), C.byref(n))
    if tok < 0:
        raise ValueError("orc_sample: bad argument")
    return int(tok), cand[:n.value].copy(), cum[:n.value].copy()


def default_threads() -> int:
    """Host threads for the batched evaluation: the CPUs this process may use,
    at most OMP_NUM_THREADS when that is set, and at most 16."""
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    env = os.environ.get("OMP_NUM_THREADS", "")
    if env.isdigit() and int(env) > 0:
        n = min(n, int(env))
    return max(1, min(n, 16))


def tensor_offsets(shape):
    cfg = config_of(shape)
    n = lib().orc_n_tensors(C.byref(cfg))
    off = (C.c_size_t * n)()
    total = lib().orc_tensor_offsets(C.byref(cfg), off, n)
    return list(off), int(total)


def cache_size(shape, B, T):
    return shape.n_layers * 2 * B * shape.n_kv_heads * T * shape.head_dim


class Model:
    """The reference decoder over one host weight arena and one host cache."""

    def __init__(self, shape, arena: np.ndarray, B: int, T: int):
        self.shape, self.B, self.T = shape, B, T
        self.cfg = config_of(shape)
        self.arena = np.ascontiguousarray(arena, np.uint8)
        self.cache = np.zeros(cache_size(shape, B, T), np.float32)

    def cache_view(self):
        s = self.shape
        return self.cache.reshape(s.n_layers, 2, self.B, s.n_kv_heads, self.T, s.head_dim)

    def forward(self, b, pos, token):
        logits = np.zeros(self.shape.vocab_size, np.float32)
        r = lib().orc_forward(C.byref(self.cfg), self.arena, self.cache, self.B, self.T, b, pos,
                              int(token), logits)
        if r < 0:
            raise ValueError(f"orc_forward failed ({r})")
        return r, logits

    def decode_step(self, lengths: np.ndarray, tok_in: np.ndarray):
        """Returns (tok_out, logits [B][V]); lengths (int32) advance in place."""
        B, V = self.B, self.shape.vocab_size
        tok_out = np.zeros(B, np.int32)
        logits = np.zeros(B * V, np.float32)
        r = lib().orc_decode_step(C.byref(self.cfg), self.arena, self.cache, B, self.T, lengths,
                                  np.ascontiguousarray(tok_in, np.int32), tok_out, logits)
        if r < 0:
            raise ValueError(f"orc_decode_step failed ({r})")
        return tok_out, logits.reshape(B, V)

    # ---- the batched evaluation (batch.c): the same numbers, computed for
    # many positions at once --------------------------------------------------
    def forward_items(self, seq, pos, tok, want, threads=None):
        """orc_forward for every item (seq[i], pos[i], tok[i]), bit for bit,
        layer by layer for all items together.  Returns (tok_out [n] with -1
        where not wanted, logits [n_wanted][V] in item order)."""
        seq = np.ascontiguousarray(seq, np.int32)
        pos = np.ascontiguousarray(pos, np.int32)
        tok = np.ascontiguousarray(tok, np.int32)
        want = np.ascontiguousarray(want, np.int32)
        n = len(seq)
        assert len(pos) == n and len(tok) == n and len(want) == n
        nw = int(np.count_nonzero(want))
        logits = np.zeros((max(nw, 1), self.shape.vocab_size), np.float32)
        tok_out = np.zeros(max(n, 1), np.int32)
        r = lib().orc_forward_items(C.byref(self.cfg), self.arena, self.cache, self.B, self.T, n, seq, pos,
                                    tok, want, logits.ctypes.data, tok_out,
                                    int(threads or default_threads()))
        if r < 0:
            raise ValueError(f"orc_forward_items failed ({r})")
        return tok_out[:n], logits[:nw]

    def prefill_fast(self, b, tokens, start=0, chunk=4096, threads=None):
        """Positions start.. of sequence b fed with `tokens`, in chunks of
        `chunk` items; returns (greedy token, logits) of the last position."""
        tokens = np.asarray(tokens, np.int32)
        n = len(tokens)
        tok, lg = None, None
        for c0 in range(0, n, chunk):
            c1 = min(n, c0 + chunk)
            k = c1 - c0
            want = np.zeros(k, np.int32)
            if c1 == n:
                want[-1] = 1
            t, l = self.forward_items(np.full(k, b, np.int32), np.arange(start + c0, start + c1, dtype=np.int32),
                                      tokens[c0:c1], want, threads)
            if c1 == n:
                tok, lg = int(t[-1]), l[0]
        return tok, lg

    def decode_fast(self, lengths: np.ndarray, tok_in: np.ndarray, threads=None):
        """decode_step for every sequence at once: same results, bit for bit."""
        B = self.B
        tok_out, logits = self.forward_items(np.arange(B, dtype=np.int32), lengths, tok_in,
                                             np.ones(B, np.int32), threads)
        lengths += 1
        return tok_out, logits

    def generate(self, b, prompt, n_new, uncached=False, want_logits=True):
        V = self.shape.vocab_size
        toks = np.zeros(n_new, np.int32)
        logits = np.zeros(n_new * V, np.float32) if want_logits else None
        passes = C.c_int64(0)
        r = lib().orc_generate(C.byref(self.cfg), self.arena, self.cache, self.B, self.T, b,
                               np.ascontiguousarray(prompt, np.int32), len(prompt), n_new,
                               1 if uncached else 0, toks,
                               logits.ctypes.data if logits is not None else None,
                               C.byref(passes))
        if r < 0:
            raise ValueError(f"orc_generate failed ({r})")
        return toks, (logits.reshape(n_new, V) if logits is not None else None), passes.value
