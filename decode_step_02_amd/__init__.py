"""Python binding of libds_decode.so, the gfx950 single-token Llama decode step.

Argument marshalling only: every step of the decode path runs in the HIP
kernels of the library.  torch supplies device memory and streams.  The
functions ``ds_*`` mirror the C ABI in ``include/ds_decode.h`` one to one;
``Model`` and ``KVCache`` are conveniences that allocate the caller-owned
buffers with torch at the sizes the library reports.

Importing this package fails loudly if the library has not been built
(``python decode_step_02_amd/build.py``).
"""
from __future__ import annotations

import ctypes as C
import os

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libds_decode.so")

DS_OK = 0
STATUS = {0: "DS_OK", -1: "DS_ERR_INVALID_ARG", -2: "DS_ERR_UNSUPPORTED", -3: "DS_ERR_ALIGNMENT",
          -4: "DS_ERR_CONTEXT_FULL", -5: "DS_ERR_BAD_TOKEN", -6: "DS_ERR_WORKSPACE", -7: "DS_ERR_HIP",
          -8: "DS_ERR_STATE", -9: "DS_ERR_DEVICE"}
DS_F32, DS_BF16, DS_Q8, DS_Q4 = 0, 1, 2, 3
DS_SAMPLE_NOALLOC_MAX_ROWS = 64  # include/ds_decode.h


class DSError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"{STATUS.get(status, status)}: {msg}")
        self.status = status


class ds_config(C.Structure):
    _fields_ = [
        ("dim", C.c_int32), ("n_layers", C.c_int32), ("n_heads", C.c_int32),
        ("n_kv_heads", C.c_int32), ("head_dim", C.c_int32), ("hidden_dim", C.c_int32),
        ("vocab_size", C.c_int32), ("tied_embeddings", C.c_int32), ("weight_dtype", C.c_int32),
        ("rope_theta", C.c_float), ("norm_eps", C.c_float), ("cache_dtype", C.c_int32),
    ]

    @classmethod
    def of(cls, shape):
        """From any object with the ds_config field names (e.g. synth.ModelShape)."""
        return cls(*[getattr(shape, n) for n, _ in cls._fields_])


if not os.path.exists(LIB_PATH):
    raise ImportError(f"{LIB_PATH} is missing: build it with `python decode_step_02_amd/build.py`")

_lib = C.CDLL(LIB_PATH)
_P = C.c_void_p
_CFG = C.POINTER(ds_config)
_SIGS = {
    "ds_weights_bytes": (C.c_size_t, [_CFG]),
    "ds_weights_count": (C.c_int32, [_CFG]),
    "ds_weights_offsets": (C.c_int, [_CFG, C.POINTER(C.c_size_t), C.c_int32]),
    "ds_kv_cache_bytes": (C.c_size_t, [_CFG, C.c_int32, C.c_int32]),
    "ds_workspace_bytes": (C.c_size_t, [_CFG, C.c_int32, C.c_int32]),
    "ds_load_weights": (C.c_int, [_CFG, _P, C.c_size_t, _P, C.POINTER(_P)]),
    "ds_model_destroy": (None, [_P]),
    "ds_kv_cache_create": (C.c_int, [_P, C.c_int32, C.c_int32, _P, C.c_size_t, _P, _P, C.c_size_t, _P,
                                     C.POINTER(_P)]),
    "ds_kv_cache_destroy": (None, [_P]),
    "ds_kv_cache_reset": (C.c_int, [_P, C.c_int32, _P]),
    "ds_kv_cache_set_lengths": (C.c_int, [_P, C.POINTER(C.c_int32), _P]),
    "ds_kv_cache_get_lengths": (C.c_int, [_P, C.POINTER(C.c_int32)]),
    "ds_kv_cache_replicate": (C.c_int, [_P, _P, C.c_int32, C.c_int32, C.c_int32, _P]),
    "ds_decode_step_rows": (C.c_int, [_P, _P, C.POINTER(C.c_int32), C.c_int32, _P, _P, _P]),
    "ds_kv_cache_check": (C.c_int, [_P, _P]),
    "ds_kv_cache_single_launch_ctx": (C.c_int32, [_P]),
    "ds_prefill": (C.c_int, [_P, _P, C.c_int32, C.POINTER(C.c_int32), C.c_int32, _P, _P]),
    "ds_prefill_batched": (C.c_int, [_P, _P, C.c_int32, C.POINTER(C.c_int32), C.c_int32, _P, _P]),
    "ds_prefill_batch": (C.c_int, [_P, _P, C.POINTER(C.c_int32), C.POINTER(C.c_int32), _P, _P]),
    "ds_decode_step": (C.c_int, [_P, _P, _P, _P, _P]),
    "ds_logits": (C.c_int, [_P, _P, _P]),
    "ds_sample": (C.c_int, [_P, _P, C.c_float, C.c_int32, C.c_float, _P, _P]),
    "ds_sample_noalloc": (C.c_int, [_P, C.c_int32, C.c_int32, _P, C.c_float, C.c_int32, C.c_float, _P, _P]),
    "ds_set_dispatch": (C.c_int, [_P, C.c_int32]),
    "ds_bench_kernel": (C.c_int, [_P, _P, C.c_int32, C.c_int32, C.c_int32, _P]),
    "ds_bench_stream": (C.c_int, [_P, C.c_size_t, _P, C.c_int32, _P]),
    "ds_last_error": (C.c_char_p, []),
}
for _name, (_res, _args) in _SIGS.items():
    _fn = getattr(_lib, _name)
    _fn.restype = _res
    _fn.argtypes = _args


def exported_symbols():
    return list(_SIGS)


def _check(status: int):
    if status != DS_OK:
        raise DSError(status, _lib.ds_last_error().decode())


def _i32(seq):
    arr = (C.c_int32 * len(seq))(*[int(v) for v in seq])
    return arr


def _ptr(t):
    return None if t is None else C.c_void_p(t.data_ptr())


def _stream(stream):
    if stream is None:
        import torch
        stream = torch.cuda.current_stream()
    return C.c_void_p(stream.cuda_stream)


# ---- the C ABI, one function each ---------------------------------------------

def ds_weights_bytes(cfg: ds_config) -> int:
    return _lib.ds_weights_bytes(C.byref(cfg))


def ds_weights_count(cfg: ds_config) -> int:
    return _lib.ds_weights_count(C.byref(cfg))


def ds_weights_offsets(cfg: ds_config) -> list[int]:
    n = ds_weights_count(cfg)
    off = (C.c_size_t * max(n, 1))()
    _check(_lib.ds_weights_offsets(C.byref(cfg), off, n))
    return list(off)[:n]


def ds_kv_cache_bytes(cfg: ds_config, B: int, T: int) -> int:
    return _lib.ds_kv_cache_bytes(C.byref(cfg), B, T)


def ds_workspace_bytes(cfg: ds_config, B: int, T: int) -> int:
    return _lib.ds_workspace_bytes(C.byref(cfg), B, T)


def ds_load_weights(cfg: ds_config, d_arena, stream=None):
    h = C.c_void_p()
    _check(_lib.ds_load_weights(C.byref(cfg), _ptr(d_arena), d_arena.numel() * d_arena.element_size(),
                                _stream(stream), C.byref(h)))
    return h


def ds_kv_cache_create(model, B, T, d_cache, d_lengths, d_workspace, stream=None):
    h = C.c_void_p()
    _check(_lib.ds_kv_cache_create(model, B, T, _ptr(d_cache), d_cache.numel() * d_cache.element_size(),
                                   _ptr(d_lengths), _ptr(d_workspace),
                                   d_workspace.numel() * d_workspace.element_size(), _stream(stream),
                                   C.byref(h)))
    return h


def ds_kv_cache_reset(kv, seq=-1, stream=None):
    _check(_lib.ds_kv_cache_reset(kv, seq, _stream(stream)))


def ds_kv_cache_set_lengths(kv, lengths, stream=None):
    _check(_lib.ds_kv_cache_set_lengths(kv, _i32(lengths), _stream(stream)))


def ds_kv_cache_get_lengths(kv, B):
    out = (C.c_int32 * B)()
    _check(_lib.ds_kv_cache_get_lengths(kv, out))
    return list(out)


def ds_kv_cache_single_launch_ctx(kv) -> int:
    return int(_lib.ds_kv_cache_single_launch_ctx(kv))


def ds_kv_cache_check(kv, stream=None):
    _check(_lib.ds_kv_cache_check(kv, _stream(stream)))


def ds_prefill(model, kv, seq, tokens, d_tok_out=None, stream=None):
    _check(_lib.ds_prefill(model, kv, seq, _i32(tokens), len(tokens), _ptr(d_tok_out), _stream(stream)))


def ds_prefill_batched(model, kv, seq, tokens, d_tok_out=None, stream=None):
    _check(_lib.ds_prefill_batched(model, kv, seq, _i32(tokens), len(tokens), _ptr(d_tok_out), _stream(stream)))


def ds_prefill_batch(model, kv, token_lists, d_tok_out=None, stream=None):
    flat = [int(t) for toks in token_lists for t in toks]
    counts = [len(toks) for toks in token_lists]
    _check(_lib.ds_prefill_batch(model, kv, _i32(flat) if flat else None, _i32(counts), _ptr(d_tok_out),
                                 _stream(stream)))


def ds_decode_step(model, kv, d_tok_in, d_tok_out, stream=None):
    _check(_lib.ds_decode_step(model, kv, _ptr(d_tok_in), _ptr(d_tok_out), _stream(stream)))


def ds_logits(kv, d_out, stream=None):
    _check(_lib.ds_logits(kv, _ptr(d_out), _stream(stream)))


def ds_set_dispatch(kv, mode: int):
    _check(_lib.ds_set_dispatch(kv, mode))


def ds_sample_noalloc(d_logits, B: int, V: int, d_uniform, temperature, top_k, top_p, d_tok_out, stream=None):
    """ds_sample from caller-owned logits [B][V], with the library's static
    device scratch instead of a workspace (allocates nothing)."""
    _check(_lib.ds_sample_noalloc(_ptr(d_logits), int(B), int(V), _ptr(d_uniform), float(temperature), int(top_k),
                                  float(top_p), _ptr(d_tok_out), _stream(stream)))


def ds_bench_kernel(model, kv, which, layer, reps, stream=None):
    _check(_lib.ds_bench_kernel(model, kv, which, layer, reps, _stream(stream)))


def ds_bench_stream(d_src, d_out, reps=1, stream=None):
    """Diagnostic streaming read of the whole tensor d_src (d_out: device
    int32/uint32 tensor of at least 2048 elements)."""
    _check(_lib.ds_bench_stream(_ptr(d_src), d_src.numel() * d_src.element_size(), _ptr(d_out), int(reps),
                                _stream(stream)))


def ds_model_destroy(model):
    _lib.ds_model_destroy(model)


def ds_kv_cache_destroy(kv):
    _lib.ds_kv_cache_destroy(kv)


def ds_last_error() -> str:
    return _lib.ds_last_error().decode()


# ---- conveniences over torch-owned buffers --------------------------------------

def _aligned_empty(nbytes, device):
    """A uint8 CUDA tensor of at least nbytes whose data pointer is 256-byte aligned."""
    import torch
    t = torch.empty(nbytes + 256, dtype=torch.uint8, device=device)
    off = (-t.data_ptr()) % 256
    return t[off:off + nbytes]


class Model:
    """Weights bound to the library.  ``arena`` is a host uint8 numpy array or a
    CUDA uint8 tensor in the canonical layout."""

    def __init__(self, shape, arena, device="cuda", stream=None):
        import torch
        self.cfg = ds_config.of(shape)
        nbytes = ds_weights_bytes(self.cfg)
        if nbytes == 0:
            raise DSError(-1, ds_last_error())
        self.arena = _aligned_empty(nbytes, device)
        src = arena if isinstance(arena, torch.Tensor) else torch.from_numpy(arena[:nbytes])
        self.arena.copy_(src[:nbytes], non_blocking=False)
        self.handle = ds_load_weights(self.cfg, self.arena, stream)

    def close(self):
        if self.handle:
            ds_model_destroy(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


class KVCache:
    """A (B, T) cache with its lengths and workspace, allocated through torch."""

    def __init__(self, model: Model, B: int, T: int, device="cuda", stream=None):
        import torch
        self.model, self.B, self.T = model, B, T
        self.cache_t = _aligned_empty(ds_kv_cache_bytes(model.cfg, B, T), device)
        self.cache = self.cache_t.view(torch.bfloat16 if model.cfg.cache_dtype == DS_BF16 else torch.float32)
        self.lengths = _aligned_empty(4 * B, device).view(torch.int32)
        self.ws = _aligned_empty(ds_workspace_bytes(model.cfg, B, T), device)
        self.logits_buf = torch.empty(B, model.cfg.vocab_size, dtype=torch.float32, device=device)
        self.handle = ds_kv_cache_create(model.handle, B, T, self.cache_t, self.lengths, self.ws, stream)

    def cache_view(self):
        """The cache as (L, 2, B, Hkv, T, D), in its element type (fp32 or bf16)."""
        c = self.model.cfg
        return self.cache.view(c.n_layers, 2, self.B, c.n_kv_heads, self.T, c.head_dim)

    def prefill(self, seq, tokens, d_tok_out=None, stream=None):
        ds_prefill(self.model.handle, self.handle, seq, tokens, d_tok_out, stream)

    def prefill_batched(self, seq, tokens, d_tok_out=None, stream=None):
        ds_prefill_batched(self.model.handle, self.handle, seq, tokens, d_tok_out, stream)

    def prefill_batch(self, token_lists, d_tok_out=None, stream=None):
        ds_prefill_batch(self.model.handle, self.handle, token_lists, d_tok_out, stream)

    def decode_step(self, d_tok_in, d_tok_out, stream=None):
        ds_decode_step(self.model.handle, self.handle, d_tok_in, d_tok_out, stream)

    def replicate_from(self, src, src_seq, dst_first, count, stream=None):
        """Copy sequence src_seq of cache `src` (a KVCache, possibly this one)
        into sequences dst_first .. dst_first + count - 1 of this cache."""
        _check(_lib.ds_kv_cache_replicate(self.handle, src.handle, int(src_seq), int(dst_first), int(count),
                                          _stream(stream)))

    def decode_step_rows(self, rows, d_tok_in, d_tok_out, stream=None):
        """A decode step of the sequences in `rows` only."""
        rows = [int(r) for r in rows]
        _check(_lib.ds_decode_step_rows(self.model.handle, self.handle, _i32(rows) if rows else None, len(rows),
                                        _ptr(d_tok_in), _ptr(d_tok_out), _stream(stream)))

    def sample(self, d_uniform, temperature, top_k, top_p, d_tok_out, stream=None):
        """Draw one token per sequence from the last step's logits (ds_sample):
        d_uniform is a device float32[B] of uniforms in [0, 1)."""
        _check(_lib.ds_sample(self.handle, _ptr(d_uniform), float(temperature), int(top_k), float(top_p),
                              _ptr(d_tok_out), _stream(stream)))

    def logits(self, stream=None):
        ds_logits(self.handle, self.logits_buf, stream)
        return self.logits_buf

    def set_lengths(self, lengths, stream=None):
        ds_kv_cache_set_lengths(self.handle, lengths, stream)

    def get_lengths(self):
        return ds_kv_cache_get_lengths(self.handle, self.B)

    def single_launch_ctx(self) -> int:
        """Longest context (positions after the step) of batch-1 steps that run
        as one persistent launch; 0 if none do."""
        return ds_kv_cache_single_launch_ctx(self.handle)

    def reset(self, seq=-1, stream=None):
        ds_kv_cache_reset(self.handle, seq, stream)

    def check(self, stream=None):
        ds_kv_cache_check(self.handle, stream)

    def bench_kernel(self, which, layer, reps, stream=None):
        ds_bench_kernel(self.model.handle, self.handle, which, layer, reps, stream)

    def set_dispatch(self, mode):
        ds_set_dispatch(self.handle, mode)

    def close(self):
        if self.handle:
            ds_kv_cache_destroy(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass
