"""Python binding of libtq.so: the C ABI of include/tq.h with the same names.

Argument marshalling only: torch tensors become device pointers and the
current HIP stream; every step of the path runs in the library's kernels.
There is no fallback: if libtq.so is missing or a call fails, this raises.
"""
from __future__ import annotations

import ctypes
import os

import torch

_LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libtq.so")

ABI_VERSION = 1
BLOCK_TOKENS = 128
OK, EINVAL, EUNSUPPORTED, ECAPACITY, EWORKSPACE, EDEVICE = range(6)
RAW_F32, POLAR, POLAR_QJL, Q8_BLOCK32, POLAR_TREE = range(5)
F32, BF16, F16 = range(3)
DEQ_QJL = 1

FORMAT_VERSION = 1
# codec names of a workload description (its k_codec / v_codec fields)
CODEC_IDS = {"raw_f32": RAW_F32, "polar": POLAR, "polar_qjl": POLAR_QJL, "q8_block32": Q8_BLOCK32,
             "polar_tree": POLAR_TREE}
_DTYPES = {torch.float32: F32, torch.bfloat16: BF16, torch.float16: F16}


class TqError(RuntimeError):
    def __init__(self, status: int, where: str):
        super().__init__(f"{where}: {status_string(status)} (status {status})")
        self.status = status


class Config(ctypes.Structure):
    _fields_ = [("abi_version", ctypes.c_uint32), ("head_dim", ctypes.c_int32),
                ("n_q_heads", ctypes.c_int32), ("n_kv_heads", ctypes.c_int32),
                ("batch", ctypes.c_int32), ("max_ctx", ctypes.c_int32),
                ("k_codec", ctypes.c_int32), ("k_bits", ctypes.c_int32), ("qjl_m", ctypes.c_int32),
                ("v_codec", ctypes.c_int32), ("v_bits", ctypes.c_int32),
                ("decode_chunk", ctypes.c_int32), ("seed", ctypes.c_uint64),
                ("layer", ctypes.c_int32), ("sparse_v", ctypes.c_int32)]


_lib = None
_vp = ctypes.c_void_p
_u64p = ctypes.POINTER(ctypes.c_uint64)
_cfgp = ctypes.POINTER(Config)


def lib() -> ctypes.CDLL:
    """Load libtq.so (built in-tree by build_lib.build())."""
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            raise RuntimeError(f"{_LIB_PATH} is missing: build it with "
                               "compressed_decode_attention_quantize_amd.build_lib.build()")
        L = ctypes.CDLL(_LIB_PATH)
        L.tq_status_string.restype = ctypes.c_char_p
        L.tq_status_string.argtypes = [ctypes.c_int]
        L.tq_cache_bytes.argtypes = [_cfgp, _u64p, _u64p]
        L.tq_params_bytes.argtypes = [_cfgp, _u64p]
        L.tq_params_host.argtypes = [_cfgp, _vp, ctypes.c_uint64]
        L.tq_init_params.argtypes = [_cfgp, _vp, ctypes.c_uint64, _vp]
        L.tq_quantize_append.argtypes = [_cfgp, _vp, _vp, _vp, _vp, ctypes.c_int32, _vp, _vp,
                                         ctypes.c_int32, ctypes.c_int32, _vp]
        L.tq_decode_workspace_bytes.argtypes = [_cfgp, ctypes.c_int32, _u64p]
        L.tq_decode_attention.argtypes = [_cfgp, _vp, _vp, _vp, _vp, ctypes.c_int32, _vp, _vp, _vp,
                                          _vp, ctypes.c_uint64, _vp]
        L.tq_dequantize.argtypes = [_cfgp, _vp, _vp, _vp, ctypes.c_int32, ctypes.c_int32,
                                    ctypes.c_int32, _vp, _vp, ctypes.c_uint32, _vp]
        L.tq_decode_attention_noalloc.argtypes = [_cfgp, _vp, _vp, _vp, _vp, ctypes.c_int32, _vp, _vp, _vp, _vp]
        L.tq_append_decode.argtypes = [_cfgp, _vp, _vp, _vp, _vp, ctypes.c_int32, _vp, _vp, ctypes.c_int32,
                                       _vp, _vp, _vp, _vp, ctypes.c_uint64, _vp]
        L.tq_stream_read.argtypes = [_vp, ctypes.c_uint64, _vp, _vp]
        for fn in ("tq_cache_bytes", "tq_params_bytes", "tq_params_host", "tq_init_params",
                   "tq_quantize_append", "tq_decode_workspace_bytes", "tq_decode_attention",
                   "tq_dequantize", "tq_append_decode", "tq_stream_read", "tq_decode_attention_noalloc"):
            getattr(L, fn).restype = ctypes.c_int
        _lib = L
    return _lib


def status_string(status: int) -> str:
    return lib().tq_status_string(status).decode()


def _check(status: int, where: str):
    if status != OK:
        raise TqError(status, where)


def _ptr(t):
    if t is None:
        return None
    return ctypes.c_void_p(t.data_ptr())


def _stream(stream=None):
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def make_config(head_dim=128, n_q_heads=8, n_kv_heads=2, batch=1, max_ctx=1024, k_codec=POLAR_QJL,
                k_bits=3, qjl_m=128, v_codec=POLAR, v_bits=3, decode_chunk=0, seed=42,
                layer=0, sparse_v=0) -> Config:
    if k_codec != POLAR_QJL:
        qjl_m = 0
    if k_codec == RAW_F32:
        k_bits = 32
    if k_codec == Q8_BLOCK32:
        k_bits = 8
    if v_codec == RAW_F32:
        v_bits = 32
    return Config(ABI_VERSION, head_dim, n_q_heads, n_kv_heads, batch, max_ctx, k_codec, k_bits,
                  qjl_m, v_codec, v_bits, decode_chunk, seed, layer, sparse_v)


def config_for(w, seed=42, layer=0, max_ctx=None, batch=None,
               decode_chunk=0, sparse_v=0) -> Config:
    return make_config(w.d, w.n_q, w.n_kv, w.batch if batch is None else batch,
                       w.ctx if max_ctx is None else max_ctx, CODEC_IDS[w.k_codec], w.k_bits, w.m,
                       CODEC_IDS[w.v_codec], w.v_bits, decode_chunk, seed, layer, sparse_v)


# --------------------------------------------------------------- ABI calls

def cache_bytes(cfg: Config):
    k, v = ctypes.c_uint64(), ctypes.c_uint64()
    _check(lib().tq_cache_bytes(ctypes.byref(cfg), ctypes.byref(k), ctypes.byref(v)), "tq_cache_bytes")
    return k.value, v.value


def params_bytes(cfg: Config) -> int:
    n = ctypes.c_uint64()
    _check(lib().tq_params_bytes(ctypes.byref(cfg), ctypes.byref(n)), "tq_params_bytes")
    return n.value


def params_host(cfg: Config):
    import numpy as np
    n = params_bytes(cfg)
    buf = np.zeros(n, np.uint8)
    _check(lib().tq_params_host(ctypes.byref(cfg), buf.ctypes.data_as(_vp), n), "tq_params_host")
    return buf


def init_params(cfg: Config, device="cuda") -> torch.Tensor:
    n = params_bytes(cfg)
    p = torch.empty(n, dtype=torch.uint8, device=device)
    _check(lib().tq_init_params(ctypes.byref(cfg), _ptr(p), n, _stream()), "tq_init_params")
    return p


def quantize_append(cfg: Config, params, k_cache, v_cache, seq_lens, max_seq_len: int, k_new, v_new,
                    stream=None):
    n_new = k_new.shape[1]
    dt = _DTYPES[k_new.dtype]
    assert v_new.dtype == k_new.dtype and k_new.is_contiguous() and v_new.is_contiguous()
    assert tuple(k_new.shape) == (cfg.batch, n_new, cfg.n_kv_heads, cfg.head_dim)
    assert tuple(v_new.shape) == tuple(k_new.shape)
    assert seq_lens.dtype == torch.int32 and seq_lens.numel() == cfg.batch
    _check(lib().tq_quantize_append(ctypes.byref(cfg), _ptr(params), _ptr(k_cache), _ptr(v_cache),
                                    _ptr(seq_lens), int(max_seq_len), _ptr(k_new), _ptr(v_new), dt,
                                    n_new, _stream(stream)), "tq_quantize_append")


def decode_workspace_bytes(cfg: Config, max_seq_len: int) -> int:
    n = ctypes.c_uint64()
    _check(lib().tq_decode_workspace_bytes(ctypes.byref(cfg), int(max_seq_len), ctypes.byref(n)),
           "tq_decode_workspace_bytes")
    return n.value


def decode_attention(cfg: Config, params, k_cache, v_cache, seq_lens, max_seq_len: int, q, out,
                     workspace, logits=None, stream=None):
    assert q.dtype == torch.float32 and q.is_contiguous()
    assert tuple(q.shape) == (cfg.batch, cfg.n_q_heads, cfg.head_dim)
    assert out.dtype == torch.float32 and out.shape == q.shape and out.is_contiguous()
    if logits is not None:
        assert logits.dtype == torch.float32 and tuple(logits.shape) == (cfg.batch, cfg.n_q_heads, cfg.max_ctx)
    _check(lib().tq_decode_attention(ctypes.byref(cfg), _ptr(params), _ptr(k_cache), _ptr(v_cache),
                                     _ptr(seq_lens), int(max_seq_len), _ptr(q), _ptr(out), _ptr(logits),
                                     _ptr(workspace), workspace.numel() * workspace.element_size(),
                                     _stream(stream)), "tq_decode_attention")


def decode_attention_noalloc(cfg: Config, params, k_cache, v_cache, seq_lens, max_seq_len: int, q, out, logits=None,
                             stream=None):
    """tq_decode_attention on the library's own per-GPU scratch array instead
    of a caller workspace (no device allocation anywhere in the call)."""
    assert q.dtype == torch.float32 and q.is_contiguous()
    assert tuple(q.shape) == (cfg.batch, cfg.n_q_heads, cfg.head_dim)
    assert out.dtype == torch.float32 and out.shape == q.shape and out.is_contiguous()
    if logits is not None:
        assert logits.dtype == torch.float32 and tuple(logits.shape) == (cfg.batch, cfg.n_q_heads, cfg.max_ctx)
    _check(lib().tq_decode_attention_noalloc(ctypes.byref(cfg), _ptr(params), _ptr(k_cache), _ptr(v_cache),
                                             _ptr(seq_lens), int(max_seq_len), _ptr(q), _ptr(out), _ptr(logits),
                                             _stream(stream)), "tq_decode_attention_noalloc")


def append_decode(cfg: Config, params, k_cache, v_cache, seq_lens, max_seq_len: int, k_new, v_new, q, out,
                  workspace, logits=None, stream=None):
    """One serving step: k_new, v_new [batch][1][n_kv][d] stored at position
    seq_lens[b] of every sequence, then q decoded over seq_lens[b] + 1
    positions.  seq_lens is not advanced."""
    dt = _DTYPES[k_new.dtype]
    assert v_new.dtype == k_new.dtype and k_new.is_contiguous() and v_new.is_contiguous()
    assert tuple(k_new.shape) == (cfg.batch, 1, cfg.n_kv_heads, cfg.head_dim) == tuple(v_new.shape)
    assert q.dtype == torch.float32 and q.is_contiguous()
    assert tuple(q.shape) == (cfg.batch, cfg.n_q_heads, cfg.head_dim)
    assert out.dtype == torch.float32 and out.shape == q.shape and out.is_contiguous()
    if logits is not None:
        assert logits.dtype == torch.float32 and tuple(logits.shape) == (cfg.batch, cfg.n_q_heads, cfg.max_ctx)
    _check(lib().tq_append_decode(ctypes.byref(cfg), _ptr(params), _ptr(k_cache), _ptr(v_cache), _ptr(seq_lens),
                                  int(max_seq_len), _ptr(k_new), _ptr(v_new), dt, _ptr(q), _ptr(out), _ptr(logits),
                                  _ptr(workspace), workspace.numel() * workspace.element_size(), _stream(stream)),
           "tq_append_decode")


def dequantize(cfg: Config, params, k_cache, v_cache, b: int, start: int, count: int, k_out=None,
               v_out=None, qjl=False, stream=None):
    for t in (k_out, v_out):
        if t is not None:
            assert t.dtype == torch.float32 and t.numel() >= count * cfg.n_kv_heads * cfg.head_dim
    _check(lib().tq_dequantize(ctypes.byref(cfg), _ptr(params), _ptr(k_cache), _ptr(v_cache), b, start,
                               count, _ptr(k_out), _ptr(v_out), DEQ_QJL if qjl else 0, _stream(stream)),
           "tq_dequantize")


def stream_read(src, sink):
    """Measurement helper (not part of the method): XOR every 32-bit word of
    the device tensor src (a multiple of 16 bytes) into the device int32 sink
    with a plain streaming read; the bench's practical HBM read ceiling."""
    assert src.is_cuda and sink.is_cuda and sink.dtype == torch.int32
    nbytes = src.numel() * src.element_size()
    _check(lib().tq_stream_read(_ptr(src), nbytes, _ptr(sink), _stream()), "tq_stream_read")


# ------------------------------------------------------------ convenience

class KVLayer:
    """One layer's packed caches, parameters, lengths and decode workspace,
    all allocated with torch on `device`."""

    def __init__(self, cfg: Config, device="cuda", zero=True):
        self.cfg = cfg
        self.device = device
        kb, vb = cache_bytes(cfg)
        alloc = torch.zeros if zero else torch.empty
        self.k_cache = alloc(kb, dtype=torch.uint8, device=device)
        self.v_cache = alloc(vb, dtype=torch.uint8, device=device)
        self.params = init_params(cfg, device)
        self.seq_lens = torch.zeros(cfg.batch, dtype=torch.int32, device=device)
        self.max_len = 0
        self.workspace = torch.zeros(decode_workspace_bytes(cfg, cfg.max_ctx), dtype=torch.uint8,
                                     device=device)

    def append(self, k_new, v_new, stream=None):
        quantize_append(self.cfg, self.params, self.k_cache, self.v_cache, self.seq_lens, self.max_len,
                        k_new, v_new, stream)
        self.seq_lens += k_new.shape[1]
        self.max_len += k_new.shape[1]

    def decode(self, q, out=None, logits=None, stream=None):
        if out is None:
            out = torch.empty_like(q)
        decode_attention(self.cfg, self.params, self.k_cache, self.v_cache, self.seq_lens, self.max_len, q,
                         out, self.workspace, logits, stream)
        return out

    def step(self, k_new, v_new, q, out=None, logits=None, stream=None):
        """Serving step: store one new position per sequence and decode q
        over the lengths that include it (one launch on the matrix-core path)."""
        if out is None:
            out = torch.empty_like(q)
        append_decode(self.cfg, self.params, self.k_cache, self.v_cache, self.seq_lens, self.max_len, k_new,
                      v_new, q, out, self.workspace, logits, stream)
        self.seq_lens += 1
        self.max_len += 1
        return out
