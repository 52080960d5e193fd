"""Python view of the C oracle (ctypes + numpy).

TEST INFRASTRUCTURE ONLY: the test suite, the smoke check and the
benchmark's CPU-baseline leg are the only code allowed to import this
module.  The product library never links or calls it, and the two share
no code.

Every numeric step runs in ``tq_oracle.c``; this file only marshals numpy
arrays.  See that file's header for the per-function parity status.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "tq_oracle.c")
_SO = os.path.join(_HERE, "liboracle.so")

RAW_F32, POLAR, POLAR_QJL, Q8_BLOCK32, POLAR_TREE = 0, 1, 2, 3, 4
BLOCK = 128

_u8p = np.ctypeslib.ndpointer(dtype=np.uint8, flags="C_CONTIGUOUS")
_i8p = np.ctypeslib.ndpointer(dtype=np.int8, flags="C_CONTIGUOUS")
_u16p = np.ctypeslib.ndpointer(dtype=np.uint16, flags="C_CONTIGUOUS")
_i32p = np.ctypeslib.ndpointer(dtype=np.int32, flags="C_CONTIGUOUS")
_f32p = np.ctypeslib.ndpointer(dtype=np.float32, flags="C_CONTIGUOUS")
_f64p = np.ctypeslib.ndpointer(dtype=np.float64, flags="C_CONTIGUOUS")
_vp = ctypes.c_void_p


def build(force: bool = False) -> str:
    """Compile the oracle with gcc (plain C99, no fast-math, no contraction)."""
    if force or not os.path.exists(_SO) or os.path.getmtime(_SO) < os.path.getmtime(_SRC):
        tmp = _SO + ".tmp"
        subprocess.check_call(
            ["gcc", "-O2", "-ffp-contract=off", "-fno-fast-math", "-std=c99",
             "-D_DEFAULT_SOURCE", "-fPIC", "-shared", "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _SO)
    return _SO


class Spec(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in
                ("d", "n_q", "n_kv", "batch", "max_ctx",
                 "k_codec", "k_bits", "m", "v_codec", "v_bits")]


class _KRec(ctypes.Structure):
    _fields_ = [("codes", _vp), ("n16", _vp), ("signs", _vp), ("rho16", _vp),
                ("k8", _vp), ("s16", _vp), ("raw", _vp)]


class _VRec(ctypes.Structure):
    _fields_ = [("codes", _vp), ("n16", _vp), ("raw", _vp)]


class TreeTab(ctypes.Structure):
    _fields_ = [("d", ctypes.c_int), ("b", ctypes.c_int), ("levels", ctypes.c_int),
                ("bits", ctypes.c_int * 13), ("cent", (ctypes.c_double * 256) * 13),
                ("bnd", (ctypes.c_double * 255) * 13)]


_lib = None


def lib() -> ctypes.CDLL:
    global _lib
    if _lib is not None:
        return _lib
    L = ctypes.CDLL(build())
    L.or_f32_to_f16.restype = ctypes.c_uint16
    L.or_f32_to_f16.argtypes = [ctypes.c_float]
    L.or_f16_to_f32.restype = ctypes.c_float
    L.or_f16_to_f32.argtypes = [ctypes.c_uint16]
    L.or_f32_to_f16_array.argtypes = [_f32p, _u16p, ctypes.c_int64]
    L.or_f16_to_f32_array.argtypes = [_u16p, _f32p, ctypes.c_int64]
    L.or_splitmix64_mix.restype = ctypes.c_uint64
    L.or_splitmix64_mix.argtypes = [ctypes.c_uint64]
    L.or_splitmix64_at.restype = ctypes.c_uint64
    L.or_splitmix64_at.argtypes = [ctypes.c_uint64, ctypes.c_uint64]
    L.or_stream_u64.restype = ctypes.c_uint64
    L.or_stream_u64.argtypes = [ctypes.c_uint64, ctypes.c_int32, ctypes.c_uint32, ctypes.c_uint64]
    L.or_make_signs.argtypes = [ctypes.c_uint64, ctypes.c_int32, ctypes.c_uint32, ctypes.c_int, _f32p]
    L.or_make_sketch.argtypes = [ctypes.c_uint64, ctypes.c_int32, ctypes.c_int, ctypes.c_int, _f32p]
    L.or_codebook.restype = ctypes.c_int
    L.or_codebook.argtypes = [ctypes.c_int, ctypes.c_int, _f64p, _u16p, _f32p,
                              ctypes.POINTER(ctypes.c_double)]
    L.or_marginal_mass.restype = ctypes.c_double
    L.or_marginal_mass.argtypes = [ctypes.c_int, ctypes.c_double, ctypes.c_double]
    L.or_marginal_moment1.restype = ctypes.c_double
    L.or_marginal_moment1.argtypes = [ctypes.c_int, ctypes.c_double, ctypes.c_double]
    L.or_fwht_f32.argtypes = [_f32p, ctypes.c_int]
    L.or_fwht_f64.argtypes = [_f64p, ctypes.c_int]
    L.or_tree_sumsq_f32.restype = ctypes.c_double
    L.or_tree_sumsq_f32.argtypes = [_f32p, ctypes.c_int]
    L.or_quantize_polar.argtypes = [_f32p, ctypes.c_int, ctypes.c_int, _f32p, _u16p, _f32p,
                                    ctypes.c_int, _vp, _u8p, ctypes.POINTER(ctypes.c_uint16),
                                    _vp, ctypes.POINTER(ctypes.c_uint16), _vp, _vp,
                                    ctypes.POINTER(ctypes.c_double)]
    L.or_quantize_q8.argtypes = [_f32p, ctypes.c_int, _i8p, _u16p, _vp]
    L.or_dequant_polar.argtypes = [ctypes.c_int, _f32p, _u16p, _u8p, ctypes.c_uint16, _f64p]
    L.or_dequant_polar_qjl.argtypes = [ctypes.c_int, ctypes.c_int, _f32p, _u16p, _f32p, _u8p,
                                       ctypes.c_uint16, _u8p, ctypes.c_uint16, _f64p]
    L.or_dequant_q8.argtypes = [ctypes.c_int, _i8p, _u16p, _f64p]
    for fn in ("or_k_record_bytes", "or_v_record_bytes", "or_k_block_bytes",
               "or_v_block_bytes", "or_k_cache_bytes", "or_v_cache_bytes"):
        getattr(L, fn).restype = ctypes.c_int64
        getattr(L, fn).argtypes = [ctypes.POINTER(Spec)]
    L.or_quantize_k_many.argtypes = [ctypes.POINTER(Spec), _f32p, _u16p, _f32p, _vp,
                                     ctypes.c_int64, _f32p, ctypes.POINTER(_KRec), ctypes.c_int64]
    L.or_quantize_v_many.argtypes = [ctypes.POINTER(Spec), _f32p, _u16p, _f32p,
                                     ctypes.c_int64, _f32p, ctypes.POINTER(_VRec), ctypes.c_int64]
    L.or_pack_cache.argtypes = [ctypes.POINTER(Spec), _i32p, ctypes.POINTER(_KRec),
                                ctypes.POINTER(_VRec), _vp, _vp]
    L.or_unpack_cache.argtypes = [ctypes.POINTER(Spec), _i32p, _vp, _vp,
                                  ctypes.POINTER(_KRec), ctypes.POINTER(_VRec)]
    L.or_decode_pairs.argtypes = [ctypes.POINTER(Spec), _f32p, _f32p, _u16p, _u16p, _vp,
                                  ctypes.POINTER(_KRec), ctypes.POINTER(_VRec), _i32p, _f32p,
                                  ctypes.c_int, _i32p, _f64p, _vp]
    for fn in ("or_angle_mass", "or_angle_moment1"):
        getattr(L, fn).restype = ctypes.c_double
        getattr(L, fn).argtypes = [ctypes.c_int, ctypes.c_double, ctypes.c_double]
    L.or_angle_codebook.restype = ctypes.c_int
    L.or_angle_codebook.argtypes = [ctypes.c_int, ctypes.c_int, _f64p, _f64p, ctypes.POINTER(ctypes.c_double)]
    L.or_tree_angles.restype = ctypes.c_double
    L.or_tree_angles.argtypes = [_f64p, ctypes.c_int, _f64p]
    L.or_tree_from_angles.argtypes = [_f64p, ctypes.c_double, ctypes.c_int, _f64p]
    L.or_tree_tables.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.POINTER(TreeTab)]
    L.or_quantize_tree.argtypes = [_f32p, ctypes.c_int, _f32p, ctypes.POINTER(TreeTab), _u8p,
                                   ctypes.POINTER(ctypes.c_uint16), _vp]
    L.or_dequant_tree.argtypes = [ctypes.c_int, _f32p, ctypes.POINTER(TreeTab), _u8p, ctypes.c_uint16, _f64p]
    L.or_tree_table.restype = ctypes.POINTER(TreeTab)
    L.or_tree_table.argtypes = [ctypes.c_int]
    L.or_tree_prepare()   # tables of the whole-cache helpers, before any threaded use
    _lib = L
    return L


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


# ---------------------------------------------------------------- fp16 ----

def f32_to_f16(x) -> np.ndarray:
    x = np.ascontiguousarray(np.asarray(x, dtype=np.float32).ravel())
    out = np.empty(x.shape, np.uint16)
    lib().or_f32_to_f16_array(x, out, x.size)
    return out


def f16_to_f32(h) -> np.ndarray:
    h = np.ascontiguousarray(np.asarray(h, dtype=np.uint16).ravel())
    out = np.empty(h.shape, np.float32)
    lib().or_f16_to_f32_array(h, out, h.size)
    return out


# ---------------------------------------------------------------- PRNG ----

def splitmix64_at(s0: int, k: int) -> int:
    return int(lib().or_splitmix64_at(s0, k))


def stream_u64(seed: int, layer: int, stream: int, k: int) -> int:
    return int(lib().or_stream_u64(seed, layer, stream, k))


def signs(seed: int, layer: int, stream: int, d: int) -> np.ndarray:
    out = np.empty(d, np.float32)
    lib().or_make_signs(seed, layer, stream, d, out)
    return out


def sketch(seed: int, layer: int, m: int, d: int) -> np.ndarray:
    out = np.empty((m, d), np.float32)
    lib().or_make_sketch(seed, layer, m, d, out)
    return out


# ------------------------------------------------------------ codebook ----

def codebook(d: int, b: int):
    """Returns (cent64, c16 bits, bounds fp32, mse, iterations)."""
    L = 1 << b
    c64 = np.zeros(L, np.float64)
    c16 = np.zeros(L, np.uint16)
    bnd = np.zeros(max(L - 1, 1), np.float32)
    mse = ctypes.c_double()
    it = lib().or_codebook(d, b, c64, c16, bnd, ctypes.byref(mse))
    if it < 0:
        raise ValueError("bad codebook arguments")
    return c64, c16, bnd[:L - 1], mse.value, it


def marginal_mass(d, a, c):
    return lib().or_marginal_mass(d, a, c)


def marginal_moment1(d, a, c):
    return lib().or_marginal_moment1(d, a, c)


# ------------------------------------------------------------ rotation ----

def fwht_f32(x) -> np.ndarray:
    y = np.array(x, dtype=np.float32, copy=True, order="C")
    lib().or_fwht_f32(y, y.size)
    return y


def fwht_f64(x) -> np.ndarray:
    y = np.array(x, dtype=np.float64, copy=True, order="C")
    lib().or_fwht_f64(y, y.size)
    return y


def tree_sumsq(x) -> float:
    x = np.ascontiguousarray(x, dtype=np.float32)
    return lib().or_tree_sumsq_f32(x, x.size)


# ---------------------------------------------------------- quantisers ----

def quantize_polar(x, D, c16, bounds, b, m=0, S=None):
    x = np.ascontiguousarray(x, np.float32)
    d = x.size
    D = np.ascontiguousarray(D, np.float32)
    c16 = np.ascontiguousarray(c16, np.uint16)
    bounds = np.ascontiguousarray(bounds, np.float32)
    codes = np.zeros(d, np.uint8)
    n16 = ctypes.c_uint16()
    rho16 = ctypes.c_uint16()
    tmargin = np.zeros(d, np.float64)
    signs_ = np.zeros(max(m, 1), np.uint8)
    z = np.zeros(max(m, 1), np.float64)
    rrot = ctypes.c_double()
    Sarr = None if S is None else np.ascontiguousarray(S, np.float32)
    lib().or_quantize_polar(x, d, b, D, c16, bounds, m, _ptr(Sarr), codes, ctypes.byref(n16),
                            _ptr(signs_), ctypes.byref(rho16), _ptr(tmargin), _ptr(z),
                            ctypes.byref(rrot))
    out = dict(codes=codes, n16=n16.value, tmargin=tmargin)
    if m:
        out.update(signs=signs_[:m], rho16=rho16.value, z=z[:m], rrot=rrot.value)
    return out


def quantize_q8(x):
    x = np.ascontiguousarray(x, np.float32)
    d = x.size
    k8 = np.zeros(d, np.int8)
    s16 = np.zeros(d // 32, np.uint16)
    qm = np.zeros(d, np.float64)
    lib().or_quantize_q8(x, d, k8, s16, _ptr(qm))
    return k8, s16, qm


def dequant_polar(D, c16, codes, n16) -> np.ndarray:
    codes = np.ascontiguousarray(codes, np.uint8)
    out = np.zeros(codes.size, np.float64)
    lib().or_dequant_polar(codes.size, np.ascontiguousarray(D, np.float32),
                           np.ascontiguousarray(c16, np.uint16), codes, int(n16), out)
    return out


def dequant_polar_qjl(D, c16, S, codes, n16, sgn, rho16) -> np.ndarray:
    codes = np.ascontiguousarray(codes, np.uint8)
    S = np.ascontiguousarray(S, np.float32)
    out = np.zeros(codes.size, np.float64)
    lib().or_dequant_polar_qjl(codes.size, S.shape[0], np.ascontiguousarray(D, np.float32),
                               np.ascontiguousarray(c16, np.uint16), S, codes, int(n16),
                               np.ascontiguousarray(sgn, np.uint8), int(rho16), out)
    return out


def dequant_q8(k8, s16) -> np.ndarray:
    k8 = np.ascontiguousarray(k8, np.int8)
    out = np.zeros(k8.size, np.float64)
    lib().or_dequant_q8(k8.size, k8, np.ascontiguousarray(s16, np.uint16), out)
    return out


# ------------------------------------------------- recursive polar ----

def angle_codebook(level: int, bits: int):
    """(centroids, boundaries, mse, Lloyd rounds) of the level's angle law."""
    n = 1 << bits
    c = np.zeros(n, np.float64)
    bnd = np.zeros(max(n - 1, 1), np.float64)
    mse = ctypes.c_double()
    it = lib().or_angle_codebook(level, bits, c, bnd, ctypes.byref(mse))
    if it < 0:
        raise ValueError("bad angle codebook arguments")
    return c, bnd[:n - 1], mse.value, it


def angle_mass(level, a, c):
    return lib().or_angle_mass(level, a, c)


def angle_moment1(level, a, c):
    return lib().or_angle_moment1(level, a, c)


def tree_angles(y):
    """(angles in heap slots [d] (slot 0 unused), radius) of a vector."""
    y = np.ascontiguousarray(y, np.float64)
    ang = np.zeros(y.size, np.float64)
    r = lib().or_tree_angles(y, y.size, ang)
    return ang, r


def tree_from_angles(ang, r):
    ang = np.ascontiguousarray(ang, np.float64)
    y = np.zeros(ang.size, np.float64)
    lib().or_tree_from_angles(ang, float(r), ang.size, y)
    return y


def tree_tables(b: int, d: int = 128) -> TreeTab:
    T = TreeTab()
    lib().or_tree_tables(d, b, ctypes.byref(T))
    return T


def tree_table_arrays(T: TreeTab):
    """Per level l = 1..levels: (bits, centroids, boundaries) as numpy arrays."""
    out = {}
    for l in range(1, T.levels + 1):
        n = 1 << T.bits[l]
        out[l] = (T.bits[l], np.array(T.cent[l][:n]), np.array(T.bnd[l][:n - 1]))
    return out


def quantize_tree(x, D, T: TreeTab):
    x = np.ascontiguousarray(x, np.float32)
    codes = np.zeros(x.size, np.uint8)
    n16 = ctypes.c_uint16()
    amargin = np.zeros(x.size, np.float64)
    lib().or_quantize_tree(x, x.size, np.ascontiguousarray(D, np.float32), ctypes.byref(T), codes,
                           ctypes.byref(n16), _ptr(amargin))
    return dict(codes=codes, n16=n16.value, amargin=amargin)


def dequant_tree(D, T: TreeTab, codes, n16) -> np.ndarray:
    codes = np.ascontiguousarray(codes, np.uint8)
    out = np.zeros(codes.size, np.float64)
    lib().or_dequant_tree(codes.size, np.ascontiguousarray(D, np.float32), ctypes.byref(T), codes,
                          int(n16), out)
    return out


# ------------------------------------------------------ whole caches ----

def make_spec(d=128, n_q=8, n_kv=2, batch=1, max_ctx=1024, k_codec=POLAR_QJL, k_bits=3,
              m=128, v_codec=POLAR, v_bits=3) -> Spec:
    if k_codec != POLAR_QJL:
        m = 0
    return Spec(d, n_q, n_kv, batch, max_ctx, k_codec, k_bits, m, v_codec, v_bits)


def spec_sizes(s: Spec) -> dict:
    L = lib()
    p = ctypes.byref(s)
    return dict(k_record=L.or_k_record_bytes(p), v_record=L.or_v_record_bytes(p),
                k_block=L.or_k_block_bytes(p), v_block=L.or_v_block_bytes(p),
                k_cache=L.or_k_cache_bytes(p), v_cache=L.or_v_cache_bytes(p))


class Params:
    """Per-layer random tables and codebooks, generated by the oracle alone."""

    def __init__(self, s: Spec, seed: int, layer: int):
        d = s.d
        self.DK = signs(seed, layer, 0, d)
        self.DV = signs(seed, layer, 1, d)
        self.S = sketch(seed, layer, s.m, d) if s.k_codec == POLAR_QJL else None
        one = np.zeros(1, np.uint16)
        if s.k_codec in (POLAR, POLAR_QJL):
            _, self.ck16, self.kbounds, _, _ = codebook(d, s.k_bits)
        else:
            self.ck16, self.kbounds = one, np.zeros(1, np.float32)
        if s.v_codec == POLAR:
            _, self.cv16, self.vbounds, _, _ = codebook(d, s.v_bits)
        else:
            self.cv16, self.vbounds = one, np.zeros(1, np.float32)


class Records:
    """Unpacked records [batch][max_ctx][n_kv][...] for one layer."""

    def __init__(self, s: Spec):
        n = s.batch * s.max_ctx * s.n_kv
        d = s.d
        self.spec = s
        self.n = n
        kc, vc = s.k_codec, s.v_codec
        self.kcodes = np.zeros((n, d) if kc in (POLAR, POLAR_QJL, POLAR_TREE) else 1, np.uint8)
        self.kn16 = np.zeros(n if kc in (POLAR, POLAR_QJL, POLAR_TREE) else 1, np.uint16)
        self.signs = np.zeros((n, s.m) if kc == POLAR_QJL else 1, np.uint8)
        self.rho16 = np.zeros(n if kc == POLAR_QJL else 1, np.uint16)
        self.k8 = np.zeros((n, d) if kc == Q8_BLOCK32 else 1, np.int8)
        self.s16 = np.zeros((n, d // 32) if kc == Q8_BLOCK32 else 1, np.uint16)
        self.kraw = np.zeros((n, d) if kc == RAW_F32 else 1, np.float32)
        self.vcodes = np.zeros((n, d) if vc in (POLAR, POLAR_TREE) else 1, np.uint8)
        self.vn16 = np.zeros(n if vc in (POLAR, POLAR_TREE) else 1, np.uint16)
        self.vraw = np.zeros((n, d) if vc == RAW_F32 else 1, np.float32)

    def _k(self):
        return _KRec(_ptr(self.kcodes), _ptr(self.kn16), _ptr(self.signs), _ptr(self.rho16),
                     _ptr(self.k8), _ptr(self.s16), _ptr(self.kraw))

    def _v(self):
        return _VRec(_ptr(self.vcodes), _ptr(self.vn16), _ptr(self.vraw))

    def rec_index(self, b, pos, h):
        s = self.spec
        return (b * s.max_ctx + pos) * s.n_kv + h


def quantize_into(s: Spec, P: Params, recs: Records, k, v, b: int, pos0: int):
    """Quantise k, v of shape [n_new][n_kv][d] (fp32) for sequence b at
    positions pos0.. into `recs`."""
    k = np.ascontiguousarray(k, np.float32)
    v = np.ascontiguousarray(v, np.float32)
    n_new = k.shape[0]
    off = recs.rec_index(b, pos0, 0)
    kr = recs._k()
    vr = recs._v()
    L = lib()
    L.or_quantize_k_many(ctypes.byref(s), P.DK, P.ck16, P.kbounds, _ptr(P.S),
                         n_new * s.n_kv, k.reshape(-1, s.d), ctypes.byref(kr), off)
    L.or_quantize_v_many(ctypes.byref(s), P.DV, P.cv16, P.vbounds, n_new * s.n_kv,
                         v.reshape(-1, s.d), ctypes.byref(vr), off)


def pack_cache(s: Spec, recs: Records, lens):
    sz = spec_sizes(s)
    kc = np.zeros(sz["k_cache"], np.uint8)
    vc = np.zeros(sz["v_cache"], np.uint8)
    lens = np.ascontiguousarray(lens, np.int32)
    kr, vr = recs._k(), recs._v()
    lib().or_pack_cache(ctypes.byref(s), lens, ctypes.byref(kr), ctypes.byref(vr),
                        _ptr(kc), _ptr(vc))
    return kc, vc


def unpack_cache(s: Spec, kc, vc, lens) -> Records:
    recs = Records(s)
    lens = np.ascontiguousarray(lens, np.int32)
    kc = None if kc is None else np.ascontiguousarray(kc, np.uint8)
    vc = None if vc is None else np.ascontiguousarray(vc, np.uint8)
    kr, vr = recs._k(), recs._v()
    lib().or_unpack_cache(ctypes.byref(s), lens, _ptr(kc), _ptr(vc), ctypes.byref(kr),
                          ctypes.byref(vr))
    return recs


def decode(s: Spec, P: Params, recs: Records, lens, q, pairs=None, want_logits=False):
    """fp64 decode attention for (b, hq) pairs (default: all).  q is
    [batch][n_q][d] fp32.  Returns out[n_pairs][d] and optionally
    logits[n_pairs][max_ctx]."""
    q = np.ascontiguousarray(q, np.float32)
    lens = np.ascontiguousarray(lens, np.int32)
    if pairs is None:
        pairs = [(b, h) for b in range(s.batch) for h in range(s.n_q)]
    pr = np.ascontiguousarray(np.asarray(pairs, np.int32).reshape(-1, 2))
    n = pr.shape[0]
    out = np.zeros((n, s.d), np.float64)
    lg = np.full((n, s.max_ctx), np.nan, np.float64) if want_logits else None
    kr, vr = recs._k(), recs._v()
    lib().or_decode_pairs(ctypes.byref(s), P.DK, P.DV, P.ck16, P.cv16, _ptr(P.S),
                          ctypes.byref(kr), ctypes.byref(vr), lens, q, n, pr, out, _ptr(lg))
    return (out, lg) if want_logits else out
