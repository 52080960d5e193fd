"""Host-only checks of the C ABI: the library loads and exports every
declared symbol; size queries and host-built parameters agree with the
oracle's independent implementation; argument checks return the documented
status before any device call (no GPU needed)."""
import ctypes
import math
import os
import re

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def tq():
    from compressed_decode_attention_quantize_amd import build_lib, tq
    if not os.path.exists(build_lib.LIB):
        build_lib.build()
    tq.lib()
    return tq


def test_every_declared_symbol_is_exported(tq):
    hdr = open(os.path.join(ROOT, "include", "tq.h")).read()
    names = set(re.findall(r"^(?:tq_status|const char\*)\s+(tq_\w+)\(", hdr, re.M))
    assert len(names) == 12
    L = tq.lib()
    for n in names:
        assert hasattr(L, n), n


def test_config_struct_layout(tq):
    assert ctypes.sizeof(tq.Config) == 64
    assert tq.Config.seed.offset == 48


CFGS = [
    dict(k_codec=2, k_bits=3, v_codec=1, v_bits=3),
    dict(k_codec=2, k_bits=3, v_codec=1, v_bits=2),
    dict(k_codec=2, k_bits=4, v_codec=1, v_bits=4),
    dict(k_codec=3, k_bits=8, v_codec=1, v_bits=2),
    dict(k_codec=1, k_bits=2, v_codec=0, v_bits=32),
    dict(k_codec=0, k_bits=32, v_codec=0, v_bits=32),
]


@pytest.mark.parametrize("kw", CFGS)
def test_sizes_match_oracle(tq, orc, kw):
    cfg = tq.make_config(n_q_heads=32, n_kv_heads=8, batch=3, max_ctx=1000, **kw)
    s = orc.make_spec(n_q=32, n_kv=8, batch=3, max_ctx=1000, k_codec=kw["k_codec"], k_bits=kw["k_bits"],
                      v_codec=kw["v_codec"], v_bits=kw["v_bits"])
    z = orc.spec_sizes(s)
    assert tq.cache_bytes(cfg) == (z["k_cache"], z["v_cache"])


@pytest.mark.parametrize("kw", CFGS[:5])
@pytest.mark.parametrize("seed,layer", [(42, 0), (42, 31), (7, 5)])
def test_params_match_oracle_tables(tq, orc, kw, seed, layer):
    cfg = tq.make_config(seed=seed, layer=layer, **kw)
    img = tq.params_host(cfg)
    f = img.view(np.float32)
    d = 128
    s = orc.make_spec(k_codec=kw["k_codec"], k_bits=kw["k_bits"], v_codec=kw["v_codec"], v_bits=kw["v_bits"])
    P = orc.Params(s, seed, layer)
    m = 128 if kw["k_codec"] == 2 else 0
    assert np.array_equal(f[0:d], P.DK) and np.array_equal(f[d:2 * d], P.DV)
    off = 2 * d
    if m:
        S = f[off:off + m * d].reshape(m, d)
        ST = f[off + m * d:off + 2 * m * d].reshape(d, m)
        assert np.array_equal(S, P.S)
        assert np.array_equal(ST, P.S.T)
    off += 2 * m * d
    ck, kb, cv, vb = (f[off + 16 * i: off + 16 * (i + 1)] for i in range(4))
    if kw["k_codec"] in (1, 2):
        L = 1 << kw["k_bits"]
        assert np.array_equal(ck[:L], orc.f16_to_f32(P.ck16))
        assert np.array_equal(kb[:L - 1], P.kbounds)
    if kw["v_codec"] == 1:
        L = 1 << kw["v_bits"]
        assert np.array_equal(cv[:L], orc.f16_to_f32(P.cv16))
        assert np.array_equal(vb[:L - 1], P.vbounds)
    if m:
        # sketch of a query before its rotation: (S H D_K / sqrt d)^T, H the
        # Sylvester matrix built here from its definition H[i][j] = (-1)^popcount(i & j)
        idx = np.arange(d)
        H = np.where(np.bitwise_count(idx[:, None] & idx[None, :]) % 2 == 1, -1.0, 1.0)
        want = (P.S.astype(np.float64) @ H * P.DK.astype(np.float64)[None, :] / math.sqrt(d)).T
        off += 4 * 16 + 2 * 8
        SHD = f[off:off + m * d].reshape(d, m)
        assert np.allclose(SHD, want, rtol=2e-7, atol=1e-6)


def _cfg(tq, **kw):
    return tq.make_config(**kw)


@pytest.mark.parametrize("field,value,status", [
    ("abi_version", 2, 1), ("head_dim", 100, 1), ("head_dim", 64, 2), ("head_dim", 512, 1),
    ("n_q_heads", 7, 1), ("n_kv_heads", 0, 1), ("batch", 0, 1), ("max_ctx", 0, 1),
    ("k_bits", 9, 1), ("k_bits", 5, 2), ("qjl_m", 96, 1), ("qjl_m", 64, 2), ("v_codec", 2, 2),
    ("v_codec", 3, 2), ("v_codec", 9, 1), ("k_codec", 7, 1), ("decode_chunk", 100, 1),
    ("sparse_v", -1, 1), ("sparse_v", 61, 1), ("v_bits", 5, 2),
])
def test_config_validation(tq, field, value, status):
    cfg = _cfg(tq)
    setattr(cfg, field, value)
    k, v = ctypes.c_uint64(), ctypes.c_uint64()
    assert tq.lib().tq_cache_bytes(ctypes.byref(cfg), ctypes.byref(k), ctypes.byref(v)) == status


def test_group_too_large_is_unsupported(tq):
    cfg = _cfg(tq, n_q_heads=34, n_kv_heads=2)
    n = ctypes.c_uint64()
    assert tq.lib().tq_params_bytes(ctypes.byref(cfg), ctypes.byref(n)) == tq.EUNSUPPORTED


FAKE = 1 << 20   # aligned, never dereferenced: every case below fails before a device call


def test_append_argument_checks(tq):
    L = tq.lib()
    cfg = _cfg(tq, max_ctx=256)
    p = ctypes.c_void_p
    args = lambda **o: dict(dict(params=p(FAKE), kc=p(FAKE), vc=p(FAKE), lens=p(FAKE), maxlen=0, k=p(FAKE),
                                 v=p(FAKE), dt=tq.F32, n=16), **o)

    def call(a):
        return L.tq_quantize_append(ctypes.byref(cfg), a["params"], a["kc"], a["vc"], a["lens"], a["maxlen"],
                                    a["k"], a["v"], a["dt"], a["n"], None)
    assert call(args(params=None)) == tq.EINVAL
    assert call(args(kc=p(FAKE + 4))) == tq.EINVAL       # cache must be 16-byte aligned
    assert call(args(dt=5)) == tq.EINVAL
    assert call(args(n=-1)) == tq.EINVAL
    assert call(args(maxlen=250, n=7)) == tq.ECAPACITY
    assert call(args(maxlen=0, n=257)) == tq.ECAPACITY
    assert call(args(n=0)) == tq.OK                      # no-op, no launch


def test_decode_argument_checks(tq):
    L = tq.lib()
    cfg = _cfg(tq, max_ctx=4096)
    need = tq.decode_workspace_bytes(cfg, 4096)
    p = ctypes.c_void_p

    def call(ws_bytes=need, maxlen=4096, q=p(FAKE), ws=p(FAKE)):
        return L.tq_decode_attention(ctypes.byref(cfg), p(FAKE), p(FAKE), p(FAKE), p(FAKE), maxlen, q, p(FAKE),
                                     None, ws, ws_bytes, None)
    assert call(ws_bytes=need - 1) == tq.EWORKSPACE
    assert call(maxlen=4097) == tq.EINVAL
    assert call(q=None) == tq.EINVAL
    assert call(ws=p(FAKE + 64)) == tq.EINVAL


def test_append_decode_argument_checks(tq):
    L = tq.lib()
    cfg = _cfg(tq, max_ctx=256)
    need = tq.decode_workspace_bytes(cfg, 256)
    p = ctypes.c_void_p

    def call(maxlen=100, dt=tq.F32, ws_bytes=need, k=p(FAKE), q=p(FAKE)):
        return L.tq_append_decode(ctypes.byref(cfg), p(FAKE), p(FAKE), p(FAKE), p(FAKE), maxlen, k, p(FAKE), dt,
                                  q, p(FAKE), None, p(FAKE), ws_bytes, None)
    assert call(maxlen=256) == tq.ECAPACITY          # the new position would pass max_ctx
    assert call(maxlen=-1) == tq.EINVAL
    assert call(dt=7) == tq.EINVAL
    assert call(k=None) == tq.EINVAL
    assert call(q=None) == tq.EINVAL
    assert call(maxlen=255, ws_bytes=tq.decode_workspace_bytes(cfg, 255) - 1) == tq.EWORKSPACE


def test_workspace_bound_covers_every_shorter_length(tq):
    # a workspace sized for a length serves every shorter call: the bound is
    # non-decreasing in the length, also across the length at which 4-bit
    # values move from two block groups per workgroup to one (batch 1, 8 KV
    # heads: 32 splits of at least 15 blocks, from 449 blocks on)
    lens = [1, 127, 128, 129, 5000, 8192, 32768, 448 * 128, 448 * 128 + 1, 449 * 128, 449 * 128 + 1, 65 * 128 * 8,
            1 << 19, 1 << 20]
    for v_bits in (2, 4):
        for batch, kv in [(1, 8), (16, 8), (1, 2)]:
            cfg = _cfg(tq, n_q_heads=4 * kv, n_kv_heads=kv, batch=batch, max_ctx=1 << 20, v_bits=v_bits)
            sizes = [tq.decode_workspace_bytes(cfg, L_) for L_ in sorted(lens)]
            assert sizes == sorted(sizes), (v_bits, batch, kv, sizes)


def test_stream_read_argument_checks(tq):
    # no launch happens for any of these: the checks run on the host
    L = tq.lib()
    p = ctypes.c_void_p
    assert L.tq_stream_read(None, 16, p(FAKE), None) == tq.EINVAL
    assert L.tq_stream_read(p(FAKE), 16, None, None) == tq.EINVAL
    assert L.tq_stream_read(p(FAKE + 8), 16, p(FAKE), None) == tq.EINVAL   # src not 16-byte aligned
    assert L.tq_stream_read(p(FAKE), 16, p(FAKE + 2), None) == tq.EINVAL   # sink not 4-byte aligned
    assert L.tq_stream_read(p(FAKE), 24, p(FAKE), None) == tq.EINVAL       # ragged length
    assert L.tq_stream_read(p(FAKE), 0, p(FAKE), None) == tq.OK            # nothing to read


def test_dequantize_argument_checks(tq):
    L = tq.lib()
    cfg = _cfg(tq, max_ctx=256)
    p = ctypes.c_void_p
    assert L.tq_dequantize(ctypes.byref(cfg), p(FAKE), p(FAKE), p(FAKE), 1, 0, 4, p(FAKE), None, 0, None) == tq.EINVAL
    assert L.tq_dequantize(ctypes.byref(cfg), p(FAKE), p(FAKE), p(FAKE), 0, 250, 7, p(FAKE), None, 0, None) == tq.EINVAL
    assert L.tq_dequantize(ctypes.byref(cfg), p(FAKE), p(FAKE), p(FAKE), 0, 0, 4, p(FAKE), None, 2, None) == tq.EINVAL
    assert L.tq_dequantize(ctypes.byref(cfg), p(FAKE), p(FAKE), p(FAKE), 0, 0, 0, p(FAKE), None, 0, None) == tq.OK


def test_status_strings(tq):
    assert tq.status_string(tq.ECAPACITY) == "append exceeds cache capacity"
    assert tq.status_string(99) == "unknown status"


@pytest.mark.parametrize("kb,vb", [(2, 4), (3, 3), (4, 2)])
def test_tree_tables_match_oracle_codebooks(tq, orc, kb, vb):
    """Recursive polar tables of the parameter image (cos / sin of every
    centroid angle, cos^2 / sin^2 of every boundary) against the oracle's
    per-level codebooks, built with another quadrature."""
    cfg = tq.make_config(k_codec=tq.POLAR_TREE, k_bits=kb, v_codec=tq.POLAR_TREE, v_bits=vb)
    img = tq.params_host(cfg)
    d = 128
    off = 4 * d * 2 + 64 * 4 + 32 * 2          # signs, no sketch, the per-coordinate codebooks
    tk = (off + 255) & ~255
    for base, b in ((tk, kb), (tk + 2048, vb)):
        raw = img[base: base + 1920]
        cs1 = raw[0:256].view(np.float32).reshape(32, 2)
        cs = raw[256:768].view(np.float32).reshape(8, 8, 2)
        c2_1, s2_1 = raw[768:832].view(np.float64), raw[832:896].view(np.float64)
        c2, s2 = raw[896:1408].view(np.float64).reshape(8, 8), raw[1408:1920].view(np.float64).reshape(8, 8)
        c, _, _, _ = orc.angle_codebook(1, b + 1)
        n1 = 1 << (b + 1)
        assert np.allclose(cs1[:n1, 0], np.cos(c), atol=1e-7) and np.allclose(cs1[:n1, 1], np.sin(c), atol=1e-7)
        per_q = n1 // 4
        beta = (np.arange(1, per_q)) * (math.pi / 2) / per_q
        assert np.allclose(c2_1[:per_q - 1], np.cos(beta) ** 2, atol=1e-15)
        assert np.allclose(s2_1[:per_q - 1], np.sin(beta) ** 2, atol=1e-15)
        for l in range(2, 8):
            c, bnd, _, _ = orc.angle_codebook(l, b - 1)
            nl = 1 << (b - 1)
            assert np.allclose(cs[l, :nl, 0], np.cos(c), atol=2e-7), l
            assert np.allclose(cs[l, :nl, 1], np.sin(c), atol=2e-7), l
            assert np.allclose(c2[l, :nl - 1], np.cos(bnd) ** 2, atol=1e-11), l
            assert np.allclose(s2[l, :nl - 1], np.sin(bnd) ** 2, atol=1e-11), l
    n = ctypes.c_uint64()
    assert tq.lib().tq_params_bytes(ctypes.byref(cfg), ctypes.byref(n)) == tq.OK and n.value == tk + 4096


def test_tree_config_validation(tq):
    k, v = ctypes.c_uint64(), ctypes.c_uint64()
    for kw, status in [(dict(k_codec=tq.POLAR_TREE, k_bits=1), tq.EINVAL),
                       (dict(k_codec=tq.POLAR_TREE, k_bits=5), tq.EUNSUPPORTED),
                       (dict(v_codec=tq.POLAR_TREE, v_bits=1), tq.EINVAL),
                       (dict(v_codec=tq.POLAR_TREE, v_bits=6), tq.EUNSUPPORTED),
                       (dict(k_codec=tq.POLAR_TREE, k_bits=3), tq.OK)]:
        cfg = tq.make_config(**kw)
        assert tq.lib().tq_cache_bytes(ctypes.byref(cfg), ctypes.byref(k), ctypes.byref(v)) == status, kw
    cfg = tq.make_config(k_codec=tq.POLAR_TREE, k_bits=3)
    cfg.qjl_m = 128
    assert tq.lib().tq_cache_bytes(ctypes.byref(cfg), ctypes.byref(k), ctypes.byref(v)) == tq.EINVAL


def test_format_version_matches_header(tq):
    """The binding's format version is the header's TQ_FORMAT_VERSION."""
    import re
    with open(os.path.join(ROOT, "include", "tq.h")) as fh:
        m = re.search(r"#define TQ_FORMAT_VERSION (\d+)u", fh.read())
    assert m and int(m.group(1)) == tq.FORMAT_VERSION


def test_noalloc_size_limits_checked_on_the_host(tq):
    """The no-allocation decode rejects configurations whose counters or
    partials do not fit the library's scratch array, before any HIP call."""
    L = tq.lib()
    fake = ctypes.c_void_p(1 << 20)   # aligned; never dereferenced by the host checks
    big_partials = tq.make_config(n_q_heads=64, n_kv_heads=8, batch=512, max_ctx=256)
    assert L.tq_decode_attention_noalloc(ctypes.byref(big_partials), fake, fake, fake, fake, 256, fake, fake, None,
                                         None) == tq.EWORKSPACE
    big_counters = tq.make_config(n_q_heads=16, n_kv_heads=16, batch=257, max_ctx=128)
    assert L.tq_decode_attention_noalloc(ctypes.byref(big_counters), fake, fake, fake, fake, 128, fake, fake, None,
                                         None) == tq.EWORKSPACE
    cfg = tq.make_config()
    assert L.tq_decode_attention_noalloc(ctypes.byref(cfg), fake, fake, fake, fake, cfg.max_ctx + 1, fake, fake,
                                         None, None) == tq.EINVAL
    assert L.tq_decode_attention_noalloc(ctypes.byref(cfg), None, fake, fake, fake, 10, fake, fake, None,
                                         None) == tq.EINVAL
