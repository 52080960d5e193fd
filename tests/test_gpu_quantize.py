"""GPU parity of tq_quantize_append and tq_dequantize against the oracle,
through the C ABI (binding = argument marshalling only)."""
import numpy as np
import pytest
import torch

from parity_util import (compare_records, gpu_records, oracle, oracle_quantize, spec_of, synth, tq,
                         upload_cache, widen_np)

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _layer(w, ctx, batch, layer_id=3, chunk=0):
    ws = synth.with_ctx(w, ctx, batch=batch)
    cfg = tq.config_for(ws, seed=42, layer=layer_id, decode_chunk=chunk)
    return ws, cfg, tq.KVLayer(cfg, DEV)


@pytest.mark.parametrize("wi,wname", list(enumerate(synth.ORDER)))
def test_append_matches_oracle_ragged_chunks(wi, wname):
    """Five appends of 1, 31, 33, 128 and 107 positions (block and group
    boundaries, ragged tail) into two sequences."""
    ws, cfg, L = _layer(synth.WORKLOADS[wname], 300, 2)
    print(f"[append] {wname} cfg k={cfg.k_codec}/{cfg.k_bits} v={cfg.v_codec}/{cfg.v_bits}", flush=True)
    k, v = synth.make_kv(ws, 300, seed=1000 + wi, batch=2)
    pos = 0
    for n in (1, 31, 33, 128, 107):
        L.append(k[:, pos:pos + n].to(DEV).contiguous(), v[:, pos:pos + n].to(DEV).contiguous())
        pos += n
    torch.cuda.synchronize()
    spec = spec_of(cfg)
    P = oracle.Params(spec, 42, 3)
    kn, vn = widen_np(k), widen_np(v)
    R = oracle_quantize(spec, P, kn, vn, [300, 300])
    G = gpu_records(spec, L.k_cache, L.v_cache, [300, 300])
    st = compare_records(spec, P, G, R, [300, 300], kn, wname)
    print(st)


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16, torch.float16])
def test_input_dtypes(dtype):
    w = synth.WORKLOADS["tiny_b1_ctx1k_h8x2"]
    ws, cfg, L = _layer(w, 256, 1)
    k, v = synth.make_kv(ws, 256, seed=7)
    k, v = k.to(dtype), v.to(dtype)
    L.append(k.to(DEV), v.to(DEV))
    torch.cuda.synchronize()
    spec = spec_of(cfg)
    P = oracle.Params(spec, 42, 3)
    kn, vn = widen_np(k), widen_np(v)
    R = oracle_quantize(spec, P, kn, vn, [256])
    compare_records(spec, P, gpu_records(spec, L.k_cache, L.v_cache, [256]), R, [256], kn, str(dtype))


@pytest.mark.parametrize("wname", ["llama8b_b1_ctx32k", "cmdr104b_b1_ctx128k"])
def test_offset_append_keeps_other_positions(wname):
    """Sequences at different lengths; positions this call does not write keep
    their bytes (value words are shared by 32 positions)."""
    ws = synth.with_ctx(synth.WORKLOADS[wname], 300, batch=2)
    cfg = tq.config_for(ws, seed=42, layer=1)
    kb, vb = tq.cache_bytes(cfg)
    g = torch.Generator(device="cpu").manual_seed(5)
    kc0 = torch.randint(0, 256, (kb,), generator=g, dtype=torch.uint8)
    vc0 = torch.randint(0, 256, (vb,), generator=g, dtype=torch.uint8)
    spec = spec_of(cfg)
    # make the pre-existing fp16 fields finite: rewrite them through the oracle's own packer
    pre = oracle.unpack_cache(spec, kc0.numpy(), vc0.numpy(), np.array([300, 300], np.int32))
    for a in (pre.kn16, pre.rho16, pre.vn16, pre.s16):
        if a.ndim and a.size > 1:
            a &= 0x3bff
    kc_np, vc_np = kc0.numpy().copy(), vc0.numpy().copy()
    oracle.lib().or_pack_cache(oracle.ctypes.byref(spec), np.array([300, 300], np.int32),
                               oracle.ctypes.byref(pre._k()), oracle.ctypes.byref(pre._v()),
                               oracle._ptr(kc_np), oracle._ptr(vc_np))
    k_cache, v_cache = upload_cache(kc_np, vc_np, DEV)
    params = tq.init_params(cfg, DEV)
    seq_lens = torch.tensor([0, 37], dtype=torch.int32, device=DEV)
    k, v = synth.make_kv(ws, 200, seed=9, batch=2)
    tq.quantize_append(cfg, params, k_cache, v_cache, seq_lens, 37, k.to(DEV), v.to(DEV))
    torch.cuda.synchronize()
    G = gpu_records(spec, k_cache, v_cache, [300, 300])
    P = oracle.Params(spec, 42, 1)
    R = oracle.Records(spec)
    kn, vn = widen_np(k), widen_np(v)
    oracle.quantize_into(spec, P, R, kn[0], vn[0], 0, 0)
    oracle.quantize_into(spec, P, R, kn[1], vn[1], 1, 37)
    # written ranges
    written = np.zeros(R.n, bool)
    untouched = np.zeros(R.n, bool)
    for b, (lo, hi) in enumerate([(0, 200), (37, 237)]):
        for pos in range(300):
            sl = slice((b * 300 + pos) * spec.n_kv, (b * 300 + pos + 1) * spec.n_kv)
            (written if lo <= pos < hi else untouched)[sl] = True
    for name in ("kcodes", "kn16", "rho16", "k8", "s16", "vcodes", "vn16"):
        a_g, a_r, a_p = getattr(G, name), getattr(R, name), getattr(pre, name)
        if a_g.shape[0] != R.n:
            continue
        assert np.array_equal(a_g[written], a_r[written]), name
        assert np.array_equal(a_g[untouched], a_p[untouched]), f"{name} changed outside the append"
    if spec.k_codec == oracle.POLAR_QJL:
        assert np.array_equal(G.signs[untouched], pre.signs[untouched])
        assert (G.signs[written] != R.signs[written]).mean() <= 1e-4


def test_incremental_equals_one_shot():
    """Appends of many sizes equal one append of everything: every field bit
    for bit, except QJL sign bits, where the one-position appends (their own
    kernel, a per-lane sketch sum) may differ from the 16-position tiles only
    within the sign band; both caches are checked against the oracle."""
    w = synth.WORKLOADS["serving_b16_ctx8k"]
    ws = synth.with_ctx(w, 520, batch=3)
    cfg = tq.config_for(ws, seed=42, layer=0)
    A, B = tq.KVLayer(cfg, DEV), tq.KVLayer(cfg, DEV)
    k, v = synth.make_kv(ws, 520, seed=11, batch=3)
    kd, vd = k.to(DEV), v.to(DEV)
    A.append(kd, vd)
    pos = 0
    for n in (3, 29, 64, 1, 1, 200, 95, 127):
        B.append(kd[:, pos:pos + n].contiguous(), vd[:, pos:pos + n].contiguous())
        pos += n
    torch.cuda.synchronize()
    assert pos == 520
    assert torch.equal(A.v_cache, B.v_cache)
    spec = spec_of(cfg)
    GA = gpu_records(spec, A.k_cache, A.v_cache, [520] * 3)
    GB = gpu_records(spec, B.k_cache, B.v_cache, [520] * 3)
    for name in ("kcodes", "kn16", "rho16"):
        assert np.array_equal(getattr(GA, name), getattr(GB, name)), name
    P = oracle.Params(spec, 42, 0)
    kn, vn = widen_np(k), widen_np(v)
    R = oracle_quantize(spec, P, kn, vn, [520] * 3)
    compare_records(spec, P, GA, R, [520] * 3, kn, "one shot")
    compare_records(spec, P, GB, R, [520] * 3, kn, "incremental")


@pytest.mark.parametrize("codecs", [(tq.POLAR_QJL, 3, tq.POLAR, 2), (tq.POLAR_QJL, 4, tq.POLAR, 4),
                                    (tq.POLAR, 2, tq.POLAR, 3), (tq.Q8_BLOCK32, 8, tq.POLAR, 4),
                                    (tq.RAW_F32, 32, tq.RAW_F32, 32), (tq.POLAR_QJL, 2, tq.RAW_F32, 32)])
@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_single_position_appends_match_oracle(codecs, dtype):
    """The one-position append (its own kernel): five sequences at ragged
    lengths, 40 appends of one position each, against the oracle."""
    kc_, kb_, vc_, vb_ = codecs
    cfg = tq.make_config(n_q_heads=32, n_kv_heads=8, batch=5, max_ctx=400, k_codec=kc_, k_bits=kb_, v_codec=vc_,
                         v_bits=vb_, seed=42, layer=2)
    L = tq.KVLayer(cfg, DEV)
    g = torch.Generator().manual_seed(kb_ * 10 + vb_)
    n0 = [0, 31, 32, 127, 300]
    k = (torch.randn((5, 340, 8, 128), generator=g) * 2.0).to(dtype)
    v = torch.randn((5, 340, 8, 128), generator=g).to(dtype)
    L.append(k[:, :300].to(DEV).contiguous(), v[:, :300].to(DEV).contiguous())
    L.seq_lens.copy_(torch.tensor(n0, dtype=torch.int32, device=DEV))
    L.max_len = 300
    lens = list(n0)
    for s in range(40):
        idx = torch.tensor(lens)
        kn = k[torch.arange(5), idx].unsqueeze(1).contiguous().to(DEV)
        vn = v[torch.arange(5), idx].unsqueeze(1).contiguous().to(DEV)
        L.append(kn, vn)
        lens = [n + 1 for n in lens]
    torch.cuda.synchronize()
    spec = spec_of(cfg)
    P = oracle.Params(spec, 42, 2)
    kn_, vn_ = widen_np(k), widen_np(v)
    R = oracle_quantize(spec, P, kn_, vn_, lens)
    G = gpu_records(spec, L.k_cache, L.v_cache, lens)
    print(compare_records(spec, P, G, R, lens, kn_, f"single {codecs}"))


def test_capacity_and_noop():
    w = synth.WORKLOADS["tiny_b1_ctx1k_h8x2"]
    ws, cfg, L = _layer(w, 300, 1)
    k, v = synth.make_kv(ws, 300, seed=2)
    before = L.k_cache.clone()
    L.append(k[:, :0].to(DEV).contiguous(), v[:, :0].to(DEV).contiguous())   # n_new = 0
    torch.cuda.synchronize()
    assert torch.equal(before, L.k_cache)
    L.append(k.to(DEV), v.to(DEV))                                            # fills to capacity
    with pytest.raises(tq.TqError) as e:
        L.append(k[:, :1].to(DEV).contiguous(), v[:, :1].to(DEV).contiguous())
    assert e.value.status == tq.ECAPACITY


# the QJL-corrected reconstruction exists for QJL keys only
@pytest.mark.parametrize("wname,qjl", [(n, False) for n in synth.ORDER] +
                         [(n, True) for n in synth.ORDER if synth.WORKLOADS[n].k_codec == synth.POLAR_QJL])
def test_dequantize_matches_oracle(wname, qjl):
    w = synth.WORKLOADS[wname]
    ws = synth.with_ctx(w, 200, batch=2)
    cfg = tq.config_for(ws, seed=42, layer=2)
    spec = spec_of(cfg)
    P = oracle.Params(spec, 42, 2)
    k, v = synth.make_kv(ws, 200, seed=21, batch=2)
    kn, vn = widen_np(k), widen_np(v)
    R = oracle_quantize(spec, P, kn, vn, [200, 200])
    kc, vc = oracle.pack_cache(spec, R, [200, 200])
    k_cache, v_cache = upload_cache(kc, vc, DEV)
    params = tq.init_params(cfg, DEV)
    start, count = 57, 140
    ko = torch.empty(count, cfg.n_kv_heads, 128, device=DEV)
    vo = torch.empty(count, cfg.n_kv_heads, 128, device=DEV)
    tq.dequantize(cfg, params, k_cache, v_cache, 1, start, count, ko, vo, qjl=qjl)
    torch.cuda.synchronize()
    ko, vo = ko.cpu().numpy(), vo.cpu().numpy()
    for t in range(count):
        for h in range(cfg.n_kv_heads):
            i = R.rec_index(1, start + t, h)
            if spec.k_codec == oracle.POLAR_QJL and qjl:
                kr = oracle.dequant_polar_qjl(P.DK, P.ck16, P.S, R.kcodes[i], R.kn16[i], R.signs[i], R.rho16[i])
            elif spec.k_codec in (oracle.POLAR, oracle.POLAR_QJL):
                kr = oracle.dequant_polar(P.DK, P.ck16, R.kcodes[i], R.kn16[i])
            elif spec.k_codec == oracle.Q8_BLOCK32:
                kr = oracle.dequant_q8(R.k8[i], R.s16[i])
            else:
                kr = R.kraw[i].astype(np.float64)
            vr = (oracle.dequant_polar(P.DV, P.cv16, R.vcodes[i], R.vn16[i]) if spec.v_codec == oracle.POLAR
                  else R.vraw[i].astype(np.float64))
            for got, ref in ((ko[t, h], kr), (vo[t, h], vr)):
                assert np.max(np.abs(got - ref)) <= 1e-5 * max(np.linalg.norm(ref), 1e-30)


APPEND_CODECS = {   # name -> (k_codec, k_bits, v_codec, v_bits)
    "qjl2_v2": (tq.POLAR_QJL, 2, tq.POLAR, 2),
    "qjl4_raw": (tq.POLAR_QJL, 4, tq.RAW_F32, 32),
    "polar2_v4": (tq.POLAR, 2, tq.POLAR, 4),
    "polar3_v3": (tq.POLAR, 3, tq.POLAR, 3),
    "polar4_raw": (tq.POLAR, 4, tq.RAW_F32, 32),
    "q8_v3": (tq.Q8_BLOCK32, 8, tq.POLAR, 3),
    "q8_raw": (tq.Q8_BLOCK32, 8, tq.RAW_F32, 32),
    "raw_polar2": (tq.RAW_F32, 32, tq.POLAR, 2),
    "raw_raw": (tq.RAW_F32, 32, tq.RAW_F32, 32),
}


@pytest.mark.parametrize("codec", list(APPEND_CODECS))
def test_append_every_codec(codec):
    """Every key/value codec pair the kernels take, appended in ragged pieces
    (a lone position, a partial 16-position tile, a whole block) into two
    sequences, against the oracle's records."""
    kc_, kb_, vc_, vb_ = APPEND_CODECS[codec]
    cfg = tq.make_config(n_q_heads=8, n_kv_heads=2, batch=2, max_ctx=300, k_codec=kc_, k_bits=kb_,
                         v_codec=vc_, v_bits=vb_, seed=42, layer=5)
    print(f"[append codec] {codec}", flush=True)
    L = tq.KVLayer(cfg, DEV)
    g = torch.Generator().manual_seed(list(APPEND_CODECS).index(codec) + 77)
    k = torch.randn((2, 300, 2, 128), generator=g)
    v = torch.randn((2, 300, 2, 128), generator=g)
    k[:, :, :, 5] *= 9.0
    pos = 0
    for n in (1, 9, 22, 128, 140):
        L.append(k[:, pos:pos + n].to(DEV).contiguous(), v[:, pos:pos + n].to(DEV).contiguous())
        pos += n
    torch.cuda.synchronize()
    spec = spec_of(cfg)
    P = oracle.Params(spec, 42, 5)
    kn, vn = widen_np(k), widen_np(v)
    R = oracle_quantize(spec, P, kn, vn, [300, 300])
    G = gpu_records(spec, L.k_cache, L.v_cache, [300, 300])
    print(compare_records(spec, P, G, R, [300, 300], kn, codec))


# ------------------------------------------------------------------ edge cases

def _tie_rows(D, bounds, sign=1.0):
    """Rows x whose rotated vector y = H (D . x) holds a coordinate equal to
    fp32(B_j n) for every positive boundary B_j (a tie, which the format sends
    to the lower cell; sign -1 mirrors it onto -B_j).  x' = D . x is
    (a, 0, 1, -1, 0, ...) for B_j < 1 (y_0 = a exactly, n^2 = a^2 + 2) and
    (a, 1, ..., 1, 0, ...) with K ones otherwise (y_0 = a + K through the
    FWHT's own rounding, computed with the oracle's fp32 transform); a starts
    at the real root of y_0 / n = B_j and is walked over consecutive fp32
    values until y_0 == fp32(B_j n) holds exactly."""
    rows = []
    D = np.asarray(D, np.float32)
    for B in np.asarray(bounds, np.float32):
        if B <= 0:
            continue

        def row(a):
            xp = np.zeros(128, np.float32)
            xp[0] = a
            if B < 1.0:
                xp[2], xp[3] = 1.0, -1.0
            else:
                xp[1:(2 if B < 1.35 else 8)] = 1.0
            return xp

        lo, hi = (0.0, 1e6) if B < 1.0 else (-1e6, 1.0)   # the branch where y_0 / n increases with a
        for _ in range(200):
            mid = 0.5 * (lo + hi)
            xm = row(mid).astype(np.float64)
            if xm.sum() / np.sqrt((xm * xm).sum()) < float(B):
                lo = mid
            else:
                hi = mid
        a = np.float32(hi)
        found = None
        for _ in range(20000):
            xp = row(a)
            y0 = oracle.fwht_f32(xp)[0]
            n = np.float32(np.sqrt(oracle.tree_sumsq(xp)))
            thr = np.float32(B * n)
            if y0 == thr:
                found = xp
                break
            a = np.nextafter(a, np.float32(np.inf) if y0 < thr else np.float32(-np.inf), dtype=np.float32)
        assert found is not None, f"no exact tie found for boundary {B}"
        rows.append(D * (np.float32(sign) * found))
    return rows


def _q8_rows():
    """q8 blocks: a zero block, exact multiples of s = 2^-4 with the block
    amax at 127 s, exact half-way points (k + 1/2) s (round half to even)."""
    rng = np.random.default_rng(99)
    rows = []
    x = rng.standard_normal(128).astype(np.float32)
    x[32:64] = 0.0                                                  # zero block
    x[64:96] = (rng.integers(-127, 128, 32) * 2.0 ** -4).astype(np.float32)
    x[64 + 7] = np.float32(127 * 2.0 ** -4)                         # block amax -> +127
    x[96:128] = ((rng.integers(-120, 120, 32) + 0.5) * 2.0 ** -4).astype(np.float32)
    x[96 + 3] = np.float32(-127 * 2.0 ** -4)                        # amax -> -127, s = 2^-4
    rows.append(x)
    y = np.zeros(128, np.float32)
    y[:32] = (np.arange(-16, 16) * 2.0 ** -3).astype(np.float32)
    y[5] = np.float32(127 * 2.0 ** -3)
    rows.append(y)
    return rows


def _special_rows(P, spec):
    """The edge cases of the format, one row per position (keys, values)."""
    rng = np.random.default_rng(7)
    base = [np.zeros(128, np.float32), np.full(128, -0.0, np.float32),
            (rng.standard_normal(128) * 1e4).astype(np.float32),          # norm > 65504: radius saturates
            np.full(128, 1e4, np.float32),
            (rng.standard_normal(128) * 3e-6).astype(np.float32),        # fp16-subnormal radius
            (rng.standard_normal(128) * 1e-30).astype(np.float32),       # radius rounds to zero
            np.eye(128, dtype=np.float32)[5] * 2.5,
            np.ones(128, np.float32)]
    kb = P.kbounds if spec.k_codec in (oracle.POLAR, oracle.POLAR_QJL) else np.zeros(0, np.float32)
    keys = base + _tie_rows(P.DK, kb) + _tie_rows(P.DK, kb, -1.0)
    if spec.k_codec == oracle.Q8_BLOCK32:
        keys += _q8_rows()
    vals = base + _tie_rows(P.DV, P.vbounds) + _tie_rows(P.DV, P.vbounds, -1.0)
    n = max(len(keys), len(vals))
    keys += [rng.standard_normal(128).astype(np.float32) for _ in range(n - len(keys))]
    vals += [rng.standard_normal(128).astype(np.float32) for _ in range(n - len(vals))]
    return np.stack(keys), np.stack(vals)


SPECIAL_CODECS = {
    "qjl2_v2": (tq.POLAR_QJL, 2, tq.POLAR, 2),
    "qjl3_v3": (tq.POLAR_QJL, 3, tq.POLAR, 3),
    "qjl4_v4": (tq.POLAR_QJL, 4, tq.POLAR, 4),
    "polar3_v2": (tq.POLAR, 3, tq.POLAR, 2),
    "q8_v2": (tq.Q8_BLOCK32, 8, tq.POLAR, 2),
    "q8_v4": (tq.Q8_BLOCK32, 8, tq.POLAR, 4),
}


@pytest.mark.parametrize("path", ["tile", "one_position", "fused_step"])
@pytest.mark.parametrize("codec", list(SPECIAL_CODECS))
def test_append_special_vectors(codec, path):
    """Zero and signed-zero vectors (codes 0, radii 0, every sign bit 1),
    exact ties y_i == fp32(B_j n) on every boundary of both signs (lower
    cell), a norm past 65504 (radius saturates), fp16-subnormal and
    underflowing radii, one-hot and constant rows, q8 zero blocks, exact
    multiples (amax -> +-127) and exact half-way points: every field of the
    records bit-exact against the oracle through the 16-position tile
    kernel (one append of every row), the one-position kernel (one append
    per row) and the fused serving step (one step per row)."""
    kc_, kb_, vc_, vb_ = SPECIAL_CODECS[codec]
    cfg = tq.make_config(n_q_heads=8, n_kv_heads=2, batch=1, max_ctx=128, k_codec=kc_, k_bits=kb_,
                         v_codec=vc_, v_bits=vb_, seed=42, layer=6)
    spec = spec_of(cfg)
    P = oracle.Params(spec, 42, 6)
    xk, xv = _special_rows(P, spec)
    n = xk.shape[0]
    # two KV heads: head 0 the rows, head 1 the rows in reverse order
    k = np.stack([xk, xk[::-1]], axis=1)[None].copy()
    v = np.stack([xv, xv[::-1]], axis=1)[None].copy()
    print(f"[special] {codec} {path} rows={n}", flush=True)
    L = tq.KVLayer(cfg, DEV)
    kd, vd = torch.from_numpy(k).to(DEV), torch.from_numpy(v).to(DEV)
    if path == "tile":
        L.append(kd, vd)
    elif path == "one_position":
        for t in range(n):
            L.append(kd[:, t:t + 1].contiguous(), vd[:, t:t + 1].contiguous())
    else:
        g = torch.Generator().manual_seed(3)
        for t in range(n):
            q = torch.randn((1, 8, 128), generator=g).to(DEV)
            out = L.step(kd[:, t:t + 1].contiguous(), vd[:, t:t + 1].contiguous(), q)
            # the fused step equals a decode of the cache it leaves behind
            ref = torch.empty_like(q)
            tq.decode_attention(cfg, L.params, L.k_cache, L.v_cache, L.seq_lens, L.max_len, q, ref,
                                torch.zeros_like(L.workspace))
            torch.cuda.synchronize()
            assert torch.equal(torch.nan_to_num(out, nan=7.0), torch.nan_to_num(ref, nan=7.0)), f"step {t}"
    torch.cuda.synchronize()
    R = oracle_quantize(spec, P, k, v, [n])
    G = gpu_records(spec, L.k_cache, L.v_cache, [n])
    st = compare_records(spec, P, G, R, [n], k, f"{codec} {path}")
    if spec.k_codec == oracle.POLAR_QJL:
        for h, t in ((0, 0), (0, 1), (1, n - 1), (1, n - 2)):   # the zero rows of either head
            i = R.rec_index(0, t, h)
            assert np.all(G.signs[i] == 1) and G.rho16[i] == 0 and G.kn16[i] == 0
            assert np.all(G.kcodes[i] == 0)
    if spec.v_codec == oracle.POLAR:
        for h, t in ((0, 0), (0, 1), (1, n - 1), (1, n - 2)):
            i = R.rec_index(0, t, h)
            assert G.vn16[i] == 0 and np.all(G.vcodes[i] == 0)
    print(st)
