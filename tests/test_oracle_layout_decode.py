"""Pins for the packed layout (byte counts, bit positions, round trips) and
for the oracle's decode attention (bypass = textbook attention, special
cases, estimator consistency)."""
import math

import numpy as np
import pytest


def _spec(orc, **kw):
    base = dict(d=128, n_q=8, n_kv=2, batch=2, max_ctx=300, k_codec=orc.POLAR_QJL, k_bits=3,
                m=128, v_codec=orc.POLAR, v_bits=3)
    base.update(kw)
    return orc.make_spec(**base)


@pytest.mark.parametrize("kc,kb,vc,vb,krec,vrec,kbpe,vbpe", [
    (2, 3, 1, 3, 68, 50, 4.25, 3.125),
    (2, 3, 1, 2, 68, 34, 4.25, 2.125),
    (2, 4, 1, 4, 84, 66, 5.25, 4.125),
    (3, 8, 1, 2, 136, 34, 8.5, 2.125),
    (1, 3, 0, 32, 50, 512, 3.125, 32.0),
])
def test_record_bytes_closed_form(orc, kc, kb, vc, vb, krec, vrec, kbpe, vbpe):
    s = _spec(orc, k_codec=kc, k_bits=kb, v_codec=vc, v_bits=vb, max_ctx=1000, batch=3, n_kv=8, n_q=32)
    z = orc.spec_sizes(s)
    assert z["k_record"] == krec and z["v_record"] == vrec
    assert 8 * krec / 128 == kbpe and 8 * vrec / 128 == vbpe
    nblk = math.ceil(1000 / 128)
    assert z["k_cache"] == 3 * 8 * nblk * 128 * krec
    assert z["v_cache"] == 3 * 8 * nblk * 128 * vrec


def test_compression_vs_bf16_matches_closed_form(orc):
    # K 3b+QJL with V 3b: (4.25 + 3.125)/2 bits vs 16 bits
    s = _spec(orc)
    z = orc.spec_sizes(s)
    assert abs(16 * 128 * 2 / (8 * (z["k_record"] + z["v_record"])) - 32 / 7.375) < 1e-12


def _random_records(orc, s, lens, seed):
    rng = np.random.default_rng(seed)
    R = orc.Records(s)
    if s.k_codec in (orc.POLAR, orc.POLAR_QJL):
        R.kcodes[:] = rng.integers(0, 1 << s.k_bits, R.kcodes.shape)
        R.kn16[:] = rng.integers(0, 0x7c00, R.kn16.shape)
    if s.k_codec == orc.POLAR_QJL:
        R.signs[:] = rng.integers(0, 2, R.signs.shape)
        R.rho16[:] = rng.integers(0, 0x7c00, R.rho16.shape)
    if s.k_codec == orc.Q8_BLOCK32:
        R.k8[:] = rng.integers(-127, 128, R.k8.shape)
        R.s16[:] = rng.integers(0, 0x7c00, R.s16.shape)
    if s.k_codec == orc.RAW_F32:
        R.kraw[:] = rng.standard_normal(R.kraw.shape)
    if s.v_codec == orc.POLAR:
        R.vcodes[:] = rng.integers(0, 1 << s.v_bits, R.vcodes.shape)
        R.vn16[:] = rng.integers(0, 0x7c00, R.vn16.shape)
    else:
        R.vraw[:] = rng.standard_normal(R.vraw.shape)
    # positions beyond each sequence's length are not stored
    for b in range(s.batch):
        for pos in range(lens[b], s.max_ctx):
            for h in range(s.n_kv):
                i = R.rec_index(b, pos, h)
                for a in (R.kcodes, R.kn16, R.signs, R.rho16, R.k8, R.s16, R.kraw,
                          R.vcodes, R.vn16, R.vraw):
                    if a.shape[0] == R.n:
                        a[i] = 0
    return R


@pytest.mark.parametrize("kc,kb,vc,vb", [(2, 3, 1, 3), (2, 4, 1, 2), (1, 2, 1, 4),
                                         (3, 8, 1, 2), (0, 32, 0, 32)])
def test_pack_unpack_round_trip(orc, kc, kb, vc, vb):
    s = _spec(orc, k_codec=kc, k_bits=kb, v_codec=vc, v_bits=vb)
    lens = np.array([300, 129], np.int32)
    R = _random_records(orc, s, lens, kc * 10 + vb)
    kcache, vcache = orc.pack_cache(s, R, lens)
    U = orc.unpack_cache(s, kcache, vcache, lens)
    for a, b in [(R.kcodes, U.kcodes), (R.kn16, U.kn16), (R.signs, U.signs), (R.rho16, U.rho16),
                 (R.k8, U.k8), (R.s16, U.s16), (R.kraw, U.kraw), (R.vcodes, U.vcodes),
                 (R.vn16, U.vn16), (R.vraw, U.vraw)]:
        assert np.array_equal(a, b)


def test_slot_permutation_is_a_bijection_per_group(orc):
    """pi(t) = 32(t/32) + 8(t%4) + (t%32)/4 permutes each group of 32 positions;
    checked through the packer: one record per position lands on distinct slots."""
    s = _spec(orc, batch=1, n_kv=1, n_q=4, max_ctx=128)
    R = orc.Records(s)
    for t in range(128):
        R.kn16[R.rec_index(0, t, 0)] = 0x3c00 + t      # distinct radii
    kc, _ = orc.pack_cache(s, R, np.array([128], np.int32))
    n16 = kc[4 * 2048:4 * 2048 + 256].view(np.uint16)
    pi = lambda t: 32 * (t // 32) + 8 * (t % 4) + (t % 32) // 4
    assert sorted(pi(t) for t in range(128)) == list(range(128))
    assert all(n16[pi(t)] == 0x3c00 + t for t in range(128))


def test_bit_positions_of_one_record(orc):
    """Hand-computed byte offsets for one record in the documented layout."""
    s = _spec(orc, batch=1, n_kv=2, max_ctx=256)
    R = orc.Records(s)
    b, pos, h = 0, 130, 1                       # block 1 of kv head 1, token 2 in block
    i = R.rec_index(b, pos, h)
    R.kcodes[i, 37] = 5                         # bits 0 and 2 set
    R.signs[i, 100] = 1
    R.kn16[i] = 0x3c00
    R.rho16[i] = 0x4000
    R.vcodes[i, 9] = 6                          # bits 1 and 2
    R.vn16[i] = 0x3555
    lens = np.array([256], np.int32)
    kc, vc = orc.pack_cache(s, R, lens)
    kblk = 128 * 68
    base = ((0 * 2 + 1) * 2 + 1) * kblk         # (b, h, block) = (0, 1, 1)
    sl = 16                                     # token 2 of the block sits at slot 32*0 + 8*2 + 0
    word = lambda p, j, s_: base + 4 * (p * 4 * 128 + j * 128 + s_)
    nz = np.flatnonzero(kc)
    want = {word(0, 1, sl) + 0: 1 << 5, word(2, 1, sl) + 0: 1 << 5,   # coord 37 = word 1 bit 5
            base + 3 * 2048 + 4 * (3 * 128 + sl) + 0: 1 << 4,        # sign row 100 = word 3 bit 4
            base + 4 * 2048 + 2 * sl + 1: 0x3c,                       # n16 high byte
            base + 4 * 2048 + 256 + 2 * sl + 1: 0x40}                 # rho16 high byte
    assert {int(k): int(kc[k]) for k in nz} == want
    vblk = 128 * 50
    vbase = ((0 * 2 + 1) * 2 + 1) * vblk
    vword = lambda p, j, i_: vbase + 4 * (p * 4 * 128 + j * 128 + i_)
    nzv = np.flatnonzero(vc)
    wantv = {vword(1, 0, 9) + 0: 1 << 2, vword(2, 0, 9) + 0: 1 << 2,   # token 2 = bit 2 of word j=0
             vbase + 3 * 2048 + 2 * sl: 0x55, vbase + 3 * 2048 + 2 * sl + 1: 0x35}
    assert {int(k): int(vc[k]) for k in nzv} == wantv


def _attention_fp64(q, K, V):
    lg = K @ q / math.sqrt(q.size)
    p = np.exp(lg - lg.max())
    p /= p.sum()
    return p @ V, lg


def test_raw_bypass_is_textbook_attention(orc):
    s = _spec(orc, k_codec=orc.RAW_F32, k_bits=32, v_codec=orc.RAW_F32, v_bits=32)
    rng = np.random.default_rng(0)
    lens = np.array([300, 77], np.int32)
    P = orc.Params(s, 42, 0)
    R = orc.Records(s)
    k = rng.standard_normal((2, 300, 2, 128)).astype(np.float32)
    v = rng.standard_normal((2, 300, 2, 128)).astype(np.float32)
    for b in range(2):
        orc.quantize_into(s, P, R, k[b, :lens[b]], v[b, :lens[b]], b, 0)
    q = rng.standard_normal((2, 8, 128)).astype(np.float32)
    out, lg = orc.decode(s, P, R, lens, q, want_logits=True)
    for idx, (b, hq) in enumerate([(b, h) for b in range(2) for h in range(8)]):
        o, l = _attention_fp64(q[b, hq].astype(np.float64), k[b, :lens[b], hq // 4].astype(np.float64),
                               v[b, :lens[b], hq // 4].astype(np.float64))
        assert np.allclose(out[idx], o, rtol=1e-12, atol=1e-12)
        assert np.allclose(lg[idx, :lens[b]], l, rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("kc", [1, 2])
def test_logits_equal_dequantised_inner_products(orc, kc):
    """POLAR: logit = <q, x_hat>/sqrt(d); POLAR_QJL: logit = <q, x_tilde>/sqrt(d)
    where x_tilde adds R^T S^T sigma (a different route than S R q)."""
    s = _spec(orc, k_codec=kc, batch=1, max_ctx=64)
    rng = np.random.default_rng(kc)
    P = orc.Params(s, 7, 3)
    R = orc.Records(s)
    k = rng.standard_normal((64, 2, 128)).astype(np.float32)
    orc.quantize_into(s, P, R, k, k, 0, 0)
    q = rng.standard_normal((1, 8, 128)).astype(np.float32)
    _, lg = orc.decode(s, P, R, np.array([64], np.int32), q, want_logits=True)
    for hq in range(8):
        for t in range(64):
            i = R.rec_index(0, t, hq // 4)
            if kc == 1:
                xt = orc.dequant_polar(P.DK, P.ck16, R.kcodes[i], R.kn16[i])
            else:
                xt = orc.dequant_polar_qjl(P.DK, P.ck16, P.S, R.kcodes[i], R.kn16[i], R.signs[i],
                                           R.rho16[i])
            want = np.dot(q[0, hq].astype(np.float64), xt) / math.sqrt(128)
            assert abs(lg[hq, t] - want) < 1e-10 * (1 + abs(want))


def test_one_token_equal_logits_and_empty(orc):
    s = _spec(orc, batch=3, max_ctx=40)
    rng = np.random.default_rng(3)
    P = orc.Params(s, 1, 0)
    R = orc.Records(s)
    v = rng.standard_normal((40, 2, 128)).astype(np.float32)
    kzero = np.zeros((40, 2, 128), np.float32)
    orc.quantize_into(s, P, R, kzero[:1], v[:1], 0, 0)       # b=0: one token
    orc.quantize_into(s, P, R, kzero, v, 1, 0)               # b=1: all-zero keys
    lens = np.array([1, 40, 0], np.int32)
    q = rng.standard_normal((3, 8, 128)).astype(np.float32)
    out = orc.decode(s, P, R, lens, q)
    for hq in range(8):
        h = hq // 4
        v0 = orc.dequant_polar(P.DV, P.cv16, R.vcodes[R.rec_index(0, 0, h)], R.vn16[R.rec_index(0, 0, h)])
        assert np.allclose(out[hq], v0, atol=1e-12)
        vm = np.mean([orc.dequant_polar(P.DV, P.cv16, R.vcodes[R.rec_index(1, t, h)],
                                        R.vn16[R.rec_index(1, t, h)]) for t in range(40)], axis=0)
        assert np.allclose(out[8 + hq], vm, atol=1e-12)
        assert np.all(out[16 + hq] == 0)


def test_corrupted_bit_changes_decode(orc):
    """A single flipped bit in a packed record changes the oracle's output,
    so a packed-byte comparison is a meaningful check."""
    s = _spec(orc, batch=1, max_ctx=128)
    rng = np.random.default_rng(4)
    P = orc.Params(s, 3, 0)
    R = orc.Records(s)
    x = rng.standard_normal((128, 2, 128)).astype(np.float32)
    orc.quantize_into(s, P, R, x, x, 0, 0)
    lens = np.array([128], np.int32)
    kc, vc = orc.pack_cache(s, R, lens)
    q = rng.standard_normal((1, 8, 128)).astype(np.float32)
    ref = orc.decode(s, P, orc.unpack_cache(s, kc, vc, lens), lens, q)
    kc2 = kc.copy()
    kc2[5] ^= 0x10
    bad = orc.decode(s, P, orc.unpack_cache(s, kc2, vc, lens), lens, q)
    assert np.max(np.abs(bad - ref)) > 1e-6
