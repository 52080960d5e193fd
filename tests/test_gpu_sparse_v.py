"""Sparse-V decode (the wis-web.com reader article on the llama.cpp fork, its
third finding: value work skipped where the attention weight is small).

A block of 128 positions skips its value work only when every weight in it
lies below 2^-T of the running maximum of its split, for every query head the
block serves; its weights still count in the softmax denominator.  Which
blocks are skipped depends on the split schedule and on ceilings of the
kernel's own logits, so the test is a property that holds whatever was
skipped: with p the oracle's softmax weights and A the positions whose weight
is below 2^-T of the largest one (widened by the logit tolerance),

    |out_sparse - out_dense| <= sum over A of p_i |v_i|       (per coordinate)

and the sparse output stays within 2e-3 of the oracle plus that envelope.
Logits are the same bits as in dense decode, T = 60 reproduces dense decode
bit for bit, and with one split per sequence a small T on peaked data changes
the output, so the skip really runs.  Inputs: N(0, 1) keys, values and queries with one planted key
per 512 positions that the group's heads score about 16 nats above the rest.
"""
import dataclasses

import numpy as np
import pytest
import torch

from parity_util import LOGIT_REL, OUT_ABS, oracle, oracle_quantize, spec_of, synth, tq, upload_cache

pytestmark = pytest.mark.gpu
DEV = "cuda"

CODECS = {
    "qjl3_v3": (tq.POLAR_QJL, 3, tq.POLAR, 3),
    "q8_v4": (tq.Q8_BLOCK32, 8, tq.POLAR, 4),
    "polar2_v2": (tq.POLAR, 2, tq.POLAR, 2),
    "qjl4_v4": (tq.POLAR_QJL, 4, tq.POLAR, 4),
}
LENS = [3000, 1700]
CTX = 3072


def _case(codec, n_q, n_kv, seed):
    kc_, kb_, vc_, vb_ = CODECS[codec]
    base = dict(n_q_heads=n_q, n_kv_heads=n_kv, batch=len(LENS), max_ctx=CTX, k_codec=kc_, k_bits=kb_,
                v_codec=vc_, v_bits=vb_, seed=42, layer=2)
    cfg = tq.make_config(**base)
    w = dataclasses.replace(synth.WORKLOADS["tiny_b1_ctx1k_h8x2"], batch=len(LENS), ctx=CTX, n_q=n_q,
                            n_kv=n_kv)
    g = torch.Generator().manual_seed(seed)
    k = torch.randn((len(LENS), CTX, n_kv, 128), generator=g)
    v = torch.randn((len(LENS), CTX, n_kv, 128), generator=g)
    q = torch.randn((len(LENS), n_q, 128), generator=g)
    k, _ = synth.plant_focus_keys(w, k, q, seed=seed + 1, every=512, logit=16.0)
    spec = spec_of(cfg)
    P = oracle.Params(spec, cfg.seed, cfg.layer)
    R = oracle_quantize(spec, P, k.numpy(), v.numpy(), LENS)
    kc, vc = oracle.pack_cache(spec, R, np.asarray(LENS, np.int32))
    return base, spec, P, R, kc, vc, q.numpy()


def _decode(cfg, caches, q):
    k_cache, v_cache = caches
    params = tq.init_params(cfg, DEV)
    seq = torch.tensor(LENS, dtype=torch.int32, device=DEV)
    ws = torch.zeros(tq.decode_workspace_bytes(cfg, max(LENS)), dtype=torch.uint8, device=DEV)
    qd = torch.from_numpy(np.ascontiguousarray(q, np.float32)).to(DEV)
    out = torch.empty_like(qd)
    lg = torch.full((cfg.batch, cfg.n_q_heads, cfg.max_ctx), float("nan"), device=DEV)
    tq.decode_attention(cfg, params, k_cache, v_cache, seq, max(LENS), qd, out, ws, lg)
    torch.cuda.synchronize()
    return out.cpu().numpy(), lg.cpu().numpy()


def _values(spec, P, R, b, n, h):
    """Dequantised values [n][d] of sequence b, KV head h (oracle)."""
    out = np.zeros((n, spec.d), np.float64)
    for t in range(n):
        i = R.rec_index(b, t, h)
        out[t] = oracle.dequant_polar(P.DV, P.cv16, R.vcodes[i], R.vn16[i])
    return out


def _envelope(spec, vabs, ref_lg, T):
    """Per (b, head, coordinate) bound on the value mass a Sparse-V decode
    with distance T may leave out; vabs[b][hk] = |dequantised values|."""
    n_q, G = spec.n_q, spec.n_q // spec.n_kv
    env = np.zeros((len(LENS), n_q, spec.d))
    for b, n in enumerate(LENS):
        for hk in range(spec.n_kv):
            for hq in range(hk * G, (hk + 1) * G):
                l = ref_lg[b * n_q + hq, :n]
                tol = LOGIT_REL * max(np.abs(l).max(), np.sqrt(np.mean(l * l)))
                p = np.exp(l - l.max())
                small = (l - l.max()) < -T * np.log(2.0) + 2.0 * tol
                env[b, hq] = (p[small] @ vabs[b][hk][small]) / p.sum()
    return env


@pytest.mark.parametrize("codec", list(CODECS))
@pytest.mark.parametrize("heads", [(8, 2), (32, 8)])
@pytest.mark.parametrize("chunk", [0, CTX])
def test_sparse_v_within_envelope(codec, heads, chunk):
    n_q, n_kv = heads
    print(f"[sparse-v] {codec} heads={heads} chunk={chunk}", flush=True)
    base, spec, P, R, kc, vc, q = _case(codec, n_q, n_kv, seed=40 + n_kv + list(CODECS).index(codec))
    caches = upload_cache(kc, vc, DEV)
    out_d, lg_d = _decode(tq.make_config(decode_chunk=chunk, **base), caches, q)
    ref_out, ref_lg = oracle.decode(spec, P, R, LENS, q, want_logits=True)
    ref_out = ref_out.reshape(len(LENS), n_q, 128)
    assert np.max(np.abs(out_d - ref_out)) <= OUT_ABS
    vabs = [[np.abs(_values(spec, P, R, b, n, hk)) for hk in range(n_kv)] for b, n in enumerate(LENS)]
    # The two decodes add different products into fp32 sums: each 128-position
    # block adds once, and a sum may hold up to 6 times the weighted value mass
    # (the value operand's elements reach 6 where the signs are +/-1), so they
    # may differ by one rounding of that size per block on top of the skipped mass.
    vmax = max(float(x.max()) for row in vabs for x in row)
    rounding = 1e-5 + 6.0 * 2.0 ** -24 * (CTX / 128) * vmax
    changed = False
    for T in (2, 6, 10):
        out_s, lg_s = _decode(tq.make_config(decode_chunk=chunk, sparse_v=T, **base), caches, q)
        assert np.array_equal(np.nan_to_num(lg_s, nan=7.0), np.nan_to_num(lg_d, nan=7.0))
        env = _envelope(spec, vabs, ref_lg, T)
        gap = np.abs(out_s - out_d) - (env * (1.0 + 1e-3) + rounding)
        assert gap.max() <= 0.0, f"T={T}: sparse-dense difference above the envelope by {gap.max():.3g}"
        assert np.max(np.abs(out_s - ref_out) - env) <= OUT_ABS
        changed |= not np.array_equal(out_s, out_d)
    if chunk == CTX:   # one split per sequence: the blocks after a planted key are skipped
        assert changed, "no block was skipped on peaked data"


@pytest.mark.parametrize("codec", ["qjl3_v3", "q8_v4"])
def test_sparse_v_far_distance_is_dense(codec):
    base, spec, P, R, kc, vc, q = _case(codec, 32, 8, seed=7)
    caches = upload_cache(kc, vc, DEV)
    out_d, lg_d = _decode(tq.make_config(**base), caches, q)
    out_s, lg_s = _decode(tq.make_config(sparse_v=60, **base), caches, q)
    assert np.array_equal(out_s, out_d)


def test_sparse_v_ignored_by_raw_codecs():
    """Quantisation bypass decodes densely whatever the distance."""
    base = dict(n_q_heads=8, n_kv_heads=2, batch=2, max_ctx=CTX, k_codec=tq.RAW_F32, v_codec=tq.RAW_F32,
                seed=42, layer=0)
    cfg = tq.make_config(**base)
    spec = spec_of(cfg)
    P = oracle.Params(spec, cfg.seed, cfg.layer)
    g = torch.Generator().manual_seed(3)
    k = torch.randn((2, CTX, 2, 128), generator=g).numpy()
    v = torch.randn((2, CTX, 2, 128), generator=g).numpy()
    q = torch.randn((2, 8, 128), generator=g).numpy()
    R = oracle_quantize(spec, P, k, v, LENS)
    kc, vc = oracle.pack_cache(spec, R, np.asarray(LENS, np.int32))
    caches = upload_cache(kc, vc, DEV)
    out_d, _ = _decode(cfg, caches, q)
    out_s, _ = _decode(tq.make_config(sparse_v=1, **base), caches, q)
    assert np.array_equal(out_s, out_d)
