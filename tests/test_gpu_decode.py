"""GPU parity of tq_decode_attention against the oracle, through the C ABI.

Decode is checked on caches the oracle itself quantised and packed, so both
sides read identical records; the end-to-end test runs the GPU append too."""
import math

import numpy as np
import pytest
import torch

from parity_util import (check_logits, check_out, compare_records, gpu_records, oracle, oracle_quantize,
                         spec_of, synth, tq, upload_cache, widen_np)

pytestmark = pytest.mark.gpu
DEV = "cuda"

CODECS = {   # name -> (k_codec, k_bits, v_codec, v_bits)
    "qjl3_v3": (tq.POLAR_QJL, 3, tq.POLAR, 3),
    "qjl3_v2": (tq.POLAR_QJL, 3, tq.POLAR, 2),
    "qjl4_v4": (tq.POLAR_QJL, 4, tq.POLAR, 4),
    "q8_v2": (tq.Q8_BLOCK32, 8, tq.POLAR, 2),
    "q8_v4": (tq.Q8_BLOCK32, 8, tq.POLAR, 4),
    "qjl2_v3": (tq.POLAR_QJL, 2, tq.POLAR, 3),
    "polar2_v2": (tq.POLAR, 2, tq.POLAR, 2),
    "polar4_raw": (tq.POLAR, 4, tq.RAW_F32, 32),
    "raw_polar3": (tq.RAW_F32, 32, tq.POLAR, 3),
    "raw_raw": (tq.RAW_F32, 32, tq.RAW_F32, 32),
}


def _oracle_cache(cfg, lens, seed, scale_heads=False):
    spec = spec_of(cfg)
    P = oracle.Params(spec, cfg.seed, cfg.layer)
    g = torch.Generator().manual_seed(seed)
    n = cfg.max_ctx
    k = torch.randn((cfg.batch, n, cfg.n_kv_heads, 128), generator=g)
    v = torch.randn((cfg.batch, n, cfg.n_kv_heads, 128), generator=g)
    if scale_heads:
        k[:, :, :, :4] *= 10.0
    kn, vn = k.numpy(), v.numpy()
    R = oracle_quantize(spec, P, kn, vn, lens)
    kc, vc = oracle.pack_cache(spec, R, np.asarray(lens, np.int32))
    q = torch.randn((cfg.batch, cfg.n_q_heads, 128), generator=g).numpy()
    return spec, P, R, kc, vc, q


def _gpu_decode(cfg, kc, vc, lens, q, max_seq_len=None, want_logits=True):
    """Decode on the GPU; with want_logits=False the plain variant (no logits
    buffer: the kernel the benchmark times) and lg is None."""
    k_cache, v_cache = upload_cache(kc, vc, DEV)
    params = tq.init_params(cfg, DEV)
    seq = torch.tensor(lens, dtype=torch.int32, device=DEV)
    msl = max(lens) if max_seq_len is None else max_seq_len
    ws = torch.zeros(tq.decode_workspace_bytes(cfg, msl), dtype=torch.uint8, device=DEV)
    qd = torch.from_numpy(np.ascontiguousarray(q, np.float32)).to(DEV)
    out = torch.empty_like(qd)
    lg = torch.full((cfg.batch, cfg.n_q_heads, cfg.max_ctx), float("nan"), device=DEV) if want_logits else None
    tq.decode_attention(cfg, params, k_cache, v_cache, seq, msl, qd, out, ws, lg)
    torch.cuda.synchronize()
    return out.cpu().numpy(), (lg.cpu().numpy() if want_logits else None), ws


@pytest.mark.parametrize("codec", list(CODECS))
# groups of 4 and 12 (whole head groups of four), 1 (no sharing), 6 (a partial
# head group) and 16 (the largest group)
@pytest.mark.parametrize("heads", [(8, 2), (32, 8), (96, 8), (16, 16), (12, 2), (64, 4)])
def test_decode_matches_oracle(codec, heads):
    kc_, kb_, vc_, vb_ = CODECS[codec]
    n_q, n_kv = heads
    lens = [300, 1, 129, 0]
    cfg = tq.make_config(n_q_heads=n_q, n_kv_heads=n_kv, batch=4, max_ctx=300, k_codec=kc_, k_bits=kb_,
                         v_codec=vc_, v_bits=vb_, seed=42, layer=4)
    print(f"[decode] {codec} heads={heads}", flush=True)
    spec, P, R, kc, vc, q = _oracle_cache(cfg, lens, seed=list(CODECS).index(codec) + 10 * n_kv, scale_heads=True)
    out, lg, _ = _gpu_decode(cfg, kc, vc, lens, q)
    # the plain variant (no logits requested): another kernel variant where
    # the grid allows (two block groups per workgroup)
    out_plain, _, _ = _gpu_decode(cfg, kc, vc, lens, q, want_logits=False)
    ref_out, ref_lg = oracle.decode(spec, P, R, lens, q, want_logits=True)
    G = n_q // n_kv
    for b, n in enumerate(lens):
        rows = slice(b * n_q, (b + 1) * n_q)
        check_out(out[b], ref_out[rows], f"{codec} b={b}")
        check_out(out_plain[b], ref_out[rows], f"{codec} b={b} (no logits)")
        if n:
            check_logits(lg[b], ref_lg[rows], n, f"{codec} b={b}")
            assert np.all(np.isnan(lg[b][:, n:])), "logits written past the sequence"
        else:
            assert np.all(out[b] == 0) and np.all(out_plain[b] == 0)


def test_raw_bypass_is_textbook_attention():
    """Quantisation bypassed on both tensors: the kernel is plain softmax
    attention; compare with an fp64 textbook computation."""
    cfg = tq.make_config(n_q_heads=32, n_kv_heads=8, batch=2, max_ctx=1000, k_codec=tq.RAW_F32,
                         v_codec=tq.RAW_F32, seed=1, layer=0)
    spec, P, R, kc, vc, q = _oracle_cache(cfg, [1000, 517], seed=3)
    out, lg, _ = _gpu_decode(cfg, kc, vc, [1000, 517], q)
    kr = R.kraw.reshape(2, 1000, 8, 128).astype(np.float64)
    vr = R.vraw.reshape(2, 1000, 8, 128).astype(np.float64)
    for b, n in enumerate([1000, 517]):
        for h in range(32):
            l = kr[b, :n, h // 4] @ q[b, h].astype(np.float64) / math.sqrt(128)
            p = np.exp(l - l.max())
            o = (p / p.sum()) @ vr[b, :n, h // 4]
            assert np.max(np.abs(lg[b, h, :n] - l)) <= 1e-5 * max(1.0, np.abs(l).max())
            assert np.max(np.abs(out[b, h] - o)) <= 1e-5 * max(1.0, np.abs(o).max())


@pytest.mark.parametrize("codec", ["qjl3_v2", "q8_v2", "raw_raw"])
def test_split_count_invariance(codec):
    kc_, kb_, vc_, vb_ = CODECS[codec]
    lens = [2000, 1500]
    base = dict(n_q_heads=32, n_kv_heads=8, batch=2, max_ctx=2000, k_codec=kc_, k_bits=kb_, v_codec=vc_,
                v_bits=vb_, seed=42, layer=0)
    cfg0 = tq.make_config(**base)
    spec, P, R, kc, vc, q = _oracle_cache(cfg0, lens, seed=5)
    outs, lgs = [], []
    for chunk in (0, 128, 384, 2048):
        cfg = tq.make_config(decode_chunk=chunk, **base)
        o, l, _ = _gpu_decode(cfg, kc, vc, lens, q)
        outs.append(o)
        lgs.append(l)
    # the merge order changes with the split count, and so do the per-32-position
    # exponents of the probability limbs (12 significant bits): results agree
    # to well below the 2e-3 output bar
    for o, l in zip(outs[1:], lgs[1:]):
        assert np.max(np.abs(o - outs[0])) <= 1e-4 * max(1.0, np.abs(outs[0]).max())
        assert np.array_equal(np.nan_to_num(l, nan=7.0), np.nan_to_num(lgs[0], nan=7.0))


def test_workspace_counters_return_to_zero_and_repeat():
    cfg = tq.make_config(n_q_heads=32, n_kv_heads=8, batch=2, max_ctx=700, seed=42, layer=0)
    spec, P, R, kc, vc, q = _oracle_cache(cfg, [700, 300], seed=8)
    k_cache, v_cache = upload_cache(kc, vc, DEV)
    params = tq.init_params(cfg, DEV)
    seq = torch.tensor([700, 300], dtype=torch.int32, device=DEV)
    ws = torch.zeros(tq.decode_workspace_bytes(cfg, 700), dtype=torch.uint8, device=DEV)
    qd = torch.from_numpy(q).to(DEV)
    outs = []
    for _ in range(3):
        out = torch.empty_like(qd)
        tq.decode_attention(cfg, params, k_cache, v_cache, seq, 700, qd, out, ws)
        outs.append(out)
    torch.cuda.synchronize()
    assert torch.equal(outs[0], outs[1]) and torch.equal(outs[0], outs[2])
    # the counters [batch][n_kv][4] u32 open the workspace; they must all be zero again
    n_cnt = 2 * 8 * 4 * 4
    assert torch.count_nonzero(ws[:n_cnt]) == 0


def test_logits_equal_dequantised_qjl_inner_products():
    """Cross-API invariant: the decode logits equal <q, x_tilde>/sqrt(d) with
    x_tilde = tq_dequantize(..., TQ_DEQ_QJL)."""
    cfg = tq.make_config(n_q_heads=8, n_kv_heads=2, batch=1, max_ctx=256, seed=42, layer=6)
    spec, P, R, kc, vc, q = _oracle_cache(cfg, [256], seed=13)
    out, lg, _ = _gpu_decode(cfg, kc, vc, [256], q)
    k_cache, v_cache = upload_cache(kc, vc, DEV)
    params = tq.init_params(cfg, DEV)
    xt = torch.empty(256, 2, 128, device=DEV)
    tq.dequantize(cfg, params, k_cache, v_cache, 0, 0, 256, xt, None, qjl=True)
    torch.cuda.synchronize()
    xt = xt.cpu().numpy().astype(np.float64)
    for h in range(8):
        want = xt[:, h // 4] @ q[0, h].astype(np.float64) / math.sqrt(128)
        check_logits(lg[0, h:h + 1], want[None], 256, f"head {h}")


@pytest.mark.parametrize("wi,wname", [(0, "tiny_b1_ctx1k_h8x2")])
def test_end_to_end_tiny_workload_full_size(wi, wname):
    """The 1K-context tiny workload at its full size: GPU append + GPU decode
    against oracle append + oracle decode from the same inputs."""
    w = synth.WORKLOADS[wname]
    cfg = tq.config_for(w, seed=42, layer=0)
    L = tq.KVLayer(cfg, DEV)
    k, v = synth.make_kv(w, w.ctx, seed=1000 + wi)
    q = synth.make_q(w, seed=2000 + wi)
    L.append(k.to(DEV), v.to(DEV))
    lg = torch.full((1, w.n_q, w.ctx), float("nan"), device=DEV)
    out = L.decode(q.to(DEV), logits=lg).cpu().numpy()
    torch.cuda.synchronize()
    spec = spec_of(cfg)
    P = oracle.Params(spec, 42, 0)
    kn, vn = widen_np(k), widen_np(v)
    R = oracle_quantize(spec, P, kn, vn, [w.ctx])
    G = gpu_records(spec, L.k_cache, L.v_cache, [w.ctx])
    st = compare_records(spec, P, G, R, [w.ctx], kn, wname)
    ref_out, ref_lg = oracle.decode(spec, P, R, [w.ctx], q.numpy(), want_logits=True)
    differ = (G.signs != R.signs).any(axis=1).reshape(w.ctx, w.n_kv)       # records with a sign exception
    skip = np.stack([differ[:, h // w.group] for h in range(w.n_q)])
    check_logits(lg.cpu().numpy()[0], ref_lg, w.ctx, wname, skip=skip)
    check_out(out[0], ref_out, wname)
    print(st)


@pytest.mark.parametrize("k_bits,v_bits,lengths", [
    (3, 2, (4096, 2048, 4096, 1, 4096)),
    # 4-bit values: 448 blocks run two block groups per workgroup, 449 one
    (4, 4, (449 * 128 + 1, 448 * 128, 449 * 128 + 1, 300, 449 * 128 + 1)),
])
def test_workspace_reuse_across_lengths(k_bits, v_bits, lengths):
    """One workspace sized for the longest call serves calls of every shorter
    length in any order: each output equals (bit for bit) a decode of the same
    length on a freshly zeroed workspace."""
    n_max = max(lengths)
    cfg = tq.make_config(n_q_heads=32, n_kv_heads=8, batch=1, max_ctx=n_max, k_codec=tq.POLAR_QJL, k_bits=k_bits,
                         v_codec=tq.POLAR, v_bits=v_bits, seed=42, layer=0)
    L = tq.KVLayer(cfg, DEV)
    g = torch.Generator(device=DEV).manual_seed(17)
    k = torch.randn((1, n_max, 8, 128), generator=g, device=DEV).to(torch.bfloat16)
    v = torch.randn((1, n_max, 8, 128), generator=g, device=DEV).to(torch.bfloat16)
    L.append(k, v)
    q = torch.randn((1, 32, 128), generator=g, device=DEV)
    ws = torch.zeros(tq.decode_workspace_bytes(cfg, n_max), dtype=torch.uint8, device=DEV)
    for n in lengths:
        seq = torch.tensor([n], dtype=torch.int32, device=DEV)
        out = torch.empty_like(q)
        tq.decode_attention(cfg, L.params, L.k_cache, L.v_cache, seq, n, q, out, ws)
        fresh = torch.empty_like(q)
        tq.decode_attention(cfg, L.params, L.k_cache, L.v_cache, seq, n, q, fresh,
                            torch.zeros(tq.decode_workspace_bytes(cfg, n), dtype=torch.uint8, device=DEV))
        torch.cuda.synchronize()
        assert torch.equal(out, fresh), f"length {n} on the shared workspace"
