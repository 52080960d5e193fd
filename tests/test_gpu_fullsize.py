"""Parity at the workloads' full sizes, in the launch configuration the
benchmark times (one prefill append of the whole context, then decode): the
records of every (sequence, KV head) bit-exact against the oracle (counted
sign exceptions inside the band), and on sampled pairs the query heads'
logits and outputs to the bars."""
import concurrent.futures as cf

import numpy as np
import pytest
import torch

from parity_util import (THREADS, check_logits, check_out, compare_records, oracle, oracle_quantize_threaded,
                         spec_of, synth, tq, widen_np)

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _sub_records(cfg, layer, b, h, n):
    """GPU records of one (sequence, KV head), unpacked by the oracle."""
    sub = spec_of(cfg, batch=1, n_kv=1, n_q=cfg.n_q_heads // cfg.n_kv_heads)
    nb = (cfg.max_ctx + 127) // 128
    kb, vb = tq.cache_bytes(cfg)
    kslot = kb // (cfg.batch * cfg.n_kv_heads)
    vslot = vb // (cfg.batch * cfg.n_kv_heads)
    idx = b * cfg.n_kv_heads + h
    kc = layer.k_cache[idx * kslot:(idx + 1) * kslot].cpu().numpy()
    vc = layer.v_cache[idx * vslot:(idx + 1) * vslot].cpu().numpy()
    assert kslot == nb * 128 * oracle.spec_sizes(sub)["k_record"]
    return sub, oracle.unpack_cache(sub, kc, vc, np.array([n], np.int32))


def _oracle_decode_threaded(sub, P, R, n, qh):
    G = qh.shape[0]
    with cf.ThreadPoolExecutor(min(G, THREADS)) as ex:
        futs = [ex.submit(oracle.decode, sub, P, R, [n], qh[None], [(0, g)], True) for g in range(G)]
        res = [f.result() for f in futs]
    return np.concatenate([r[0] for r in res]), np.concatenate([r[1] for r in res])


def _check_all_records(cfg, layer, k, v, lens, label):
    """Records of every (sequence, KV head) of the layer against the oracle,
    one sequence at a time (the oracle quantises in parallel chunks)."""
    kb, vb = tq.cache_bytes(cfg)
    kseq, vseq = kb // cfg.batch, vb // cfg.batch
    sub = spec_of(cfg, batch=1)
    P = oracle.Params(sub, cfg.seed, cfg.layer)
    tot = dict(records=0, sign_mismatch=0, sign_total=0)
    for b in range(cfg.batch):
        n = int(lens[b])
        kc = layer.k_cache[b * kseq:(b + 1) * kseq].cpu().numpy()
        vc = layer.v_cache[b * vseq:(b + 1) * vseq].cpu().numpy()
        Gr = oracle.unpack_cache(sub, kc, vc, np.array([n], np.int32))
        kn = widen_np(k[b, :n])
        vn = widen_np(v[b, :n])
        R = oracle_quantize_threaded(sub, P, kn, vn, n)
        st = compare_records(sub, P, Gr, R, [n], kn[None], f"{label} b={b}")
        for key in tot:
            tot[key] += st[key]
        del Gr, R
    print(f"{label}: every record of {cfg.batch} x {cfg.n_kv_heads} (sequence, KV head) pairs bit-exact: {tot}",
          flush=True)
    return tot


def _check_pair(cfg, layer, k, v, q, lg, out, b, h, n, label, out_plain=None):
    G = cfg.n_q_heads // cfg.n_kv_heads
    sub, Gr = _sub_records(cfg, layer, b, h, n)
    P = oracle.Params(sub, cfg.seed, cfg.layer)
    kn = widen_np(k[b, :n, h])[:, None, :]
    vn = widen_np(v[b, :n, h])[:, None, :]
    R = oracle_quantize_threaded(sub, P, kn, vn, n)
    st = compare_records(sub, P, Gr, R, [n], kn[None], label)
    qh = q[b, h * G:(h + 1) * G].cpu().numpy()
    ref_out, ref_lg = _oracle_decode_threaded(sub, P, R, n, qh)
    skip = None
    if sub.k_codec == oracle.POLAR_QJL:
        differ = (Gr.signs[:n] != R.signs[:n]).any(axis=1)
        skip = np.repeat(differ[None], G, axis=0)
    worst = check_logits(lg[b, h * G:(h + 1) * G].cpu().numpy(), ref_lg, n, label, skip=skip)
    err = check_out(out[b, h * G:(h + 1) * G].cpu().numpy(), ref_out, label)
    if out_plain is not None:   # the decode without logits (the launch the benchmark times)
        err = max(err, check_out(out_plain[b, h * G:(h + 1) * G].cpu().numpy(), ref_out, label + " (no logits)"))
    print(f"{label}: records={st['records']} sign exceptions={st['sign_mismatch']}/{st['sign_total']} "
          f"worst logit rel={worst:.2e} max out err={err:.2e}", flush=True)


@pytest.mark.parametrize("wi,wname", [(i, n) for i, n in enumerate(synth.ORDER) if n != "serving_b16_ctx8k"])
def test_full_size_prefill_then_decode(wi, wname):
    w = synth.WORKLOADS[wname]
    print(f"[fullsize] {wname}", flush=True)
    cfg = tq.config_for(w, seed=42, layer=0)
    L = tq.KVLayer(cfg, DEV)
    k, v = synth.make_kv(w, w.ctx, seed=1000 + wi, device=DEV)
    q = synth.make_q(w, seed=2000 + wi, device=DEV)
    L.append(k, v)
    lg = torch.full((w.batch, w.n_q, w.ctx), float("nan"), device=DEV)
    out = L.decode(q, logits=lg)
    out_plain = L.decode(q)
    torch.cuda.synchronize()
    assert torch.isfinite(out).all() and torch.isfinite(out_plain).all()
    rng = np.random.default_rng(wi)
    h = int(rng.integers(0, w.n_kv))
    _check_pair(cfg, L, k, v, q, lg, out, 0, h, w.ctx, f"{wname} kv={h}", out_plain=out_plain)


@pytest.mark.parametrize("wi,wname", [(i, n) for i, n in enumerate(synth.ORDER) if n != "serving_b16_ctx8k"])
def test_full_size_records_every_head(wi, wname):
    """The prefill of the benchmark's launch configuration: the records of
    every KV head of the workload against the oracle."""
    w = synth.WORKLOADS[wname]
    print(f"[fullsize records] {wname}", flush=True)
    cfg = tq.config_for(w, seed=42, layer=0)
    L = tq.KVLayer(cfg, DEV)
    k, v = synth.make_kv(w, w.ctx, seed=1000 + wi, device=DEV)
    L.append(k, v)
    torch.cuda.synchronize()
    _check_all_records(cfg, L, k, v, [w.ctx] * w.batch, wname)


def test_full_size_serving_steps():
    """Batched serving: 16 x 8192 prefill, then 64 steps of one appended
    position per sequence followed by decode; steps 0, 31 and 63 checked on
    two sampled (sequence, KV head) pairs, and at step 63 the records of
    every (sequence, KV head)."""
    wi, w = 2, synth.WORKLOADS["serving_b16_ctx8k"]
    cfg = tq.config_for(w, seed=42, layer=0, max_ctx=w.ctx + w.steps)
    L = tq.KVLayer(cfg, DEV)
    n_tot = w.ctx + w.steps
    k, v = synth.make_kv(w, n_tot, seed=1000 + wi, device=DEV)
    L.append(k[:, :w.ctx].contiguous(), v[:, :w.ctx].contiguous())
    pairs = [(3, 5), (11, 0)]
    for step in range(w.steps):
        L.append(k[:, w.ctx + step:w.ctx + step + 1].contiguous(), v[:, w.ctx + step:w.ctx + step + 1].contiguous())
        q = synth.make_q(w, seed=5000 + step, device=DEV)
        lg = torch.full((w.batch, w.n_q, cfg.max_ctx), float("nan"), device=DEV)
        out = L.decode(q, logits=lg)
        if step in (0, 31, 63):
            torch.cuda.synchronize()
            n = w.ctx + step + 1
            for b, h in pairs:
                _check_pair(cfg, L, k, v, q, lg, out, b, h, n, f"serving step {step} b={b} kv={h}")
            if step == w.steps - 1:
                _check_all_records(cfg, L, k, v, [n] * w.batch, f"serving step {step}")


def test_full_size_fused_serving_steps():
    """The same 64 serving steps through the fused step (tq_append_decode:
    the new position stored and attended to in one launch, the launch the
    serving bench times): steps 0, 31 and 63 against the oracle on two
    sampled (sequence, KV head) pairs, records included, and at step 63 the
    records of every (sequence, KV head)."""
    wi, w = 2, synth.WORKLOADS["serving_b16_ctx8k"]
    cfg = tq.config_for(w, seed=42, layer=0, max_ctx=w.ctx + w.steps)
    L = tq.KVLayer(cfg, DEV)
    n_tot = w.ctx + w.steps
    k, v = synth.make_kv(w, n_tot, seed=1000 + wi, device=DEV)
    L.append(k[:, :w.ctx].contiguous(), v[:, :w.ctx].contiguous())
    pairs = [(6, 2), (15, 7)]
    for step in range(w.steps):
        q = synth.make_q(w, seed=5000 + step, device=DEV)
        lg = torch.full((w.batch, w.n_q, cfg.max_ctx), float("nan"), device=DEV)
        out = L.step(k[:, w.ctx + step:w.ctx + step + 1].contiguous(),
                     v[:, w.ctx + step:w.ctx + step + 1].contiguous(), q, logits=lg)
        if step in (0, 31, 63):
            torch.cuda.synchronize()
            n = w.ctx + step + 1
            for b, h in pairs:
                _check_pair(cfg, L, k, v, q, lg, out, b, h, n, f"fused serving step {step} b={b} kv={h}")
            if step == w.steps - 1:
                _check_all_records(cfg, L, k, v, [n] * w.batch, f"fused serving step {step}")


def test_full_size_sparse_v_1m():
    """Sparse-V at the 1M-context workload in the benchmark's peaked setting
    (one planted key per 1024 positions, skip distance T = 8): on two sampled
    (sequence, KV head) pairs the sparse output stays within the mass of the
    weights below 2^-T of the largest (the oracle's weights and dequantised
    values) of the dense output, and within 2e-3 plus that mass of the
    oracle; logits are the dense launch's bits."""
    wi, w = 4, synth.WORKLOADS["long_b1_ctx1m"]
    T = 8
    k, v = synth.make_kv(w, w.ctx, seed=1000 + wi, device=DEV)
    q = synth.make_q(w, seed=2000 + wi, device=DEV)
    k, _ = synth.plant_focus_keys(w, k, q, seed=3000 + wi, every=1024)
    outs, lgs, layer = [], [], None
    for sv in (0, T):
        cfg = tq.config_for(w, seed=42, layer=0, sparse_v=sv)
        if layer is None:
            layer = tq.KVLayer(cfg, DEV)
            layer.append(k, v)
        lg = torch.full((w.batch, w.n_q, cfg.max_ctx), float("nan"), device=DEV)
        out = torch.empty_like(q)
        tq.decode_attention(cfg, layer.params, layer.k_cache, layer.v_cache, layer.seq_lens, layer.max_len, q, out,
                            torch.zeros(tq.decode_workspace_bytes(cfg, layer.max_len), dtype=torch.uint8, device=DEV),
                            lg)
        torch.cuda.synchronize()
        outs.append(out.cpu().numpy())
        lgs.append(lg.cpu().numpy())
    assert np.array_equal(np.nan_to_num(lgs[0], nan=7.0), np.nan_to_num(lgs[1], nan=7.0))
    assert not np.array_equal(outs[0], outs[1]), "no block was skipped on peaked data"
    n = w.ctx
    G = w.n_q // w.n_kv
    for b, h in [(0, 5)]:
        label = f"sparse-v 1M b={b} kv={h}"
        sub, Gr = _sub_records(cfg, layer, b, h, n)
        P = oracle.Params(sub, cfg.seed, cfg.layer)
        kn = widen_np(k[b, :n, h])[:, None, :]
        vn = widen_np(v[b, :n, h])[:, None, :]
        R = oracle_quantize_threaded(sub, P, kn, vn, n)
        qh = q[b, h * G:(h + 1) * G].cpu().numpy()
        ref_out, ref_lg = _oracle_decode_threaded(sub, P, R, n, qh)
        vabs = np.empty((n, 128))

        def _deq(lo, hi):
            for t in range(lo, hi):
                vabs[t] = np.abs(oracle.dequant_polar(P.DV, P.cv16, R.vcodes[t], R.vn16[t]))

        step = (n + THREADS - 1) // THREADS
        with cf.ThreadPoolExecutor(THREADS) as ex:
            for f in [ex.submit(_deq, s0, min(n, s0 + step)) for s0 in range(0, n, step)]:
                f.result()
        for g in range(G):
            l = ref_lg[g, :n]
            tol = 1e-3 * max(np.abs(l).max(), np.sqrt(np.mean(l * l)))
            p = np.exp(l - l.max())
            small = (l - l.max()) < -T * np.log(2.0) + 2.0 * tol
            env = (p[small] @ vabs[small]) / p.sum()
            d_s, d_d = outs[1][b, h * G + g], outs[0][b, h * G + g]
            rounding = 1e-5 + 6.0 * 2.0 ** -24 * (n / 128) * float(vabs.max())
            assert np.all(np.abs(d_s - d_d) <= env * (1.0 + 1e-3) + rounding), label
            assert np.max(np.abs(d_s - ref_out[g]) - env) <= 2e-3, label
        print(f"{label}: max |sparse - dense| = {np.abs(outs[1][b, h * G:(h + 1) * G] - outs[0][b, h * G:(h + 1) * G]).max():.2e}",
              flush=True)
