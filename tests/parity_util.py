"""Shared helpers for the GPU parity tests: build oracle views of a library
configuration, compare packed records and decode results to the documented
bars.

Bars:
  codes, fp16 radii, q8 codes/scales: bit-exact;
  QJL sign bits: bit-exact except entries whose oracle sketch value lies
    within 1e-5 of zero in units of the rotated residual norm, and at most
    floor(1e-4 x the sign bits compared) of them;
  recursive polar angle codes: the same rule, for angles within 1e-5 rad of
    a decision boundary (the wrap-around at 0 = 2 pi included);
  logits: |gpu - oracle| <= 1e-3 * max(|oracle|, rms of that head's logits);
  outputs: |gpu - oracle| <= 2e-3.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import sys

import numpy as np
import torch

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, os.path.join(ROOT, "oracle"))
import oracle  # noqa: E402

from compressed_decode_attention_quantize_amd import synth, tq  # noqa: E402

LOGIT_REL = 1e-3
OUT_ABS = 2e-3
SIGN_BAND = 1e-5
SIGN_FRACTION = 1e-4
THREADS = min(16, os.cpu_count() or 1)


def spec_of(cfg, batch=None, max_ctx=None, n_kv=None, n_q=None):
    return oracle.make_spec(d=cfg.head_dim, n_q=cfg.n_q_heads if n_q is None else n_q,
                            n_kv=cfg.n_kv_heads if n_kv is None else n_kv,
                            batch=cfg.batch if batch is None else batch,
                            max_ctx=cfg.max_ctx if max_ctx is None else max_ctx,
                            k_codec=cfg.k_codec, k_bits=cfg.k_bits, m=cfg.qjl_m, v_codec=cfg.v_codec,
                            v_bits=cfg.v_bits)


def widen_np(x: torch.Tensor) -> np.ndarray:
    return x.detach().to("cpu").to(torch.float32).contiguous().numpy()


def oracle_quantize(spec, P, k, v, lens_done, n_new_list=None):
    """Oracle records for inputs k, v [batch][n][n_kv][d] (numpy fp32) written
    at positions 0..n-1 of every sequence (per-sequence lengths `lens_done`
    say how many positions of each sequence are real)."""
    R = oracle.Records(spec)
    for b in range(spec.batch):
        n = int(lens_done[b])
        if n:
            oracle.quantize_into(spec, P, R, k[b, :n], v[b, :n], b, 0)
    return R


def oracle_quantize_threaded(spec, P, k, v, n):
    """Batch-1 spec: quantise positions 0..n-1 in parallel chunks (the oracle
    itself stays single-threaded per call; ctypes releases the GIL)."""
    R = oracle.Records(spec)
    chunk = max(256, (n + THREADS - 1) // THREADS)
    with cf.ThreadPoolExecutor(THREADS) as ex:
        futs = [ex.submit(oracle.quantize_into, spec, P, R, k[s:s + chunk], v[s:s + chunk], 0, s)
                for s in range(0, n, chunk)]
        for f in futs:
            f.result()
    return R


def _tree_mismatches(spec, D, bits, Gc, Rc, sel, x, label):
    """Angle codes of the recursive polar codec: equal except within the
    band of a decision boundary (checked on the oracle's own margins)."""
    diff = (Gc != Rc) & sel[:, None]
    n_bad = int(diff.sum())
    assert n_bad <= int(SIGN_FRACTION * int(sel.sum()) * spec.d), f"{label}: {n_bad} angle codes differ"
    if n_bad:
        assert x is not None, f"{label}: angle codes differ and no inputs to check the band"
        T = oracle.tree_tables(bits, spec.d)
        for rec in np.unique(np.nonzero(diff)[0]):
            h = rec % spec.n_kv
            pos = (rec // spec.n_kv) % spec.max_ctx
            b = rec // (spec.n_kv * spec.max_ctx)
            r = oracle.quantize_tree(x[b, pos, h], D, T)
            bad = np.nonzero(diff[rec])[0]
            assert np.all(r["amargin"][bad] < SIGN_BAND), f"{label}: angle code outside the band"
    return n_bad


def compare_records(spec, P, G, R, lens, x_k=None, label="", x_v=None):
    """Compare GPU-unpacked records G with oracle records R over positions
    [0, lens[b]).  x_k, x_v (numpy [batch][n][n_kv][d]) let sign and angle
    code mismatches be checked against the oracle's margins.  Returns a
    stats dict."""
    sel = np.zeros(R.n, bool)
    for b in range(spec.batch):
        for pos in range(int(lens[b])):
            base = (b * spec.max_ctx + pos) * spec.n_kv
            sel[base:base + spec.n_kv] = True
    st = dict(records=int(sel.sum()), sign_mismatch=0, sign_total=0)
    kc, vc = spec.k_codec, spec.v_codec
    if kc in (oracle.POLAR, oracle.POLAR_QJL):
        assert np.array_equal(G.kcodes[sel], R.kcodes[sel]), f"{label}: key codes differ"
        assert np.array_equal(G.kn16[sel], R.kn16[sel]), f"{label}: key radii differ"
    if kc == oracle.POLAR_QJL:
        assert np.array_equal(G.rho16[sel], R.rho16[sel]), f"{label}: residual norms differ"
        diff = (G.signs != R.signs) & sel[:, None]
        st["sign_mismatch"] = int(diff.sum())
        st["sign_total"] = int(sel.sum()) * spec.m
        assert st["sign_mismatch"] <= int(SIGN_FRACTION * st["sign_total"]), f"{label}: {st}"
        if st["sign_mismatch"]:
            assert x_k is not None, f"{label}: sign bits differ and no inputs to check the band"
            recs = np.unique(np.nonzero(diff)[0])
            for rec in recs:
                h = rec % spec.n_kv
                pos = (rec // spec.n_kv) % spec.max_ctx
                b = rec // (spec.n_kv * spec.max_ctx)
                r = oracle.quantize_polar(x_k[b, pos, h], P.DK, P.ck16, P.kbounds, spec.k_bits, spec.m, P.S)
                bad = np.nonzero(diff[rec])[0]
                assert np.all(np.abs(r["z"][bad]) < SIGN_BAND * r["rrot"]), f"{label}: sign outside band"
    if kc == oracle.POLAR_TREE:
        assert np.array_equal(G.kn16[sel], R.kn16[sel]), f"{label}: key radii differ"
        st["k_angle_mismatch"] = _tree_mismatches(spec, P.DK, spec.k_bits, G.kcodes, R.kcodes, sel, x_k,
                                                  label + " keys")
    if kc == oracle.Q8_BLOCK32:
        assert np.array_equal(G.k8[sel], R.k8[sel]), f"{label}: q8 codes differ"
        assert np.array_equal(G.s16[sel], R.s16[sel]), f"{label}: q8 scales differ"
    if kc == oracle.RAW_F32:
        assert np.array_equal(G.kraw[sel], R.kraw[sel])
    if vc == oracle.POLAR:
        assert np.array_equal(G.vcodes[sel], R.vcodes[sel]), f"{label}: value codes differ"
        assert np.array_equal(G.vn16[sel], R.vn16[sel]), f"{label}: value radii differ"
    elif vc == oracle.POLAR_TREE:
        assert np.array_equal(G.vn16[sel], R.vn16[sel]), f"{label}: value radii differ"
        st["v_angle_mismatch"] = _tree_mismatches(spec, P.DV, spec.v_bits, G.vcodes, R.vcodes, sel, x_v,
                                                  label + " values")
    else:
        assert np.array_equal(G.vraw[sel], R.vraw[sel])
    return st


MIN_RMS_POSITIONS = 16


def check_logits(gpu_lg, ref_lg, n, label="", skip=None):
    """gpu_lg, ref_lg: [n_pairs][>=n]; skip: optional bool mask [n_pairs][n]
    of positions excluded (records that differ by a counted sign exception).

    Bar: |d| <= LOGIT_REL * max(|ref|, rms of that head's logits).  A row of
    fewer than MIN_RMS_POSITIONS positions takes the rms over every row of
    the call instead: over one position the row rms is |ref| itself, and the
    bar would turn back into the pure relative error that is undefined near 0."""
    g = np.asarray(gpu_lg, np.float64)[:, :n]
    r = np.asarray(ref_lg, np.float64)[:, :n]
    if n >= MIN_RMS_POSITIONS:
        rms = np.sqrt(np.mean(r * r, axis=1, keepdims=True))
    else:
        rms = np.full((r.shape[0], 1), np.sqrt(np.mean(r * r)) if r.size else 0.0)
    tol = LOGIT_REL * np.maximum(np.abs(r), rms)
    bad = np.abs(g - r) > tol
    if skip is not None:
        bad &= ~skip
    worst = float(np.max(np.abs(g - r) / np.maximum(np.abs(r), rms))) if n else 0.0
    assert not bad.any(), f"{label}: {int(bad.sum())} logits beyond the bar (worst rel {worst:.3g})"
    return worst


def check_out(gpu_out, ref_out, label=""):
    err = float(np.max(np.abs(np.asarray(gpu_out, np.float64) - np.asarray(ref_out, np.float64))))
    assert err <= OUT_ABS, f"{label}: output error {err}"
    return err


def upload_cache(kc: np.ndarray, vc: np.ndarray, dev):
    return torch.from_numpy(kc).to(dev), torch.from_numpy(vc).to(dev)


def gpu_records(spec, k_cache: torch.Tensor, v_cache: torch.Tensor, lens):
    return oracle.unpack_cache(spec, k_cache.cpu().numpy(), v_cache.cpu().numpy(), np.asarray(lens, np.int32))
