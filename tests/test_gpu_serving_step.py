"""The fused serving step (tq_append_decode): one new position per sequence
stored and attended to in one launch.  Its cache bytes and outputs must equal
those of tq_quantize_append followed by tq_decode_attention (the same kernels'
arithmetic), step after step, and the outputs must match the oracle's decode
over everything appended."""
import numpy as np
import pytest
import torch

from parity_util import check_logits, check_out, oracle, oracle_quantize, spec_of, tq, widen_np

pytestmark = pytest.mark.gpu
DEV = "cuda"

CODECS = {   # name -> (k_codec, k_bits, v_codec, v_bits)
    "qjl3_v2": (tq.POLAR_QJL, 3, tq.POLAR, 2),
    "qjl4_v4": (tq.POLAR_QJL, 4, tq.POLAR, 4),
    "qjl2_v3": (tq.POLAR_QJL, 2, tq.POLAR, 3),
    "q8_v4": (tq.Q8_BLOCK32, 8, tq.POLAR, 4),
    "q8_v2": (tq.Q8_BLOCK32, 8, tq.POLAR, 2),            # G = 12: one workgroup for the three head groups
    "polar2_v2": (tq.POLAR, 2, tq.POLAR, 2),
    "raw_raw": (tq.RAW_F32, 32, tq.RAW_F32, 32),        # two launches
    "tree3_tree2": (tq.POLAR_TREE, 3, tq.POLAR_TREE, 2),  # two launches
}
LENS0 = [0, 127, 128, 300]
STEPS = 5


def _pair(codec, heads, chunk, max_ctx=320):
    kc, kb, vc, vb = CODECS[codec]
    cfg = tq.make_config(n_q_heads=heads[0], n_kv_heads=heads[1], batch=len(LENS0), max_ctx=max_ctx, k_codec=kc,
                         k_bits=kb, v_codec=vc, v_bits=vb, decode_chunk=chunk, seed=42, layer=9)
    return cfg, tq.KVLayer(cfg, DEV), tq.KVLayer(cfg, DEV)


def _prefill(L, k, v):
    """Ragged prefill: one append of max(LENS0) positions into every
    sequence, then the lengths cut back to LENS0 (later appends overwrite the
    positions past them)."""
    n = max(LENS0)
    L.append(k[:, :n].contiguous(), v[:, :n].contiguous())
    L.seq_lens.copy_(torch.tensor(LENS0, dtype=torch.int32, device=DEV))
    L.max_len = n


@pytest.mark.parametrize("codec", list(CODECS))
@pytest.mark.parametrize("heads", [(32, 8), (96, 8), (12, 2)])
@pytest.mark.parametrize("chunk", [0, 128])
def test_fused_step_equals_append_then_decode(codec, heads, chunk):
    print(f"[serving step] {codec} heads={heads} chunk={chunk}", flush=True)
    cfg, A, B = _pair(codec, heads, chunk)
    g = torch.Generator(device="cpu").manual_seed(100 * list(CODECS).index(codec) + heads[0] + chunk)
    n0 = max(LENS0)
    k = torch.randn((cfg.batch, n0 + STEPS, cfg.n_kv_heads, 128), generator=g).to(torch.bfloat16).to(DEV)
    v = torch.randn((cfg.batch, n0 + STEPS, cfg.n_kv_heads, 128), generator=g).to(torch.bfloat16).to(DEV)
    _prefill(A, k, v)
    _prefill(B, k, v)
    torch.cuda.synchronize()
    lens = list(LENS0)
    for s in range(STEPS):
        q = torch.randn((cfg.batch, cfg.n_q_heads, 128), generator=g).to(DEV)
        # the new position of sequence b comes from row lens[b] of the inputs
        idx = torch.tensor(lens, device=DEV)
        kn = k[torch.arange(cfg.batch, device=DEV), idx].unsqueeze(1).contiguous()
        vn = v[torch.arange(cfg.batch, device=DEV), idx].unsqueeze(1).contiguous()
        la = torch.full((cfg.batch, cfg.n_q_heads, cfg.max_ctx), float("nan"), device=DEV)
        lb = torch.full_like(la, float("nan"))
        oa = A.step(kn, vn, q, logits=la)
        B.append(kn, vn)
        ob = B.decode(q, logits=lb)
        torch.cuda.synchronize()
        assert torch.equal(A.k_cache, B.k_cache) and torch.equal(A.v_cache, B.v_cache), f"step {s}: caches differ"
        assert torch.equal(oa, ob), f"step {s}: outputs differ by {float((oa - ob).abs().max())}"
        assert torch.equal(torch.nan_to_num(la, nan=7.0), torch.nan_to_num(lb, nan=7.0)), f"step {s}: logits"
        assert torch.equal(A.seq_lens, B.seq_lens)
        lens = [n + 1 for n in lens]


@pytest.mark.parametrize("codec", ["qjl3_v2", "q8_v4"])
def test_fused_steps_match_oracle(codec):
    """Prefill, then steps through the fused call only; the last step's
    output against the oracle's decode over every position it stored."""
    cfg, A, _ = _pair(codec, (32, 8) if codec != "q8_v4" else (96, 8), 0)
    g = torch.Generator(device="cpu").manual_seed(11)
    n0 = max(LENS0)
    k = torch.randn((cfg.batch, n0 + STEPS, cfg.n_kv_heads, 128), generator=g).to(torch.bfloat16)
    v = torch.randn((cfg.batch, n0 + STEPS, cfg.n_kv_heads, 128), generator=g).to(torch.bfloat16)
    kd, vd = k.to(DEV), v.to(DEV)
    _prefill(A, kd, vd)
    lens = list(LENS0)
    for s in range(STEPS):
        q = torch.randn((cfg.batch, cfg.n_q_heads, 128), generator=g)
        idx = torch.tensor(lens)
        kn = kd[torch.arange(cfg.batch, device=DEV), idx.to(DEV)].unsqueeze(1).contiguous()
        vn = vd[torch.arange(cfg.batch, device=DEV), idx.to(DEV)].unsqueeze(1).contiguous()
        lg = torch.full((cfg.batch, cfg.n_q_heads, cfg.max_ctx), float("nan"), device=DEV)
        out = A.step(kn, vn, q.to(DEV), logits=lg)
        lens = [n + 1 for n in lens]
    torch.cuda.synchronize()
    # the oracle's records: sequence b holds rows 0 .. lens[b] - 1 of its inputs
    spec = spec_of(cfg)
    P = oracle.Params(spec, cfg.seed, cfg.layer)
    R = oracle_quantize(spec, P, widen_np(k), widen_np(v), lens)
    ref_out, ref_lg = oracle.decode(spec, P, R, lens, q.numpy(), want_logits=True)
    out, lg = out.cpu().numpy(), lg.cpu().numpy()
    for b, n in enumerate(lens):
        rows = slice(b * cfg.n_q_heads, (b + 1) * cfg.n_q_heads)
        check_out(out[b], ref_out[rows], f"{codec} b={b}")
        check_logits(lg[b], ref_lg[rows], n, f"{codec} b={b}")


def test_fused_step_long_splits():
    """4-bit keys and values over sequences of up to 15000 positions, so that
    every split runs several steps, with the new position in the middle of a
    split: the fused step must still equal append then decode, step after
    step."""
    lens0 = [15000, 9000, 300, 14000]
    cfg = tq.make_config(n_q_heads=32, n_kv_heads=8, batch=4, max_ctx=15104, k_codec=tq.POLAR_QJL, k_bits=4,
                         v_codec=tq.POLAR, v_bits=4, seed=42, layer=3)
    A, B = tq.KVLayer(cfg, DEV), tq.KVLayer(cfg, DEV)
    g = torch.Generator(device="cpu").manual_seed(77)
    n0 = max(lens0)
    k = torch.randn((cfg.batch, n0 + 3, cfg.n_kv_heads, 128), generator=g).to(torch.bfloat16).to(DEV)
    v = torch.randn((cfg.batch, n0 + 3, cfg.n_kv_heads, 128), generator=g).to(torch.bfloat16).to(DEV)
    for L in (A, B):
        L.append(k[:, :n0].contiguous(), v[:, :n0].contiguous())
        L.seq_lens.copy_(torch.tensor(lens0, dtype=torch.int32, device=DEV))
        L.max_len = n0
    torch.cuda.synchronize()
    lens = list(lens0)
    for s in range(3):
        print(f"[serving step, one group] step {s}", flush=True)
        q = torch.randn((cfg.batch, cfg.n_q_heads, 128), generator=g).to(DEV)
        idx = torch.tensor(lens, device=DEV)
        kn = k[torch.arange(cfg.batch, device=DEV), idx].unsqueeze(1).contiguous()
        vn = v[torch.arange(cfg.batch, device=DEV), idx].unsqueeze(1).contiguous()
        oa = A.step(kn, vn, q)
        B.append(kn, vn)
        ob = B.decode(q)
        torch.cuda.synchronize()
        assert torch.equal(A.k_cache, B.k_cache) and torch.equal(A.v_cache, B.v_cache), f"step {s}: caches differ"
        assert torch.equal(oa, ob), f"step {s}: outputs differ by {float((oa - ob).abs().max())}"
        lens = [n + 1 for n in lens]
