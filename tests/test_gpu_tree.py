"""GPU parity of the recursive polar codec (POLAR_TREE: the radius + angle
step of the wis-web.com reader article read as a pairwise tree) against the
oracle, through the C ABI: append (angle codes bit-exact outside the 1e-5 rad
band of a decision boundary, radii bit-exact), decode (logits and outputs to
the usual bars) and dequantisation."""
import numpy as np
import pytest
import torch

from parity_util import (check_logits, check_out, compare_records, gpu_records, oracle, oracle_quantize, spec_of,
                         synth, tq, upload_cache, widen_np)

pytestmark = pytest.mark.gpu
DEV = "cuda"

PAIRS = {   # name -> (k_codec, k_bits, v_codec, v_bits)
    "tree3_tree3": (tq.POLAR_TREE, 3, tq.POLAR_TREE, 3),
    "tree2_tree4": (tq.POLAR_TREE, 2, tq.POLAR_TREE, 4),
    "tree4_tree2": (tq.POLAR_TREE, 4, tq.POLAR_TREE, 2),
    "qjl3_tree3": (tq.POLAR_QJL, 3, tq.POLAR_TREE, 3),
    "tree3_polar2": (tq.POLAR_TREE, 3, tq.POLAR, 2),
    "q8_tree2": (tq.Q8_BLOCK32, 8, tq.POLAR_TREE, 2),
    "raw_tree3": (tq.RAW_F32, 32, tq.POLAR_TREE, 3),
}


def _cfg(pair, n_q=8, n_kv=2, batch=2, ctx=300, layer=5, chunk=0):
    kc, kb, vc, vb = PAIRS[pair]
    return tq.make_config(n_q_heads=n_q, n_kv_heads=n_kv, batch=batch, max_ctx=ctx, k_codec=kc, k_bits=kb,
                          v_codec=vc, v_bits=vb, seed=42, layer=layer, decode_chunk=chunk)


@pytest.mark.parametrize("pair", list(PAIRS))
@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_tree_append_matches_oracle(pair, dtype):
    """Appends of 1, 31, 33, 128 and 107 positions into two sequences; inputs
    N(0, 1) with a few large channels (the 1M workload's Student-t recipe)."""
    cfg = _cfg(pair)
    print(f"[tree append] {pair} {dtype}", flush=True)
    L = tq.KVLayer(cfg, DEV)
    ws = synth.with_ctx(synth.WORKLOADS["long_b1_ctx1m"], 300, batch=2)
    ws = synth.dataclasses.replace(ws, n_q=8, n_kv=2)
    k, v = synth.make_kv(ws, 300, seed=31 + list(PAIRS).index(pair), batch=2)
    k, v = k.to(dtype), v.to(dtype)
    pos = 0
    for n in (1, 31, 33, 128, 107):
        L.append(k[:, pos:pos + n].to(DEV).contiguous(), v[:, pos:pos + n].to(DEV).contiguous())
        pos += n
    torch.cuda.synchronize()
    spec = spec_of(cfg)
    P = oracle.Params(spec, cfg.seed, cfg.layer)
    kn, vn = widen_np(k), widen_np(v)
    R = oracle_quantize(spec, P, kn, vn, [300, 300])
    G = gpu_records(spec, L.k_cache, L.v_cache, [300, 300])
    print(compare_records(spec, P, G, R, [300, 300], kn, pair, x_v=vn))


def test_tree_append_special_vectors():
    """Zero vectors, signed zeros, pairs on the axes (angles exactly on the
    quadrant boundaries, which close on their upper end) and one huge radius
    (fp16 saturation)."""
    cfg = _cfg("tree3_tree3", batch=1, ctx=64)
    L = tq.KVLayer(cfg, DEV)
    x = np.random.default_rng(2).standard_normal((1, 8, 2, 128)).astype(np.float32)
    x[0, 0] = 0.0
    x[0, 1] = -0.0
    x[0, 2, :, 1::2] = 0.0                  # y pairs built from a single axis after rotation are not
    x[0, 3, :, :] = 1.0                     # axis-aligned; constant and one-hot inputs are
    x[0, 4, :, :] = 0.0
    x[0, 4, :, 5] = -2.5
    x[0, 5] *= 1e5
    x[0, 6] *= 1e-30
    k = torch.from_numpy(x)
    L.append(k.to(DEV), (-k).to(DEV))
    torch.cuda.synchronize()
    spec = spec_of(cfg)
    P = oracle.Params(spec, cfg.seed, cfg.layer)
    R = oracle_quantize(spec, P, x, -x, [8])
    G = gpu_records(spec, L.k_cache, L.v_cache, [8])
    compare_records(spec, P, G, R, [8], x, "special", x_v=-x)


def test_tree_offset_append_keeps_other_positions():
    """A sequence that starts at position 37 shares value words with 5
    positions written earlier: their bits stay."""
    cfg = _cfg("tree3_tree3", batch=2, ctx=200)
    L = tq.KVLayer(cfg, DEV)
    rng = np.random.default_rng(4)
    k = rng.standard_normal((2, 200, 2, 128)).astype(np.float32)
    v = rng.standard_normal((2, 200, 2, 128)).astype(np.float32)
    tq.quantize_append(cfg, L.params, L.k_cache, L.v_cache, torch.zeros(2, dtype=torch.int32, device=DEV), 0,
                       torch.from_numpy(k[:, :37]).to(DEV), torch.from_numpy(v[:, :37]).to(DEV))
    tq.quantize_append(cfg, L.params, L.k_cache, L.v_cache, torch.full((2,), 37, dtype=torch.int32, device=DEV),
                       37, torch.from_numpy(k[:, 37:150]).contiguous().to(DEV),
                       torch.from_numpy(v[:, 37:150]).contiguous().to(DEV))
    torch.cuda.synchronize()
    spec = spec_of(cfg)
    P = oracle.Params(spec, cfg.seed, cfg.layer)
    R = oracle_quantize(spec, P, k, v, [150, 150])
    G = gpu_records(spec, L.k_cache, L.v_cache, [150, 150])
    compare_records(spec, P, G, R, [150, 150], k, "offset", x_v=v)


def _oracle_cache(cfg, lens, seed):
    spec = spec_of(cfg)
    P = oracle.Params(spec, cfg.seed, cfg.layer)
    g = torch.Generator().manual_seed(seed)
    k = torch.randn((cfg.batch, cfg.max_ctx, cfg.n_kv_heads, 128), generator=g)
    v = torch.randn((cfg.batch, cfg.max_ctx, cfg.n_kv_heads, 128), generator=g)
    k[:, :, :, :4] *= 10.0
    R = oracle_quantize(spec, P, k.numpy(), v.numpy(), lens)
    kc, vc = oracle.pack_cache(spec, R, np.asarray(lens, np.int32))
    q = torch.randn((cfg.batch, cfg.n_q_heads, 128), generator=g).numpy()
    return spec, P, R, kc, vc, q


@pytest.mark.parametrize("pair", list(PAIRS))
# groups of 4 and 12 (whole head groups of four), 1 (no sharing), 6 (a partial
# head group) and 16 (the largest group)
@pytest.mark.parametrize("heads", [(8, 2), (32, 8), (96, 8), (16, 16), (12, 2), (64, 4)])
def test_tree_decode_matches_oracle(pair, heads):
    n_q, n_kv = heads
    lens = [300, 1, 129, 0]
    cfg = _cfg(pair, n_q=n_q, n_kv=n_kv, batch=4, ctx=300, layer=6)
    print(f"[tree decode] {pair} heads={heads}", flush=True)
    spec, P, R, kc, vc, q = _oracle_cache(cfg, lens, seed=50 + list(PAIRS).index(pair) + n_kv)
    k_cache, v_cache = upload_cache(kc, vc, DEV)
    params = tq.init_params(cfg, DEV)
    seq = torch.tensor(lens, dtype=torch.int32, device=DEV)
    ws = torch.zeros(tq.decode_workspace_bytes(cfg, 300), dtype=torch.uint8, device=DEV)
    qd = torch.from_numpy(q).to(DEV)
    out = torch.empty_like(qd)
    lg = torch.full((4, n_q, 300), float("nan"), device=DEV)
    tq.decode_attention(cfg, params, k_cache, v_cache, seq, 300, qd, out, ws, lg)
    torch.cuda.synchronize()
    out, lg = out.cpu().numpy(), lg.cpu().numpy()
    ref_out, ref_lg = oracle.decode(spec, P, R, lens, q, want_logits=True)
    for b, n in enumerate(lens):
        rows = slice(b * n_q, (b + 1) * n_q)
        check_out(out[b], ref_out[rows], f"{pair} b={b}")
        if n:
            check_logits(lg[b], ref_lg[rows], n, f"{pair} b={b}")
            assert np.all(np.isnan(lg[b][:, n:]))
        else:
            assert np.all(out[b] == 0)


@pytest.mark.parametrize("pair", ["tree3_tree3", "tree2_tree4", "tree4_tree2"])
def test_tree_dequantize_matches_oracle(pair):
    cfg = _cfg(pair, batch=2, ctx=260)
    lens = [260, 200]
    spec, P, R, kc, vc, _ = _oracle_cache(cfg, lens, seed=70)
    k_cache, v_cache = upload_cache(kc, vc, DEV)
    params = tq.init_params(cfg, DEV)
    Tk, Tv = oracle.tree_tables(cfg.k_bits), oracle.tree_tables(cfg.v_bits)
    for b, (start, count) in enumerate([(0, 260), (61, 139)]):
        ko = torch.empty((count, 2, 128), device=DEV)
        vo = torch.empty((count, 2, 128), device=DEV)
        tq.dequantize(cfg, params, k_cache, v_cache, b, start, count, ko, vo)
        torch.cuda.synchronize()
        ko, vo = ko.cpu().numpy(), vo.cpu().numpy()
        for t in range(count):
            for h in range(2):
                rec = R.rec_index(b, start + t, h)
                rk = oracle.dequant_tree(P.DK, Tk, R.kcodes[rec], R.kn16[rec])
                rv = oracle.dequant_tree(P.DV, Tv, R.vcodes[rec], R.vn16[rec])
                sk = max(1.0, np.abs(rk).max())
                sv = max(1.0, np.abs(rv).max())
                assert np.max(np.abs(ko[t, h] - rk)) <= 2e-5 * sk, (b, t, h)
                assert np.max(np.abs(vo[t, h] - rv)) <= 2e-5 * sv, (b, t, h)
