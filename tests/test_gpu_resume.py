"""Checkpoint and resume of a packed cache: the caches and lengths of a
serving run copied device -> host mid-stream, restored into freshly
allocated device buffers (with parameters rebuilt from the same seed and
layer), and the run continued.  Every later output and the final cache bytes
equal those of the uninterrupted run, bit for bit."""
import numpy as np
import pytest
import torch

from parity_util import tq

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _inputs(cfg, n_steps, seed):
    g = torch.Generator().manual_seed(seed)
    k0 = torch.randn((cfg.batch, 300, cfg.n_kv_heads, 128), generator=g).to(torch.bfloat16)
    v0 = torch.randn((cfg.batch, 300, cfg.n_kv_heads, 128), generator=g).to(torch.bfloat16)
    ks = torch.randn((n_steps, cfg.batch, 1, cfg.n_kv_heads, 128), generator=g).to(torch.bfloat16)
    vs = torch.randn((n_steps, cfg.batch, 1, cfg.n_kv_heads, 128), generator=g).to(torch.bfloat16)
    qs = torch.randn((n_steps, cfg.batch, cfg.n_q_heads, 128), generator=g)
    return k0, v0, ks, vs, qs


def _step(L, fused, k, v, q):
    if fused:
        return L.step(k, v, q)
    L.append(k, v)
    return L.decode(q)


@pytest.mark.parametrize("codecs,fused", [((tq.POLAR_QJL, 4, tq.POLAR, 4), True),
                                          ((tq.POLAR_QJL, 3, tq.POLAR, 2), False),
                                          ((tq.Q8_BLOCK32, 8, tq.POLAR, 2), True),
                                          ((tq.POLAR_TREE, 3, tq.POLAR_TREE, 3), False)])
def test_checkpoint_resume_is_bit_identical(codecs, fused):
    kc, kb, vc, vb = codecs
    cfg = tq.make_config(n_q_heads=32, n_kv_heads=8, batch=3, max_ctx=400, k_codec=kc, k_bits=kb, v_codec=vc,
                         v_bits=vb, seed=42, layer=7)
    n_steps, cut = 24, 11
    k0, v0, ks, vs, qs = _inputs(cfg, n_steps, seed=kb * 10 + vb)
    dk0, dv0 = k0.to(DEV), v0.to(DEV)

    # uninterrupted run
    A = tq.KVLayer(cfg, DEV)
    A.append(dk0, dv0)
    outs_a = [_step(A, fused, ks[s].to(DEV), vs[s].to(DEV), qs[s].to(DEV)).cpu() for s in range(n_steps)]

    # interrupted run: checkpoint after `cut` steps
    B = tq.KVLayer(cfg, DEV)
    B.append(dk0, dv0)
    outs_b = [_step(B, fused, ks[s].to(DEV), vs[s].to(DEV), qs[s].to(DEV)).cpu() for s in range(cut)]
    torch.cuda.synchronize()
    ckpt = {"format_version": tq.FORMAT_VERSION, "k": B.k_cache.cpu().numpy().copy(),
            "v": B.v_cache.cpu().numpy().copy(), "lens": B.seq_lens.cpu().numpy().copy(), "max_len": B.max_len}
    del B
    torch.cuda.empty_cache()

    # resume: new buffers, parameters rebuilt from (seed, layer), cache restored
    assert ckpt["format_version"] == tq.FORMAT_VERSION
    C = tq.KVLayer(cfg, DEV, zero=False)
    C.k_cache.copy_(torch.from_numpy(ckpt["k"]))
    C.v_cache.copy_(torch.from_numpy(ckpt["v"]))
    C.seq_lens.copy_(torch.from_numpy(ckpt["lens"]))
    C.max_len = ckpt["max_len"]
    outs_b += [_step(C, fused, ks[s].to(DEV), vs[s].to(DEV), qs[s].to(DEV)).cpu() for s in range(cut, n_steps)]
    torch.cuda.synchronize()
    for s in range(n_steps):
        assert torch.equal(outs_a[s], outs_b[s]), f"step {s}"
    assert torch.equal(A.k_cache, C.k_cache) and torch.equal(A.v_cache, C.v_cache)
    assert np.array_equal(A.seq_lens.cpu().numpy(), C.seq_lens.cpu().numpy())
