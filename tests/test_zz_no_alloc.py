"""tq_decode_attention_noalloc -- the decode on the library's own per-GPU
scratch array, for callers that cannot allocate -- against
tq_decode_attention with a caller workspace on the same inputs: outputs and
logits bit-identical, on consecutive calls (the second with a smaller input)
of codecs served by the matrix-core kernel (polar and q8 keys) and by the
vector-ALU kernel (raw keys and values)."""
import pytest
import torch

from parity_util import tq

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _layer(cfg, lens, seed):
    L = tq.KVLayer(cfg, DEV)
    g = torch.Generator(device=DEV).manual_seed(seed)
    n = max(lens)
    k = torch.randn((cfg.batch, n, cfg.n_kv_heads, 128), generator=g, device=DEV).to(torch.bfloat16)
    v = torch.randn((cfg.batch, n, cfg.n_kv_heads, 128), generator=g, device=DEV).to(torch.bfloat16)
    L.append(k, v)
    L.seq_lens.copy_(torch.tensor(lens, dtype=torch.int32, device=DEV))
    q = torch.randn((cfg.batch, cfg.n_q_heads, 128), generator=g, device=DEV)
    return L, q


def _both(cfg, L, q, n_max):
    lg_a = torch.full((cfg.batch, cfg.n_q_heads, cfg.max_ctx), float("nan"), device=DEV)
    lg_b = lg_a.clone()
    out_a = torch.empty_like(q)
    out_b = torch.empty_like(q)
    tq.decode_attention(cfg, L.params, L.k_cache, L.v_cache, L.seq_lens, n_max, q, out_a,
                        torch.zeros(tq.decode_workspace_bytes(cfg, n_max), dtype=torch.uint8, device=DEV), lg_a)
    tq.decode_attention_noalloc(cfg, L.params, L.k_cache, L.v_cache, L.seq_lens, n_max, q, out_b, lg_b)
    torch.cuda.synchronize()
    assert torch.equal(out_a, out_b)
    assert torch.equal(torch.nan_to_num(lg_a, nan=7.0), torch.nan_to_num(lg_b, nan=7.0))


CASES = [
    # (k_codec, k_bits, v_codec, v_bits, n_q, n_kv, first call lens, second call lens)
    (tq.POLAR_QJL, 3, tq.POLAR, 2, 32, 8, [5000, 3000, 4100], [900, 2]),
    (tq.POLAR_QJL, 4, tq.POLAR, 4, 32, 8, [8192, 8000], [1500]),
    (tq.Q8_BLOCK32, 8, tq.POLAR, 2, 96, 8, [4000, 2500], [300]),
    (tq.RAW_F32, 32, tq.RAW_F32, 32, 16, 4, [2000, 1200], [129]),
]


@pytest.mark.parametrize("case", CASES)
def test_noalloc_equals_workspace_decode(case):
    kc, kb, vc, vb, n_q, n_kv, lens1, lens2 = case
    print(f"[noalloc] {case}", flush=True)
    cfg1 = tq.make_config(n_q_heads=n_q, n_kv_heads=n_kv, batch=len(lens1), max_ctx=max(lens1), k_codec=kc,
                          k_bits=kb, v_codec=vc, v_bits=vb, seed=42, layer=1)
    L1, q1 = _layer(cfg1, lens1, seed=kb + vb)
    _both(cfg1, L1, q1, max(lens1))
    # a second call, smaller (fewer sequences, shorter), on the same scratch
    cfg2 = tq.make_config(n_q_heads=n_q, n_kv_heads=n_kv, batch=len(lens2), max_ctx=max(lens2), k_codec=kc,
                          k_bits=kb, v_codec=vc, v_bits=vb, seed=42, layer=2)
    L2, q2 = _layer(cfg2, lens2, seed=kb + vb + 1)
    _both(cfg2, L2, q2, max(lens2))
    # and the first again: the scratch keeps no state between calls
    _both(cfg1, L1, q1, max(lens1))


def test_noalloc_rejects_what_does_not_fit():
    cfg = tq.make_config(n_q_heads=64, n_kv_heads=8, batch=512, max_ctx=256, seed=42, layer=0)
    t = torch.zeros(1024, dtype=torch.uint8, device=DEV)
    q = torch.zeros((512, 64, 128), device=DEV)
    with pytest.raises(tq.TqError) as e:
        tq.decode_attention_noalloc(cfg, t, t, t, torch.zeros(512, dtype=torch.int32, device=DEV), 256, q,
                                    torch.empty_like(q))
    assert e.value.status == tq.EWORKSPACE
