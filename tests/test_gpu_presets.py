"""A mixed-codec layer stack built from the cache-type presets (keys turbo3,
values turbo2, the first and last two layers in q8_0): every layer's append
and decode against the oracle, through the C ABI."""
import numpy as np
import pytest
import torch

from compressed_decode_attention_quantize_amd import presets
from parity_util import (check_logits, check_out, compare_records, gpu_records, oracle, oracle_quantize, spec_of,
                         tq, widen_np)

pytestmark = pytest.mark.gpu
DEV = "cuda"


def test_policy_stack_matches_oracle():
    n_layers, lens = 6, [300, 300]
    base = tq.make_config(n_q_heads=32, n_kv_heads=8, batch=2, max_ctx=300, seed=42)
    policy = presets.layer_policy(n_layers, "turbo3", "turbo2", protect=2)
    g = torch.Generator().manual_seed(4242)
    for l, codecs in enumerate(policy):
        cfg = presets.config(base, codecs, l)
        print(f"[policy] layer {l}: {codecs.k_type}/{codecs.v_type}", flush=True)
        L = tq.KVLayer(cfg, DEV)
        k = torch.randn((2, 300, 8, 128), generator=g).to(torch.bfloat16)
        v = torch.randn((2, 300, 8, 128), generator=g).to(torch.bfloat16)
        q = torch.randn((2, 32, 128), generator=g).to(torch.bfloat16).float()
        for a, b in ((0, 113), (113, 300)):
            L.append(k[:, a:b].to(DEV).contiguous(), v[:, a:b].to(DEV).contiguous())
        lg = torch.full((2, 32, 300), float("nan"), device=DEV)
        out = L.decode(q.to(DEV), logits=lg).cpu().numpy()
        torch.cuda.synchronize()
        spec = spec_of(cfg)
        P = oracle.Params(spec, 42, l)
        kn, vn = widen_np(k), widen_np(v)
        R = oracle_quantize(spec, P, kn, vn, lens)
        G = gpu_records(spec, L.k_cache, L.v_cache, lens)
        compare_records(spec, P, G, R, lens, kn, f"layer {l}")
        ref_out, ref_lg = oracle.decode(spec, P, R, lens, q.numpy(), want_logits=True)
        for b in range(2):
            rows = slice(b * 32, (b + 1) * 32)
            check_out(out[b], ref_out[rows], f"layer {l} b={b}")
            differ = (G.signs != R.signs).any(axis=1) if spec.k_codec == oracle.POLAR_QJL else None
            skip = None
            if differ is not None and differ.any():
                d = differ.reshape(2, 300, 8)[b]
                skip = np.stack([d[:, h // 4] for h in range(32)])
            check_logits(lg[b].cpu().numpy(), ref_lg[rows], 300, f"layer {l} b={b}", skip=skip)
