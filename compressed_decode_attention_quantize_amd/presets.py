"""Named KV-cache types and per-layer codec policies.

The wis-web.com reader page (the llama.cpp fork article) sets the key and
value cache types separately (its -ctk / -ctv options), names three TurboQuant
modes, turbo4, turbo3 and turbo2 (the last meant for values only), keeps keys
in q8_0 in its asymmetric configuration, and protects the first two and the
last two layers of a model in q8_0 while the other layers use a compressed
type.  This module maps those names onto the codecs of this library; it only
builds configurations (host side, no kernels of its own).

Reading of the names (the page gives compression ratios, not formats):
  * turboN stores N bits per coordinate of the rotated direction: for keys
    N - 1 codebook bits plus the 1-bit QJL sign sketch (m = d), for values N
    codebook bits.  turbo2 therefore exists for values only (a 1-bit
    codebook is not a key codec here), as the page advises.
  * q8_0 is the per-32 block 8-bit key codec.  This library has no q8 value
    codec; a q8_0 value type is served by the 4-bit value codebook, the
    closest-to-lossless value type it has.
  * f32 is the quantisation bypass (RAW_F32).
"""
from __future__ import annotations

from dataclasses import dataclass

from . import tq

# type name -> (codec, bits)
KEY_TYPES = {
    "turbo4": (tq.POLAR_QJL, 3),
    "turbo3": (tq.POLAR_QJL, 2),
    "q8_0": (tq.Q8_BLOCK32, 8),
    "f32": (tq.RAW_F32, 32),
}
VALUE_TYPES = {
    "turbo4": (tq.POLAR, 4),
    "turbo3": (tq.POLAR, 3),
    "turbo2": (tq.POLAR, 2),
    "q8_0": (tq.POLAR, 4),
    "f32": (tq.RAW_F32, 32),
}


@dataclass(frozen=True)
class LayerCodecs:
    k_type: str
    v_type: str
    k_codec: int
    k_bits: int
    v_codec: int
    v_bits: int


def layer_codecs(k_type: str, v_type: str) -> LayerCodecs:
    if k_type not in KEY_TYPES:
        raise ValueError(f"unknown key cache type {k_type!r} (turbo2 is a value type only)")
    if v_type not in VALUE_TYPES:
        raise ValueError(f"unknown value cache type {v_type!r}")
    kc, kb = KEY_TYPES[k_type]
    vc, vb = VALUE_TYPES[v_type]
    return LayerCodecs(k_type, v_type, kc, kb, vc, vb)


def layer_policy(n_layers: int, k_type: str = "turbo3", v_type: str = "turbo3", protect: int = 0,
                 protect_type: str = "q8_0"):
    """Per-layer codecs of an n_layers stack: the first `protect` and the last
    `protect` layers use `protect_type` for keys and values, the others
    (k_type, v_type)."""
    if n_layers <= 0 or protect < 0:
        raise ValueError("n_layers must be positive and protect non-negative")
    inner = layer_codecs(k_type, v_type)
    edge = layer_codecs(protect_type, protect_type)
    return [edge if (l < protect or l >= n_layers - protect) else inner for l in range(n_layers)]


def config(base: tq.Config, codecs: LayerCodecs, layer: int) -> tq.Config:
    """A copy of `base` with the layer's codecs and layer index (the seeded
    rotation and sketch are per layer)."""
    return tq.make_config(base.head_dim, base.n_q_heads, base.n_kv_heads, base.batch, base.max_ctx,
                          codecs.k_codec, codecs.k_bits, base.qjl_m or 128, codecs.v_codec, codecs.v_bits,
                          base.decode_chunk, base.seed, layer, base.sparse_v)


def record_bits(codecs: LayerCodecs, d: int = 128, m: int = 128):
    """Bits per (position, KV head) record of keys and of values, in closed
    form: b·d + m + 32 (codes, signs, two fp16 norms) for keys with QJL,
    b·d + 16 without, 8·d + 16·d/32 for q8 keys, 32·d for f32."""
    def one(codec, bits, is_key):
        if codec == tq.RAW_F32:
            return 32 * d
        if codec == tq.Q8_BLOCK32:
            return 8 * d + 16 * (d // 32)
        if codec == tq.POLAR_QJL:
            return bits * d + m + 32
        return bits * d + 16
    return one(codecs.k_codec, codecs.k_bits, True), one(codecs.v_codec, codecs.v_bits, False)


def compression_vs_fp16(codecs: LayerCodecs, d: int = 128, m: int = 128) -> float:
    """fp16 K + V bytes over this layer's packed K + V bytes."""
    kb, vb = record_bits(codecs, d, m)
    return (2 * 16 * d) / (kb + vb)
