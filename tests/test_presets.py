"""Cache-type presets and per-layer codec policies (host side; the size
closed forms are checked against the library's own size query)."""
import pytest

from compressed_decode_attention_quantize_amd import presets, tq


def test_type_mapping():
    assert presets.layer_codecs("turbo4", "turbo4") == presets.LayerCodecs("turbo4", "turbo4", tq.POLAR_QJL, 3,
                                                                           tq.POLAR, 4)
    assert presets.layer_codecs("turbo3", "turbo2") == presets.LayerCodecs("turbo3", "turbo2", tq.POLAR_QJL, 2,
                                                                           tq.POLAR, 2)
    c = presets.layer_codecs("q8_0", "q8_0")
    assert (c.k_codec, c.k_bits, c.v_codec, c.v_bits) == (tq.Q8_BLOCK32, 8, tq.POLAR, 4)
    with pytest.raises(ValueError):
        presets.layer_codecs("turbo2", "turbo2")   # a value type only
    with pytest.raises(ValueError):
        presets.layer_codecs("turbo3", "q4_0")


def test_boundary_protection():
    pol = presets.layer_policy(32, "turbo3", "turbo2", protect=2)
    kinds = [(c.k_type, c.v_type) for c in pol]
    assert kinds[:2] == kinds[-2:] == [("q8_0", "q8_0")] * 2
    assert kinds[2:30] == [("turbo3", "turbo2")] * 28
    assert all(c.k_type == "turbo4" for c in presets.layer_policy(5, "turbo4", "turbo4", protect=0))
    # protection wider than the stack covers every layer
    assert all(c.k_type == "q8_0" for c in presets.layer_policy(3, "turbo3", "turbo3", protect=2))


@pytest.mark.parametrize("kt", list(presets.KEY_TYPES))
@pytest.mark.parametrize("vt", list(presets.VALUE_TYPES))
def test_record_bits_match_library_sizes(kt, vt):
    c = presets.layer_codecs(kt, vt)
    base = tq.make_config(n_q_heads=32, n_kv_heads=8, batch=2, max_ctx=1000)
    cfg = presets.config(base, c, layer=7)
    assert (cfg.k_codec, cfg.k_bits, cfg.v_codec, cfg.v_bits, cfg.layer) == (c.k_codec, c.k_bits, c.v_codec,
                                                                           c.v_bits, 7)
    kb, vb = tq.cache_bytes(cfg)
    records = 2 * 8 * ((1000 + 127) // 128) * 128
    kbits, vbits = presets.record_bits(c)
    assert kb * 8 == records * kbits and vb * 8 == records * vbits


def test_compression_closed_forms():
    # fp16 K + V (2 x 16 bits per coordinate) over the packed record bits
    assert presets.compression_vs_fp16(presets.layer_codecs("turbo4", "turbo4")) == pytest.approx(32 / 8.375)
    assert presets.compression_vs_fp16(presets.layer_codecs("turbo3", "turbo3")) == pytest.approx(32 / 6.375)
    assert presets.compression_vs_fp16(presets.layer_codecs("turbo3", "turbo2")) == pytest.approx(32 / 5.375)
    assert presets.compression_vs_fp16(presets.layer_codecs("q8_0", "turbo3")) == pytest.approx(32 / (8.5 + 3.125))
