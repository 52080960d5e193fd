"""Pins for the oracle's recursive polar codec (POLAR_TREE): the radius +
angle reading of the wis-web.com reader article's Cartesian-to-polar
paragraph.

What fixes each function from outside the oracle:
  * angle laws: Wallis integrals (closed form masses), the level-2 one-bit
    codebook in closed form, and the Lloyd-Max optimality conditions checked
    against Monte Carlo angles of Gaussian vectors (pins the law the
    codebooks are built for, the exponent included);
  * the tree transform: angles recomputed here from block norms of the
    vector (numpy), and the exact inverse;
  * quantisation: codes against #{boundaries below the angle} of those
    recomputed angles, with y = H D x from scipy's Sylvester Hadamard matrix;
  * dequantisation: reconstruction from the centroid angles done here
    top-down, and |x_hat| = the stored radius;
  * layout: one bit at a hand-computed word and position for K and V.
"""
import math

import numpy as np
import pytest
from scipy.linalg import hadamard
from scipy.special import beta

D128 = 128
LEVELS = 7


def _np_tree_angles(y):
    """Heap-slot angles of y: slot 2^(L-l) + k is node k of level l, whose
    angle compares the norms of the two halves of coordinates
    [k 2^l, (k + 1) 2^l); level 1 keeps the signed pair."""
    d = y.size
    ang = np.zeros(d)
    for l in range(1, LEVELS + 1):
        w = 1 << l
        blocks = y.reshape(d // w, w)
        if l == 1:
            th = np.arctan2(blocks[:, 1], blocks[:, 0])
            th = np.where(th < 0, th + 2 * np.pi, th)
        else:
            left = np.linalg.norm(blocks[:, : w // 2], axis=1)
            right = np.linalg.norm(blocks[:, w // 2:], axis=1)
            th = np.arctan2(right, left)
        first = 1 << (LEVELS - l)
        ang[first: first + d // w] = th
    return ang


def _np_unit_from_angles(ang):
    """Coordinate i of the unit vector: product over levels of cos or sin of
    its ancestor's angle, cos for a left child and sin for a right one."""
    d = ang.size
    u = np.ones(d)
    for i in range(d):
        for l in range(1, LEVELS + 1):
            node = i >> l
            slot = (1 << (LEVELS - l)) + node
            right = (i >> (l - 1)) & 1
            u[i] *= math.sin(ang[slot]) if right else math.cos(ang[slot])
    return u


@pytest.mark.parametrize("level", [2, 3, 4, 5, 6, 7])
def test_angle_law_mass_is_wallis(orc, level):
    # int_0^{pi/2} sin(2t)^n dt = B((n+1)/2, 1/2) / 2, n = 2^(l-1) - 1
    n = (1 << (level - 1)) - 1
    assert abs(orc.angle_mass(level, 0.0, math.pi / 2) - beta((n + 1) / 2, 0.5) / 2) < 1e-12
    # symmetric about pi/4
    assert abs(orc.angle_mass(level, 0.0, math.pi / 4) - orc.angle_mass(level, math.pi / 4, math.pi / 2)) < 1e-12


def test_level2_one_bit_codebook_closed_form(orc):
    # density sin(2t) on [0, pi/2]: cells [0, pi/4], [pi/4, pi/2]; centroid of
    # the lower cell = int t sin 2t / int sin 2t = (1/4) / (1/2) = 1/2
    c, b, mse, _ = orc.angle_codebook(2, 1)
    assert abs(c[0] - 0.5) < 1e-12 and abs(c[1] - (math.pi / 2 - 0.5)) < 1e-12
    assert abs(b[0] - math.pi / 4) < 1e-15
    # E[(t - 1/2)^2 | t < pi/4] = (int t^2 sin 2t - 1/4 ... ) in closed form:
    # int_0^{pi/4} t^2 sin 2t dt = pi/8 - 1/4
    m2 = (math.pi / 8 - 0.25) / 0.5
    assert abs(mse - (m2 - 0.25)) < 1e-10


@pytest.mark.parametrize("bits", [1, 2, 3, 4, 5])
def test_level1_is_uniform_quantiser(orc, bits):
    c, b, mse, it = orc.angle_codebook(1, bits)
    n = 1 << bits
    w = 2 * math.pi / n
    assert it == 0
    assert np.allclose(c, (np.arange(n) + 0.5) * w, atol=1e-15, rtol=0)
    assert np.allclose(b, (np.arange(1, n)) * w, atol=1e-15, rtol=0)
    assert abs(mse - w * w / 12) < 1e-15


@pytest.mark.slow
def test_codebooks_meet_lloyd_conditions_on_gaussian_angles(orc):
    """Angles of N(0, I_128) vectors: every centroid is the mean of the angles
    falling in its cell, every boundary the midpoint of its neighbours."""
    rng = np.random.default_rng(7)
    y = rng.standard_normal((6000, D128))
    angs = np.stack([_np_tree_angles(v) for v in y])
    for l in range(2, LEVELS + 1):
        first = 1 << (LEVELS - l)
        th = angs[:, first: 2 * first].ravel()
        for bits in (1, 2, 3):
            c, b, _, _ = orc.angle_codebook(l, bits)
            assert np.allclose(b, 0.5 * (c[1:] + c[:-1]), atol=1e-12)
            cell = np.searchsorted(b, th, side="left")
            for j in range(c.size):
                sel = th[cell == j]
                se = sel.std() / math.sqrt(sel.size)
                assert abs(sel.mean() - c[j]) < 5 * se + 1e-4, (l, bits, j)
    # level 1 is uniform on the circle: its mean is pi, and its quadrants are equally likely
    th1 = angs[:, 64:128].ravel()
    assert abs(th1.mean() - math.pi) < 5 * (2 * math.pi / math.sqrt(12)) / math.sqrt(th1.size)
    q = np.bincount((th1 // (math.pi / 2)).astype(int), minlength=4) / th1.size
    assert np.all(np.abs(q - 0.25) < 0.01)


def test_tree_angles_and_inverse(orc):
    rng = np.random.default_rng(3)
    for _ in range(20):
        y = rng.standard_normal(D128) * rng.uniform(0.1, 10)
        ang, r = orc.tree_angles(y)
        ref = _np_tree_angles(y)
        assert np.allclose(ang[1:], ref[1:], atol=1e-12, rtol=0)
        assert abs(r - np.linalg.norm(y)) < 1e-12 * np.linalg.norm(y)
        assert np.allclose(orc.tree_from_angles(ang, r), y, atol=1e-12, rtol=0)
        # and the unit vector of the angles, built here coordinate by coordinate
        assert np.allclose(_np_unit_from_angles(ang) * r, y, atol=1e-12, rtol=0)


def test_tree_angles_zero_and_signed_zero(orc):
    ang, r = orc.tree_angles(np.zeros(D128))
    assert r == 0.0 and np.all(ang == 0.0)
    y = np.zeros(D128)
    y[0] = -0.0
    y[1] = 0.0
    ang, _ = orc.tree_angles(y)
    assert ang[64] == 0.0   # read as (+0, +0), not atan2(+0, -0) = pi


@pytest.mark.parametrize("b", [2, 3, 4])
def test_quantize_tree_codes_are_the_cells_of_the_angles(orc, b):
    rng = np.random.default_rng(10 + b)
    T = orc.tree_tables(b)
    tabs = orc.tree_table_arrays(T)
    D = orc.signs(42, 1, 0, D128)
    H = hadamard(D128).astype(np.float64)
    n_close = 0
    for k in range(60):
        x = (rng.standard_normal(D128) * (0.01 if k % 3 == 0 else 3.0)).astype(np.float32)
        r = orc.quantize_tree(x, D, T)
        y = H @ (D.astype(np.float64) * x.astype(np.float64))
        ang = _np_tree_angles(y)
        # the oracle rotates in fp32: every coordinate is off by at most 7
        # roundings of partial sums bounded by |x|_1; an angle of a node whose
        # block has norm r moves by at most that times sqrt(block size) / r
        dy = 7 * 2.0 ** -24 * float(np.sum(np.abs(x)))
        for s in range(1, D128):
            l = LEVELS - int(math.floor(math.log2(s)))
            bits, c, bnd = tabs[l]
            assert bits == (b + 1 if l == 1 else b - 1)
            node = s - (1 << (LEVELS - l))
            r_node = np.linalg.norm(y[node << l: (node + 1) << l])
            dth = 2 * dy * math.sqrt(1 << l) / max(r_node, 1e-30)
            want = int(np.sum(bnd < ang[s]))
            dist = np.min(np.abs(bnd - ang[s]))
            if l == 1:
                dist = min(dist, ang[s], 2 * math.pi - ang[s])
            if dist < dth:
                n_close += 1
                continue
            assert r["codes"][s] == want, (k, s, l)
            assert abs(r["amargin"][s] - dist) <= dth
        assert r["codes"][0] == 0
        n = math.sqrt(float(np.sum(x.astype(np.float64) ** 2)))
        assert r["n16"] == int(orc.f32_to_f16(np.float32(n))[0])
    assert n_close < 20


@pytest.mark.parametrize("b", [2, 3, 4])
def test_dequant_tree_reconstruction(orc, b):
    rng = np.random.default_rng(20 + b)
    T = orc.tree_tables(b)
    tabs = orc.tree_table_arrays(T)
    D = orc.signs(7, 3, 1, D128).astype(np.float64)
    H = hadamard(D128).astype(np.float64)
    for _ in range(10):
        codes = np.zeros(D128, np.uint8)
        ang = np.zeros(D128)
        for s in range(1, D128):
            l = LEVELS - int(math.floor(math.log2(s)))
            bits, c, _ = tabs[l]
            codes[s] = rng.integers(0, 1 << bits)
            ang[s] = c[codes[s]]
        n16 = int(orc.f32_to_f16(np.float32(rng.uniform(0.5, 20)))[0])
        n = float(orc.f16_to_f32(np.array([n16], np.uint16))[0])
        xh = orc.dequant_tree(D, T, codes, n16)
        ref = D * (H @ (_np_unit_from_angles(ang) * math.sqrt(D128) * n)) / D128
        assert np.allclose(xh, ref, atol=1e-12 * n, rtol=0)
        assert abs(np.linalg.norm(xh) - n) < 1e-12 * n


def test_tree_distortion_against_per_coordinate_codebook(orc):
    """The comparison at equal bits per coordinate: relative MSE of the
    recursive polar codec and of the per-coordinate codebook on Gaussian
    vectors.  The per-coordinate one matches its codebook's own MSE (an
    outside check of the estimate); the recursive one lands within 12 % of
    it at b = 2, 3, 4 (measured 0.124 / 0.116, 0.0351 / 0.0341, 0.0095 /
    0.0093)."""
    rng = np.random.default_rng(5)
    D = orc.signs(42, 0, 0, D128)
    for b in (2, 3, 4):
        T = orc.tree_tables(b)
        _, c16, bnd, mse_cb, _ = orc.codebook(D128, b)
        et, ep = [], []
        for _ in range(400):
            x = rng.standard_normal(D128).astype(np.float32)
            n2 = float(np.sum(x.astype(np.float64) ** 2))
            r = orc.quantize_tree(x, D, T)
            et.append(np.sum((x - orc.dequant_tree(D, T, r["codes"], r["n16"])) ** 2) / n2)
            p = orc.quantize_polar(x, D, c16, bnd, b)
            ep.append(np.sum((x - orc.dequant_polar(D, c16, p["codes"], p["n16"])) ** 2) / n2)
        mt, mp = float(np.mean(et)), float(np.mean(ep))
        assert abs(mp - mse_cb) < 0.05 * mse_cb
        assert mp <= mt < 1.12 * mp, (b, mt, mp)


@pytest.mark.parametrize("tensor", ["k", "v"])
def test_tree_layout_bit_positions(orc, tensor):
    """One record of the b = 3 tree codec at position t = 37 of a block: the
    bit of a level-2 slot (plane 1 of the b - 1 = 2 shared planes) and of a
    level-1 slot (its top bit, in the second level-1 plane) at the words the
    layout defines."""
    s = orc.make_spec(d=128, n_q=2, n_kv=1, batch=1, max_ctx=128, k_codec=orc.POLAR_TREE, k_bits=3,
                      v_codec=orc.POLAR_TREE, v_bits=3)
    R = orc.Records(s)
    t = 37
    codes = R.kcodes if tensor == "k" else R.vcodes
    codes[t, 40] = 0b10          # level-2 slot 40: bit 1 set
    codes[t, 100] = 0b1000       # level-1 slot 100: bit 3 = b - 1 + 1 -> second level-1 plane
    (R.kn16 if tensor == "k" else R.vn16)[t] = 0x3C00
    lens = np.array([t + 1], np.int32)
    kc, vc = orc.pack_cache(s, R, lens)
    img = (kc if tensor == "k" else vc).view(np.uint32)
    pi = 32 * (t // 32) + 8 * (t % 4) + (t % 32) // 4
    if tensor == "k":
        # plane p < 2: word [p][j][pi], j = slot / 32; level-1 planes after 2 * 4 * 128 words
        w1 = 1 * 4 * 128 + (40 // 32) * 128 + pi
        w2 = 2 * 4 * 128 + 1 * 2 * 128 + ((100 - 64) // 32) * 128 + pi
        assert img[w1] == 1 << (40 % 32) and img[w2] == 1 << (100 % 32)
        n16_off = 2 * 4 * 128 * 4 + 2 * 2 * 128 * 4
    else:
        # plane p < 2: word [p][t / 32][slot], bit t % 32; level-1 planes: [x][t / 32][slot - 64]
        w1 = 1 * 4 * 128 + (t // 32) * 128 + 40
        w2 = 2 * 4 * 128 + 1 * 4 * 64 + (t // 32) * 64 + (100 - 64)
        assert img[w1] == 1 << (t % 32) and img[w2] == 1 << (t % 32)
        n16_off = 2 * 4 * 128 * 4 + 2 * 4 * 64 * 4
    assert np.count_nonzero(img[: n16_off // 4]) == 2
    n16 = (kc if tensor == "k" else vc)[n16_off + 2 * pi: n16_off + 2 * pi + 2].view(np.uint16)[0]
    assert n16 == 0x3C00
    back = orc.unpack_cache(s, kc, vc, lens)
    assert np.array_equal((back.kcodes if tensor == "k" else back.vcodes)[t], codes[t])


def test_tree_record_bytes_equal_per_coordinate_codec(orc):
    for b in (2, 3, 4):
        s = orc.make_spec(k_codec=orc.POLAR_TREE, k_bits=b, v_codec=orc.POLAR_TREE, v_bits=b)
        z = orc.spec_sizes(s)
        assert z["k_record"] == z["v_record"] == 16 * b + 2


def test_tree_decode_is_attention_over_dequantised_records(orc):
    """The oracle's decode with tree codecs equals softmax attention computed
    here from its dequantised keys and values."""
    s = orc.make_spec(d=128, n_q=4, n_kv=1, batch=1, max_ctx=200, k_codec=orc.POLAR_TREE, k_bits=3,
                      v_codec=orc.POLAR_TREE, v_bits=2)
    P = orc.Params(s, 42, 0)
    rng = np.random.default_rng(1)
    n = 150
    k = rng.standard_normal((n, 1, 128)).astype(np.float32)
    v = rng.standard_normal((n, 1, 128)).astype(np.float32)
    q = rng.standard_normal((1, 4, 128)).astype(np.float32)
    R = orc.Records(s)
    orc.quantize_into(s, P, R, k, v, 0, 0)
    out, lg = orc.decode(s, P, R, [n], q, want_logits=True)
    Tk, Tv = orc.tree_tables(3), orc.tree_tables(2)
    K = np.stack([orc.dequant_tree(P.DK, Tk, R.kcodes[t], R.kn16[t]) for t in range(n)])
    V = np.stack([orc.dequant_tree(P.DV, Tv, R.vcodes[t], R.vn16[t]) for t in range(n)])
    for h in range(4):
        l = K @ q[0, h].astype(np.float64) / math.sqrt(128)
        p = np.exp(l - l.max())
        assert np.allclose(lg[h, :n], l, atol=1e-12, rtol=0)
        assert np.allclose(out[h], (p / p.sum()) @ V, atol=1e-12, rtol=0)
