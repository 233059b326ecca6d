"""Pins of the exponent-palette oracle (lossless BF16 weight format of the
Unweight page): palette choice, index layout, row classification, lossless
round trip and the reference product."""
import collections

import numpy as np
import torch

import workloads as W
from oracle import palette_ref as P


def _bits(a):
    return W.bf16_bits(torch.from_numpy(np.asarray(a, dtype=np.float32)).to(torch.bfloat16))


def test_exponent_field():
    # 1.0 = 0x3F80 (exponent 127), -1.5 = 0xBFC0 (127), 2^-100, -0, a subnormal
    b = np.array([0x3F80, 0xBFC0, 0x0D80, 0x8000, 0x0001], dtype=np.uint16)
    assert P.exponent(b).tolist() == [127, 127, 27, 0, 0]


def test_palette_is_the_16_most_common_ties_to_smaller():
    # exponent e appears count[e] times; 20 distinct exponents with ties
    counts = {100 + i: c for i, c in enumerate([5, 9, 9, 1, 7, 7, 7, 3, 2, 2, 2, 2, 4, 6, 8, 8, 1, 1, 10, 3])}
    vals = []
    for e, c in counts.items():
        vals += [e << 7] * c                       # +1.x with mantissa 0 at exponent e
    rng = np.random.default_rng(0)
    w = np.array(vals, dtype=np.uint16)
    rng.shuffle(w)
    w = w.reshape(1, -1)
    pal = P.palette_select(w)
    ranked = sorted(counts, key=lambda e: (-counts[e], e))[:16]
    assert pal.tolist() == ranked
    # against collections.Counter on the exponent list (its order for equal counts is first-seen,
    # so compare as sets of the top counts)
    top = collections.Counter(P.exponent(w).ravel().tolist()).most_common()
    assert sorted(c for _, c in top[:16]) == sorted(counts[e] for e in pal.tolist())
    assert pal[0] == 118 and pal[1] == 101 and pal[2] == 102     # counts 10, 9, 9


def test_fewer_than_16_exponents_pad_with_unused():
    w = _bits([[1.0, 2.0, -4.0, 0.5, 1.5, 3.0, -6.0, 0.75]])
    pal = P.palette_select(w)
    assert set(pal[:4].tolist()) == {126, 127, 128, 129}
    assert (pal[4:] == P.UNUSED).all()
    enc = P.palette_encode(w)
    assert len(enc["verb_rows"]) == 0 and enc["pal_rows"].tolist() == [0]


def test_index_word_layout_hand_example():
    idx = np.array([list(range(8)) + list(range(8, 16))], dtype=np.uint8)
    words = P.pack_indices(idx)
    assert words.tolist() == [[0x73625140, 0xFBEAD9C8]]
    assert np.array_equal(P.unpack_indices(words, 16), idx)


def test_sign_mantissa_byte_and_reconstruction():
    # -1.5 = 0xBFC0: sign 1, exponent 127, mantissa 0x40 -> byte 0xC0
    w = np.array([[0xBFC0, 0x3F80, 0x8000, 0x0001, 0x4049, 0xC049, 0x3F80, 0x3F80]], dtype=np.uint16)
    enc = P.palette_encode(w)
    assert enc["sm"].tolist() == [[0xC0, 0x00, 0x80, 0x01, 0x49, 0xC9, 0x00, 0x00]]
    assert np.array_equal(P.palette_decode(enc), w)


def test_rare_exponent_makes_its_row_verbatim():
    # every row holds 16 distinct exponents (2^0 .. 2^15, four times each); a 17th, rare one
    # (2^-100, once) in row 3 cannot join the palette
    w = _bits(np.tile(2.0 ** (np.arange(64) % 16), (6, 1)).astype(np.float32))
    w[3, 10] = _bits([2.0 ** -100])[0]
    enc = P.palette_encode(w)
    assert enc["verb_rows"].tolist() == [3]
    assert enc["pal_rows"].tolist() == [0, 1, 2, 4, 5]
    assert np.array_equal(enc["verb"][0], w[3])
    assert np.array_equal(P.palette_decode(enc), w)


def test_round_trip_is_lossless_on_gaussian_weights(rng):
    w = W.bf16_bits(W.randn_bf16((64, 1024), seed=7, std=0.02))
    enc = P.palette_encode(w)
    assert 0 < len(enc["verb_rows"]) < 64            # long rows: a few hold a rare exponent
    assert np.array_equal(P.palette_decode(enc), w)
    # every stored index points at the element's own exponent
    pe = enc["palette"][P.unpack_indices(enc["ix"], 1024)]
    assert np.array_equal(pe, P.exponent(w[enc["pal_rows"]]))
    n_p, n_v = len(enc["pal_rows"]), len(enc["verb_rows"])
    assert P.encoded_bytes(enc) == (16 + enc["sm"].nbytes + enc["ix"].nbytes + enc["verb"].nbytes
                                    + 4 * (n_p + n_v))


def test_round_trip_special_values(rng):
    # +-0, subnormals, the largest finite values, all in one tensor
    specials = np.array([0x0000, 0x8000, 0x0001, 0x807F, 0x7F7F, 0xFF7F, 0x0080, 0x8080], dtype=np.uint16)
    w = rng.choice(specials, size=(8, 64)).astype(np.uint16)
    enc = P.palette_encode(w)
    assert len(enc["verb_rows"]) == 0                 # only 3 distinct exponents: 0, 1, 254
    assert np.array_equal(P.palette_decode(enc), w)


def test_gemm_ref_against_triple_loop(rng):
    x = _bits(rng.standard_normal((3, 16)).astype(np.float32))
    w = _bits(rng.standard_normal((5, 16)).astype(np.float32))
    ref, mag = P.gemm_ref(x, w)
    xf = (x.astype(np.uint32) << 16).view(np.float32)
    wf = (w.astype(np.uint32) << 16).view(np.float32)
    for i in range(3):
        for j in range(5):
            s = sum(float(xf[i, t]) * float(wf[j, t]) for t in range(16))
            a = sum(abs(float(xf[i, t]) * float(wf[j, t])) for t in range(16))
            assert abs(ref[i, j] - s) <= 1e-12 * a and abs(mag[i, j] - a) <= 1e-12 * a


def test_storage_order_hand_example():
    """One block of 16 rows, K = 128 (one chunk of T = 1): lane group q holds K [32q, 32q + 32);
    piece j of (q, r16) sits at 16 * (64 j + 16 q + r16)."""
    k = 128
    sm = (np.arange(16 * k, dtype=np.int64) % 251).astype(np.uint8).reshape(16, k)
    enc = {"k": k, "sm": sm, "ix": np.zeros((16, k // 8), np.uint32), "verb": np.zeros((0, k), np.uint16)}
    st, _, _ = P.palette_store(enc)
    for j in range(2):
        for q in range(4):
            for r in range(16):
                o = 16 * (64 * j + 16 * q + r)
                assert np.array_equal(st[o:o + 16], sm[r, 32 * q + 16 * j: 32 * q + 16 * j + 16])


def test_storage_order_is_a_permutation_with_padding(rng):
    """Every byte of every row appears once; padded rows are zero; K tails of 1-3 units."""
    for n, k in ((5, 384), (16, 640), (33, 1536)):
        sm = rng.integers(1, 256, size=(n, k)).astype(np.uint8)
        ix = rng.integers(1, 2 ** 32, size=(n, k // 8), dtype=np.uint64).astype(np.uint32)
        verb = rng.integers(1, 2 ** 16, size=(n, k)).astype(np.uint16)
        st_sm, st_ix, st_v = P.palette_store({"k": k, "sm": sm, "ix": ix, "verb": verb})
        npad = (n + 15) // 16 * 16
        assert st_sm.size == npad * k and st_ix.size == npad * k // 8 and st_v.size == npad * k
        assert np.array_equal(np.sort(st_sm[st_sm != 0]), np.sort(sm.ravel()))
        assert np.array_equal(np.sort(st_ix[st_ix != 0]), np.sort(ix.ravel()))
        assert np.array_equal(np.sort(st_v[st_v != 0]), np.sort(verb.ravel()))
        assert (st_sm == 0).sum() == (npad - n) * k
        # the first chunk of block 0: lane group 1, piece 0 of row 0 = row 0's K [32T, 32T + 16)
        t = min(4, k // 128)
        assert np.array_equal(st_sm[16 * 16:16 * 17], sm[0, 32 * t:32 * t + 16])
