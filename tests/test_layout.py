"""Layout pins (4-bit layout v1 and the 3-bit bit-plane layout): hand-derived worked words,
the pair-extraction masks, bijection."""

import os

import numpy as np

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "layout_v1_words.txt")
GOLDEN3 = os.path.join(os.path.dirname(__file__), "golden", "layout_3bit_words.txt")


def _golden():
    rows = []
    for line in open(GOLDEN):
        line = line.strip()
        if not line or line.startswith("#"):
            continue
        codes, word = line.split("|")
        rows.append(([int(c) for c in codes.split()], int(word, 16)))
    return rows


def test_worked_words():
    rows = _golden()
    assert len(rows) >= 8
    q = np.array([r[0] for r in rows])
    words = oracle.pack_codes(q.reshape(len(rows), 8))
    assert [int(w) for w in words[:, 0]] == [r[1] for r in rows]
    back = oracle.unpack_codes(words, 8)
    assert np.array_equal(back, q)


def test_pair_mask_yields_input_pairs():
    rng = np.random.default_rng(0)
    q = rng.integers(0, 16, size=(3, 64))
    words = oracle.pack_codes(q)
    for r in range(3):
        for j in range(8):
            w = int(words[r, j])
            for i in range(4):
                pair = (w >> (4 * i)) & 0x000F000F
                assert pair & 0xFFFF == q[r, 8 * j + 2 * i]
                assert pair >> 16 == q[r, 8 * j + 2 * i + 1]


def test_pack_unpack_bijection():
    rng = np.random.default_rng(1)
    q = rng.integers(0, 16, size=(17, 1024))
    assert np.array_equal(oracle.unpack_codes(oracle.pack_codes(q), 1024), q)
    w = rng.integers(0, 2 ** 32, size=(5, 40), dtype=np.uint64).astype(np.uint32)
    assert np.array_equal(oracle.pack_codes(oracle.unpack_codes(w)), w)


def test_layout_version():
    assert oracle.LAYOUT_VERSION == 1


def _golden3():
    rows = []
    for line in open(GOLDEN3):
        line = line.strip()
        if not line or line.startswith("#"):
            continue
        codes, words = line.split("|")
        rows.append(([int(c) for c in codes.split()], [int(w, 16) for w in words.split()]))
    return rows


def test_worked_words_3bit():
    rows = _golden3()
    assert len(rows) >= 6
    q = np.array([r[0] for r in rows])
    assert q.shape[1] == 32
    words = oracle.pack_codes3(q)
    assert [[int(w) for w in row] for row in words] == [r[1] for r in rows]
    assert np.array_equal(oracle.unpack_codes3(words, 32), q)


def test_pair_masks_yield_input_pairs_3bit():
    # the property a kernel relies on: low-plane pair | high-plane pair << 2 is the code pair
    rng = np.random.default_rng(2)
    q = rng.integers(0, 8, size=(3, 96))
    words = oracle.pack_codes3(q)
    for r in range(3):
        for b in range(3):
            lo = [int(words[r, 3 * b]), int(words[r, 3 * b + 1])]
            hi = int(words[r, 3 * b + 2])
            for jj in range(16):
                h, i = divmod(jj, 8)
                pair = ((lo[h] >> (2 * i)) & 0x00030003) | (((hi >> jj) & 0x00010001) << 2)
                assert pair & 0xFFFF == q[r, 32 * b + 2 * jj]
                assert pair >> 16 == q[r, 32 * b + 2 * jj + 1]


def test_pack_unpack_bijection_3bit():
    rng = np.random.default_rng(3)
    q = rng.integers(0, 8, size=(11, 512))
    assert np.array_equal(oracle.unpack_codes3(oracle.pack_codes3(q), 512), q)
    w = rng.integers(0, 2 ** 32, size=(4, 30), dtype=np.uint64).astype(np.uint32)
    assert np.array_equal(oracle.pack_codes3(oracle.unpack_codes3(w)), w)
