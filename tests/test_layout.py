"""Layout v1 pins: hand-derived worked words, the pair-extraction mask, bijection."""

import os

import numpy as np

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "layout_v1_words.txt")


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
