"""The seeded input generator: determinism, random access, distributions."""
import numpy as np

import synth


def test_splitmix64_reference_values():
    # SplitMix64 with state 0: the first outputs of Vigna's splitmix64.c
    z = np.array([1, 2, 3], dtype=np.uint64) * synth.GAMMA
    with np.errstate(over="ignore"):
        out = synth._mix64(z)
    assert [int(v) for v in out] == [0xE220A8397B1DCDAF, 0x6E789E6AA1B965F4, 0x06C45D188009454F]


def test_streams_are_deterministic_and_distinct():
    a = synth.draws("a", 0, 0, 100)
    assert np.array_equal(a, synth.draws("a", 0, 0, 100))
    assert not np.array_equal(a, synth.draws("a", 1, 0, 100))
    assert not np.array_equal(a, synth.draws("b", 0, 0, 100))


def test_random_access_matches_full_generation():
    m = synth.Matrix("ra", 37, 96, seed=3)
    w, s = m.words(), m.scales()
    rows = [0, 5, 36, 5]
    assert np.array_equal(m.word_rows(rows), w[rows])
    assert np.array_equal(m.scale_rows(rows), s[rows])
    big = synth.draws("c", 0, 0, 5_000_000)
    assert np.array_equal(big[4_194_300:4_194_310], synth.draws("c", 0, 4_194_300, 10))


def test_distributions():
    c = synth.codes("d", 0, 1 << 16)
    assert c.min() == 0 and c.max() == 15
    assert abs(np.bincount(c, minlength=16) / len(c) - 1 / 16).max() < 0.01
    z = synth.normal("n", 0, 0, 200_000)
    assert abs(z.mean()) < 0.01 and abs(z.std() - 1) < 0.01
    s = synth.half_bits_to_f64(synth.scales_halfnormal("s", 0, 0, 100_000))
    assert s.min() >= 1e-3 * (1 - 2 ** -11) and abs(s.mean() - (0.01 * np.sqrt(2 / np.pi) + 1e-3)) < 2e-4
    _, sc, x = synth.small_config(0)
    sv = synth.half_bits_to_f64(sc)
    assert sc.shape == (256, 16) and x.shape == (512,)
    assert sv.min() >= 0.005 * (1 - 2 ** -11) and sv.max() <= 0.02 * (1 + 2 ** -11)


def test_torch_words_match_numpy():
    import torch
    for count in (1, 2, 7, 1000, 33_333):
        a = synth.words("tw", 5, count)
        b = synth.words_torch("tw", 5, count, device="cpu").numpy().view(np.uint32)
        assert np.array_equal(a, b), count
    m = synth.Matrix("tw/m", 9, 96, seed=2)
    assert np.array_equal(m.words(), m.words_torch("cpu").numpy().view(np.uint32))
