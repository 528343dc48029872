"""The seeded generator: known-answer vectors of Philox4x32-10 (Random123's
published test vectors), determinism, and that any slice regenerates alone."""
import numpy as np

import synth


def test_philox_known_answers():
    kat = [
        ((0, 0, 0, 0), (0, 0), (0x6627e8d5, 0xe169c58d, 0xbc57ac4c, 0x9b00dbd8)),
        ((0xffffffff,) * 4, (0xffffffff, 0xffffffff), (0x408f276d, 0x41c83b0e, 0xa20bc7c6, 0x6d5451fd)),
        ((0x243f6a88, 0x85a308d3, 0x13198a2e, 0x03707344), (0xa4093822, 0x299f31d0),
         (0xd16cfe09, 0x94fdcceb, 0x5001e420, 0x24126ea1)),
    ]
    for ctr, key, want in kat:
        got = synth.philox4x32_10(*ctr, *key)
        assert tuple(int(v) for v in got) == want


def test_leaves_ascending_and_sliceable():
    full = synth.leaves(1, 1, 0, 3, 2, 16, 8)
    assert full.dtype == np.float32 and full.shape == (16, 8, 256)
    assert np.all(np.diff(full, axis=-1) > 0)
    part = synth.leaves(1, 1, 0, 3, 2, 16, 8, 5, 9)
    assert np.array_equal(part, full[5:9])
    q, gap = synth.leaf_quantiles()
    assert np.all(np.abs(full.astype(np.float64) - q) <= 0.25 * gap + 1e-9)


def test_codes_sliceable_and_uniform():
    full = synth.codes(1, 1, 0, 3, 1, 64, 256)
    part = synth.codes(1, 1, 0, 3, 1, 64, 256, 10, 20)
    assert np.array_equal(part, full[10:20])
    h = np.bincount(full.ravel(), minlength=256)
    assert h.min() > 0 and h.max() < 3 * h.mean()
    assert not np.array_equal(full, synth.codes(1, 1, 0, 3, 0, 64, 256))


def test_normals_moments():
    z = synth.activation(5, 1, 0, 0, 1 << 16)
    assert abs(z.mean()) < 0.02 and abs(z.std() - 1) < 0.02
    assert np.array_equal(z, synth.activation(5, 1, 0, 0, 1 << 16))


def test_uniform_k_range():
    k = synth.uniform_k(3, 0, 0, 0, 4000)
    assert k.min() == 1 and k.max() == 8
    assert np.all(np.bincount(k)[1:] > 350)


def test_zipf_trace_draws_by_rank():
    rank = synth.expert_popularity_rank(3, 1, 7, 512)
    assert sorted(rank.tolist()) == list(range(1, 513))
    n = 4000
    top = np.array([int(np.argmax(synth.zipf_router_logits(3, 1, 7, t % 4096, 512, 1.0,
                                                            step=t // 4096)))
                    for t in range(n)])
    # Gumbel-max: the top expert is rank r with probability r^-1 / H_512
    h = np.sum(1.0 / np.arange(1, 513))
    for r in (1, 2, 5):
        p = 1.0 / r / h
        got = np.mean(rank[top] == r)
        assert abs(got - p) <= 4.0 * np.sqrt(p * (1 - p) / n)
    again = synth.zipf_router_logits(3, 1, 7, 11, 512, 1.0)
    assert np.array_equal(again, synth.zipf_router_logits(3, 1, 7, 11, 512, 1.0))
