"""The seeded generator: reproducible, exact ignore counts, the stated value
distributions, and round-to-nearest-even bf16 conversion."""
import math

import numpy as np
import pytest

from linear_cross_entropy_cce_amd import inputs


def test_bf16_rounding_is_nearest_even():
    f = np.array([1.0, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, 1.0 + 2 ** -8 + 2 ** -20, -2.5, 3.0e38], dtype=np.float32)
    bits = inputs.round_to_bf16_bits(f)
    # 1 + 2^-8 is halfway between 1 and 1 + 2^-7: ties go to the even mantissa (1.0).
    # 1 + 3*2^-8 is halfway between 1 + 2^-7 and 1 + 2^-6: ties to even (1 + 2^-6).
    want = np.array([1.0, 1.0, 1.0 + 2 ** -6, 1.0 + 2 ** -7, -2.5, 2.9975336e38], dtype=np.float32)
    got = inputs.bf16_bits_as_f32(bits)
    np.testing.assert_array_equal(got[:5], want[:5])
    assert abs(got[5] - 3.0e38) / 3.0e38 < 2 ** -8


def test_reproducible_and_seed_sensitive():
    a = inputs.make_workload(3, N=300, D=64, V=1000)
    b = inputs.make_workload(3, N=300, D=64, V=1000)
    c = inputs.make_workload(3, seed=99, N=300, D=64, V=1000)
    assert np.array_equal(a.H, b.H) and np.array_equal(a.E, b.E) and np.array_equal(a.labels, b.labels)
    assert not np.array_equal(a.E, c.E)


@pytest.mark.parametrize("k,frac", [(1, 0.10), (3, 0.40)])
def test_ignore_count_exact(k, frac):
    x = inputs.make_workload(k, N=1000, D=32, V=500)
    assert int(np.sum(x.labels == inputs.IGNORE_INDEX)) == round(frac * 1000)


def test_full_size_ignore_counts():
    # 26 of 256 rows (workload 1), 6554 of 16384 (workload 3): count from the recipe.
    assert round(0.10 * 256) == 26 and round(0.40 * 16384) == 6554


def test_zipf_head_mass():
    # P(id < 256) for Zipf(1.1) over 256 000 ids is H_256 / H_256000 ~= 0.628.
    rng = np.random.default_rng(0)
    y = inputs.zipf_labels(rng, 200_000, 256_000)
    r = np.arange(1, 256_001, dtype=np.float64) ** -1.1
    want = r[:256].sum() / r.sum()
    assert abs(np.mean(y < 256) - want) < 0.005
    assert y.min() >= 0 and y.max() < 256_000


def test_distributions():
    x = inputs.make_workload(1)  # full tiny workload, f32
    assert x.H.dtype == np.float32 and x.E.dtype == np.float32
    assert abs(x.E.std() - 1 / math.sqrt(128)) < 0.002
    assert abs(x.H.std() - 1.0) < 0.01
    y = inputs.make_workload(4, N=512, V=2000)  # bf16 bits, E ~ N(0, 0.02^2)
    assert y.E.dtype == np.uint16
    assert abs(inputs.bf16_bits_as_f32(y.E).std() - 0.02) < 0.0005


def test_peaked_hidden_states_point_at_label():
    x = inputs.make_workload(2, N=64, D=256, V=3000)
    H = inputs.bf16_bits_as_f32(x.H).astype(np.float64)
    E = inputs.bf16_bits_as_f32(x.E).astype(np.float64)
    z = H @ E.T
    # The label logit is the row maximum by a wide margin (about 0.06 D).
    assert np.all(np.argmax(z, axis=1) == x.labels)
    margin = z[np.arange(64), x.labels] - np.sort(z, axis=1)[:, -2]
    assert np.median(margin) > 0.04 * 256


def test_scattered_zipf_is_a_relabelled_zipf():
    # Workload 6 draws the same Zipf ranks as workload 5 and sends them through
    # a permutation of the ids: same multiset of counts, head spread out.
    a = inputs.make_workload(5, N=4000, D=16, V=20000)
    b = inputs.make_workload(6, N=4000, D=16, V=20000, seed=5)
    ca = np.sort(np.bincount(a.labels, minlength=20000))
    cb = np.sort(np.bincount(b.labels, minlength=20000))
    assert np.array_equal(ca, cb)
    assert np.mean(a.labels < 256) > 0.4 and np.mean(b.labels < 256) < 0.05
    # one id map: equal ranks give equal ids
    ids = {}
    for ra, rb in zip(a.labels, b.labels):
        assert ids.setdefault(int(ra), int(rb)) == int(rb)


def test_partially_peaked_recipe_regime():
    # workload 7: about 0.02 % of the non-label softmax entries at or above
    # 2^-12 and the label a large but not overwhelming share.  The first 32
    # rows of the full workload (same seeds), logits in float32 from the
    # exact bf16 values (a regime check, not parity).
    import numpy as np
    x = inputs.make_workload(7, N=32)
    H = inputs.bf16_bits_as_f32(x.H)
    E = inputs.bf16_bits_as_f32(x.E)
    z = (H @ E.T).astype(np.float64)
    m = z.max(axis=1, keepdims=True)
    lse = m + np.log(np.exp(z - m).sum(axis=1, keepdims=True))
    p = np.exp(z - lse)
    rows = np.arange(x.N)
    py = p[rows, x.labels].copy()
    p[rows, x.labels] = 0.0
    frac = (p >= 2.0 ** -12).sum() / (x.N * (x.V - 1))
    assert 1e-4 <= frac <= 4e-4, frac
    assert 0.05 <= np.median(1.0 - py) <= 0.5, np.median(1.0 - py)
