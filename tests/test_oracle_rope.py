"""Pins of the rotary / query-scaling / cache-append oracle (oracle/rope.py)
to the concept page's "Positions" section and its example's assertions, and
to properties of rotations that any correct implementation has."""
import math

import numpy as np
import pytest

import oracle
from oracle import rope


def wavelengths(freq):
    return 2 * math.pi / np.asarray(freq)


def test_page_wavelength_assertions():
    """The page's example asserts pair 3 turns in under 16 positions and
    pair 16 in over 2^20."""
    w = wavelengths(rope.yarn_frequencies())
    assert w[3] < 16 and w[16] > 2 ** 20


def test_yarn_kept_divided_and_blended_pairs():
    """Pairs completing at least 32 turns in 512 positions keep their
    frequency; pairs completing less than one turn are divided by 2,048; in
    between the ratio moves linearly in the pair index."""
    base = rope.base_frequencies()
    f = rope.yarn_frequencies()
    turns = 512 * base / (2 * math.pi)
    kept = turns >= 32
    divided = turns < 1
    assert list(np.nonzero(kept)[0]) == [0, 1, 2, 3]
    assert list(np.nonzero(divided)[0]) == list(range(16, 32))
    np.testing.assert_array_equal(f[kept], base[kept])
    np.testing.assert_allclose(f[divided], base[divided] / 2048, rtol=1e-15)
    keep = (f / base - 1 / 2048) / (1 - 1 / 2048)    # blend weight of the original frequency
    mid = np.arange(3, 17)
    np.testing.assert_allclose(np.diff(keep[mid]), -1 / 13, rtol=1e-12)
    assert np.all(np.diff(f) < 0)                     # frequencies still fall with the pair index


def test_lerope_multiplier():
    """LeRoPE multiplies frequency i by e^{alpha_i}: the page's e^0.9336 at
    frequency 16 divides its wavelength by that factor, and the summary
    page's 1.8x rise makes a wavelength 44% shorter."""
    alpha = np.zeros(32)
    alpha[16] = 0.9336
    w0, w1 = wavelengths(rope.rope_frequencies()), wavelengths(rope.rope_frequencies(alpha))
    np.testing.assert_allclose(w1[16], w0[16] / math.exp(0.9336), rtol=1e-14)
    np.testing.assert_array_equal(np.delete(w1, 16), np.delete(w0, 16))
    alpha[16] = math.log(1.8)
    assert round(1 - wavelengths(rope.rope_frequencies(alpha))[16] / w0[16], 2) == 0.44


def test_rotation_properties():
    rng = np.random.default_rng(3)
    f = rope.rope_frequencies(rng.standard_normal(32) * 0.3)
    x, y = rng.standard_normal(64), rng.standard_normal(64)
    np.testing.assert_array_equal(rope.rotate(x, 0, f), x)                 # position 0: identity
    r = rope.rotate(x, 1234, f)
    np.testing.assert_allclose(np.hypot(r[0::2], r[1::2]), np.hypot(x[0::2], x[1::2]), rtol=1e-13)
    np.testing.assert_allclose(rope.rotate(rope.rotate(x, 300, f), 77, f), rope.rotate(x, 377, f), atol=1e-12)
    # relative position: <R(p)x, R(q)y> = <R(p-q)x, y>
    for p, q in ((1000, 10), (70000, 69000), (5, 900)):
        np.testing.assert_allclose(rope.rotate(x, p, f) @ rope.rotate(y, q, f),
                                   rope.rotate(x, p - q, f) @ y if p >= q else x @ rope.rotate(y, q - p, f),
                                   atol=1e-10)
    # a single pair, against the textbook 2-D rotation
    e = np.zeros(64)
    e[10] = 1.0
    a = 9 * f[5]
    np.testing.assert_allclose(rope.rotate(e, 9, f)[10:12], [math.cos(a), math.sin(a)], atol=1e-15)


def test_query_scaling_and_append_row():
    rng = np.random.default_rng(4)
    f = rope.rope_frequencies()
    q = rng.standard_normal((64, 576))
    s, b = rng.standard_normal(64), rng.standard_normal(64)
    t = 4095
    out = rope.prepare_query(q, t, f, s, b)
    m = s * math.log(4096) + b
    np.testing.assert_allclose(out[:, :512], q[:, :512] * m[:, None], rtol=1e-14)
    for h in (0, 33):
        np.testing.assert_allclose(out[h, 512:], rope.rotate(q[h, 512:] * m[h], t, f), rtol=1e-13, atol=1e-14)
    # s = 0, b = 1: no scaling; rotary-free queries are only scaled
    np.testing.assert_allclose(rope.prepare_query(q, t, f, np.zeros(64), np.ones(64)), rope.prepare_query(q, t, f))
    q512 = q[:, :512]
    np.testing.assert_allclose(rope.prepare_query(q512, t, f, s, b), q512 * m[:, None], rtol=1e-14)
    lat, kr = rng.standard_normal(512), rng.standard_normal(64)
    row = rope.append_row(lat, kr, t, f)
    np.testing.assert_array_equal(row[:512], lat)
    np.testing.assert_allclose(row[512:], rope.rotate(kr, t, f))
    np.testing.assert_array_equal(rope.append_row(lat, None, t, f), lat)


@pytest.mark.parametrize("n", [2, 7, 4096, 70001])
def test_query_scaling_bounds_the_competitors(n):
    """The concept page's "Query scaling" section: a key that beats n - 1
    competitors by a logit gap Delta gets weight 1/(1 + (n - 1) e^-Delta);
    with the logits multiplied by c ln n the competitors' total becomes
    (n - 1) n^(-c Delta).  Composing the oracle's query preparation at the
    last position t = n - 1 (s_h = c_h, b_h = 0) with its attention over all
    n visible positions must give the leader exactly that weight, for every
    head's own c_h: this ties query_scale to the log of the number of
    visible positions, t + 1, and to the factor multiplying the whole logit.

    Construction: 512-wide rows without rotary part (a rotary-free layer) and
    one with a zero rotary part; the leader's latent is e_0, the others' have
    a zero first value (their other values are free), and every head's query
    is e_0 * Delta / tau, so the unscaled logits are Delta and 0.  The
    leader's weight is then the first value of each head's output."""
    rng = np.random.default_rng(60 + n)
    tau = 1.0 / math.sqrt(192.0)
    t = n - 1
    c = np.linspace(0.25, 2.0, 64)                 # per-head learned slope s_h
    delta = 1.3
    lead = int(rng.integers(0, n))
    for width in (512, 576):
        kv = rng.standard_normal((n, width)).astype(np.float32)
        kv[:, 0] = 0.0
        kv[lead] = 0.0
        kv[lead, 0] = 1.0
        if width == 576:
            kv[:, 512:] = 0.0                      # the rotary key plays no part
        q = np.zeros((64, width))
        q[:, 0] = delta / tau
        qs = rope.prepare_query(q, t, rope.rope_frequencies(), c, np.zeros(64))
        q32 = qs.astype(np.float32)
        o, lse = oracle.mla_attend(q32, kv, np.arange(n, dtype=np.int32), tau)
        # given the float32 query the attention passes on, the leader's logit
        # is tau * q32[h][0] exactly and its weight follows
        gap = tau * q32[:, 0].astype(np.float64)
        # (to the rounding of the oracle's n-term sum in double)
        np.testing.assert_allclose(o[:, 0], 1.0 / (1.0 + (n - 1) * np.exp(-gap)), rtol=1e-12 + 2e-16 * n, atol=0)
        # the page's identity, up to the one float32 rounding of the scaled
        # query (a relative 6e-8 of a logit below 40)
        expect = 1.0 / (1.0 + (n - 1) * float(n) ** (-c * delta))
        np.testing.assert_allclose(o[:, 0], expect, rtol=5e-6, atol=0)


def test_query_scaling_leader_weight_exact_in_double():
    """The same identity with the composition carried out in float64 end to
    end (the oracle's attention widens float32 inputs, so the query is
    applied to the logits here by hand with the oracle's query_scale): the
    leader's weight equals 1/(1 + (n - 1) n^(-c Delta)) to 1e-12."""
    for n in (3, 100, 1 << 20):
        for c, delta in ((0.5, 2.0), (1.0, 1.0), (1.7, 0.4)):
            m = float(rope.query_scale(n - 1, np.array([c]), np.array([0.0]))[0])
            logits = np.zeros(n)
            logits[0] = m * delta                  # the leader; n - 1 competitors at 0
            p = np.exp(logits - logits.max())
            p /= p.sum()
            assert abs(p[0] - 1.0 / (1.0 + (n - 1) * float(n) ** (-c * delta))) <= 1e-12
