"""Pins of the prologue oracle (RMSNorm + 3-D RoPE, readings R27-R29): a hand-worked
token, closed forms and invariants a mistake in the norm, the pair layout, the axis
split, the frequencies or the sign of the rotation would break."""
import math

import numpy as np

from oracle.prologue import qk_prologue, rmsnorm, rope_angles, rope_split, rotate


def test_split():
    assert rope_split(128) == (22, 21, 21)
    assert rope_split(64) == (12, 10, 10)
    assert rope_split(6) == (1, 1, 1)


def test_hand_worked_token():
    # d = 6: one pair per axis, each turning by its position (i = 0 -> frequency 1).
    # x = (1,0,1,0,1,0): mean square 1/2, so with eps = 0 the norm scales by sqrt(2).
    x = np.array([1.0, 0.0, 1.0, 0.0, 1.0, 0.0]).reshape(1, 1, 1, 6)
    # a 3 x 4 latent frame (12 tokens) at clip frame 1; token 7 is row 1, column 3
    out = qk_prologue(np.tile(x, (1, 1, 12, 1)), np.ones(6), tpf=12, lat_w=4, frame0=1, eps=0.0)
    tok = 7
    r2 = math.sqrt(2.0)
    want = r2 * np.array([math.cos(1), math.sin(1), math.cos(1), math.sin(1), math.cos(3), math.sin(3)])
    assert np.allclose(out[0, 0, tok], want, rtol=0, atol=1e-14)
    # a second pair per axis turns at theta^(-1/2) = 0.01 (d = 12: two pairs per axis)
    ang = rope_angles(np.array([5]), np.array([2]), np.array([7]), 12)
    assert np.allclose(ang[0], [5, 0.05, 2, 0.02, 7, 0.07], rtol=0, atol=1e-15)


def test_rmsnorm_closed_form():
    rng = np.random.default_rng(1)
    x = rng.standard_normal((3, 5, 64)) * 3
    eps = 1e-6
    y = rmsnorm(x, np.ones(64), eps)
    ms = (x * x).mean(-1)
    assert np.allclose((y * y).mean(-1), ms / (ms + eps), rtol=0, atol=1e-12)
    g = rng.standard_normal(64)
    assert np.allclose(rmsnorm(x, g, eps), y * g, rtol=0, atol=1e-12)
    assert np.allclose(rmsnorm(7 * x, np.ones(64), 0.0), rmsnorm(x, np.ones(64), 0.0), rtol=0, atol=1e-12)


def test_rope_invariants():
    rng = np.random.default_rng(2)
    d = 128
    a, b = rng.standard_normal(d), rng.standard_normal(d)
    # identity at the origin, norm kept everywhere
    z = rope_angles(np.array([0]), np.array([0]), np.array([0]), d)
    assert np.allclose(rotate(a[None], z)[0], a, rtol=0, atol=0)
    pos = [(3, 10, 40), (0, 29, 51), (20, 0, 1)]
    for t, h, w in pos:
        ang = rope_angles(np.array([t]), np.array([h]), np.array([w]), d)
        assert abs(np.linalg.norm(rotate(a[None], ang)[0]) - np.linalg.norm(a)) < 1e-12
    # scores depend only on the position difference, along every axis
    def score(p, q):
        ap = rope_angles(*[np.array([v]) for v in p], d)
        aq = rope_angles(*[np.array([v]) for v in q], d)
        return float(rotate(a[None], ap)[0] @ rotate(b[None], aq)[0])
    base = score((5, 7, 9), (2, 3, 4))
    for shift in ((4, 0, 0), (0, 6, 0), (0, 0, 11), (1, 2, 3)):
        s = score(tuple(u + v for u, v in zip((5, 7, 9), shift)), tuple(u + v for u, v in zip((2, 3, 4), shift)))
        assert abs(s - base) < 1e-10
    # the rotation sense: a pair (1, 0) at angle phi goes to (cos phi, sin phi)
    e = np.zeros(d)
    e[0] = 1.0
    ang = rope_angles(np.array([2]), np.array([0]), np.array([0]), d)
    r = rotate(e[None], ang)[0]
    assert np.allclose(r[:2], [math.cos(2), math.sin(2)], rtol=0, atol=1e-15)


def test_positions_follow_frames_rows_columns():
    # token t of the chunk: frame frame0 + t // tpf, row (t % tpf) // lat_w, column t % lat_w
    d, tpf, lat_w = 12, 6, 3
    x = np.zeros((1, 1, 2 * tpf, d))
    x[..., 0] = 1.0                                      # only the first temporal pair is set
    x[..., 2 * 2] = 1.0                                  # first row pair (pair index n_t = 2)
    out = qk_prologue(x, np.ones(d), tpf=tpf, lat_w=lat_w, frame0=4, eps=0.0)
    r2 = math.sqrt(6.0)                                  # mean square 2/12
    for t in range(2 * tpf):
        f, p = 4 + t // tpf, t % tpf
        assert np.allclose(out[0, 0, t, 0:2], r2 * np.array([math.cos(f), math.sin(f)]), atol=1e-13)
        hr = p // lat_w
        assert np.allclose(out[0, 0, t, 4:6], r2 * np.array([math.cos(hr), math.sin(hr)]), atol=1e-13)
