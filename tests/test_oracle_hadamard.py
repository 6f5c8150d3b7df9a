"""Pins for the oracle's Hadamard matrices, fast transform and rotation.

Each check ties the oracle to something other than itself: a closed form,
the defining property H H^T = d I, brute-force dense products, the
invariance identities of the pages, or a value the pages print.
"""
import json
import os

import numpy as np
import pytest

from oracle import hadamard as had

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def popcount_sign(i, j):
    return -1 if bin(i & j).count("1") % 2 else 1


@pytest.mark.parametrize("n", [0, 1, 2, 3, 5, 7])
def test_sylvester_closed_form(n):
    # Sylvester order: H[i, j] = (-1)^popcount(i & j), entry by entry in Python integers.
    h = had.sylvester(n)
    d = 1 << n
    expect = np.array([[popcount_sign(i, j) for j in range(d)] for i in range(d)])
    assert np.array_equal(h, expect)


@pytest.mark.parametrize("n", range(0, 12))
def test_sylvester_orthogonal(n):
    h = had.sylvester(n).astype(np.float64)
    d = 1 << n
    assert np.array_equal(h @ h.T, d * np.eye(d))


@pytest.mark.parametrize("m", [28, 172])
def test_known_hadamard_orthogonal(m):
    h = had.known_hadamard(m)
    assert h.shape == (m, m)
    assert set(np.unique(h)) == {-1, 1}
    assert np.array_equal(h @ h.T, m * np.eye(m, dtype=np.int64))


def test_williamson_blocks_are_symmetric_circulants():
    seqs = had.williamson_sequences()
    assert len(seqs) == 4 and all(s.shape == (43,) for s in seqs)
    for s in seqs:
        # symmetric first row <=> symmetric circulant
        assert np.array_equal(s[1:], s[1:][::-1])
    # Williamson condition: periodic autocorrelations sum to zero off the origin.
    for shift in range(1, 43):
        assert sum(int(np.dot(s, np.roll(s, shift))) for s in seqs) == 0


def test_paley_h28_from_conference_matrix():
    # The conference matrix built from the quadratic character mod 13 has C C^T = 13 I.
    q = 13
    qr = {(x * x) % q for x in range(1, q)}
    chi = lambda a: 0 if a % q == 0 else (1 if a % q in qr else -1)  # noqa: E731
    conf = np.zeros((q + 1, q + 1), dtype=np.int64)
    conf[0, 1:] = 1
    conf[1:, 0] = 1
    for i in range(q):
        for j in range(q):
            conf[1 + i, 1 + j] = chi(j - i)
    assert np.array_equal(conf @ conf.T, q * np.eye(q + 1, dtype=np.int64))
    h = had.known_hadamard(28)
    # block (i, j) of H_28 is C[i, j] [[1,1],[1,-1]] (+ [[1,-1],[-1,-1]] on the diagonal)
    for i in range(q + 1):
        for j in range(q + 1):
            blk = h[2 * i:2 * i + 2, 2 * j:2 * j + 2]
            expect = conf[i, j] * np.array([[1, 1], [1, -1]])
            if i == j:
                expect = expect + np.array([[1, -1], [-1, -1]])
            assert np.array_equal(blk, expect)


@pytest.mark.parametrize("d", [2 * 28, 8 * 28, 172, 2 * 172])
def test_kronecker_orthogonal(d):
    h = had.hadamard_dense(d).astype(np.float64)
    assert np.array_equal(h @ h.T, d * np.eye(d))


@pytest.mark.parametrize("d", [1, 2, 4, 8, 16, 32, 64, 128, 256, 28, 56, 112, 224, 172])
def test_fast_transform_equals_dense_exactly(d):
    rng = np.random.default_rng(d)
    x = rng.integers(-1000, 1000, size=(3, d)).astype(np.float64)
    dense = had.hadamard_dense(d).astype(np.float64)
    assert np.array_equal(had.hadamard_apply(x, d), x @ dense.T)


def test_hadamard_rows_match_dense():
    for d in (64, 224, 344):
        dense = had.hadamard_dense(d).astype(np.float64)
        rows = np.array([0, 1, d // 2, d - 1])
        assert np.array_equal(had.hadamard_rows(d, rows), dense[rows])


@pytest.mark.parametrize("d", [128, 4096, 8192, 11008, 28672])
def test_fast_transform_equals_dense_rows_at_config_widths(d):
    # Dense rows of H_d built on the fly from the Kronecker/popcount definition.
    rng = np.random.default_rng(1000 + d)
    x = rng.standard_normal((4, d))
    fast = had.hadamard_apply(x, d)
    block = 1024 if d <= 8192 else 512
    for r0 in range(0, d, block):
        rows = np.arange(r0, min(d, r0 + block))
        dense_rows = had.hadamard_rows(d, rows)
        np.testing.assert_allclose(fast[:, rows], x @ dense_rows.T, rtol=0, atol=1e-9 * np.sqrt(d))


@pytest.mark.parametrize("d", [64, 4 * 28, 172])
def test_rotation_applies_signs_before_transform(d):
    # R = H diag(s) / sqrt(d): the image of e_j is s_j H[:, j] / sqrt(d).
    rng = np.random.default_rng(7)
    s = np.where(rng.integers(0, 2, d) == 0, 1, -1)
    dense = had.hadamard_dense(d)
    for j in (0, 1, d - 1):
        e = np.zeros(d)
        e[j] = 1.0
        np.testing.assert_allclose(had.rotate(e, s), s[j] * dense[:, j] / np.sqrt(d), atol=1e-15)


@pytest.mark.parametrize("d", [128, 4096, 11008, 28672])
def test_rotation_is_orthogonal(d):
    rng = np.random.default_rng(11)
    s = np.where(rng.integers(0, 2, d) == 0, 1, -1)
    x = rng.standard_normal((3, d))
    y = had.rotate(x, s)
    np.testing.assert_allclose(y @ y.T, x @ x.T, rtol=1e-12, atol=1e-9)


@pytest.mark.parametrize("d", [4096, 11008, 28672])
def test_computational_invariance(d):
    # (X R^T)(W R^T)^T = X W^T: rotating the GEMM input rows and the weight rows
    # by the same R leaves the product unchanged (QuaRot paper, computational
    # invariance; QuaRot blog, "Computational invariance: rotation is free").
    rng = np.random.default_rng(12)
    s = np.where(rng.integers(0, 2, d) == 0, 1, -1)
    x = rng.standard_normal((4, d))
    x[:, rng.choice(d, 5, replace=False)] *= 50
    w = rng.standard_normal((6, d)) * 0.02
    ref = x @ w.T
    got = had.rotate(x, s) @ had.rotate(w, s).T
    rel = np.abs(got - ref).max() / np.abs(ref).max()
    assert rel <= 1e-4
    assert rel <= 1e-12  # fp64 reaches far below the 1e-4 bound


def test_factorisation():
    assert had.factor(4096) == (12, 1)
    assert had.factor(8192) == (13, 1)
    assert had.factor(128) == (7, 1)
    assert had.factor(11008) == (6, 172)
    assert had.factor(28672) == (10, 28)
    with pytest.raises(ValueError):
        had.factor(43)


def test_blog_incoherence_demo():
    g = json.load(open(os.path.join(GOLDEN, "blog_incoherence_demo.json")))
    st = g["setup"]
    v = np.random.default_rng(st["seed"]).standard_normal(st["length"])
    v[st["outlier_index"]] = st["outlier_value"]
    n = len(v)
    rotated = had.fwht(v) / np.sqrt(n)
    # the fast transform of this very vector against the dense Sylvester product
    np.testing.assert_allclose(rotated, had.sylvester(10) @ v / np.sqrt(n), atol=1e-12)
    before = np.abs(v).max() / np.linalg.norm(v)
    after = np.abs(rotated).max() / np.linalg.norm(v)
    tol = g["tolerance"]
    assert abs(before - g["printed"]["incoherence_before"]) <= tol["before_abs"]
    assert abs(after - g["printed"]["incoherence_after"]) <= tol["after_abs"]
    assert before / after >= tol["min_drop_factor"]
    assert had.incoherence(v) == pytest.approx(before)


def test_blog_fwht_cost():
    g = json.load(open(os.path.join(GOLDEN, "fwht_cost_4096.json")))
    assert had.fwht_passes(g["d"]) == g["passes"]
    assert g["d"] ** 2 == g["dense_macs"]
