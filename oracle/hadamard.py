"""Hadamard matrices, the fast Walsh-Hadamard transform and the randomized
Hadamard rotation, in float64 / exact integers.  TEST INFRASTRUCTURE ONLY
(see ``oracle/__init__.py``).

Definitions followed:

* Sylvester recursion H_1 = [1], H_2k = [[H_k, H_k], [H_k, -H_k]] in natural
  (not sequency) order, unnormalised so that H H^T = d I.  QuaRot blog,
  "Hadamard matrices: orthogonal and fast" (the recursion and the in-place
  butterfly transform); QuaRot paper, background on Hadamard matrices (a
  Walsh-Hadamard matrix has size 2^n and H x costs O(d log d)).
* Widths d != 2^n: factor d = 2^n m with m the order of a known Hadamard
  matrix and use H_d = H_{2^n} (x) H_m, cost O(d (m + n)).  QuaRot paper,
  background on Hadamard matrices.  Index convention i = a m + b (numpy
  ``kron``): H_m acts on the contiguous index b, H_{2^n} on a with stride m.
* Randomized Hadamard H~ = H diag(s), s in {+1, -1}^d; it is orthogonal after
  the 1/sqrt(d) normalisation.  QuaRot paper, background on Hadamard matrices
  (randomized Hadamard after Tseng et al.).  A row x maps to
  y = H (s * x) / sqrt(d): signs first, then the transform.
* H_28 by Paley's second construction over GF(13), H_172 by Williamson's
  construction from the sequences in ``data/williamson43.txt`` (found by
  ``williamson_search.c``).  The pages name Sloane's list but print no
  matrix; any H with H H^T = m I is valid.
"""
from __future__ import annotations

import functools
from pathlib import Path

import numpy as np

DATA = Path(__file__).resolve().parent / "data"


# ---------------------------------------------------------------------------
# Matrices
# ---------------------------------------------------------------------------

def sylvester(n: int) -> np.ndarray:
    """Sylvester-Hadamard matrix of order 2**n (int64 entries +-1)."""
    h = np.ones((1, 1), dtype=np.int64)
    for _ in range(n):
        h = np.block([[h, h], [h, -h]])
    return h


def _legendre(a: int, p: int) -> int:
    a %= p
    if a == 0:
        return 0
    return 1 if pow(a, (p - 1) // 2, p) == 1 else -1


def paley2(q: int) -> np.ndarray:
    """Paley's second construction: Hadamard matrix of order 2(q+1), q prime, q = 1 mod 4.

    Jacobsthal matrix Q[i, j] = chi(j - i) (chi = quadratic character mod q),
    symmetric conference matrix C = [[0, 1^T], [1, Q]] with C C^T = q I, then
    H = C (x) [[1, 1], [1, -1]] + I (x) [[1, -1], [-1, -1]].
    """
    assert q % 4 == 1
    jac = np.array([[_legendre(j - i, q) for j in range(q)] for i in range(q)], dtype=np.int64)
    conf = np.zeros((q + 1, q + 1), dtype=np.int64)
    conf[0, 1:] = 1
    conf[1:, 0] = 1
    conf[1:, 1:] = jac
    a = np.array([[1, 1], [1, -1]], dtype=np.int64)
    b = np.array([[1, -1], [-1, -1]], dtype=np.int64)
    return np.kron(conf, a) + np.kron(np.eye(q + 1, dtype=np.int64), b)


def _circulant(first_row: np.ndarray) -> np.ndarray:
    n = first_row.shape[0]
    idx = (np.arange(n)[None, :] - np.arange(n)[:, None]) % n
    return first_row[idx]


def williamson(seqs: list[np.ndarray]) -> np.ndarray:
    """Williamson array of four symmetric circulants A, B, C, D -> order 4n."""
    a, b, c, d = (_circulant(s) for s in seqs)
    return np.block([
        [a, b, c, d],
        [-b, a, -d, c],
        [-c, d, a, -b],
        [-d, -c, b, a],
    ])


def williamson_sequences() -> list[np.ndarray]:
    rows = [ln.strip() for ln in (DATA / "williamson43.txt").read_text().splitlines()
            if ln.strip() and not ln.startswith("#")]
    return [np.array([1 if ch == "+" else -1 for ch in r], dtype=np.int64) for r in rows]


@functools.lru_cache(maxsize=None)
def known_hadamard(m: int) -> np.ndarray:
    """The H_m used for the non-power-of-two factor (read-only int64 array)."""
    if m == 1:
        h = np.ones((1, 1), dtype=np.int64)
    elif m == 28:
        h = paley2(13)
    elif m == 172:
        h = williamson(williamson_sequences())
    else:
        raise ValueError(f"no known Hadamard matrix of order {m} in this oracle")
    h.setflags(write=False)
    return h


KNOWN_M = (1, 28, 172)


def factor(d: int) -> tuple[int, int]:
    """d = 2**n * m with m in KNOWN_M; m = 1 when d is a power of two."""
    for m in KNOWN_M:
        if d % m == 0:
            r = d // m
            if r >= 1 and r & (r - 1) == 0:
                return r.bit_length() - 1, m
    raise ValueError(f"width {d} is not 2^n * m for a known m")


def hadamard_dense(d: int) -> np.ndarray:
    """Dense H_d = H_{2^n} (x) H_m (int64).  Only for small d (brute force)."""
    n, m = factor(d)
    return np.kron(sylvester(n), known_hadamard(m))


def hadamard_rows(d: int, rows: np.ndarray) -> np.ndarray:
    """Selected rows of H_d as float64, built directly from the Kronecker
    definition H_d[a m + b, a' m + b'] = H_2n[a, a'] H_m[b, b'] with the
    Sylvester entries (-1)^popcount(a & a')."""
    n, m = factor(d)
    hm = known_hadamard(m).astype(np.float64)
    rows = np.asarray(rows, dtype=np.int64)
    a, b = rows // m, rows % m
    a2 = np.arange(1 << n, dtype=np.int64)
    anded = a[:, None] & a2[None, :]
    par = np.zeros_like(anded)
    while np.any(anded):
        par ^= anded & 1
        anded >>= 1
    h2 = 1.0 - 2.0 * par  # [len(rows), 2^n]
    return (h2[:, :, None] * hm[b][:, None, :]).reshape(len(rows), d)


# ---------------------------------------------------------------------------
# Fast transform
# ---------------------------------------------------------------------------

def fwht(x: np.ndarray) -> np.ndarray:
    """Unnormalised fast Walsh-Hadamard transform along the last axis (float64).

    The butterfly passes of the QuaRot blog ("Hadamard matrices: orthogonal and
    fast"): for h = 1, 2, 4, ... each pair (x[j], x[j + h]) inside a block of
    2h becomes (x[j] + x[j + h], x[j] - x[j + h]).  Natural (Sylvester) order.
    The blog's 1/sqrt(n) is applied by the caller.
    """
    x = np.array(x, dtype=np.float64, copy=True)
    d = x.shape[-1]
    assert d & (d - 1) == 0, "fwht needs a power-of-two length"
    lead = x.shape[:-1]
    h = 1
    while h < d:
        v = x.reshape(*lead, d // (2 * h), 2, h)
        a = v[..., 0, :].copy()
        b = v[..., 1, :]
        v[..., 0, :] = a + b
        v[..., 1, :] = a - b
        h *= 2
    return x


def fwht_passes(d: int) -> int:
    """Number of butterfly passes the fast transform makes for length d."""
    passes, h = 0, 1
    while h < d:
        passes += 1
        h *= 2
    return passes


def hadamard_apply(x: np.ndarray, d: int | None = None) -> np.ndarray:
    """z = H_d x along the last axis, float64, via H_{2^n} (x) H_m.

    The row is viewed as [2^n, m] (i = a m + b); H_m multiplies every
    contiguous m-chunk (dense matrix product) and the fast transform runs over
    a.  The two factors commute.
    """
    x = np.asarray(x, dtype=np.float64)
    d = x.shape[-1] if d is None else d
    assert x.shape[-1] == d
    n, m = factor(d)
    lead = x.shape[:-1]
    v = x.reshape(*lead, 1 << n, m)
    if m > 1:
        v = v @ known_hadamard(m).T.astype(np.float64)
    v = np.moveaxis(v, -1, -2)           # [..., m, 2^n]
    v = fwht(v)
    v = np.moveaxis(v, -1, -2)           # [..., 2^n, m]
    return np.ascontiguousarray(v).reshape(*lead, d)


def rotate(x: np.ndarray, signs: np.ndarray | None) -> np.ndarray:
    """y = H_d diag(s) x / sqrt(d) row-wise, float64 (signs None means all +1)."""
    x = np.asarray(x, dtype=np.float64)
    d = x.shape[-1]
    if signs is not None:
        x = x * np.asarray(signs, dtype=np.float64)
    return hadamard_apply(x, d) / np.sqrt(d)


def rotate_unnormalised(x: np.ndarray, signs: np.ndarray | None) -> np.ndarray:
    """z = H_d diag(s) x (no 1/sqrt(d)), float64."""
    x = np.asarray(x, dtype=np.float64)
    if signs is not None:
        x = x * np.asarray(signs, dtype=np.float64)
    return hadamard_apply(x, x.shape[-1])


def incoherence(v: np.ndarray) -> float:
    """max |v| / ||v||_2: the QuaRot blog's incoherence ratio (its outlier demo)."""
    v = np.asarray(v, dtype=np.float64)
    return float(np.abs(v).max() / np.linalg.norm(v))
