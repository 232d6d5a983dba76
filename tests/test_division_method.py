"""The encoder divides the rANS state by a symbol frequency with one IEEE
double multiply: q = trunc(double(x) * r_f), r_f = (1 + 2^-44) / f rounded to
double.  This is exact for every f in [1, 4096] and every state the encoder
divides (x < f * 2^20, so q < 2^20):

  the product is at least x/f (the 2^-44 bias exceeds both roundings), so
  trunc never falls below floor(x/f); and it exceeds x/f by at most
  (x/f) * 2^-43 < 2^20 * 2^-43 = 2^-23, while x/f sits at least 1/f >= 2^-12
  below the next integer, so trunc never reaches floor(x/f) + 1.

numpy's float64 arithmetic is the same IEEE binary64 round-to-nearest as the
GPU's v_mul_f64, so checking the method here on the boundary states (every
multiple of f and its neighbours at the bottom, middle and top of the range,
for every f) checks the kernel's arithmetic.  No GPU needed."""
import numpy as np


def test_reciprocal_division_exact_on_boundaries():
    f = np.arange(1, 4097, dtype=np.float64)
    r = (1.0 + 2.0 ** -44) / f
    fi = f.astype(np.uint64)
    ks = np.concatenate([np.arange(0, 40), (1 << 20) - np.arange(1, 40), np.array([1 << 10, 1 << 15, 777_777])])
    for k in ks.astype(np.uint64):
        for d in (0, 1, 2):
            base = k * fi
            for x in (base + fi - np.uint64(d) - np.uint64(1), base + np.uint64(d)):
                ok = x < fi * np.uint64(1 << 20)
                x = x[ok]
                q = np.trunc(x.astype(np.float64) * r[ok]).astype(np.uint64)
                assert np.array_equal(q, x // fi[ok])


def test_reciprocal_division_exact_random_states():
    rng = np.random.default_rng(0)
    f = rng.integers(1, 4097, 2_000_000).astype(np.uint64)
    x = (rng.random(f.size) * (f.astype(np.float64) * (1 << 20))).astype(np.uint64)
    x = np.minimum(x, f * np.uint64(1 << 20) - np.uint64(1))
    r = (1.0 + 2.0 ** -44) / f.astype(np.float64)
    q = np.trunc(x.astype(np.float64) * r).astype(np.uint64)
    assert np.array_equal(q, x // f)
