"""Pins of the oracle's projection (stage 3) and gate (stage 4).

Projection (metrale "deepseek_v41_ref/engram.rs", linear_bf16: f32
accumulation, bf16 output):
* wkv = identity gives kv = x exactly; a one-hot x gives a column of wkv;
* against numpy's float64 matmul rounded by torch's bf16 cast: within one bf16
  step (the f32 sum and the exact sum round to neighbouring bf16 values at
  most).

Gate (metrale gate_and_add; f32 highway per atlas "engram_v41.rs" stage 4):
* value = 0 leaves h bit for bit;
* key = 0 gives dot = 0 and gate = sigmoid(1e-3);
* key = lambda * h with q = k = 1 has the closed form
  s = lambda*S / (sqrt(S/d + eps) * sqrt(lambda^2*S/d + eps) * sqrt(d)),
  S = sum h^2, evaluated in float64;
* a float64 re-evaluation of the formula bounds the oracle's f32 error;
* 0 < gate < 1 always.
"""
import numpy as np
import torch


def bf16(x):
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


def widen(b):
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


# ------------------------------------------------------------- projection
def test_linear_identity(orc):
    rng = np.random.default_rng(0)
    x = bf16(rng.standard_normal((5, 96)))
    eye = bf16(np.eye(96))
    np.testing.assert_array_equal(orc.linear_bf16(x, eye), x)


def test_linear_one_hot(orc):
    rng = np.random.default_rng(1)
    w = bf16(rng.standard_normal((40, 64)) * 0.02)
    x = np.zeros((64, 64), dtype=np.float32)
    x[np.arange(64), np.arange(64)] = 1.0
    y = orc.linear_bf16(bf16(x), w)
    np.testing.assert_array_equal(y, w.T)


def test_linear_vs_float64(orc):
    rng = np.random.default_rng(2)
    for rows, K, N in ((3, 1024, 257), (17, 512, 64), (1, 6144, 33)):
        x = bf16(rng.standard_normal((rows, K)))
        w = bf16(rng.standard_normal((N, K)) * 0.02)
        y = widen(orc.linear_bf16(x, w)).astype(np.float64)
        exact = widen(x).astype(np.float64) @ widen(w).astype(np.float64).T
        # one bf16 step at the exact value's magnitude
        ulp = 2.0 ** (np.floor(np.log2(np.abs(exact) + 1e-300)) - 7)
        assert (np.abs(y - exact) <= ulp * 1.0000001).all()
        # and most outputs are the correctly rounded exact sum
        assert (bf16(exact) == bf16(y)).mean() > 0.95


def test_linear_equals_sequential_f32_sum(orc):
    """The pages accumulate in f32 in index order.  numpy's cumsum in float32
    is that sequential sum (each prefix rounded to f32); a bf16 x bf16 product
    is exact in f32, so the oracle must match it bit for bit."""
    rng = np.random.default_rng(10)
    x = bf16(rng.standard_normal((3, 768)))
    w = bf16(rng.standard_normal((50, 768)) * 0.02)
    xf, wf = widen(x), widen(w)
    want = np.empty((3, 50), dtype=np.float32)
    for r in range(3):
        for o in range(50):
            want[r, o] = np.cumsum(xf[r] * wf[o], dtype=np.float32)[-1]
    np.testing.assert_array_equal(orc.linear_bf16(x, w), bf16(want))
    # where the order shows through the bf16 result: in f32, 2^24 + 1 is a tie
    # that rounds back to 2^24 (even), while -2^24 + 1 is exact.  In index
    # order 2^24 + 1 - 2^24 gives 0 and -2^24 + 1 + 2^24 gives 1; the reversed
    # order swaps the two
    ones = bf16(np.ones((1, 3)))
    wc = bf16(np.array([[2.0 ** 24, 1.0, -(2.0 ** 24)], [-(2.0 ** 24), 1.0, 2.0 ** 24],
                        [1.0, 2.0 ** 24, -(2.0 ** 24)]]))
    np.testing.assert_array_equal(widen(orc.linear_bf16(ones, wc)), [[0.0, 1.0, 0.0]])


def test_linear_threads_invariant(orc):
    rng = np.random.default_rng(3)
    x = bf16(rng.standard_normal((4, 256)))
    w = bf16(rng.standard_normal((100, 256)))
    np.testing.assert_array_equal(orc.linear_bf16(x, w, nthreads=1),
                                  orc.linear_bf16(x, w, nthreads=7))


# ------------------------------------------------------------------- gate
def gate_f64(h, kv, q, k, eps):
    """The gate formula in float64 (independent re-evaluation)."""
    T, hc, dim = h.shape
    h = h.astype(np.float64)
    kvf = widen(kv).astype(np.float64).reshape(T, hc + 1, dim)
    qk = widen(q).astype(np.float64) * widen(k).astype(np.float64)
    out = h.copy()
    gates = np.zeros((T, hc))
    for t in range(T):
        for c in range(hc):
            key, val, hh = kvf[t, c], kvf[t, hc], h[t, c]
            s = (hh * qk[c] * key).sum() / np.sqrt((hh * hh).sum() / dim + eps) \
                / np.sqrt((key * key).sum() / dim + eps) / np.sqrt(dim)
            g = np.copysign(np.sqrt(max(abs(s), 1e-6)), s)
            gate = 1.0 / (1.0 + np.exp(-g))
            gates[t, c] = gate
            out[t, c] = hh + gate * val
    return out, gates


def make_gate_inputs(rng, T, hc, dim):
    h = rng.standard_normal((T, hc, dim)).astype(np.float32)
    kv = bf16(rng.standard_normal((T, dim * (hc + 1))) * 0.5)
    q = bf16(1 + 0.05 * rng.standard_normal((hc, dim)))
    k = bf16(1 + 0.05 * rng.standard_normal((hc, dim)))
    return h, kv, q, k


def test_gate_zero_value(orc):
    rng = np.random.default_rng(4)
    h, kv, q, k = make_gate_inputs(rng, 3, 4, 256)
    kv = kv.reshape(3, 5, 256)
    kv[:, 4] = 0
    out = orc.gate_and_add(h, kv.reshape(3, -1), q, k, 1e-6)
    np.testing.assert_array_equal(out.view(np.uint32), h.view(np.uint32))


def test_gate_zero_key(orc):
    rng = np.random.default_rng(5)
    h, kv, q, k = make_gate_inputs(rng, 2, 3, 128)
    kv = kv.reshape(2, 4, 128)
    kv[:, :3] = 0
    out = orc.gate_and_add(h, kv.reshape(2, -1), q, k, 1e-6)
    gate = (out.astype(np.float64) - h) / widen(kv[:, 3])[:, None, :]
    mask = np.abs(widen(kv[:, 3])) > 0.1
    want = 1.0 / (1.0 + np.exp(-1e-3))
    g = gate[np.broadcast_to(mask[:, None, :], gate.shape)]
    assert np.abs(g - want).max() < 1e-5


def test_gate_closed_form(orc):
    rng = np.random.default_rng(6)
    dim, hc = 256, 2
    one = bf16(np.ones((hc, dim)))
    for lam in (2.0, -0.5, 0.25):
        hb = widen(bf16(rng.standard_normal((1, hc, dim)))).copy()     # bf16-valued h
        kv = np.zeros((1, hc + 1, dim), dtype=np.float32)
        kv[0, :hc] = lam * hb[0]                                         # exact in bf16
        kv[0, hc] = 1.0
        eps = 1e-6
        out = orc.gate_and_add(hb, bf16(kv.reshape(1, -1)), one, one, eps)
        for c in range(hc):
            S = float((hb[0, c].astype(np.float64) ** 2).sum())
            s = lam * S / (np.sqrt(S / dim + eps) * np.sqrt(lam * lam * S / dim + eps)
                           * np.sqrt(dim))
            g = np.copysign(np.sqrt(abs(s)), s)
            gate = 1 / (1 + np.exp(-g))
            assert abs(np.sign(lam) * dim ** 0.25 - g) < 1e-3
            got = (out[0, c].astype(np.float64) - hb[0, c]).mean()
            assert abs(got - gate) < 2e-6


def test_gate_vs_float64_and_bounds(orc):
    rng = np.random.default_rng(7)
    for T, hc, dim in ((4, 4, 256), (2, 1, 4096), (3, 3, 1024)):
        h, kv, q, k = make_gate_inputs(rng, T, hc, dim)
        out = orc.gate_and_add(h, kv, q, k, 1e-6)
        want, gates = gate_f64(h, kv, q, k, 1e-6)
        assert ((gates > 0) & (gates < 1)).all()
        assert np.abs(out - want).max() < 1e-5


def test_gate_bf16_flag(orc):
    rng = np.random.default_rng(8)
    h, kv, q, k = make_gate_inputs(rng, 2, 4, 256)
    a = orc.gate_and_add(h, kv, q, k, 1e-6)
    b = orc.gate_and_add(h, kv, q, k, 1e-6, round_bf16=True)
    np.testing.assert_array_equal(widen(bf16(a)), b)


def test_gate_threads_invariant(orc):
    rng = np.random.default_rng(9)
    h, kv, q, k = make_gate_inputs(rng, 9, 4, 256)
    a = orc.gate_and_add(h, kv, q, k, 1e-6, nthreads=1)
    b = orc.gate_and_add(h, kv, q, k, 1e-6, nthreads=4)
    np.testing.assert_array_equal(a.view(np.uint32), b.view(np.uint32))
