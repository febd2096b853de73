"""Pins of the attention oracle, O = softmax(scale Q K^T) V (CPU only).

Nothing here re-types the oracle's loop:
  * brute force in exact rationals and 60-digit decimals: scores as exact
    rationals of the decoded inputs, weights exp(s_j - m) from Python's decimal
    module, the quotient rounded once to fp32 / fp16 / bf16 by an exact
    nearest-value search -- compared bit for bit;
  * closed forms: equal keys (or scale 0) give the mean row of V; one key far
    ahead of the rest selects its row of V exactly; V = identity gives the
    softmax weights, non-negative and summing to 1;
  * invariances: a shift of every score of a row (an extra constant column in Q
    and K) and a permutation of the keys with their values leave O unchanged;
  * selected rows == the full computation, batch strides and padded leading
    dimensions, thread-count invariance, rejected arguments.
"""
from decimal import Decimal, localcontext
from fractions import Fraction

import numpy as np
import pytest

import oracle
import workloads
from tests import exact


def draw(rng, shape, t, lo=-1.0, hi=1.0):
    return workloads.to_bits(rng.uniform(lo, hi, shape), t)


def vals(bits, t):
    return exact.f16_values(bits) if t == "f16" else (exact.bf16_values(bits) if t == "bf16" else
                                                       np.asarray(bits, np.float64))


def brute(batch, sq, sk, d, dv, Q, ldq, sqs, K, ldk, sks, V, ldv, svs, t, out_t, scale):
    """Exact-rational scores, 60-digit decimal weights, one exact rounding per output."""
    out = np.zeros((batch, sq, dv), dtype=np.uint16 if out_t != "f32" else np.float32)
    sc = Fraction(float(np.float32(scale)))
    with localcontext() as ctx:
        ctx.prec = 60
        for b in range(batch):
            for i in range(sq):
                s = []
                for j in range(sk):
                    dot = sum(exact.exact_value(Q[b * sqs + i * ldq + k], t) *
                              exact.exact_value(K[b * sks + j * ldk + k], t) for k in range(d))
                    s.append(sc * dot)
                m = max(s)
                w = [(Decimal((x - m).numerator) / Decimal((x - m).denominator)).exp() for x in s]
                tot = sum(w)
                for c in range(dv):
                    num = sum(w[j] * Decimal(float(exact.exact_value(V[b * svs + j * ldv + c], t)))
                              for j in range(sk))
                    q = Fraction(num / tot)
                    out[b, i, c] = exact.round32(q) if out_t == "f32" else exact.round16(q, out_t)
    return out


@pytest.mark.parametrize("t,out_t", [("f16", "f32"), ("bf16", "f32"), ("f16", "f16"), ("bf16", "bf16")])
def test_brute_force_exact(t, out_t):
    rng = np.random.default_rng([5, ord(t[0]), ord(out_t[-1])])
    batch, sq, sk, d, dv = 2, 3, 5, 4, 3
    ldq, ldk, ldv = d + 1, d + 2, dv + 3  # padded leading dimensions
    sqs, sks, svs = sq * ldq + 2, sk * ldk + 1, sk * ldv + 4
    Q = draw(rng, batch * sqs, t, -2, 2)
    K = draw(rng, batch * sks, t, -2, 2)
    V = draw(rng, batch * svs, t)
    scale = 0.6
    ldo, so = dv + 2, sq * (dv + 2) + 3  # padded output
    got = oracle.attention(batch, sq, sk, d, dv, Q, ldq, sqs, K, ldk, sks, V, ldv, svs, in_type=t, out_type=out_t,
                           scale=scale, ldo=ldo, stride_o=so)
    want = brute(batch, sq, sk, d, dv, Q, ldq, sqs, K, ldk, sks, V, ldv, svs, t, out_t, scale)
    got = np.stack([got[b * so: b * so + sq * ldo].reshape(sq, ldo)[:, :dv] for b in range(batch)])
    if out_t == "f32":
        assert np.array_equal(got.view(np.uint32), want.view(np.uint32)), (got, want)
    else:
        assert np.array_equal(got, want), (got, want)


def test_equal_keys_give_the_mean_of_v():
    rng = np.random.default_rng(1)
    sq, sk, d, dv = 4, 37, 16, 8
    Q = draw(rng, sq * d, "f16")
    krow = draw(rng, d, "f16")
    K = np.tile(krow, sk)
    V = draw(rng, sk * dv, "f16")
    got = oracle.attention(1, sq, sk, d, dv, Q, d, 0, K, d, 0, V, dv, 0, in_type="f16", out_type="f32", scale=0.3)
    mean = [sum(Fraction(float(x)) for x in vals(V, "f16").reshape(sk, dv)[:, c]) / sk for c in range(dv)]
    want = np.array([exact.round32(m) for m in mean], dtype=np.float32)
    assert np.array_equal(got.reshape(sq, dv).view(np.uint32), np.tile(want, (sq, 1)).view(np.uint32))


def test_scale_zero_gives_the_mean_of_v():
    rng = np.random.default_rng(2)
    sq, sk, d, dv = 3, 10, 8, 5
    Q, K, V = draw(rng, sq * d, "bf16"), draw(rng, sk * d, "bf16"), draw(rng, sk * dv, "bf16")
    got = oracle.attention(1, sq, sk, d, dv, Q, d, 0, K, d, 0, V, dv, 0, in_type="bf16", out_type="f32", scale=0.0)
    mean = vals(V, "bf16").reshape(sk, dv).mean(axis=0)
    assert np.allclose(got.reshape(sq, dv), np.tile(mean, (sq, 1)), rtol=0, atol=1e-7)


def test_dominant_key_selects_its_value_row():
    """Query i's scores: key (3 i) mod sk is 200 ahead of every other; exp(-200) is far
    below half an ulp of 1, so O(i) is exactly that key's row of V."""
    sq, sk, dv = 6, 11, 7
    rng = np.random.default_rng(3)
    d = sk + 1  # K(j, .) = one-hot at j; Q(i, .) = one-hot at (3 i) mod sk
    K = np.zeros(sk * d)
    for j in range(sk):
        K[j * d + j] = 1.0
    Q = np.zeros(sq * d)
    for i in range(sq):
        Q[i * d + (3 * i) % sk] = 1.0
    Vf = rng.uniform(-1, 1, sk * dv)
    V = workloads.to_bits(Vf, "f16")
    got = oracle.attention(1, sq, sk, d, dv, workloads.to_bits(Q, "f16"), d, 0, workloads.to_bits(K, "f16"), d, 0,
                           V, dv, 0, in_type="f16", out_type="f16", scale=200.0)
    for i in range(sq):
        assert np.array_equal(got.reshape(sq, dv)[i], V.reshape(sk, dv)[(3 * i) % sk]), i


def test_identity_v_gives_softmax_weights():
    rng = np.random.default_rng(4)
    sq, sk, d = 5, 9, 6
    Q, K = draw(rng, sq * d, "f16", -3, 3), draw(rng, sk * d, "f16", -3, 3)
    V = workloads.to_bits(np.eye(sk).ravel(), "f16")
    got = oracle.attention(1, sq, sk, d, sk, Q, d, 0, K, d, 0, V, sk, 0, in_type="f16", out_type="f32",
                           scale=0.8).reshape(sq, sk)
    assert np.all(got >= 0)
    assert np.allclose(got.sum(axis=1), 1.0, rtol=0, atol=1e-6)
    # and they are the softmax of the scores, recomputed here in fp64 from the decoded inputs
    s = 0.8 * vals(Q, "f16").reshape(sq, d) @ vals(K, "f16").reshape(sk, d).T
    w = np.exp(s - s.max(axis=1, keepdims=True))
    assert np.allclose(got, w / w.sum(axis=1, keepdims=True), rtol=1e-6, atol=0)


def test_shift_of_the_scores_leaves_o_unchanged():
    """An extra column, 1 in Q and the same value c in every row of K, adds scale c to every
    score of a row: the softmax and O do not change (fp64 rounding aside)."""
    rng = np.random.default_rng(6)
    sq, sk, d, dv = 4, 13, 8, 6
    Qf, Kf, Vf = rng.uniform(-1, 1, (sq, d)), rng.uniform(-1, 1, (sk, d)), rng.uniform(-1, 1, (sk, dv))
    base = oracle.attention(1, sq, sk, d, dv, workloads.to_bits(Qf, "f16"), d, 0, workloads.to_bits(Kf, "f16"),
                            d, 0, workloads.to_bits(Vf, "f16"), dv, 0, in_type="f16", out_type="f32", scale=0.5)
    Q2 = np.hstack([Qf, np.ones((sq, 1))])
    K2 = np.hstack([Kf, np.full((sk, 1), 37.0)])
    shifted = oracle.attention(1, sq, sk, d + 1, dv, workloads.to_bits(Q2, "f16"), d + 1, 0,
                               workloads.to_bits(K2, "f16"), d + 1, 0, workloads.to_bits(Vf, "f16"), dv, 0,
                               in_type="f16", out_type="f32", scale=0.5)
    assert np.allclose(base, shifted, rtol=1e-6, atol=1e-7)


def test_key_permutation_leaves_o_unchanged():
    rng = np.random.default_rng(7)
    sq, sk, d, dv = 4, 17, 8, 6
    Q, K, V = draw(rng, sq * d, "bf16"), draw(rng, sk * d, "bf16"), draw(rng, sk * dv, "bf16")
    perm = rng.permutation(sk)
    Kp = K.reshape(sk, d)[perm].ravel()
    Vp = V.reshape(sk, dv)[perm].ravel()
    a = oracle.attention(1, sq, sk, d, dv, Q, d, 0, K, d, 0, V, dv, 0, in_type="bf16", out_type="f32", scale=0.7)
    b = oracle.attention(1, sq, sk, d, dv, Q, d, 0, Kp, d, 0, Vp, dv, 0, in_type="bf16", out_type="f32", scale=0.7)
    assert np.allclose(a, b, rtol=1e-6, atol=1e-7)


def test_rows_equal_full_and_threads_invariant():
    rng = np.random.default_rng(8)
    batch, sq, sk, d, dv = 3, 7, 19, 16, 12
    Q = draw(rng, batch * sq * d, "f16")
    K = draw(rng, batch * sk * d, "f16")
    V = draw(rng, batch * sk * dv, "f16")
    args = (batch, sq, sk, d, dv, Q, d, sq * d, K, d, sk * d, V, dv, sk * dv)
    full = oracle.attention(*args, in_type="f16", out_type="f16", scale=0.25).reshape(batch, sq, dv)
    one = oracle.attention(*args, in_type="f16", out_type="f16", scale=0.25, nthreads=1).reshape(batch, sq, dv)
    assert np.array_equal(full, one)
    rows = np.array([[b, i] for b in range(batch) for i in range(sq)][::3])
    sel = oracle.attention_rows(*args, rows, in_type="f16", out_type="f16", scale=0.25)
    for r, (b, i) in enumerate(rows):
        assert np.array_equal(sel[r], full[b, i])


def test_batches_are_independent():
    """Each batch slice uses its own Q, K and V: slice 1 alone equals slice 1 of the batch."""
    rng = np.random.default_rng(9)
    batch, sq, sk, d, dv = 2, 5, 9, 8, 4
    Q, K, V = draw(rng, batch * sq * d, "f16"), draw(rng, batch * sk * d, "f16"), draw(rng, batch * sk * dv, "f16")
    both = oracle.attention(batch, sq, sk, d, dv, Q, d, sq * d, K, d, sk * d, V, dv, sk * dv, in_type="f16",
                            out_type="f32", scale=1.0).reshape(batch, sq, dv)
    alone = oracle.attention(1, sq, sk, d, dv, Q[sq * d:], d, 0, K[sk * d:], d, 0, V[sk * dv:], dv, 0,
                             in_type="f16", out_type="f32", scale=1.0).reshape(sq, dv)
    assert np.array_equal(both[1], alone)
    assert not np.array_equal(both[0], alone)


def test_large_scores_do_not_overflow():
    """Scores near 700 (exp would overflow fp64 without the row maximum subtracted)."""
    sq, sk, d, dv = 2, 4, 1, 2
    Q = workloads.to_bits(np.array([1.0, -1.0]), "f16")
    K = workloads.to_bits(np.array([1.0, 2.0, 3.0, 4.0]), "f16")
    V = workloads.to_bits(np.arange(8, dtype=np.float64) / 8, "f16")
    got = oracle.attention(1, sq, sk, d, dv, Q, d, 0, K, d, 0, V, dv, 0, in_type="f16", out_type="f32",
                           scale=700.0).reshape(sq, dv)
    assert np.all(np.isfinite(got))
    assert np.array_equal(got[0], vals(V, "f16").reshape(sk, dv)[3].astype(np.float32))
    assert np.array_equal(got[1], vals(V, "f16").reshape(sk, dv)[0].astype(np.float32))


@pytest.mark.parametrize("kw", [dict(sk=0), dict(sq=-1), dict(in_type="i8"), dict(out_type="i32")])
def test_rejections(kw):
    base = dict(batch=1, sq=2, sk=3, d=4, dv=4, in_type="f16", out_type="f32")
    base.update(kw)
    Q = np.zeros(64, np.uint16 if base["in_type"] != "i8" else np.int8)
    with pytest.raises((ValueError, KeyError, TypeError)):
        oracle.attention(base["batch"], base["sq"], base["sk"], base["d"], base["dv"], Q, 4, 0, Q, 4, 0, Q, 4, 0,
                         in_type=base["in_type"], out_type=base["out_type"], scale=1.0)
