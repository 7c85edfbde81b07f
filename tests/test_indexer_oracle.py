"""Pins for the indexer-score oracle (no GPU).

The oracle computes Eq. (1) of page "LiteTopK: Exploiting the Curse of
Dimensionality for a Fused Indexer-TopK Kernel ..." (section 核心公式):
I[t, s] = sum_h w[t, h] * ReLU(q[t, h] . k[s]) over FP8 (OCP E4M3) q and k, with
-inf past each query's valid length. It is pinned here to things other than
itself: the E4M3 code points the OCP format fixes, torch's own float8_e4m3fn
conversion, a pure-Python loop over the formula on tiny shapes, closed-form
cases built from one-hot vectors (each one chosen so that a dropped ReLU, a
swapped head / weight index, a transposed operand or a wrong suffix fails it),
and the magnitude bound that scales the float32 tolerance. Mutated copies of the
oracle with those mistakes planted must fail the same pins.
"""
import math

import numpy as np
import pytest
import torch

from oracle import indexer_scores as O

ONE = 0x38  # E4M3 code of 1.0 (exponent field 7 = bias, mantissa 0)


def test_e4m3_code_points_from_the_format():
    # sign | 4 exponent bits (bias 7) | 3 mantissa bits; subnormals at exponent 0
    cases = {
        0x00: 0.0, 0x01: 2.0 ** -9, 0x07: 7 * 2.0 ** -9, 0x08: 2.0 ** -6,
        0x38: 1.0, 0x39: 1.125, 0x3F: 1.875, 0x40: 2.0, 0x30: 0.5,
        0x7E: 448.0, 0x77: 240.0, 0x78: 256.0,
        0x80: -0.0, 0xB8: -1.0, 0xFE: -448.0, 0x81: -(2.0 ** -9),
    }
    got = O.decode_e4m3(np.array(list(cases), dtype=np.uint8))
    assert np.array_equal(got, np.array(list(cases.values())))
    assert np.signbit(O.decode_e4m3(np.uint8(0x80)))
    assert np.isnan(O.decode_e4m3(np.array([0x7F, 0xFF], dtype=np.uint8))).all()
    assert np.isfinite(O.decode_e4m3(np.arange(256, dtype=np.uint8)[np.arange(256) % 128 != 127])).all()


def test_e4m3_matches_torch_for_every_code():
    codes = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = O.decode_e4m3(codes)
    same = (got == ref) | (np.isnan(got) & np.isnan(ref))
    assert same.all(), codes[~same]
    num = ~np.isnan(ref)
    assert np.array_equal(np.signbit(got[num]), np.signbit(ref[num]))


def _python_loop_scores(q, k, w, L):
    """The formula written as nested Python loops over exact float values."""
    T, H, D = q.shape
    S = k.shape[0]
    qv = [[[float(O.decode_e4m3(q[t, h, d])) for d in range(D)] for h in range(H)] for t in range(T)]
    kv = [[float(O.decode_e4m3(k[s, d])) for d in range(D)] for s in range(S)]
    out = np.full((T, S), -math.inf)
    for t in range(T):
        for s in range(min(max(int(L[t]), 0), S)):
            acc = 0.0
            for h in range(H):
                dot = math.fsum(qv[t][h][d] * kv[s][d] for d in range(D))
                acc += float(np.float32(w[t, h])) * max(dot, 0.0)
            out[t, s] = acc
    return out


def _random_case(T, H, D, S, seed):
    rng = np.random.default_rng(seed)
    # finite codes only (no NaN patterns), both signs, subnormals included
    q = rng.integers(0, 0x7F, size=(T, H, D), dtype=np.uint8) | (rng.integers(0, 2, (T, H, D)) << 7).astype(np.uint8)
    k = rng.integers(0, 0x7F, size=(S, D), dtype=np.uint8) | (rng.integers(0, 2, (S, D)) << 7).astype(np.uint8)
    w = rng.standard_normal((T, H)).astype(np.float32)
    L = rng.integers(-1, S + 2, size=T).astype(np.int32)
    return q, k, w, L


@pytest.mark.parametrize("shape", [(2, 3, 5, 7), (3, 4, 8, 6), (1, 16, 4, 3)])
def test_matches_python_loops_on_tiny_shapes(shape):
    T, H, D, S = shape
    for seed in range(4):
        q, k, w, L = _random_case(T, H, D, S, seed)
        ref = _python_loop_scores(q, k, w, L)
        got = O.indexer_scores(q, k, w, L)
        fin = np.isfinite(ref)
        assert np.array_equal(fin, np.isfinite(got))
        assert np.array_equal(got[~fin], ref[~fin])
        assert np.allclose(got[fin], ref[fin], rtol=1e-12, atol=1e-12 * np.abs(ref[fin]).max(initial=1.0))


def _one_hot_case():
    """T=2 queries, H=3 heads, D=4, S=5 keys, built from one-hot +-1 vectors.

    q[t, h] = sign(t, h) * e_{h+t}: head h of query t points along axis (h + t) % 4.
    k[s] = (s + 1) * ... is not representable for all s, so k[s] = e_{s % 4} * c_s with
    c_s in {1, 2, 4, 0.5, 1} (exact E4M3 values)."""
    T, H, D, S = 2, 3, 4, 5
    sign = np.array([[1, -1, 1], [-1, 1, 1]])
    code = {1.0: 0x38, 2.0: 0x40, 4.0: 0x48, 0.5: 0x30, -1.0: 0xB8}
    q = np.zeros((T, H, D), dtype=np.uint8)
    for t in range(T):
        for h in range(H):
            q[t, h, (h + t) % D] = code[float(sign[t, h])]
    c = [1.0, 2.0, 4.0, 0.5, 1.0]
    k = np.zeros((S, D), dtype=np.uint8)
    for s in range(S):
        k[s, s % D] = code[c[s]]
    w = np.array([[0.5, 3.0, -2.0], [1.5, -0.25, 8.0]], dtype=np.float32)
    L = np.array([5, 3], dtype=np.int32)
    # dot(t, h, s) = sign[t, h] * c[s] * [(h + t) % 4 == s % 4]; I = sum_h w * max(dot, 0)
    want = np.full((T, S), -np.inf)
    for t in range(T):
        for s in range(L[t]):
            want[t, s] = sum(w[t, h] * max(sign[t, h] * c[s] * ((h + t) % D == s % D), 0.0) for h in range(H))
    return q, k, w, L, want


def test_one_hot_closed_form():
    q, k, w, L, want = _one_hot_case()
    # written out: query 0 heads point at axes 0, 1, 2 with signs +, -, +
    assert want[0].tolist() == [0.5 * 1, 0.0, -2.0 * 4, 0.0, 0.5 * 1]
    # query 1 heads at axes 1, 2, 3 with signs -, +, +; length 3
    assert want[1, :3].tolist() == [0.0, 0.0, -0.25 * 4]
    assert np.isneginf(want[1, 3:]).all()
    got = O.indexer_scores(q, k, w, L)
    assert np.array_equal(got, want)


def test_relu_drops_negative_heads_and_weights_sign():
    # q[0, 0] = +x, q[0, 1] = -x, k = x: dots +|x|^2 and -|x|^2
    D = 8
    x = np.array([0x38, 0x40, 0xB8, 0x30, 0x00, 0x48, 0xC0, 0x38], dtype=np.uint8)  # 1,2,-1,.5,0,4,-2,1
    xv = O.decode_e4m3(x)
    q = np.stack([x, x ^ 0x80])[None]          # flip the sign bit of every code
    k = x[None]
    w = np.array([[0.75, 100.0]], dtype=np.float32)
    got = O.indexer_scores(q, k, w, np.array([1]))
    assert got[0, 0] == 0.75 * float(xv @ xv)
    w2 = np.array([[-0.75, 100.0]], dtype=np.float32)
    assert O.indexer_scores(q, k, w2, np.array([1]))[0, 0] == -0.75 * float(xv @ xv)


def test_lengths_clamp_and_suffix():
    q, k, w, L = _random_case(4, 2, 4, 6, 11)
    L = np.array([-3, 0, 4, 99], dtype=np.int32)
    got = O.indexer_scores(q, k, w, L)
    assert np.isneginf(got[0]).all() and np.isneginf(got[1]).all()
    assert np.isfinite(got[2, :4]).all() and np.isneginf(got[2, 4:]).all()
    assert np.isfinite(got[3]).all()


def test_magnitude_bound_dominates():
    q, k, w, L = _random_case(3, 5, 16, 40, 3)
    I = O.indexer_scores(q, k, w, L)
    B = O.abs_magnitude(q, k, w, L)
    fin = np.isfinite(I)
    assert (np.abs(I[fin]) <= B[fin] * (1 + 1e-12)).all()
    assert (B[~fin] == 0).all()
    # all-positive inputs: no ReLU clipping and no cancellation, so I == B
    qp, kp, wp = q & 0x7F, k & 0x7F, np.abs(w)
    assert np.allclose(O.indexer_scores(qp, kp, wp, L)[fin], O.abs_magnitude(qp, kp, wp, L)[fin], rtol=1e-13)


def test_float32_reference_sits_inside_the_tolerance():
    # A float32 evaluation in a fixed order (products exact, sums rounded) must stay inside
    # the derived tolerance; a wrong-by-one-head value must not.
    q, k, w, L = _random_case(3, 16, 128, 50, 5)
    L = np.full(3, 50, dtype=np.int32)
    qf = O.decode_e4m3(q).astype(np.float32)
    kf = O.decode_e4m3(k).astype(np.float32)
    dots = np.einsum("thd,sd->ths", qf, kf, dtype=np.float32)
    f32 = np.zeros((3, 50), dtype=np.float32)
    for h in range(16):
        f32 = f32 + w[:, h, None] * np.maximum(dots[:, h], np.float32(0))
    ref = O.indexer_scores(q, k, w, L)
    tol = O.float32_tolerance(q, k, w, L)
    assert (np.abs(f32 - ref) <= tol).all()
    off = f32 - w[:, 0, None] * np.maximum(dots[:, 0], np.float32(0))
    bad = np.abs(off - ref) > tol
    assert bad.any()


# ---- planted mistakes: each mutated oracle must fail a pin above -------------------------

def _mut_no_relu(q, k, w, L):
    qd, kd = O.decode_e4m3(q), O.decode_e4m3(k)
    T, S = qd.shape[0], kd.shape[0]
    out = np.full((T, S), -np.inf)
    for t in range(T):
        n = int(np.clip(L[t], 0, S))
        out[t, :n] = w[t].astype(np.float64) @ (qd[t] @ kd[:n].T)
    return out


def _mut_head_shift(q, k, w, L):
    return O.indexer_scores(q, k, np.roll(np.asarray(w), 1, axis=1), L)


def _mut_transposed_key(q, k, w, L):
    qd, kd = O.decode_e4m3(q), O.decode_e4m3(k)
    T, H, D = qd.shape
    S = kd.shape[0]
    kt = kd.reshape(D, S).T if S != D else kd.T  # reads k column-major
    out = np.full((T, S), -np.inf)
    for t in range(T):
        n = int(np.clip(L[t], 0, S))
        out[t, :n] = w[t].astype(np.float64) @ np.maximum(qd[t] @ kt[:n].T, 0)
    return out


def _mut_suffix_off_by_one(q, k, w, L):
    return O.indexer_scores(q, k, w, np.asarray(L) + 1)


def _mut_bias_8(q, k, w, L):
    saved = O.E4M3_BIAS
    O.E4M3_BIAS = 8
    try:
        return O.indexer_scores(q, k, w, L)
    finally:
        O.E4M3_BIAS = saved


@pytest.mark.parametrize("mutant", [_mut_no_relu, _mut_head_shift, _mut_transposed_key,
                                    _mut_suffix_off_by_one, _mut_bias_8])
def test_planted_mistakes_fail_the_pins(mutant):
    q, k, w, L, want = _one_hot_case()
    fails = not np.array_equal(mutant(q, k, w, L), want)
    if not fails:
        qr, kr, wr, Lr = _random_case(2, 3, 5, 7, 1)
        fails = not np.allclose(np.nan_to_num(mutant(qr, kr, wr, Lr), neginf=-1e300),
                                np.nan_to_num(_python_loop_scores(qr, kr, wr, Lr), neginf=-1e300))
    assert fails
