"""CPU oracle for the indexer score producer that feeds the Top-K selector.

TEST INFRASTRUCTURE ONLY: imported by tests, the package smoke check and the
benchmark's CPU-baseline leg, never by the product path. It shares no code with
the HIP library.

What it computes: the DSA-style indexer score of page "LiteTopK: Exploiting the
Curse of Dimensionality for a Fused Indexer-TopK Kernel ..." (section 核心公式,
Eq. (1)): for query token t and preceding key token s,

    I[t, s] = sum over heads h of  w[t, h] * ReLU( q[t, h, :] . k[s, :] )

with FP8 key vectors (same passage) and FP8 query vectors (the score operator of
page "几何平均快 1.55 倍，但短行采样会输：腾讯怎么测精确 Top-K", section "框架轨迹",
is an FP8 multi-query attention score kernel). Positions s at or past the
query's valid length L_t are -inf, the invalid suffix the selector expects
(same page, section "什么叫精确，时间怎么量").

Readings taken where the pages are silent:
  * FP8 means OCP E4M3 (1 sign bit, 4 exponent bits with bias 7, 3 mantissa
    bits, subnormals, the all-ones pattern S.1111.111 is NaN, no infinities,
    largest finite magnitude 448).
  * Weights w are FP32 and are applied as given (no extra softmax scale).
  * The sum runs over all H heads; D is the head dimension of q and k.

Arithmetic: every q*k product of two E4M3 values is exact in float64, and a sum
of D <= 128 of them spans at most 36 + 7 bits, so the dot products below are
exact; only the final weighting by w rounds (at float64 precision). The result
is therefore the definition's value to about 1e-16 relative.
"""
import numpy as np

E4M3_BIAS = 7


def decode_e4m3(codes) -> np.ndarray:
    """Float64 value of each OCP E4M3 byte (NaN for the two NaN patterns)."""
    b = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = np.where(b >> 7, -1.0, 1.0)
    e = (b >> 3) & 0xF
    m = (b & 0x7).astype(np.float64)
    normal = sign * np.ldexp(1.0 + m / 8.0, (e - E4M3_BIAS).astype(np.int32))
    subnormal = sign * np.ldexp(m / 8.0, 1 - E4M3_BIAS)
    v = np.where(e == 0, subnormal, normal)
    return np.where((e == 0xF) & ((b & 0x7) == 0x7), np.nan, v)


def _lengths(row_len, T: int, S: int) -> np.ndarray:
    return np.clip(np.asarray(row_len, dtype=np.int64).reshape(T), 0, S)


def indexer_scores(q_codes, k_codes, w, row_len) -> np.ndarray:
    """I[t, s] in float64, shape [T, S]; -inf for s >= clamp(row_len[t], 0, S).

    q_codes [T, H, D] uint8 (E4M3), k_codes [S, D] uint8 (E4M3), w [T, H] float32,
    row_len [T] int32."""
    q = decode_e4m3(q_codes)
    k = decode_e4m3(k_codes)
    T, H, D = q.shape
    S = k.shape[0]
    assert k.shape == (S, D)
    wt = np.asarray(w, dtype=np.float32).astype(np.float64).reshape(T, H)
    L = _lengths(row_len, T, S)
    out = np.full((T, S), -np.inf)
    for t in range(T):
        n = int(L[t])
        if n == 0:
            continue
        dots = q[t] @ k[:n].T                     # [H, n]: q[t, h] . k[s]
        out[t, :n] = wt[t] @ np.maximum(dots, 0.0)  # sum_h w[t, h] * ReLU(dot)
    return out


def abs_magnitude(q_codes, k_codes, w, row_len) -> np.ndarray:
    """B[t, s] = sum_h |w[t, h]| * sum_d |q[t, h, d] * k[s, d]| (float64, 0 past L_t).

    Any float32 evaluation of I[t, s] that sums the D products of each head and then
    the H weighted ReLU terms, in any order, with exact products, is within
    (D + H + 2) * 2^-24 * B[t, s] of the exact value (standard summation error bound;
    ReLU is 1-Lipschitz), so B scales the tolerance of a float32 implementation."""
    q = np.abs(decode_e4m3(q_codes))
    k = np.abs(decode_e4m3(k_codes))
    T, H, D = q.shape
    S = k.shape[0]
    wt = np.abs(np.asarray(w, dtype=np.float32).astype(np.float64).reshape(T, H))
    L = _lengths(row_len, T, S)
    out = np.zeros((T, S))
    for t in range(T):
        n = int(L[t])
        if n:
            out[t, :n] = wt[t] @ (q[t] @ k[:n].T)
    return out


def float32_tolerance(q_codes, k_codes, w, row_len) -> np.ndarray:
    """Per-element absolute tolerance for a float32 implementation (see abs_magnitude)."""
    D = np.asarray(q_codes).shape[2]
    H = np.asarray(q_codes).shape[1]
    return (D + H + 2) * 2.0 ** -24 * abs_magnitude(q_codes, k_codes, w, row_len)
