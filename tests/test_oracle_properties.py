"""Property-based pins for the CPU oracle (hypothesis, a fixed derandomized
example set so every run checks the same cases).

The combine is `_lse_weighted_combine` on the page
"vllm.v1.attention.ops.dcp_alltoall"; the pack layout is that page's
`dcp_a2a_lse_reduce` (`_dcp_a2a_pack_send`). Random shard counts, row counts,
widths, LSE values and non-finite LSEs (NaN, +inf, -inf) are drawn, and each
property below is a fact of the mathematics or of the page's layout rather than
the oracle's own formula:

* a row with a finite shard LSE is a convex combination of the outputs of its
  finite shards (between their elementwise minimum and maximum), and its global
  LSE lies between the largest finite shard LSE and that plus ln(count);
* the global LSE is scipy's logsumexp over the finite shards;
* a row whose shard LSEs are all NaN or +-inf gives zeros and -inf;
* adding one constant to every LSE shifts the global LSE by it and leaves the
  output unchanged; reordering the shards changes nothing;
* base 2 with LSEs l2 equals base e with l2 * ln 2, the global LSE scaled back;
* the send buffer equals numpy's reshape of the output to [B, N, H/N, D] moved
  to plane-major order, with the LSE's four bytes after each row in memory
  order.
"""
import math

import numpy as np
from hypothesis import HealthCheck, given, settings
from hypothesis import strategies as st
from scipy.special import logsumexp

SETTINGS = settings(max_examples=300, deadline=None, derandomize=True,
                    suppress_health_check=[HealthCheck.too_slow, HealthCheck.data_too_large])

LSE_VALUE = st.one_of(
    st.floats(-60.0, 60.0, allow_nan=False, allow_infinity=False),
    st.sampled_from([-math.inf, math.inf, math.nan]),
)
OUT_VALUE = st.floats(-1e3, 1e3, allow_nan=False, allow_infinity=False)


@st.composite
def combine_case(draw):
    N = draw(st.integers(1, 12))
    R = draw(st.integers(1, 6))
    D = draw(st.integers(1, 5))
    lse = np.array(draw(st.lists(LSE_VALUE, min_size=N * R, max_size=N * R)),
                   dtype=np.float64).reshape(N, R)
    o = np.array(draw(st.lists(OUT_VALUE, min_size=N * R * D, max_size=N * R * D)),
                 dtype=np.float64).reshape(N, R, D)
    return o, lse


def _scale(o):
    return 1.0 + float(np.max(np.abs(o)))


@SETTINGS
@given(case=combine_case())
def test_rows_are_convex_combinations_and_lse_is_logsumexp(oracle_mod, case):
    o, lse = case
    y, L = oracle_mod.combine_f64(o, lse)
    tol = 1e-12 * _scale(o)
    for r in range(lse.shape[1]):
        fin = np.isfinite(lse[:, r])
        if not fin.any():
            assert np.all(y[r] == 0.0) and L[r] == -math.inf
            continue
        lo = o[fin, r].min(axis=0)
        hi = o[fin, r].max(axis=0)
        assert np.all(y[r] >= lo - tol) and np.all(y[r] <= hi + tol)
        top = lse[fin, r].max()
        assert top - 1e-12 <= L[r] <= top + math.log(int(fin.sum())) + 1e-12
        assert math.isclose(L[r], logsumexp(lse[fin, r]), rel_tol=1e-13, abs_tol=1e-12)


@SETTINGS
@given(case=combine_case(), shift=st.floats(-200.0, 200.0, allow_nan=False),
       seed=st.integers(0, 2 ** 32 - 1))
def test_shift_and_permutation_invariance(oracle_mod, case, shift, seed):
    o, lse = case
    y, L = oracle_mod.combine_f64(o, lse)
    tol = 1e-11 * _scale(o)
    ys, Ls = oracle_mod.combine_f64(o, lse + shift)
    np.testing.assert_allclose(ys, y, rtol=0, atol=tol)
    fin_row = np.isfinite(L)
    np.testing.assert_allclose(Ls[fin_row], L[fin_row] + shift, rtol=1e-13, atol=1e-10)
    assert np.all(Ls[~fin_row] == -math.inf)
    perm = np.random.default_rng(seed).permutation(o.shape[0])
    yp, Lp = oracle_mod.combine_f64(o[perm], lse[perm])
    np.testing.assert_allclose(yp, y, rtol=0, atol=tol)
    np.testing.assert_allclose(Lp[fin_row], L[fin_row], rtol=1e-14, atol=1e-12)
    assert np.all(Lp[~fin_row] == -math.inf)


@SETTINGS
@given(case=combine_case())
def test_base2_is_base_e_of_scaled_lses(oracle_mod, case):
    o, lse2 = case
    y2, L2 = oracle_mod.combine_f64(o, lse2, base2=True)
    ye, Le = oracle_mod.combine_f64(o, lse2 * math.log(2.0))
    np.testing.assert_allclose(y2, ye, rtol=0, atol=1e-11 * _scale(o))
    fin = np.isfinite(Le)
    np.testing.assert_allclose(L2[fin] * math.log(2.0), Le[fin], rtol=1e-13, atol=1e-11)
    assert np.all(L2[~fin] == -math.inf) and np.all(Le[~fin] == -math.inf)


@st.composite
def pack_case(draw):
    dtype = draw(st.sampled_from(["bf16", "f16", "f32"]))
    N = draw(st.integers(1, 6))
    Hl = draw(st.integers(1, 4))
    B = draw(st.integers(1, 5))
    D = draw(st.integers(1, 9))
    seed = draw(st.integers(0, 2 ** 32 - 1))
    return dtype, N, Hl, B, D, seed


@SETTINGS
@given(case=pack_case())
def test_pack_is_the_plane_major_reshape(oracle_mod, case):
    dtype, N, Hl, B, D, seed = case
    H = N * Hl
    rng = np.random.default_rng(seed)
    elem = np.uint32 if dtype == "f32" else np.uint16
    out = rng.integers(0, np.iinfo(elem).max, size=(B, H, D), dtype=elem, endpoint=True)
    lse = rng.integers(0, 2 ** 32 - 1, size=(B, H), dtype=np.uint32, endpoint=True).view(np.float32)
    send = oracle_mod.pack_send(out, lse, N, dtype=dtype)
    P = 4 // np.dtype(elem).itemsize
    # [B, H, D] -> [B, N, Hl, D] -> plane-major [N, B, Hl, D]; the LSE's bytes in memory order
    body = out.reshape(B, N, Hl, D).transpose(1, 0, 2, 3)
    tail = lse.view(np.uint32).view(elem).reshape(B, N, Hl, P).transpose(1, 0, 2, 3)
    want = np.concatenate([body, tail], axis=3)
    assert send.shape == (N, B, Hl, D + P)
    assert np.array_equal(send, want)
