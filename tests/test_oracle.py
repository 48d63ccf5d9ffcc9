"""Pins for the CPU oracle, checked against things other than itself.

The combine being pinned is `_lse_weighted_combine` on the page
"vllm.v1.attention.ops.dcp_alltoall"; the pack / unpack layout is that page's
`dcp_a2a_lse_reduce`. Each test below would fail on a plausible slip in the
oracle (a dropped term, a wrong sign or base, a swapped index, a wrong plane):

* hand-derived closed forms (tests/golden/closed_forms.json);
* brute-force attention: splitting the keys of one softmax attention into
  shards and combining the per-shard results must give the unsharded result;
* library routines: scipy's logsumexp for the global LSE, torch.softmax for
  the weights, and numpy's own float16 decoding;
* the second statement of the merge on the page
  "vllm_ascend/attention/context_parallel/sfa_cp.py",
  `_merge_dcp_outputs_with_torch` (softmax over shards, NaN -> 0);
* invariants (permutation, shift, dropping a +inf / NaN shard);
* the simulated all-to-all for the packed path.
"""
import json
import math
import os

import numpy as np
import pytest
import torch
from scipy.special import logsumexp

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "closed_forms.json")


# ---------------------------------------------------------------- conversions

def test_bf16_decoding_all_patterns(oracle_mod):
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    got = oracle_mod.bits_to_f64(bits, "bf16")
    # library route: numpy reinterprets the widened bits as float32
    with np.errstate(invalid="ignore"):
        want = (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    assert np.array_equal(np.isnan(got), np.isnan(want))
    m = ~np.isnan(want)
    assert np.array_equal(got[m], want[m])
    # a few values known from the format itself
    assert got[0x3F80] == 1.0 and got[0xC000] == -2.0 and got[0x7F80] == math.inf
    assert got[0x0001] == 2.0 ** -133 and got[0x8000] == 0.0 and math.copysign(1, got[0x8000]) < 0


def test_f16_decoding_all_patterns(oracle_mod):
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    got = oracle_mod.bits_to_f64(bits, "f16")
    want = bits.view(np.float16).astype(np.float64)  # numpy's own binary16 decoder
    assert np.array_equal(np.isnan(got), np.isnan(want))
    m = ~np.isnan(want)
    assert np.array_equal(got[m], want[m])
    assert got[0x3C00] == 1.0 and got[0x0001] == 2.0 ** -24 and got[0x7BFF] == 65504.0


def test_f32_decoding(oracle_mod):
    rng = np.random.default_rng(17)
    bits = rng.integers(0, 2 ** 32, size=200000, dtype=np.uint64).astype(np.uint32)
    special = np.array([0, 0x80000000, 0x00000001, 0x007FFFFF, 0x00800000, 0x3F800000,
                        0x7F7FFFFF, 0x7F800000, 0xFF800000, 0x7FC00000, 0xFFC12345],
                       dtype=np.uint32)
    bits = np.concatenate([special, bits])
    got = oracle_mod.bits_to_f64(bits, "f32")
    with np.errstate(invalid="ignore"):
        want = bits.view(np.float32).astype(np.float64)  # numpy's binary32 decoder
    assert np.array_equal(np.isnan(got), np.isnan(want))
    m = ~np.isnan(want)
    assert np.array_equal(got[m], want[m])
    assert got[2] == 2.0 ** -149 and got[5] == 1.0 and got[7] == math.inf
    # float32 values and their patterns are the same input
    vals = bits[m].view(np.float32)
    assert np.array_equal(oracle_mod.bits_to_f64(vals, "f32"), want[m])


# ---------------------------------------------------------------- closed forms

def _golden_cases():
    with open(GOLDEN) as f:
        return json.load(f)["cases"]


@pytest.mark.parametrize("case", _golden_cases(), ids=lambda c: c["name"])
def test_closed_forms(oracle_mod, case):
    lse = np.array([float(v) for v in case["lse"]], dtype=np.float64)
    o = np.array([[float(v) for v in row] for row in case["o"]], dtype=np.float64)
    N, D = o.shape
    y, L = oracle_mod.combine_f64(o.reshape(N, 1, D), lse.reshape(N, 1), base2=case["base2"])
    want_y = np.array([float(v) for v in case["y"]])
    want_L = float(case["L"])
    assert np.array_equal(np.isnan(y[0]), np.isnan(want_y))
    m = ~np.isnan(want_y)
    np.testing.assert_allclose(y[0][m], want_y[m], rtol=1e-14, atol=1e-14)
    if math.isinf(want_L):
        assert L[0] == want_L
    else:
        assert abs(L[0] - want_L) <= 1e-14 * max(1.0, abs(want_L))


# ---------------------------------------------------------------- brute force

def _attention(q, k, v):
    """Softmax attention of one query over keys k [L, dk], values v [L, D], fp64.

    Returns (output [D], lse) with lse = ln sum exp(scores); an empty key set
    gives output 0 and lse -inf (what an attention kernel reports for no keys).
    """
    if k.shape[0] == 0:
        return np.zeros(v.shape[1]), -math.inf
    s = k @ q / math.sqrt(q.shape[0])
    lse = float(logsumexp(s))
    p = np.exp(s - lse)
    return p @ v, lse


def _shard_sets(L, N, how, rng):
    idx = np.arange(L)
    if how == "contiguous":
        return np.array_split(idx, N)
    if how == "interleaved":
        # round-robin chunks of `interleave` tokens, the way a DCP rank owns its
        # local KV (Ascend SFA page, `_get_dcp_local_seq_lens`)
        interleave = 4
        owner = (idx // interleave) % N
        return [idx[owner == r] for r in range(N)]
    if how == "with_empty":
        cuts = np.sort(rng.choice(np.arange(1, L), size=N - 3, replace=False))
        parts = np.split(idx, cuts)
        return [np.array([], dtype=int)] + parts[:1] + [np.array([], dtype=int)] + parts[1:]
    raise ValueError(how)


_SPLITS = [(h, n) for h in ("contiguous", "interleaved") for n in (1, 2, 5, 8)] + \
    [("with_empty", 5), ("with_empty", 8)]


@pytest.mark.parametrize("how,N", _SPLITS)
@pytest.mark.parametrize("base2", [False, True])
def test_brute_force_sharded_attention(oracle_mod, how, base2, N):
    rng = np.random.default_rng(1000 * N + (7 if base2 else 0) + len(how))
    B, H, dk, D, L = 3, 2, 8, 5, 37
    q = rng.normal(size=(B, H, dk))
    k = rng.normal(size=(L, H, dk)) * 2.0
    v = rng.normal(size=(L, H, D))
    sets = _shard_sets(L, N, how, rng)
    assert sum(len(s) for s in sets) == L
    Nn = len(sets)
    o = np.zeros((Nn, B * H, D))
    lse = np.zeros((Nn, B * H))
    full_o = np.zeros((B * H, D))
    full_l = np.zeros(B * H)
    for b in range(B):
        for h in range(H):
            r = b * H + h
            full_o[r], full_l[r] = _attention(q[b, h], k[:, h], v[:, h])
            for n, s in enumerate(sets):
                o[n, r], lse[n, r] = _attention(q[b, h], k[s, h], v[s, h])
    scale = 1.0 / math.log(2.0) if base2 else 1.0  # ln -> log2
    y, Lg = oracle_mod.combine_f64(o, lse * scale, base2=base2)
    np.testing.assert_allclose(y, full_o, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(Lg, full_l * scale, rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("N", [2, 5])
def test_brute_force_fp32_storage(oracle_mod, N):
    """Sharded attention whose partial outputs and LSEs are stored in fp32 (the
    fp32-output case of the packed exchange): the storage entry point must
    reproduce unsharded attention up to the fp32 rounding of its inputs.

    Bound: each partial is off by at most 2^-24 |o| <= 2^-24 M (M = max |v|);
    each stored LSE by 2^-24 |l|, which moves a normalised weight by at most
    2 * 2^-24 * max|l| relative; so |y - y*| <= (1 + 4 max|l|) 2^-24 M.
    """
    rng = np.random.default_rng(90 + N)
    B, H, dk, D, L = 2, 3, 8, 6, 41
    q = rng.normal(size=(B, H, dk))
    k = rng.normal(size=(L, H, dk)) * 2.0
    v = rng.normal(size=(L, H, D)) * 3.0
    sets = np.array_split(rng.permutation(L), N)
    o = np.zeros((N, B, H, D), dtype=np.float32)
    lse = np.zeros((N, B, H), dtype=np.float32)
    full = np.zeros((B, H, D))
    for b in range(B):
        for h in range(H):
            full[b, h] = _attention(q[b, h], k[:, h], v[:, h])[0]
            for n, sset in enumerate(sets):
                on, ln = _attention(q[b, h], k[sset, h], v[sset, h])
                o[n, b, h], lse[n, b, h] = on, ln
    y, _ = oracle_mod.lse_combine(o, lse, "f32")
    M = np.abs(v).max()
    bound = (1 + 4 * np.abs(lse).max()) * 2.0 ** -24 * M
    assert np.abs(y - full).max() <= bound
    # the same inputs as raw patterns
    y2, _ = oracle_mod.lse_combine(o.view(np.uint32), lse, "f32")
    assert np.array_equal(y, y2)


# ---------------------------------------------------------------- library routines

@pytest.mark.parametrize("base2", [False, True])
def test_global_lse_is_logsumexp(oracle_mod, base2):
    rng = np.random.default_rng(5)
    N, R, D = 6, 200, 3
    lse = rng.uniform(-30, 40, size=(N, R))
    o = rng.normal(size=(N, R, D))
    _, L = oracle_mod.combine_f64(o, lse, base2=base2)
    if base2:
        want = logsumexp(lse * math.log(2.0), axis=0) / math.log(2.0)
    else:
        want = logsumexp(lse, axis=0)
    np.testing.assert_allclose(L, want, rtol=1e-13, atol=1e-12)


def _page2_merge(o, lse):
    """Second statement of the merge (Ascend SFA page, `_merge_dcp_outputs_with_torch`):
    non-finite LSE -> -inf, softmax over shards, NaN weights -> 0, weighted sum."""
    lt = torch.from_numpy(lse)
    lt = lt.masked_fill(~torch.isfinite(lt), float("-inf"))
    w = torch.nan_to_num(torch.softmax(lt, dim=0), nan=0.0)
    return (torch.from_numpy(o) * w.unsqueeze(-1)).sum(dim=0).numpy()


def test_agrees_with_softmax_formulation(oracle_mod, synth_mod):
    rng = np.random.default_rng(11)
    N, R, D = 7, 300, 4
    lse = rng.uniform(-10, 30, size=(N, R))
    u = rng.uniform(size=(N, R))
    lse[u < 0.05] = np.nan
    lse[(u >= 0.05) & (u < 0.1)] = np.inf
    lse[(u >= 0.1) & (u < 0.15)] = -np.inf
    lse[:, 0] = -np.inf  # an all -inf row
    lse[:, 1] = np.nan   # an all NaN row
    o = rng.normal(size=(N, R, D))
    y, _ = oracle_mod.combine_f64(o, lse, base2=False)
    np.testing.assert_allclose(y, _page2_merge(o, lse), rtol=1e-12, atol=1e-13)
    assert np.all(y[0] == 0) and np.all(y[1] == 0)


# ---------------------------------------------------------------- invariants

def test_invariants(oracle_mod):
    rng = np.random.default_rng(3)
    N, R, D = 5, 64, 6
    lse = rng.uniform(-5, 15, size=(N, R))
    o = rng.normal(size=(N, R, D))
    y, L = oracle_mod.combine_f64(o, lse)
    # permutation of shards
    perm = rng.permutation(N)
    y2, L2 = oracle_mod.combine_f64(o[perm], lse[perm])
    np.testing.assert_allclose(y2, y, rtol=1e-13, atol=1e-14)
    np.testing.assert_allclose(L2, L, rtol=1e-14, atol=1e-13)
    # common shift of all LSEs
    c = 123.25
    y3, L3 = oracle_mod.combine_f64(o, lse + c)
    np.testing.assert_allclose(y3, y, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(L3, L + c, rtol=1e-14, atol=1e-12)
    # a +inf or NaN shard contributes nothing
    for bad in (np.inf, np.nan):
        lse4 = np.concatenate([lse, np.full((1, R), bad)])
        o4 = np.concatenate([o, rng.normal(size=(1, R, D)) * 1e6])
        y4, L4 = oracle_mod.combine_f64(o4, lse4)
        np.testing.assert_allclose(y4, y, rtol=1e-13, atol=1e-14)
        np.testing.assert_allclose(L4, L, rtol=1e-14, atol=1e-13)
    # N = 1 is the identity for a finite LSE
    y5, L5 = oracle_mod.combine_f64(o[:1], lse[:1])
    assert np.array_equal(y5, o[0]) and np.array_equal(L5, lse[0])
    # equal LSEs give the mean and lse + ln N
    eq = np.repeat(lse[:1], N, axis=0)
    y6, L6 = oracle_mod.combine_f64(o, eq)
    np.testing.assert_allclose(y6, o.mean(axis=0), rtol=1e-13, atol=1e-14)
    np.testing.assert_allclose(L6, lse[0] + math.log(N), rtol=1e-14, atol=1e-13)


def test_storage_entry_matches_f64_entry(oracle_mod, synth_mod):
    """The storage-typed entry point equals the fp64 entry point on decoded inputs."""
    for dt in ("bf16", "f16", "f32"):
        o, l = synth_mod.custom_inputs(3, 5, 4, 16, dtype=dt, seed=2,
                                       special=((0.1, float("nan")), (0.1, float("inf"))))
        y, L = oracle_mod.lse_combine(o, l, dt, base2=(dt == "f16"))
        of = oracle_mod.bits_to_f64(o, dt).reshape(3, 20, 16)
        y2, L2 = oracle_mod.combine_f64(of, l.astype(np.float64).reshape(3, 20), base2=(dt == "f16"))
        assert np.array_equal(y.reshape(20, 16), y2)
        assert np.array_equal(L.reshape(20), L2)


# ---------------------------------------------------------------- pack / unpack

def test_pack_dim():
    import oracle
    assert oracle.pack_dim(2) == 2 and oracle.pack_dim(4) == 1


def test_pack_layout_and_round_trip(oracle_mod, synth_mod):
    N, B, H, D = 4, 6, 8, 10
    o, _ = synth_mod.custom_inputs(1, B, H, D, seed=9)
    o = o[0]
    rng = np.random.default_rng(2)
    lse = rng.uniform(-5, 15, size=(B, H)).astype(np.float32)
    # NaN payloads and infinities must move as raw bits
    lse_bits = lse.view(np.uint32)
    lse_bits[0, 0] = 0x7FC12345
    lse_bits[1, 3] = 0xFFA00001
    lse_bits[2, 5] = 0x7F800000
    send = oracle_mod.pack_send(o, lse, N)
    Hl = H // N
    assert send.shape == (N, B, Hl, D + 2)
    for r in range(N):
        # plane r holds heads [r*Hl, (r+1)*Hl): the chunk the all-to-all gives rank r
        assert np.array_equal(send[r, :, :, :D], o[:, r * Hl:(r + 1) * Hl, :])
        # the tail is the fp32 LSE's bytes in memory order (numpy's own view)
        tail = np.ascontiguousarray(send[r, :, :, D:]).view(np.uint32)[..., 0]
        assert np.array_equal(tail, lse_bits[:, r * Hl:(r + 1) * Hl])
    outs, lses = oracle_mod.unpack(send, D)
    for r in range(N):
        assert np.array_equal(outs[r], o[:, r * Hl:(r + 1) * Hl])
        assert np.array_equal(lses[r].view(np.uint32), lse_bits[:, r * Hl:(r + 1) * Hl])


def test_pack_layout_f32(oracle_mod, synth_mod):
    """fp32 elements: P = 1, the tail element is the LSE's own pattern."""
    N, B, H, D = 2, 3, 6, 5
    o, _ = synth_mod.custom_inputs(1, B, H, D, dtype="f32", seed=19)
    o = o[0]
    assert o.dtype == np.float32
    rng = np.random.default_rng(4)
    lse = rng.uniform(-5, 15, size=(B, H)).astype(np.float32)
    lse.view(np.uint32)[1, 2] = 0x7FC00ABC  # NaN payload moves as bits
    send = oracle_mod.pack_send(o, lse, N, dtype="f32")
    Hl = H // N
    assert send.shape == (N, B, Hl, D + 1) and send.dtype == np.uint32
    for r in range(N):
        assert np.array_equal(send[r, :, :, :D], o[:, r * Hl:(r + 1) * Hl].view(np.uint32))
        assert np.array_equal(send[r, :, :, D], lse.view(np.uint32)[:, r * Hl:(r + 1) * Hl])
    outs, lses = oracle_mod.unpack(send, D, dtype="f32")
    for r in range(N):
        assert np.array_equal(outs[r], o[:, r * Hl:(r + 1) * Hl].view(np.uint32))
        assert np.array_equal(lses[r].view(np.uint32), lse.view(np.uint32)[:, r * Hl:(r + 1) * Hl])
    with pytest.raises(ValueError):
        oracle_mod.unpack(send, D + 1, dtype="f32")


@pytest.mark.parametrize("dt,base2", [("bf16", False), ("f16", True), ("f32", False)])
def test_simulated_all_to_all(oracle_mod, synth_mod, dt, base2):
    """pack on N ranks -> all-to-all -> unpack_combine on rank p equals the
    combine over the N ranks' outputs for rank p's head slice."""
    N, B, H, D = 4, 5, 8, 12
    Hl = H // N
    outs, lses = [], []
    for r in range(N):
        o, l = synth_mod.custom_inputs(1, B, H, D, dtype=dt, seed=40 + r,
                                       special=((0.1, float("nan")), (0.05, float("-inf"))))
        outs.append(o[0])
        lses.append(l[0])
    sends = [oracle_mod.pack_send(outs[r], lses[r], N, dtype=dt) for r in range(N)]
    recvs = oracle_mod.exchange(sends)
    stacked_o = np.stack(outs)   # [N, B, H, D]: rank r's partial output
    stacked_l = np.stack(lses)
    for p in range(N):
        y, L = oracle_mod.unpack_combine(recvs[p], D, dt, base2)
        sl = slice(p * Hl, (p + 1) * Hl)
        y_ref, L_ref = oracle_mod.lse_combine(stacked_o[:, :, sl], stacked_l[:, :, sl], dt, base2)
        assert np.array_equal(y, y_ref)
        assert np.array_equal(L, L_ref)


def test_bad_arguments(oracle_mod):
    o = np.zeros((2, 6, 4), dtype=np.uint16)
    l = np.zeros((2, 6), dtype=np.float32)
    with pytest.raises(ValueError):
        oracle_mod.pack_send(o, l, 4)  # H = 6 not divisible by 4
    with pytest.raises(ValueError):
        oracle_mod.unpack(np.zeros((2, 1, 1, 5), dtype=np.uint16), 4)


# ---------------------------------------------------------------- token-major merge

def _page2_merge_layout(o, lse, token_dim):
    """`_merge_dcp_outputs_with_torch` written with torch library calls: mask
    non-finite LSEs to -inf, softmax over shards, NaN -> 0, weighted sum over
    dim 0, then move dimension token_dim - 1 to the front."""
    lt = torch.from_numpy(lse)
    lt = lt.masked_fill(~torch.isfinite(lt), float("-inf"))
    w = torch.nan_to_num(torch.softmax(lt, dim=0), nan=0.0)
    out = (torch.from_numpy(o) * w.unsqueeze(-1)).sum(dim=0)
    return out.movedim(token_dim - 1, 0).contiguous().numpy()


@pytest.mark.parametrize("token_dim", [1, 2])
@pytest.mark.parametrize("dt", ["bf16", "f32"])
def test_merge_matches_page2_layout(oracle_mod, synth_mod, token_dim, dt):
    N, A, C, D = 4, 3, 5, 8
    o, l = synth_mod.custom_inputs(N, A, C, D, dtype=dt, seed=60 + token_dim,
                                   special=((0.1, float("nan")), (0.1, float("inf")),
                                            (0.1, float("-inf"))))
    l[:, 1, 2] = -np.inf   # an all -inf row
    y, L = oracle_mod.merge(o, l, dt, token_dim)
    want = _page2_merge_layout(oracle_mod.bits_to_f64(o, dt), l.astype(np.float64), token_dim)
    assert y.shape == want.shape
    np.testing.assert_allclose(y, want, rtol=1e-12, atol=1e-13)
    # the LSE follows the same layout and equals the plain combine's
    _, Lc = oracle_mod.lse_combine(o, l, dt)
    assert np.array_equal(L, Lc if token_dim == 1 else Lc.T)
    with pytest.raises(ValueError):
        oracle_mod.merge(o, l, dt, 3)


# ---------------------------------------------------------------- all-gather + reduce-scatter local step

@pytest.mark.parametrize("base2,dt", [(False, "bf16"), (True, "bf16"), (False, "f32")])
def test_corrected_partials_sum_to_the_combine(oracle_mod, synth_mod, base2, dt):
    """The reduce-scatter / all-reduce sums every rank's corrected partial; the
    sum must be the combine of all ranks' partials (and L its global LSE)."""
    N, B, H, D = 5, 6, 4, 16
    o, l = synth_mod.custom_inputs(N, B, H, D, dtype=dt, seed=71,
                                   special=((0.1, float("nan")), (0.1, float("inf")),
                                            (0.1, float("-inf"))))
    l[:, 0, 0] = -np.inf  # all -inf row: every corrected partial is 0
    y_ref, L_ref = oracle_mod.lse_combine(o, l, dt, base2)
    total = np.zeros_like(y_ref)
    for r in range(N):
        y, L = oracle_mod.correct_partial(l, r, o[r], dt, base2)
        assert np.array_equal(L, L_ref)
        total += y
    np.testing.assert_allclose(total, y_ref, rtol=1e-12, atol=1e-13)
    assert np.all(total[0, 0] == 0)


def test_corrected_partial_closed_form(oracle_mod):
    """Two shards, base e, lse = [0, ln 3]: normalised weights [1/4, 3/4]."""
    l = np.array([0.0, math.log(3.0)], dtype=np.float32).reshape(2, 1, 1)
    o = np.array([[0x4080, 0xBF80], [0x4100, 0x4040]], dtype=np.uint16)  # [4, -1], [8, 3] in bf16
    w3 = float(np.float32(math.log(3.0)))  # the fp32 LSE actually stored
    w = np.array([1.0, math.exp(w3)]) / (1.0 + math.exp(w3))
    for r, want in ((0, np.array([4.0, -1.0]) * w[0]), (1, np.array([8.0, 3.0]) * w[1])):
        y, L = oracle_mod.correct_partial(l, r, o[r].reshape(1, 1, 2), "bf16")
        np.testing.assert_allclose(y.ravel(), want, rtol=1e-15)
        assert abs(L[0, 0] - math.log(1.0 + math.exp(w3))) < 1e-15
    with pytest.raises(ValueError):
        oracle_mod.correct_partial(l, 2, o[0].reshape(1, 1, 2), "bf16")


# ---------------------------------------------------------------- valid tokens of a padded step
#
# Reading of DirectDCPA2AWorkspace.lse_reduce (page "vllm.v1.attention.ops.dcp"),
# whose seq_lens / query_start_loc arguments the page passes without showing
# the op's body: entry num_reqs of query_start_loc counts the real tokens, the
# rest of the capacity is padding with no result.

VALID_GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "valid_tokens.json")


def _valid_cases():
    with open(VALID_GOLDEN) as f:
        return json.load(f)["cases"]


@pytest.mark.parametrize("case", _valid_cases(), ids=lambda c: c["name"])
def test_valid_tokens_hand_derived(oracle_mod, case):
    q = np.array(case["query_start_loc"], dtype=np.int32)
    assert oracle_mod.valid_tokens(q, case["capacity"], case["num_reqs"]) == case["valid"]
    if case["num_reqs"] == len(q) - 1:  # the default is the last entry
        assert oracle_mod.valid_tokens(q, case["capacity"]) == case["valid"]


def _padded_step(rng, req_lens, T, N, H, dk, D, keys_per_req):
    """A step of requests padded to T tokens, as the direct exchange delivers
    it: every real token attends to its request's keys, which are split over N
    shards (contiguous runs; a shard may hold none of a request's keys, and
    then reports output 0 and LSE -inf). Partials and LSEs are stored in fp32.
    Padding tokens hold NaN outputs and arbitrary LSEs. Returns the planes,
    query_start_loc and the unsharded attention (output, LSE) of the real
    tokens."""
    qsl = np.concatenate([[0], np.cumsum(req_lens)]).astype(np.int32)
    Tv = int(qsl[-1])
    o = np.full((N, T, H, D), np.nan, dtype=np.float32)
    lse = rng.uniform(-50, 50, size=(N, T, H)).astype(np.float32)
    lse[:, Tv:][rng.random((N, T - Tv, H)) < 0.3] = np.inf
    full = np.zeros((Tv, H, D))
    full_l = np.zeros((Tv, H))
    for r, n_tok in enumerate(req_lens):
        L = keys_per_req[r]
        k = rng.normal(size=(L, H, dk)) * 2.0
        v = rng.normal(size=(L, H, D)) * 3.0
        cuts = np.sort(rng.integers(0, L + 1, size=N - 1))  # may leave shards empty
        sets = np.split(np.arange(L), cuts)
        for t in range(qsl[r], qsl[r] + n_tok):
            q = rng.normal(size=(H, dk))
            for h in range(H):
                full[t, h], full_l[t, h] = _attention(q[h], k[:, h], v[:, h])
                for n, s in enumerate(sets):
                    on, ln = _attention(q[h], k[s, h], v[s, h])
                    o[n, t, h], lse[n, t, h] = on, ln
    return o, lse, qsl, full, full_l


@pytest.mark.parametrize("req_lens,T,N", [([3, 0, 4], 10, 3), ([1, 1, 1, 1], 6, 4),
                                          ([5, 2], 7, 2), ([], 5, 2)])
def test_valid_combine_is_attention_of_the_real_tokens(oracle_mod, req_lens, T, N):
    """The real tokens of a padded step combine to the unsharded attention of
    each token over its request's keys, whatever the padding holds; Tv is the
    number of real tokens and no padding row is returned."""
    rng = np.random.default_rng(sum(req_lens) * 31 + T + N)
    H, dk, D = 2, 8, 6
    o, lse, qsl, full, full_l = _padded_step(rng, req_lens, T, N, H, dk, D,
                                                keys_per_req=[7 + 3 * i for i in range(len(req_lens))])
    y, Lg, tv = oracle_mod.lse_combine_valid(o, lse, qsl, "f32")
    assert tv == sum(req_lens) and y.shape == (tv, H, D) and Lg.shape == (tv, H)
    if tv:
        # fp32 storage of partials and LSEs: |y - y*| <= (1 + 4 max|l|) 2^-24 M
        # (as in test_brute_force_fp32_storage), M = max |partial| of the real tokens
        real_l = lse[:, :tv][np.isfinite(lse[:, :tv])]
        M = np.nanmax(np.abs(o[:, :tv]))
        bound = (1 + 4 * np.abs(real_l).max()) * 2.0 ** -24 * M
        assert np.abs(y - full).max() <= bound
        np.testing.assert_allclose(Lg, full_l, rtol=0, atol=4 * 2.0 ** -24 * np.abs(real_l).max() + 1e-12)
        # the same as the plain combine of the first tv tokens
        y2, L2 = oracle_mod.lse_combine(np.ascontiguousarray(o[:, :tv]),
                                        np.ascontiguousarray(lse[:, :tv]), "f32")
        assert np.array_equal(y, y2) and np.array_equal(Lg, L2)
    # padding contents do not matter
    o2, lse2 = o.copy(), lse.copy()
    o2[:, tv:] = 1e30
    lse2[:, tv:] = -np.inf
    y3, L3, tv3 = oracle_mod.lse_combine_valid(o2, lse2, qsl, "f32")
    assert tv3 == tv and np.array_equal(y3, y) and np.array_equal(L3, Lg)


def test_valid_combine_counts_entry_num_reqs(oracle_mod, synth_mod):
    """A query_start_loc longer than num_reqs + 1 (a buffer sized for more
    requests): the count comes from entry num_reqs, and the capacity clamps it."""
    o, l = synth_mod.custom_inputs(3, 9, 2, 8, dtype="bf16", seed=5)
    q = np.array([0, 2, 5, 9, 9], dtype=np.int32)
    for nr, want in ((0, 0), (1, 2), (2, 5), (3, 9), (4, 9)):
        y, L, tv = oracle_mod.lse_combine_valid(o, l, q, "bf16", num_reqs=nr)
        assert tv == want and y.shape[0] == want
        if want:
            y2, L2 = oracle_mod.lse_combine(np.ascontiguousarray(o[:, :want]),
                                            np.ascontiguousarray(l[:, :want]), "bf16")
            assert np.array_equal(y, y2) and np.array_equal(L, L2)
    _, _, tv = oracle_mod.lse_combine_valid(o, l, np.array([0, 40], dtype=np.int32), "bf16")
    assert tv == 9
    with pytest.raises(ValueError):
        oracle_mod.valid_tokens(q, 9, num_reqs=5)
