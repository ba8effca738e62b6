"""Pins for the fp64 oracle (O1 and O2), CPU only.

Each test pins the oracle to something other than itself: brute force over a
differently-built mask, closed forms, a library routine, or an invariant.  The
comment on each test names the plausible mistake it is meant to catch.
"""
import math

import numpy as np
import pytest
import scipy.special
import torch

from oracle import attention as O1
from oracle import brute as O2


def rnd(rng, *shape, std=1.0):
    return rng.standard_normal(shape) * std


# --------------------------------------------------------------------------
# visible set and its size: closed forms
# --------------------------------------------------------------------------

def test_visible_chunks_examples():
    # W = 2: chunk 0 sees nothing earlier; chunk 1 sees the sink; chunk 2 sees
    # the sink and chunk 1; from chunk 3 on the window slides (sink + 2 newest).
    assert O1.visible_chunks(0, 2) == []
    assert O1.visible_chunks(1, 2) == [0]
    assert O1.visible_chunks(2, 2) == [0, 1]
    assert O1.visible_chunks(3, 2) == [0, 1, 2]
    assert O1.visible_chunks(4, 2) == [0, 2, 3]
    assert O1.visible_chunks(9, 2) == [0, 7, 8]
    # W = 0: only the sink besides the chunk itself.
    assert O1.visible_chunks(5, 0) == [0]
    # the sink is never duplicated by the window
    for t in range(12):
        for W in range(6):
            ids = O1.visible_chunks(t, W)
            assert len(ids) == len(set(ids))
            assert all(j < t for j in ids)


def test_kv_length_closed_form():
    # |S(t)| = m + n * (1[t>=1] + min(W, max(t-1, 0)) + 1), worked by hand:
    # tiny (m=16, n=64, W=2): 16+64, +64, +64, then flat at 16 + 4*64.
    assert [O1.kv_length(t, 16, 64, 2) for t in range(6)] == [80, 144, 208, 272, 272, 272]
    # 720p (m=256, n=1620, W=3): 256+1620=1876, 3496, 5116, 6736, then 8356.
    assert [O1.kv_length(t, 256, 1620, 3) for t in range(7)] == \
        [1876, 3496, 5116, 6736, 8356, 8356, 8356]
    # long stream (W=6) saturates at 256 + 8*1620 = 13216 from t = 7.
    assert O1.kv_length(7, 256, 1620, 6) == 13216
    assert O1.kv_length(224, 256, 1620, 6) == 13216
    assert O1.kv_length(6, 256, 1620, 6) == 256 + 7 * 1620


# --------------------------------------------------------------------------
# O1 against O2 (catches wrong window bounds, a duplicated or missing sink,
# history taken from the wrong chunk, cond dropped)
# --------------------------------------------------------------------------

@pytest.mark.parametrize("window", [0, 1, 2, 3, 5])
@pytest.mark.parametrize("m", [0, 5])
def test_o1_equals_brute_force(window, m):
    rng = np.random.default_rng(100 + 10 * window + m)
    T, n, H, d = 7, 6, 2, 8
    scale = 1 / math.sqrt(d)
    qs = [rnd(rng, n, H, d) for _ in range(T)]
    ks = [rnd(rng, n, H, d) for _ in range(T)]
    vs = [rnd(rng, n, H, d) for _ in range(T)]
    ck = rnd(rng, m, H, d) if m else None
    cv = rnd(rng, m, H, d) if m else None
    ref = O2.stream_attention(qs, ks, vs, ck, cv, window, scale)
    so = O1.StreamOracle(window, scale, ck, cv)
    for t in range(T):
        o, _ = so.attend(t, qs[t], ks[t], vs[t])
        so.commit(t, ks[t], vs[t])
        np.testing.assert_allclose(o, ref[t], rtol=0, atol=1e-12)


def test_o1_equals_brute_force_tiny_workload_shape():
    # the tiny workload's own shape: 1 head x 64, n = 64, m = 16, W = 2, 6 chunks
    rng = np.random.default_rng(7)
    T, n, H, d, m, W = 6, 64, 1, 64, 16, 2
    scale = 1 / 8.0
    qs = [rnd(rng, n, H, d) for _ in range(T)]
    ks = [rnd(rng, n, H, d) for _ in range(T)]
    vs = [rnd(rng, n, H, d) for _ in range(T)]
    ck, cv = rnd(rng, m, H, d), rnd(rng, m, H, d)
    ref = O2.stream_attention(qs, ks, vs, ck, cv, W, scale)
    so = O1.StreamOracle(W, scale, ck, cv)
    for t in range(T):
        o, _ = so.attend(t, qs[t], ks[t], vs[t])
        so.commit(t, ks[t], vs[t])
        np.testing.assert_allclose(o, ref[t], rtol=0, atol=1e-12)


def test_brute_mask_counts_match_closed_form():
    # the mask's row counts equal |S(t)| for every chunk (independent of O1's
    # list-based assembly)
    m, n, T, W = 3, 4, 9, 2
    mask = O2.stream_mask(m, n, T, W)
    for t in range(T):
        assert mask[t * n].sum() == O1.kv_length(t, m, n, W)
        # no future chunk is visible
        assert not mask[t * n, m + (t + 1) * n:].any()


# --------------------------------------------------------------------------
# normalisation and lse (catches a missing max shift, a wrong normaliser, a
# wrong log base)
# --------------------------------------------------------------------------

def test_rows_sum_to_one_and_output_is_prob_times_v():
    rng = np.random.default_rng(3)
    n, S, H, d = 9, 23, 3, 16
    q, k, v = rnd(rng, n, H, d, std=2), rnd(rng, S, H, d, std=2), rnd(rng, S, H, d)
    o, lse, p = O1.softmax_attention(q, k, v, 0.3, return_probs=True)
    np.testing.assert_allclose(p.sum(-1), 1.0, rtol=0, atol=1e-12)
    assert (p >= 0).all()
    for h in range(H):
        np.testing.assert_allclose(o[:, h], p[h] @ v[:, h], rtol=0, atol=1e-12)


def test_lse_matches_scipy_logsumexp():
    rng = np.random.default_rng(4)
    n, S, H, d = 5, 31, 2, 8
    q, k, v = rnd(rng, n, H, d, std=3), rnd(rng, S, H, d, std=3), rnd(rng, S, H, d)
    scale = 0.7
    _, lse = O1.softmax_attention(q, k, v, scale)
    for h in range(H):
        z = scale * np.einsum("nd,sd->ns", q[:, h], k[:, h])
        np.testing.assert_allclose(lse[h], scipy.special.logsumexp(z, axis=1),
                                   rtol=0, atol=1e-12)


def test_huge_logit_gap_is_one_hot_and_finite():
    # one key 800 above the rest in logit: exp(800) overflows float64, so a
    # dropped max shift yields inf/nan here; the result must be that key's V.
    rng = np.random.default_rng(5)
    S, H, d = 17, 1, 4
    q = np.zeros((1, H, d)); q[0, 0, 0] = 1.0
    k = rnd(rng, S, H, d) * 0.1
    k[:, 0, 0] = 0.0
    k[11, 0, 0] = 800.0
    v = rnd(rng, S, H, d)
    o, lse = O1.softmax_attention(q, k, v, 1.0)
    assert np.isfinite(o).all() and np.isfinite(lse).all()
    np.testing.assert_allclose(o[0, 0], v[11, 0], rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse[0, 0], 800.0, rtol=0, atol=1e-9)


def test_hand_worked_two_key_example():
    # d = 1, scale = 1, q = 1, keys 0 and ln 3: weights 1:3, values 4 and 8
    # -> o = (4 + 3*8) / 4 = 7, lse = ln(1 + 3) = ln 4.
    q = np.array([[[1.0]]])
    k = np.array([[[0.0]], [[math.log(3.0)]]])
    v = np.array([[[4.0]], [[8.0]]])
    o, lse = O1.softmax_attention(q, k, v, 1.0)
    assert abs(o[0, 0, 0] - 7.0) < 1e-14
    assert abs(lse[0, 0] - math.log(4.0)) < 1e-14


# --------------------------------------------------------------------------
# special cases that reduce to textbook routines (catches a transposed operand,
# a wrong scale, q/k swapped)
# --------------------------------------------------------------------------

def test_single_chunk_is_sdpa():
    # one chunk, W = 0, no condition tokens: plain softmax attention.
    rng = np.random.default_rng(6)
    n, H, d = 13, 3, 32
    q, k, v = rnd(rng, n, H, d), rnd(rng, n, H, d), rnd(rng, n, H, d)
    so = O1.StreamOracle(0, 1 / math.sqrt(d))
    o, _ = so.attend(0, q, k, v)
    tq = torch.from_numpy(q).permute(1, 0, 2)
    tk = torch.from_numpy(k).permute(1, 0, 2)
    tv = torch.from_numpy(v).permute(1, 0, 2)
    ref = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv).permute(1, 0, 2).numpy()
    np.testing.assert_allclose(o, ref, rtol=0, atol=1e-12)


def test_nonsquare_sdpa_with_explicit_kv():
    # more keys than queries, non-default scale: catches a transposed operand
    rng = np.random.default_rng(8)
    n, S, H, d = 7, 19, 2, 16
    q, k, v = rnd(rng, n, H, d), rnd(rng, S, H, d), rnd(rng, S, H, d)
    o, _ = O1.softmax_attention(q, k, v, 0.37)
    tq, tk, tv = (torch.from_numpy(x).permute(1, 0, 2) for x in (q, k, v))
    ref = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, scale=0.37)
    np.testing.assert_allclose(o, ref.permute(1, 0, 2).numpy(), rtol=0, atol=1e-12)


def test_zero_scale_gives_mean_of_visible_values():
    rng = np.random.default_rng(9)
    T, n, H, d, m, W = 5, 4, 2, 8, 3, 2
    qs = [rnd(rng, n, H, d) for _ in range(T)]
    ks = [rnd(rng, n, H, d) for _ in range(T)]
    vs = [rnd(rng, n, H, d) for _ in range(T)]
    ck, cv = rnd(rng, m, H, d), rnd(rng, m, H, d)
    so = O1.StreamOracle(W, 0.0, ck, cv)
    for t in range(T):
        o, _ = so.attend(t, qs[t], ks[t], vs[t])
        so.commit(t, ks[t], vs[t])
        vis = [cv] + [vs[j] for j in O1.visible_chunks(t, W)] + [vs[t]]
        mean = np.concatenate(vis, axis=0).mean(axis=0)
        np.testing.assert_allclose(o, np.broadcast_to(mean, o.shape), rtol=0, atol=1e-12)


def test_identical_keys_give_mean_of_values():
    rng = np.random.default_rng(10)
    n, S, H, d = 6, 21, 2, 8
    q = rnd(rng, n, H, d, std=5)
    k = np.broadcast_to(rnd(rng, 1, H, d, std=5), (S, H, d)).copy()
    v = rnd(rng, S, H, d)
    o, _ = O1.softmax_attention(q, k, v, 1.0)
    np.testing.assert_allclose(o, np.broadcast_to(v.mean(0), o.shape), rtol=0, atol=1e-12)


# --------------------------------------------------------------------------
# invariants
# --------------------------------------------------------------------------

def test_permuting_kv_within_a_segment_leaves_output_unchanged():
    rng = np.random.default_rng(11)
    n, H, d, m = 8, 2, 16, 10
    q = rnd(rng, n, H, d)
    ck, cv = rnd(rng, m, H, d), rnd(rng, m, H, d)
    hk = [rnd(rng, n, H, d) for _ in range(3)]
    hv = [rnd(rng, n, H, d) for _ in range(3)]
    kc, vc = rnd(rng, n, H, d), rnd(rng, n, H, d)
    o, lse = O1.chunk_attention(q, ck, cv, hk, hv, kc, vc, 0.25)
    pc, ph = rng.permutation(m), rng.permutation(n)
    hk2 = list(hk); hv2 = list(hv)
    hk2[1], hv2[1] = hk[1][ph], hv[1][ph]
    o2, lse2 = O1.chunk_attention(q, ck[pc], cv[pc], hk2, hv2, kc[ph], vc[ph], 0.25)
    np.testing.assert_allclose(o2, o, rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse2, lse, rtol=0, atol=1e-12)


def test_permuting_queries_permutes_outputs():
    rng = np.random.default_rng(12)
    n, S, H, d = 9, 14, 2, 8
    q, k, v = rnd(rng, n, H, d), rnd(rng, S, H, d), rnd(rng, S, H, d)
    o, _ = O1.softmax_attention(q, k, v, 0.5)
    p = rng.permutation(n)
    o2, _ = O1.softmax_attention(q[p], k, v, 0.5)
    np.testing.assert_array_equal(o2, o[p])


def test_stream_length_invariance():
    # chunk t's output depends only on cond, chunk 0 and chunks t-W..t: two
    # streams that agree on those and differ on every other chunk give
    # bitwise-identical output at chunk t.
    rng = np.random.default_rng(13)
    T, n, H, d, m, W = 9, 5, 2, 8, 4, 2
    ck, cv = rnd(rng, m, H, d), rnd(rng, m, H, d)
    A = [(rnd(rng, n, H, d), rnd(rng, n, H, d)) for _ in range(T)]
    B = [(rnd(rng, n, H, d), rnd(rng, n, H, d)) for _ in range(T)]
    t = T - 1
    for j in [0] + list(range(t - W, t + 1)):
        B[j] = A[j]
    q = rnd(rng, n, H, d)
    outs = []
    for S_ in (A, B):
        so = O1.StreamOracle(W, 0.35, ck, cv)
        for j in range(t):
            so.commit(j, *S_[j])
        outs.append(so.attend(t, q, *S_[t])[0])
    np.testing.assert_array_equal(outs[0], outs[1])
    # and a stream that differs inside the window does change the output
    C = list(A)
    C[t - 1] = (rnd(rng, n, H, d), rnd(rng, n, H, d))
    so = O1.StreamOracle(W, 0.35, ck, cv)
    for j in range(t):
        so.commit(j, *C[j])
    assert np.abs(so.attend(t, q, *C[t])[0] - outs[0]).max() > 1e-6


def test_current_chunk_is_bidirectional():
    # every query of the current chunk sees every key of the current chunk:
    # changing the LAST key of the chunk changes the FIRST query's output.
    rng = np.random.default_rng(14)
    n, H, d = 6, 1, 8
    q, k, v = rnd(rng, n, H, d), rnd(rng, n, H, d), rnd(rng, n, H, d)
    so = O1.StreamOracle(1, 0.5)
    o1, _ = so.attend(0, q, k, v)
    v2 = v.copy(); v2[-1] += 1.0
    o2, _ = so.attend(0, q, k, v2)
    assert abs(o2[0] - o1[0]).max() > 1e-6


def test_golden_visible_sets():
    import os
    path = os.path.join(os.path.dirname(__file__), "golden", "visible_sets.txt")
    rows = 0
    for line in open(path):
        line = line.split("#")[0].strip()
        if not line:
            continue
        head, rest = line.split(":")
        ids_s, sizes = rest.split("|")
        W, t = map(int, head.split())
        ids = [] if ids_s.strip() == "-" else list(map(int, ids_s.split()))
        m, n, S = map(int, sizes.split())
        assert O1.visible_chunks(t, W) == ids, line
        assert O1.kv_length(t, m, n, W) == S, line
        rows += 1
    assert rows >= 15


# --------------------------------------------------------------------------
# token groups: reference tokens R (always visible) and the chunk's source
# tokens S_t (queried with the chunk, visible to it only).  O1's explicit
# assembly against O2's label mask catches a source segment leaking into the
# history, R placed after the sink but dropped for chunk 0, source queries
# seeing a different set than the chunk's own queries.
# --------------------------------------------------------------------------

@pytest.mark.parametrize("window", [0, 1, 2, 4])
@pytest.mark.parametrize("m,r,s", [(0, 3, 0), (4, 0, 5), (4, 3, 5), (0, 0, 2)])
def test_o1_equals_brute_force_with_token_groups(window, m, r, s):
    rng = np.random.default_rng(1000 + 100 * window + 10 * r + s + m)
    T, n, H, d = 6, 5, 2, 8
    scale = 1 / math.sqrt(d)
    qs = [rnd(rng, n + s, H, d) for _ in range(T)]
    ks = [rnd(rng, n + s, H, d) for _ in range(T)]
    vs = [rnd(rng, n + s, H, d) for _ in range(T)]
    ck = rnd(rng, m, H, d) if m else None
    cv = rnd(rng, m, H, d) if m else None
    rk = rnd(rng, r, H, d) if r else None
    rv = rnd(rng, r, H, d) if r else None
    ref = O2.group_stream_attention(qs, ks, vs, ck, cv, rk, rv, n, window, scale)
    so = O1.StreamOracle(window, scale, ck, cv, rk, rv)
    for t in range(T):
        src_k = ks[t][n:] if s else None
        src_v = vs[t][n:] if s else None
        o, _ = so.attend(t, qs[t], ks[t][:n], vs[t][:n], src_k=src_k, src_v=src_v)
        so.commit(t, ks[t][:n], vs[t][:n])
        np.testing.assert_allclose(o, ref[t], rtol=0, atol=1e-12)


def test_group_mask_without_groups_is_the_plain_stream_mask():
    # with no reference and no source tokens the label mask is the chunk mask
    m, n, T, W = 3, 4, 8, 2
    kg, kc = O2.group_labels(m, 0, n, 0, T)
    qc = np.repeat(np.arange(T), n)
    np.testing.assert_array_equal(O2.group_mask(kg, kc, qc, W), O2.stream_mask(m, n, T, W))


def test_group_mask_counts_match_closed_form():
    # every query of chunk t (target or source) sees |S(t)| =
    # m + r + n * (visible chunks + 1) + s keys, and never another chunk's
    # source tokens
    m, r, n, s, T, W = 2, 3, 4, 5, 9, 2
    kg, kc = O2.group_labels(m, r, n, s, T)
    qc = np.repeat(np.arange(T), n + s)
    mask = O2.group_mask(kg, kc, qc, W)
    for t in range(T):
        for row in (t * (n + s), t * (n + s) + n + s - 1):
            assert mask[row].sum() == O1.kv_length(t, m, n, W, r, s)
            src_seen = (kg == O2.SOURCE) & mask[row]
            assert set(kc[src_seen]) <= {t}
    # hand count, 720p-shaped groups (m=256, R = S = one latent frame of
    # 1620 tokens, W=3, steady): cond 256 + ref 1620 + sink, 3 window chunks
    # and the current chunk 5 * 1620 + source 1620 = 11596 keys
    assert O1.kv_length(4, 256, 1620, 3, 1620, 1620) == 11596


def test_source_queries_see_the_same_keys_as_the_chunk():
    # a source-token query and a chunk-token query with the same vector get the
    # same output: both attend the same set
    rng = np.random.default_rng(3)
    n, s, H, d = 4, 3, 1, 8
    ck, cv = rnd(rng, 2, H, d), rnd(rng, 2, H, d)
    hk, hv = [rnd(rng, n, H, d)], [rnd(rng, n, H, d)]
    cur_k, cur_v = rnd(rng, n, H, d), rnd(rng, n, H, d)
    src_k, src_v = rnd(rng, s, H, d), rnd(rng, s, H, d)
    q = rnd(rng, n + s, H, d)
    q[n + 1] = q[2]
    o, lse = O1.chunk_attention(q, ck, cv, hk, hv, cur_k, cur_v, 0.5, src_k=src_k, src_v=src_v)
    np.testing.assert_array_equal(o[n + 1], o[2])
    np.testing.assert_array_equal(lse[:, n + 1], lse[:, 2])
