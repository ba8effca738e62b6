"""GPU parity with every token group of the editing model: reference tokens R
(always visible) and the chunk's source tokens S_t (queried with the chunk and
attended by it only), against the fp64 oracle on the same seeded inputs.
bf16 tolerances as elsewhere (max-abs <= 2e-2 and rel-L2 <= 5e-3 per call);
fp8 rings max-abs <= 6e-2."""
import dataclasses

import numpy as np
import pytest
import torch

import chunked_attention_amd as kv
import synth
from helpers import FP8_MAX_ABS, LSE_BF16_BOUND, StreamRun, assert_bf16_parity, compare, fp8_roundtrip_tokens
from oracle import attention as O1

pytestmark = pytest.mark.gpu


def ring_for(w):
    return kv.Ring(w.heads, w.head_dim, w.chunk_tokens, w.cond_tokens, w.window,
                   kv_dtype=w.kv_dtype, ref_tokens=w.ref_tokens, source_tokens=w.source_tokens)


GROUP_SHAPES = [
    # ragged everywhere: 64-token chunks, 40 source and 24 reference tokens
    dict(heads=1, head_dim=64, chunk_tokens=64, cond_tokens=16, window=2, ref_tokens=24,
         source_tokens=40),
    # source only, no cond; queries span two 128-query rows
    dict(heads=3, head_dim=128, chunk_tokens=100, cond_tokens=0, window=1, ref_tokens=0,
         source_tokens=100),
    # reference only, one-query chunks
    dict(heads=2, head_dim=128, chunk_tokens=1, cond_tokens=5, window=3, ref_tokens=65,
         source_tokens=0),
    # one source token
    dict(heads=2, head_dim=64, chunk_tokens=70, cond_tokens=1, window=0, ref_tokens=1,
         source_tokens=1),
]


@pytest.mark.parametrize("shape", GROUP_SHAPES)
@pytest.mark.parametrize("dist", ["baseline", "sharp", "peaky"])
def test_token_groups_stream_parity(shape, dist):
    w = synth.Workload("groups-small", chunks=shape["window"] + 4, seed=21, **shape)
    print(f"groups {shape} {dist}", flush=True)
    run = StreamRun(synth.Stream(w, dist), ring_for(w))
    for t in range(w.chunks):
        (o, ref, st), = run.chunk(t, lse=True)
        assert o.shape[0] == w.chunk_tokens + w.source_tokens
        assert_bf16_parity(st, f"groups {shape} {dist} t={t}")
        assert st["lse_max_abs"] < LSE_BF16_BOUND, st


@pytest.mark.parametrize("dist", ["baseline", "sharp"])
def test_token_groups_720p_sampled_heads(dist):
    # 40 heads x 128, 1620 chunk tokens + 1620 source tokens as queries,
    # 256 cond + 1620 reference tokens, W = 3: 11596 keys from chunk 4.  The
    # oracle runs on 3 heads; the GPU computes all 40.
    w = synth.WORKLOADS["groups"]
    heads = [0, 17, 39]
    run = StreamRun(synth.Stream(w, dist), ring_for(w), heads=heads)
    for t in range(5):
        check = t in (0, 1, 4)
        res, = run.chunk(t, check=check, lse=check)
        if check:
            assert_bf16_parity(res[2], f"groups 720p {dist} t={t}")
            assert res[2]["lse_max_abs"] < LSE_BF16_BOUND, res[2]
    assert O1.kv_length(4, 256, 1620, 3, 1620, 1620) == 11596


def test_clean_pass_sees_committed_source_tokens():
    # an attention call after COMMIT (the clean pass) attends the committed
    # chunk and the source rows passed with the commit
    shape = GROUP_SHAPES[0]
    w = synth.Workload("groups-clean", chunks=5, seed=23, **shape)
    s = synth.Stream(w, "sharp")
    ring = ring_for(w)
    run = StreamRun(s, ring)
    for t in range(3):
        run.chunk(t, check=False)
    t = 3
    k, v = s.kv_clean(t)
    sk, sv = s.kv_src_clean(t)
    ring.commit(torch.cat([k, sk]).cuda(), torch.cat([v, sv]).cuda())
    q = torch.cat([s.q(t), s.q_src(t)])
    o = ring.attention(q.cuda())
    ref, _ = run.oracle.attend(t, O1.as_f64(q), O1.as_f64(k), O1.as_f64(v),
                               src_k=O1.as_f64(sk), src_v=O1.as_f64(sv))
    assert_bf16_parity(compare(o, ref), "clean pass with source tokens")


@pytest.mark.parametrize("dist", ["baseline", "sharp"])
def test_token_groups_fp8(dist):
    shape = GROUP_SHAPES[0]
    w = synth.Workload("groups-fp8", chunks=6, seed=25, kv_dtype="fp8_e4m3", **shape)
    run = StreamRun(synth.Stream(w, dist), ring_for(w), fp8=True)
    worst = 0.0
    for t in range(w.chunks):
        (o, ref, st), = run.chunk(t)
        assert st["finite"]
        assert st["max_abs"] <= FP8_MAX_ABS, (t, st)
        worst = max(worst, st["rel_l2"])
    print(f"fp8 groups {dist}: worst rel-L2 {worst:.3e}")


@pytest.mark.parametrize("kv_dtype", ["bf16", "fp8_e4m3"])
def test_largest_window_uses_every_segment(kv_dtype):
    # W = KVC_MAX_WINDOW with condition, reference and source tokens: from
    # chunk W+1 on the segment table holds KVC_MAX_SEGMENTS entries (cond, ref,
    # sink, W window chunks, current, source).  Ragged sizes; the last chunks
    # are checked against the oracle.
    W = kv.KVC_MAX_WINDOW
    w = synth.Workload("maxwin", 2, 64, 40, 20, W, W + 4, seed=33, kv_dtype=kv_dtype,
                       ref_tokens=10, source_tokens=12)
    fp8 = kv_dtype != "bf16"
    print(f"max window {kv_dtype}", flush=True)
    run = StreamRun(synth.Stream(w, "baseline"), ring_for(w), fp8=fp8)
    for t in range(w.chunks):
        check = t >= W + 1
        res, = run.chunk(t, check=check, lse=check and not fp8)
        if check:
            # cond + ref + sink + W window chunks + current + source
            assert O1.kv_length(t, 20, 40, W, 10, 12) == 20 + 10 + 40 * (W + 2) + 12
            o, ref, st = res
            if fp8:
                assert st["finite"] and st["max_abs"] <= FP8_MAX_ABS, (t, st)
            else:
                assert_bf16_parity(st, f"max window t={t}")
                assert st["lse_max_abs"] < LSE_BF16_BOUND, st
