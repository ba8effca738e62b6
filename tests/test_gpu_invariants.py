"""GPU invariants of the HIP path that hold at any size: normalisation,
determinism, logical-order and stream-length invariance (bitwise)."""
import numpy as np
import pytest
import torch

import chunked_attention_amd as kv
import synth
from helpers import to_f64

pytestmark = pytest.mark.gpu


def ring_for(w):
    return kv.Ring(w.heads, w.head_dim, w.chunk_tokens, w.cond_tokens, w.window)


def test_constant_values_give_constant_output():
    # V = 1 everywhere -> O = 1 (softmax rows sum to one), any logits
    w = synth.Workload("ones", 8, 128, 1620, 256, 3, 6, seed=3)
    s = synth.Stream(w, "peaky")
    r = ring_for(w)
    ck, _ = s.kv_cond()
    ones_c = torch.ones_like(ck)
    r.cond(ck.cuda(), ones_c.cuda())
    for t in range(w.chunks):
        k, _ = s.kv_noisy(t)
        one = torch.ones_like(k).cuda()
        r.stage(k.cuda(), one)
        o = r.attention(s.q(t).cuda()).float()
        assert torch.allclose(o, torch.ones_like(o), atol=2 ** -8, rtol=0), (t, o.min(), o.max())
        kc, _ = s.kv_clean(t)
        r.commit(kc.cuda(), one)
        r.evict()


def run_stream(w, chunks_kv, q, cond):
    """Commit chunks_kv[0..t-1], stage chunks_kv[t], attend q; return O."""
    r = ring_for(w)
    r.cond(cond[0].cuda(), cond[1].cuda())
    for j, (k, v) in enumerate(chunks_kv[:-1]):
        r.commit(k.cuda(), v.cuda())
        r.evict()
    k, v = chunks_kv[-1]
    r.stage(k.cuda(), v.cuda())
    o = r.attention(q.cuda())
    torch.cuda.synchronize()
    return o.cpu()


def test_stream_length_invariance_bitwise():
    # output at chunk t depends only on cond, chunk 0 and chunks t-W..t:
    # streams differing elsewhere give bitwise-identical output.
    w = synth.Workload("inv", 6, 128, 300, 64, 2, 9, seed=4)
    sa = synth.Stream(w, "sharp", seed=40)
    sb = synth.Stream(w, "sharp", seed=41)
    t = 8
    A = [sa.kv_clean(j) for j in range(t + 1)]
    B = [sb.kv_clean(j) for j in range(t + 1)]
    for j in [0] + list(range(t - w.window, t + 1)):
        B[j] = A[j]
    q = sa.q(t)
    cond = sa.kv_cond()
    oa = run_stream(w, A, q, cond)
    ob = run_stream(w, B, q, cond)
    assert torch.equal(oa.view(torch.int16), ob.view(torch.int16))
    # ... while a change inside the window changes it
    C = list(A)
    C[t - 1] = sb.kv_clean(t - 1)
    oc = run_stream(w, C, q, cond)
    assert not torch.equal(oa.view(torch.int16), oc.view(torch.int16))


def test_physical_slot_order_does_not_matter_bitwise():
    # The same logical KV [cond, sink, window, current] laid out in different
    # physical slots: a long stream (window slots rotated) vs a fresh ring that
    # commits only the sink and the window chunks.
    w = synth.Workload("slots", 4, 128, 200, 32, 3, 12, seed=5)
    s = synth.Stream(w, "sharp")
    t = 11
    chunks = [s.kv_clean(j) for j in range(t + 1)]
    q = s.q(t)
    cond = s.kv_cond()
    o_long = run_stream(w, chunks, q, cond)
    short = [chunks[0]] + chunks[t - w.window:t + 1]
    o_short = run_stream(w, short, q, cond)
    assert torch.equal(o_long.view(torch.int16), o_short.view(torch.int16))


def test_repeat_runs_are_bitwise_deterministic():
    w = synth.WORKLOADS["720p"]
    s = synth.Stream(w, "baseline")
    r = ring_for(w)
    ck, cv = s.kv_cond()
    r.cond(ck.cuda(), cv.cuda())
    for t in range(5):
        k, v = s.kv_clean(t)
        if t < 4:
            r.commit(k.cuda(), v.cuda())
            r.evict()
        else:
            r.stage(k.cuda(), v.cuda())
    q = s.q(4).cuda()
    lse1 = torch.empty(w.heads, w.chunk_tokens, device="cuda")
    lse2 = torch.empty_like(lse1)
    o1 = r.attention(q, lse=lse1)
    o2 = r.attention(q, lse=lse2)
    for _ in range(3):
        o3 = r.attention(q)
    torch.cuda.synchronize()
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16))
    assert torch.equal(o1.view(torch.int16), o3.view(torch.int16))
    assert torch.equal(lse1, lse2)


def test_attention_after_commit_uses_clean_current():
    # clean-pass attention (after COMMIT, before evict) equals staging the same
    # clean K/V and attending.
    w = synth.Workload("clean", 2, 128, 100, 16, 2, 5, seed=6)
    s = synth.Stream(w, "sharp")
    r1, r2 = ring_for(w), ring_for(w)
    ck, cv = s.kv_cond()
    for r in (r1, r2):
        r.cond(ck.cuda(), cv.cuda())
    for t in range(w.chunks):
        kc, vc = s.kv_clean(t)
        q = s.q(t).cuda()
        r1.commit(kc.cuda(), vc.cuda())
        o1 = r1.attention(q)
        r2.stage(kc.cuda(), vc.cuda())
        o2 = r2.attention(q)
        r2.commit(kc.cuda(), vc.cuda())
        torch.cuda.synchronize()
        assert torch.equal(o1.view(torch.int16), o2.view(torch.int16))
        r1.evict()
        r2.evict()
