"""chunk_attn_fwd_noalloc (the entry point for callers that cannot
allocate: its split-row scratch is the library's static device array)
against chunk_attn_fwd on the same ring and inputs, through the C ABI.

Same kernels and work split, so the outputs must be bitwise equal (which
meets the bf16 parity bar a fortiori).  Two calls in a row, the second on a
smaller ring, then the first ring again: the array keeps the last call's
contents and each call must only see its own."""
import numpy as np
import pytest
import torch

import chunked_attention_amd as kv
import synth

pytestmark = pytest.mark.gpu


def steady_ring(w, t, dist="sharp"):
    s = synth.Stream(w, dist, pool=4)
    r = kv.Ring(w.heads, w.head_dim, w.chunk_tokens, w.cond_tokens, w.window)
    if w.cond_tokens:
        ck, cv = s.kv_cond()
        r.cond(ck.cuda(), cv.cuda())
    for c in range(t):
        kc, vc = s.kv_clean(c)
        r.commit(kc.cuda(), vc.cuda())
        r.evict()
    k, v = s.kv_noisy(t)
    r.stage(k.cuda(), v.cuda())
    return r, s.q(t).cuda()


def both(r, q):
    o_ref = torch.empty_like(q)
    o_na = torch.full_like(q, float("nan"))
    nq = q.shape[0]
    lse_ref = torch.empty(r.cfg.heads, nq, dtype=torch.float32, device=q.device)
    lse_na = torch.full_like(lse_ref, float("nan"))
    kv.chunk_attn_fwd(r.handle, r.cfg, q, o_ref, lse_ref)
    kv.chunk_attn_fwd_noalloc(r.handle, r.cfg, q, o_na, lse_na)
    torch.cuda.synchronize()
    return o_ref, o_na, lse_ref, lse_na


def check(o_ref, o_na, lse_ref, lse_na, what):
    assert torch.isfinite(o_na.float()).all(), what
    d = (o_na.float() - o_ref.float()).abs().max().item()
    assert d <= 2e-2, (what, d)
    assert torch.equal(o_na.view(torch.int16), o_ref.view(torch.int16)), what
    assert torch.equal(lse_na.view(torch.int32), lse_ref.view(torch.int32)), what


def test_noalloc_matches_chunk_attn_fwd_twice_then_smaller():
    big = synth.WORKLOADS["720p"]                              # 40 x 128, 1620 q, 8356 keys
    small = synth.Workload("small", 8, 128, 300, 64, 2, 4, seed=17)
    ra, qa = steady_ring(big, 4)
    rb, qb = steady_ring(small, 3)
    check(*both(ra, qa), "720p first call")
    check(*both(rb, qb), "smaller ring, second call")
    check(*both(ra, qa), "720p again")
    ra.close()
    rb.close()


def test_noalloc_refuses_calls_beyond_its_scratch():
    # 41 heads x ceil(25600 / 128) = 8200 rows > KVC_NOALLOC_MAX_ROWS: refused
    # before any launch, o untouched
    w = synth.Workload("big", 41, 128, 25600, 0, 0, 1, seed=19)
    r = kv.Ring(w.heads, w.head_dim, w.chunk_tokens, w.cond_tokens, w.window)
    k = torch.zeros(w.chunk_tokens, w.heads, w.head_dim, dtype=torch.bfloat16, device="cuda")
    r.stage(k, k)
    o = torch.full_like(k, 7.0)
    with pytest.raises(kv.KvcError) as e:
        kv.chunk_attn_fwd_noalloc(r.handle, r.cfg, k, o)
    assert e.value.status == kv.KVC_E_SCRATCH
    torch.cuda.synchronize()
    assert (o.float() == 7.0).all()
    r.close()
