"""GPU parity of the full-depth denoise pattern: one KV ring per layer, two
denoise steps per chunk (STAGE, attend, STAGE again into the same staging
slot, attend), then the clean-KV rewrite (COMMIT) and eviction of every
layer's ring, chunk after chunk.

The per-chunk loop follows discuss.pytorch.kr "JoyAI-Video-Edit 소개",
section on the real-time deployment pipeline (a two-step DiT denoise per
chunk, with saving the clean KV cache as a stage of its own), and
ta-paperlens "論文解説: JoyAI-Video-Edit", section 5 (each chunk denoised with
the cache as history, then the cache updated to window + sink).

The 720p shape runs on three rings (layers 0, 23 and 47 of a 48-layer model),
interleaved as a model runs them: for each denoise step every layer stages
and attends, then every layer commits and evicts.  Inputs come from a pool of
four sets per role, keyed by (layer + chunk + step) mod 4 (the pool the
benchmark streams from).  The oracle checks layers 0 and 47 at chunks
{0, 3, 4, 63} (both steps) and layer 23 at chunk 63, on heads {0, 17, 39};
the GPU computes every head.  Tolerances: bf16 max-abs <= 2e-2 and rel-L2 <=
5e-3 over the sampled heads of a call.
"""
import numpy as np
import pytest
import torch

import chunked_attention_amd as kv
import synth
from helpers import assert_bf16_parity, compare
from oracle import attention as O1

pytestmark = pytest.mark.gpu

LAYERS = (0, 23, 47)
HEADS = [0, 17, 39]
POOL = 4


def _checked(layer: int, chunks: int):
    if layer == 23:
        return {chunks - 1}
    return {0, 3, 4, chunks - 1}


def test_depth_two_steps_three_rings():
    w = synth.WORKLOADS["depth"]
    assert w.steps == 2 and w.layers == 48
    chunks = w.chunks                                   # 64
    s = synth.Stream(w, "baseline", pool=POOL)

    # the pool on the device once (the stream keeps its pool tensors alive,
    # so their addresses identify them)
    dev = {}

    def gpu(x):
        key = x.data_ptr()
        if key not in dev:
            dev[key] = x.cuda()
        return dev[key]

    rings = {}
    oracles = {}
    for layer in LAYERS:
        r = kv.Ring(w.heads, w.head_dim, w.chunk_tokens, w.cond_tokens, w.window)
        ck, cv = s.kv_cond(layer)
        r.cond(ck.cuda(), cv.cuda())
        rings[layer] = r
        oracles[layer] = O1.StreamOracle(w.window, w.scale, O1.as_f64(ck)[:, HEADS],
                                         O1.as_f64(cv)[:, HEADS])
    # committed chunks the checked calls read (the sink and their windows)
    keep = {layer: set() for layer in LAYERS}
    for layer in LAYERS:
        for t in _checked(layer, chunks):
            keep[layer].update(O1.visible_chunks(t, w.window))

    worst = 0.0
    checked = 0
    for t in range(chunks):
        for step in range(w.steps):
            for layer in LAYERS:
                r = rings[layer]
                k, v = s.kv_noisy(t, step, layer)
                q = s.q(t, step, layer)
                r.stage(gpu(k), gpu(v))
                o = r.attention(gpu(q))
                if t in _checked(layer, chunks):
                    ref, _ = oracles[layer].attend(t, O1.as_f64(q)[:, HEADS],
                                                   O1.as_f64(k)[:, HEADS],
                                                   O1.as_f64(v)[:, HEADS])
                    st = compare(o, ref, HEADS)
                    assert_bf16_parity(st, f"depth layer={layer} t={t} step={step}")
                    worst = max(worst, st["rel_l2"])
                    checked += 1
        for layer in LAYERS:
            r = rings[layer]
            kc, vc = s.kv_clean(t, layer)
            r.commit(gpu(kc), gpu(vc))
            if t in keep[layer]:
                oracles[layer].commit(t, O1.as_f64(kc)[:, HEADS], O1.as_f64(vc)[:, HEADS])
            r.evict()
    for layer in LAYERS:
        info = rings[layer].info()
        assert info.n_window == w.window and info.sink_valid
        rings[layer].close()
    assert checked == 2 * (4 + 4 + 1)
    print(f"depth: {checked} calls checked, worst rel-L2 {worst:.2e}")


def test_depth_second_step_overwrites_the_staged_chunk():
    # The second denoise step re-stages the same slot: its call must see the
    # second step's K/V only.  Checked bitwise against a fresh ring that only
    # ever staged the second step's K/V (same history, same work split).
    w = synth.Workload("depth2", 8, 128, 300, 64, 2, 4, steps=2,
                       std=1.0 / np.sqrt(128), seed=21)
    s = synth.Stream(w, "sharp")
    a = kv.Ring(w.heads, w.head_dim, w.chunk_tokens, w.cond_tokens, w.window)
    b = kv.Ring(w.heads, w.head_dim, w.chunk_tokens, w.cond_tokens, w.window)
    ck, cv = s.kv_cond()
    for r in (a, b):
        r.cond(ck.cuda(), cv.cuda())
    for t in range(w.chunks):
        k0, v0 = s.kv_noisy(t, 0)
        k1, v1 = s.kv_noisy(t, 1)
        q1 = s.q(t, 1)
        a.stage(k0.cuda(), v0.cuda())
        a.attention(s.q(t, 0).cuda())
        a.stage(k1.cuda(), v1.cuda())
        oa = a.attention(q1.cuda())
        b.stage(k1.cuda(), v1.cuda())
        ob = b.attention(q1.cuda())
        assert torch.equal(oa.view(torch.int16), ob.view(torch.int16)), t
        kc, vc = s.kv_clean(t)
        for r in (a, b):
            r.commit(kc.cuda(), vc.cuda())
            r.evict()
    a.close()
    b.close()
