"""GPU parity of LiveEdit's active-row path through the C ABI.

- kvc_edit_mask: the rows array (active indices, then -1) and the count bit
  for bit equal to the oracle's (O4), in threshold and top-k mode, with ties
  and NaN rows.
- chunk_attn_fwd_rows: the active rows of the output against the fp64
  oracle (bf16 max-abs <= 2e-2 and rel-L2 <= 5e-3 over the active rows;
  fp8 rings max-abs <= 6e-2), every other row of o and lse bitwise untouched.
  The mask is produced on the device and consumed by the attention kernel
  without a host round trip.
"""
import numpy as np
import pytest
import torch

import chunked_attention_amd as kv
import synth
from helpers import FP8_MAX_ABS, LSE_BF16_BOUND, StreamRun, assert_bf16_parity, compare, to_f64
from oracle import attention as O1
from oracle import liveedit as O4

pytestmark = pytest.mark.gpu


def expected_rows(active, tokens):
    out = np.full(tokens, -1, dtype=np.int32)
    out[:len(active)] = active
    return out


def check_mask(zs, ze, tau=None, keep=None):
    rows, count = kv.kvc_edit_mask(zs.cuda(), ze.cuda(), tau=tau, keep=keep)
    if keep is None:
        active = O4.active_rows_threshold(zs, ze, tau)
    else:
        active = O4.active_rows_topk(zs, ze, keep)
    got = rows.cpu().numpy()
    assert int(count.item()) == len(active)
    np.testing.assert_array_equal(got, expected_rows(active, zs.shape[0]))
    return active


@pytest.mark.parametrize("frames,grid,channels", [
    (1, (8, 8), 16), (1, (30, 54), 16), (3, (30, 54), 16), (1, (30, 54), 48),
    (1, (128, 128), 4), (1, (1, 1), 1), (1, (10, 100), 4096), (1, (50, 60), 24),
])
def test_edit_mask_bit_exact(frames, grid, channels):
    zs, ze = synth.edit_latents(3, 0, grid, frames, channels)
    tokens = zs.shape[0]
    print(f"mask {frames}x{grid}x{channels}", flush=True)
    dsq = O4.distance_sq(zs, ze)
    # thresholds around the pruning point, and the edges
    for tau in (0.0, float(np.sqrt(max(np.median(dsq), 0.0))), 1.0, 3.0, float("inf")):
        check_mask(zs, ze, tau=tau)
    for keep in sorted({0, 1, int(0.3 * tokens), tokens - 1, tokens, tokens + 5}):
        if keep >= 0:
            check_mask(zs, ze, keep=keep)


def test_edit_mask_ties_and_nan():
    zs, ze = synth.edit_latents(4, 0, (20, 20), 1, 8)
    ze = ze.clone()
    ze[10:20] = ze[0]          # ten tokens with the same edit ...
    zs[10:20] = zs[0]          # ... and the same source: equal distances
    ze[50, 3] = float("nan")   # one NaN distance
    for keep in (0, 5, 11, 120, 399, 400):
        check_mask(zs, ze, keep=keep)
    for tau in (0.0, 0.5, 2.0):
        check_mask(zs, ze, tau=tau)


def test_edit_mask_ties_across_rounds():
    # 5000 tokens (five rounds of 1024 owner threads, a part-filled last
    # round) holding only five distinct distances, spread by a multiplicative
    # hash so that every tie group spans every round and wave: the top-k cut
    # falls inside a tie group, and the lowest indices of the group must win
    # across rounds; three NaN distances sit in later rounds
    tokens = 5000
    idx = torch.arange(tokens)
    level = (idx * 7919) % 5                      # 0..4
    zs = torch.zeros(tokens, 3, dtype=torch.bfloat16)
    ze = torch.zeros(tokens, 3, dtype=torch.float32)
    ze[:, 0] = level.to(torch.float32)            # distance level^2
    ze = ze.to(torch.bfloat16)
    ze[1500, 1] = float("nan")
    ze[3071, 2] = float("nan")
    ze[4999, 0] = float("nan")
    counts = [int((level == v).sum()) for v in range(5)]
    print(f"mask ties across rounds, level counts {counts}", flush=True)
    above = 0
    keeps = {0, 1, tokens - 3, tokens}
    for v in (4, 3, 2, 1, 0):
        keeps |= {above + 1, above + counts[v] // 2, above + counts[v] - 1}
        above += counts[v]
    for keep in sorted(k for k in keeps if 0 <= k <= tokens + 5):
        check_mask(zs, ze, keep=keep)
    for tau in (0.0, 1.0, 1.5, 3.5):
        check_mask(zs, ze, tau=tau)


def test_edit_mask_deep_digits():
    # distances 1 + (k 2^-20)^2 (k = token mod 256): equal in their top 40
    # bits, so the top-k select runs through most digits before a bin holds
    # exactly the keys still wanted; with 400 tokens, 144 values tie twice
    tokens = 400
    zs = torch.zeros(tokens, 2, dtype=torch.bfloat16)
    ze = torch.zeros(tokens, 2, dtype=torch.float32)
    ze[:, 0] = 1.0
    ze[:, 1] = torch.tensor([(i % 256) * 2.0 ** -20 for i in range(tokens)])
    ze = ze.to(torch.bfloat16)
    assert torch.equal(ze[:, 1].float(), torch.tensor([(i % 256) * 2.0 ** -20 for i in range(tokens)]))
    for keep in (1, 37, 144, 200, 257, 399):
        check_mask(zs, ze, keep=keep)


def test_edit_mask_rejects_bad_arguments():
    z = torch.zeros(4, 2, dtype=torch.bfloat16, device="cuda")
    with pytest.raises(kv.KvcError):
        kv.kvc_edit_mask(z, z, tau=-1.0)
    with pytest.raises(kv.KvcError):
        kv.kvc_edit_mask(z, z, tau=float("nan"))
    big = torch.zeros(kv.KVC_MAX_MASK_TOKENS + 1, 1, dtype=torch.bfloat16, device="cuda")
    with pytest.raises(kv.KvcError):
        kv.kvc_edit_mask(big, big, keep=3)


def ring_for(w):
    return kv.Ring(w.heads, w.head_dim, w.chunk_tokens, w.cond_tokens, w.window,
                   kv_dtype=w.kv_dtype, ref_tokens=w.ref_tokens, source_tokens=w.source_tokens)


def run_rows_stream(w, dist, grid, frames, channels, keep_frac=None, tau=1.0, heads=None,
                    check_chunks=None, fp8=False, lse=True):
    """Streams chunks; from chunk 1 on, each chunk's queries go through
    chunk_attn_fwd_rows with the mask of the previous chunk's latents."""
    s = synth.Stream(w, dist)
    ring = ring_for(w)
    run = StreamRun(s, ring, fp8=fp8, heads=heads)
    nq = w.chunk_tokens + w.source_tokens
    H = w.heads
    g = torch.Generator().manual_seed(7)
    for t in range(w.chunks):
        if t == 0 or (check_chunks is not None and t not in check_chunks):
            run.chunk(t, check=False)
            continue
        zs, ze = synth.edit_latents(11, t - 1, grid, frames, channels)
        assert zs.shape[0] == nq
        keep = None if keep_frac is None else int(round(keep_frac * nq))
        rows, count = kv.kvc_edit_mask(zs.cuda(), ze.cuda(),
                                       tau=None if keep is not None else tau, keep=keep)
        active = (O4.active_rows_topk(zs, ze, keep) if keep is not None
                  else O4.active_rows_threshold(zs, ze, tau))
        k, v = s.kv_noisy(t)
        q = s.q(t)
        ring.stage(k.cuda(), v.cuda())
        prev = (torch.randn(nq, H, w.head_dim, generator=g)).to(torch.bfloat16)
        prev_lse = torch.randn(H, nq, generator=g)
        o = prev.cuda()
        lse_t = prev_lse.cuda() if lse else None
        ring.attention_rows(q.cuda(), rows, count, out=o, lse=lse_t)
        qr = O1.as_f64(q)
        if heads is not None:
            qr = qr[:, heads]
        ref, ref_lse = run.oracle.attend(t, qr, run._ref(k), run._ref(v))
        o_cpu = o.cpu()
        inactive = np.setdiff1d(np.arange(nq), active)
        # untouched rows: bitwise the previous contents
        assert torch.equal(o_cpu[inactive].view(torch.int16), prev[inactive].view(torch.int16))
        if lse:
            lse_cpu = lse_t.cpu()
            assert torch.equal(lse_cpu[:, inactive], prev_lse[:, inactive])
        # active rows against the oracle
        if len(active):
            st = compare(o_cpu[active], ref[active], heads)
            if fp8:
                assert st["finite"] and st["max_abs"] <= FP8_MAX_ABS, (t, st)
            else:
                assert_bf16_parity(st, f"rows {w.name} {dist} t={t} active={len(active)}")
        if lse and len(active):
            gl = to_f64(lse_t)[:, active]
            if heads is not None:
                gl = gl[heads]
            assert np.abs(gl - ref_lse[:, active]).max() < LSE_BF16_BOUND
        # finish the chunk like the stream does (commit clean K/V, evict)
        kc, vc = s.kv_clean(t)
        ring.commit(kc.cuda(), vc.cuda())
        run.oracle.commit(t, run._ref(kc), run._ref(vc))
        ring.evict()
    return run


@pytest.mark.parametrize("dist", ["baseline", "sharp", "peaky"])
@pytest.mark.parametrize("mode", ["threshold", "topk"])
def test_rows_attention_small(dist, mode):
    # 8x12 latent grid = 96 tokens per chunk, 2 heads: ragged row tiles
    w = synth.Workload("rows-small", 2, 128, 96, 16, 2, 6, seed=31)
    run_rows_stream(w, dist, (8, 12), 1, 16, keep_frac=0.3 if mode == "topk" else None,
                    tau=1.0)


@pytest.mark.parametrize("keep_frac", [0.0, 1 / 96, 1.0])
def test_rows_attention_edge_counts(keep_frac):
    # no active row (o untouched), one row, every row
    w = synth.Workload("rows-edge", 2, 64, 96, 16, 1, 4, seed=33)
    run_rows_stream(w, "sharp", (8, 12), 1, 16, keep_frac=keep_frac)


def test_rows_attention_skips_bad_indices_and_clamps_count():
    w = synth.Workload("rows-bad", 3, 128, 100, 8, 1, 3, seed=35)
    s = synth.Stream(w, "sharp")
    ring = ring_for(w)
    run = StreamRun(s, ring)
    run.chunk(0, check=False)
    k, v = s.kv_noisy(1)
    q = s.q(1)
    ring.stage(k.cuda(), v.cuda())
    idx = torch.tensor([5, -1, 99, 100, 1 << 20, 7, 0] + [-3] * 93, dtype=torch.int32)
    rows = idx.cuda()
    count = torch.tensor([1000], dtype=torch.int32, device="cuda")   # clamped to 100
    prev = torch.randn(100, 3, 128).to(torch.bfloat16)
    o = prev.cuda()
    ring.attention_rows(q.cuda(), rows, count, out=o)
    ref, _ = run.oracle.attend(1, O1.as_f64(q), O1.as_f64(k), O1.as_f64(v))
    o_cpu = o.cpu()
    good = [0, 5, 7, 99]
    assert_bf16_parity(compare(o_cpu[good], ref[good]), "valid listed rows")
    others = [i for i in range(100) if i not in good]
    assert torch.equal(o_cpu[others].view(torch.int16), prev[others].view(torch.int16))


def test_rows_attention_fp8():
    w = synth.Workload("rows-fp8", 2, 128, 96, 16, 2, 5, seed=37, kv_dtype="fp8_e4m3")
    run_rows_stream(w, "baseline", (8, 12), 1, 16, keep_frac=0.3, fp8=True, lse=False)


@pytest.mark.parametrize("keep_frac", [0.3, 0.1])
def test_rows_attention_720p_chunk_row_aligned_split(keep_frac):
    # 1620-token chunks, 40 heads x 128, W = 3: 486 (or 162) active rows make
    # 160 (80) rows of 131 steps, which the active-row call splits over 480
    # workgroups, three (six) to a row, each range inside one row.  Oracle on
    # 3 heads at chunks 1 and 4 (8356 keys).
    w = synth.WORKLOADS["720p"]
    w = synth.Workload("720p", w.heads, w.head_dim, w.chunk_tokens, w.cond_tokens, w.window,
                       5, std=w.std, seed=w.seed)
    run_rows_stream(w, "baseline", (30, 54), 1, 16, keep_frac=keep_frac, heads=[0, 17, 39],
                    check_chunks={1, 4})


def test_rows_attention_three_frame_chunks_sampled_heads():
    # the LiveEdit chunk: three latent frames of a 30x54 grid (4860 tokens),
    # 40 heads x 128, 256 condition tokens, W = 3, about 30% of rows active
    # (top-k); the oracle runs on 3 heads at chunks 1 and 4 (24556 keys)
    w = synth.WORKLOADS["edit3"]
    w = synth.Workload("edit3", w.heads, w.head_dim, w.chunk_tokens, w.cond_tokens, w.window,
                       5, std=w.std, seed=w.seed)
    run_rows_stream(w, "baseline", (30, 54), 3, 16, keep_frac=0.3, heads=[0, 17, 39],
                    check_chunks={1, 4})
