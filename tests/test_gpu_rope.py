"""GPU parity of the fused rotary encoding (kvc_append_chunk_rope,
chunk_attn_fwd_rope) through the C ABI.

- K1 with a rotation table: stored keys bit for bit equal to the oracle's
  stored values (O5: float32 products and sum, bf16 nearest-even), fp8 codes
  and scales equal to O3 applied to them; V untouched by the rotation.
- Fused rotation = plain calls on keys and queries rotated beforehand with
  the oracle's stored values: bitwise the same outputs (same kernels, same
  bf16 operands).
- Attention with rotation against the fp64 oracle on the rotated values,
  with token groups (the source rows take the table from row n on) and with
  active rows.
"""
import numpy as np
import pytest
import torch

import chunked_attention_amd as kv
import synth
from helpers import FP8_MAX_ABS, LSE_BF16_BOUND, assert_bf16_parity, compare
from oracle import attention as O1
from oracle import fp8 as O3
from oracle import rope as O5

pytestmark = pytest.mark.gpu


def ring(H, d, n, m, W, dtype="bf16", r=0, s=0):
    return kv.Ring(H, d, n, m, W, kv_dtype=dtype, ref_tokens=r, source_tokens=s)


@pytest.mark.parametrize("H,d,n,m,s", [(3, 128, 100, 40, 0), (2, 64, 64, 16, 24),
                                       (40, 128, 1620, 256, 0), (1, 128, 1, 1, 1)])
@pytest.mark.parametrize("dtype", ["bf16", "fp8_e4m3"])
def test_cache_write_rope_bit_exact(H, d, n, m, s, dtype):
    w = synth.Workload("k1rope", H, d, n, m, 1, 3, seed=41)
    st = synth.Stream(w, "sharp")
    rg = ring(H, d, n, m, 1, dtype, s=s)
    ck, cv = st.kv_cond()
    k, v = st.kv_noisy(0)
    sk = torch.randn(s, H, d).to(torch.bfloat16)
    sv = torch.randn(s, H, d).to(torch.bfloat16)
    kall, vall = torch.cat([k, sk]), torch.cat([v, sv])
    tc = synth.rope_table(41, 0, m, d)
    tk = synth.rope_table(41, 1, n + s, d)
    rg.cond(ck.cuda(), cv.cuda(), rope=tc.cuda())
    rg.stage(kall.cuda(), vall.cuda(), rope=tk.cuda())
    torch.cuda.synchronize()
    cases = [(-1, ck, cv, tc), (-2, k, v, tk[:n])]
    if s:
        cases.append((-4, sk, sv, tk[n:]))
    for which, kk, vv, tab in cases:
        K, Vt, ks, vs, rows = rg.slot_tensors(which)
        krot = O5.rotate_stored(kk, tab.numpy())
        if dtype == "bf16":
            assert torch.equal(K.cpu()[:, :rows].view(torch.int16),
                               krot.permute(1, 0, 2).contiguous().view(torch.int16))
            # V is not rotated: its plane holds the plain values
            P = Vt.shape[1] * Vt.shape[3]
            p = torch.arange(P)
            kappa = (p & ~0xC) | ((p & 4) << 1) | ((p & 8) >> 1)
            vpad = torch.zeros(P, H, d, dtype=torch.bfloat16)
            vpad[:rows] = vv
            expect = vpad[kappa].view(P // 32, 32, H, d).permute(2, 0, 3, 1).contiguous()
            assert torch.equal(Vt.cpu().view(torch.int16), expect.view(torch.int16))
        else:
            codes, scales = O3.quantize_segment(krot.float().numpy())
            assert np.array_equal(ks.cpu().numpy().view(np.uint32), scales.view(np.uint32))
            got = K.cpu().numpy()[:, :rows]
            assert np.array_equal(got, codes.transpose(1, 0, 2))


@pytest.mark.parametrize("dtype", ["bf16", "fp8_e4m3"])
@pytest.mark.parametrize("groups", [False, True])
def test_fused_rope_equals_prerotated_inputs(dtype, groups):
    H, d, n, m, W = 3, 128, 150, 20, 2
    r, s = (30, 50) if groups else (0, 0)
    w = synth.Workload("rope-eq", H, d, n, m, W, 5, seed=43, ref_tokens=r, source_tokens=s)
    st = synth.Stream(w, "sharp")
    fused = ring(H, d, n, m, W, dtype, r, s)
    plain = ring(H, d, n, m, W, dtype, r, s)
    ck, cv = st.kv_cond()
    tc = synth.rope_table(43, 100, m, d)
    fused.cond(ck.cuda(), cv.cuda(), rope=tc.cuda())
    plain.cond(O5.rotate_stored(ck, tc.numpy()).cuda(), cv.cuda())
    if r:
        rk, rv = st.kv_ref()
        tr = synth.rope_table(43, 101, r, d)
        fused.ref(rk.cuda(), rv.cuda(), rope=tr.cuda())
        plain.ref(O5.rotate_stored(rk, tr.numpy()).cuda(), rv.cuda())
    for t in range(w.chunks):
        k, v = st.kv_noisy(t)
        q = st.q(t)
        if s:
            sk, sv = st.kv_src(t)
            k, v = torch.cat([k, sk]), torch.cat([v, sv])
            q = torch.cat([q, st.q_src(t)])
        tk = synth.rope_table(43, t, n + s, d)
        tq = synth.rope_table(43, 1000 + t, n + s, d)
        fused.stage(k.cuda(), v.cuda(), rope=tk.cuda())
        plain.stage(O5.rotate_stored(k, tk.numpy()).cuda(), v.cuda())
        lf = torch.empty(H, n + s, device="cuda")
        lp = torch.empty(H, n + s, device="cuda")
        of = fused.attention(q.cuda(), lse=lf, rope=tq.cuda())
        op = plain.attention(O5.rotate_stored(q, tq.numpy()).cuda(), lse=lp)
        assert torch.equal(of.view(torch.int16), op.view(torch.int16)), f"t={t}"
        assert torch.equal(lf, lp)
        kc, vc = st.kv_clean(t)
        if s:
            skc, svc = st.kv_src_clean(t)
            kc, vc = torch.cat([kc, skc]), torch.cat([vc, svc])
        fused.commit(kc.cuda(), vc.cuda(), rope=tk.cuda())
        plain.commit(O5.rotate_stored(kc, tk.numpy()).cuda(), vc.cuda())
        fused.evict()
        plain.evict()


@pytest.mark.parametrize("dtype", ["bf16", "fp8_e4m3"])
def test_fused_rope_three_frame_chunk_whole_rows_first(dtype):
    # 4860-query chunks over 40 heads: 1520 query rows on 512 workgroups, so
    # every range spans three or more rows and the RoPE call walks its
    # pieces whole rows first, like the plain call on pre-rotated inputs.
    # The two must agree bit for bit (chunk 0, then chunk 1 after a COMMIT).
    w = synth.WORKLOADS["edit3"]
    H, d, n, m, W = w.heads, w.head_dim, w.chunk_tokens, w.cond_tokens, w.window
    st = synth.Stream(w, "baseline")
    fused = ring(H, d, n, m, W, dtype)
    plain = ring(H, d, n, m, W, dtype)
    ck, cv = st.kv_cond()
    tc = synth.rope_table(49, 100, m, d)
    fused.cond(ck.cuda(), cv.cuda(), rope=tc.cuda())
    plain.cond(O5.rotate_stored(ck, tc.numpy()).cuda(), cv.cuda())
    for t in range(2):
        k, v = st.kv_noisy(t)
        q = st.q(t)
        tk = synth.rope_table(49, t, n, d)
        tq = synth.rope_table(49, 1000 + t, n, d)
        fused.stage(k.cuda(), v.cuda(), rope=tk.cuda())
        plain.stage(O5.rotate_stored(k, tk.numpy()).cuda(), v.cuda())
        lf = torch.empty(H, n, device="cuda")
        lp = torch.empty(H, n, device="cuda")
        of = fused.attention(q.cuda(), lse=lf, rope=tq.cuda())
        op = plain.attention(O5.rotate_stored(q, tq.numpy()).cuda(), lse=lp)
        assert torch.equal(of.view(torch.int16), op.view(torch.int16)), f"t={t}"
        assert torch.equal(lf, lp), f"t={t}"
        of2 = fused.attention(q.cuda(), rope=tq.cuda())
        op2 = plain.attention(O5.rotate_stored(q, tq.numpy()).cuda())
        assert torch.equal(of2.view(torch.int16), op2.view(torch.int16)), f"t={t} no lse"
        kc, vc = st.kv_clean(t)
        fused.commit(kc.cuda(), vc.cuda(), rope=tk.cuda())
        plain.commit(O5.rotate_stored(kc, tk.numpy()).cuda(), vc.cuda())
        fused.evict()
        plain.evict()


@pytest.mark.parametrize("dist", ["baseline", "sharp", "peaky"])
def test_rope_stream_parity(dist):
    # bf16 ring with reference and source groups, rotated keys and queries,
    # against the fp64 oracle on the rotated (stored) values
    H, d, n, m, W, r, s = 2, 128, 96, 16, 2, 24, 40
    w = synth.Workload("rope-par", H, d, n, m, W, 5, seed=45, ref_tokens=r, source_tokens=s)
    st = synth.Stream(w, dist)
    rg = ring(H, d, n, m, W, "bf16", r, s)
    ck, cv = st.kv_cond()
    rk, rv = st.kv_ref()
    tc = synth.rope_table(45, 100, m, d)
    tr = synth.rope_table(45, 101, r, d)
    rg.cond(ck.cuda(), cv.cuda(), rope=tc.cuda())
    rg.ref(rk.cuda(), rv.cuda(), rope=tr.cuda())
    orc = O1.StreamOracle(W, w.scale, O5.rotate_stored(ck, tc.numpy()), cv,
                          O5.rotate_stored(rk, tr.numpy()), rv)
    for t in range(w.chunks):
        k, v = st.kv_noisy(t)
        sk, sv = st.kv_src(t)
        q = torch.cat([st.q(t), st.q_src(t)])
        tk = synth.rope_table(45, t, n + s, d)
        tq = synth.rope_table(45, 1000 + t, n + s, d)
        rg.stage(torch.cat([k, sk]).cuda(), torch.cat([v, sv]).cuda(), rope=tk.cuda())
        lse = torch.empty(H, n + s, device="cuda")
        o = rg.attention(q.cuda(), lse=lse, rope=tq.cuda())
        krot = O5.rotate_stored(torch.cat([k, sk]), tk.numpy())
        ref, ref_lse = orc.attend(t, O5.rotate_stored(q, tq.numpy()), krot[:n], v,
                                  src_k=krot[n:], src_v=sv)
        stats = compare(o, ref)
        assert_bf16_parity(stats, f"rope {dist} t={t}")
        assert np.abs(lse.cpu().double().numpy() - ref_lse).max() < LSE_BF16_BOUND
        kc, vc = st.kv_clean(t)
        skc, svc = st.kv_src_clean(t)
        tkc = synth.rope_table(45, 500 + t, n + s, d)
        rg.commit(torch.cat([kc, skc]).cuda(), torch.cat([vc, svc]).cuda(), rope=tkc.cuda())
        orc.commit(t, O5.rotate_stored(kc, tkc.numpy()[:n]), vc)
        rg.evict()


def test_rope_with_active_rows_and_fp8():
    H, d, n, m, W = 2, 128, 96, 16, 1
    w = synth.Workload("rope-rows", H, d, n, m, W, 3, seed=47, kv_dtype="fp8_e4m3")
    st = synth.Stream(w, "baseline")
    rg = ring(H, d, n, m, W, "fp8_e4m3")
    ck, cv = st.kv_cond()
    tc = synth.rope_table(47, 100, m, d)
    rg.cond(ck.cuda(), cv.cuda(), rope=tc.cuda())
    rt = lambda x: O3.roundtrip_segment(x.float().numpy())
    orc = O1.StreamOracle(W, w.scale, rt(O5.rotate_stored(ck, tc.numpy())), rt(cv))
    for t in range(w.chunks):
        k, v = st.kv_noisy(t)
        q = st.q(t)
        tk = synth.rope_table(47, t, n, d)
        tq = synth.rope_table(47, 1000 + t, n, d)
        rg.stage(k.cuda(), v.cuda(), rope=tk.cuda())
        active = np.arange(3, n, 4).astype(np.int32)
        rows = torch.full((n,), -1, dtype=torch.int32)
        rows[:len(active)] = torch.from_numpy(active)
        count = torch.tensor([len(active)], dtype=torch.int32)
        prev = torch.randn(n, H, d).to(torch.bfloat16)
        o = prev.cuda()
        rg.attention_rows(q.cuda(), rows.cuda(), count.cuda(), out=o, rope=tq.cuda())
        krot = O5.rotate_stored(k, tk.numpy())
        ref, _ = orc.attend(t, O5.rotate_stored(q, tq.numpy()), rt(krot), rt(v))
        oc = o.cpu()
        st_ = compare(oc[active], ref[active])
        assert st_["finite"] and st_["max_abs"] <= FP8_MAX_ABS, (t, st_)
        inactive = np.setdiff1d(np.arange(n), active)
        assert torch.equal(oc[inactive].view(torch.int16), prev[inactive].view(torch.int16))
        kc, vc = st.kv_clean(t)
        rg.commit(kc.cuda(), vc.cuda(), rope=tk.cuda())
        orc.commit(t, rt(O5.rotate_stored(kc, tk.numpy())), rt(vc))
        rg.evict()
