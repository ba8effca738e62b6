"""Host logic of the ring and the C ABI, on the CPU.

Drives the product's ring.cpp / plan.cpp through the C ABI, linked against
the recording launcher in tests/fake_launch.cpp (no GPU, no kernels).  The
device buffer is a fake, aligned address that the host code never
dereferences.
"""
import ctypes
import os
import math

import numpy as np
import pytest

import chunked_attention_amd as kv
from chunked_attention_amd import build as kbuild
from oracle import attention as O1
from oracle import fp8 as O3

BASE = 0x7F0000000000     # fake, 256-aligned device address


class Record(ctypes.Structure):
    _fields_ = [("kind", ctypes.c_int32), ("rows", ctypes.c_int32), ("pitch", ctypes.c_int32),
                ("nseg", ctypes.c_int32), ("dst_k", ctypes.c_uint64),
                ("dst_vt", ctypes.c_uint64), ("src_k", ctypes.c_uint64),
                ("src_v", ctypes.c_uint64), ("seg_k", ctypes.c_uint64 * kv.KVC_MAX_SEGMENTS),
                ("seg_rows", ctypes.c_int32 * kv.KVC_MAX_SEGMENTS),
                ("seg_pitch", ctypes.c_int32 * kv.KVC_MAX_SEGMENTS),
                ("scale", ctypes.c_float), ("kv_dtype", ctypes.c_int32),
                ("k_scale", ctypes.c_uint64), ("stream", ctypes.c_uint64),
                ("qrows", ctypes.c_uint64), ("qcount", ctypes.c_uint64),
                ("rope", ctypes.c_uint64), ("epoch", ctypes.c_uint32),
                ("ws_ready", ctypes.c_int32)]


@pytest.fixture(scope="module")
def lib():
    # KVC_HOST_SANITIZE=1: the AddressSanitizer + UBSan build of the same
    # sources (run by test_host_sanitizers.py in a process that preloads the
    # sanitizer runtime)
    sanitize = os.environ.get("KVC_HOST_SANITIZE") == "1"
    path = kbuild.HOST_LIB_SAN if sanitize else kbuild.HOST_LIB
    if kbuild.host_lib_stale(path):
        kbuild.build_host(sanitize=sanitize)
    L = kv.declare(ctypes.CDLL(path))
    L.kvcfake_record_size.restype = ctypes.c_int32
    L.kvcfake_count.restype = ctypes.c_int32
    L.kvcfake_get.argtypes = [ctypes.c_int32, ctypes.c_void_p]
    L.kvcfake_fail_next.argtypes = [ctypes.c_int32]
    L.kvcfake_e4m3_encode.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64]
    assert L.kvcfake_record_size() == ctypes.sizeof(Record)
    return L


class FakeRing:
    def __init__(self, L, H=2, d=128, n=100, m=40, W=2, dtype=kv.KVC_KV_BF16, scale=0.0,
                 r=0, s=0):
        self.L = L
        self.cfg = kv.kvc_config(H, d, n, m, W, dtype, scale, r, s)
        self.bytes = L.kvc_required_bytes(ctypes.byref(self.cfg))
        assert self.bytes > 0
        self.h = ctypes.c_void_p()
        L.kvcfake_reset()
        assert L.kvc_create(ctypes.byref(self.cfg), ctypes.c_void_p(BASE), self.bytes,
                            ctypes.byref(self.h)) == kv.KVC_OK

    def append(self, kind, k=0x1000, v=0x2000):
        return self.L.kvc_append_chunk(self.h, kind, ctypes.c_void_p(k), ctypes.c_void_p(v),
                                       ctypes.c_void_p(0x77))

    def attn(self, q=0x3000, o=0x4000, lse=None):
        return self.L.chunk_attn_fwd(self.h, ctypes.c_void_p(q), ctypes.c_void_p(o),
                                     ctypes.c_void_p(lse), ctypes.c_void_p(0x77))

    def evict(self):
        ev = ctypes.c_int32(-7)
        st = self.L.kvc_evict(self.h, ctypes.byref(ev))
        return st, ev.value

    def info(self):
        i = kv.kvc_info()
        assert self.L.kvc_get_info(self.h, ctypes.byref(i)) == kv.KVC_OK
        return {f: getattr(i, f) for f, _ in kv.kvc_info._fields_}

    def segments(self):
        buf = (kv.kvc_segment * 32)()
        cnt = ctypes.c_int32()
        st = self.L.kvc_get_segments(self.h, buf, 32, ctypes.byref(cnt))
        if st != kv.KVC_OK:
            return st
        return [(s.chunk, s.slot, s.rows, s.role) for s in buf[:cnt.value]]

    def slot(self, which):
        v = kv.kvc_slot_view()
        st = self.L.kvc_get_slot(self.h, which, ctypes.byref(v))
        return st, v

    def last(self):
        r = Record()
        n = self.L.kvcfake_count()
        assert self.L.kvcfake_get(n - 1, ctypes.byref(r)) == 0
        return r

    def count(self):
        return self.L.kvcfake_count()

    def close(self):
        self.L.kvc_destroy(self.h)


def expected_bytes(H, d, n, m, W, e, fp8, r=0, s=0):
    al = lambda x: (x + 255) // 256 * 256
    P = lambda r: (r + 63) // 64 * 64
    def slot(r):
        b = 2 * al(H * P(r) * d * e)
        if fp8:
            b += al(8 * H)
        return b
    total = (slot(m) if m else 0) + (slot(r) if r else 0) + (W + 2) * slot(n) + \
        (slot(s) if s else 0)
    if fp8:
        total += al(4 * 2 * H * (P(max(n, m, r, s)) // 64))
    # attention workspace: one 64-bit arrival word per 128-query row (n + s
    # queries), one 32-bit tag per partial slot (2 per persistent workgroup,
    # 512 at most), then per slot the reference and sum of 128 queries and the
    # fp32 O [128][d]
    rows = H * ((n + s + 127) // 128)
    total += al(8 * rows) + al(4 * 2 * 512) + al(4 * 2 * 512 * 2 * 128) + \
        4 * 2 * 512 * 128 * d
    return total


@pytest.mark.parametrize("H,d,n,m,W", [(40, 128, 1620, 256, 3), (1, 64, 64, 16, 2),
                                       (3, 128, 7, 0, 0), (2, 64, 65, 1, 29)])
@pytest.mark.parametrize("fp8", [False, True])
@pytest.mark.parametrize("r,s", [(0, 0), (30, 0), (0, 70), (1620, 1620)])
def test_required_bytes_matches_layout(lib, H, d, n, m, W, fp8, r, s):
    cfg = kv.kvc_config(H, d, n, m, W, int(fp8), 0.0, r, s)
    assert lib.kvc_required_bytes(ctypes.byref(cfg)) == \
        expected_bytes(H, d, n, m, W, 1 if fp8 else 2, fp8, r, s)


def test_720p_ring_size():
    # 720p bf16: cond 256 rows + 5 slots of 1620 rows (padded to 1664), 40
    # heads, plus the attention workspace (520 rows; 512 workgroups x 2 slots)
    assert expected_bytes(40, 128, 1620, 256, 3, 2, False) == \
        2 * 40 * 128 * 2 * (256 + 5 * 1664) + 4352 + 4096 + 1048576 + 67108864


@pytest.mark.parametrize("bad", [
    dict(heads=0), dict(head_dim=96), dict(chunk_tokens=0), dict(cond_tokens=-1),
    dict(window=-1), dict(window=30), dict(kv_dtype=2), dict(softmax_scale=-1.0),
    dict(softmax_scale=float("nan")), dict(softmax_scale=float("inf")),
    dict(ref_tokens=-1), dict(source_tokens=-5), dict(source_tokens=(1 << 20) + 1),
])
def test_bad_configs_rejected(lib, bad):
    f = dict(heads=2, head_dim=128, chunk_tokens=10, cond_tokens=4, window=2, kv_dtype=0,
             softmax_scale=0.0)
    f.update(bad)
    cfg = kv.kvc_config(**f)
    assert lib.kvc_required_bytes(ctypes.byref(cfg)) == 0
    h = ctypes.c_void_p()
    assert lib.kvc_create(ctypes.byref(cfg), ctypes.c_void_p(BASE), 1 << 40,
                          ctypes.byref(h)) == kv.KVC_E_INVAL


def test_create_errors(lib):
    cfg = kv.kvc_config(2, 128, 10, 4, 2, 0, 0.0)
    need = lib.kvc_required_bytes(ctypes.byref(cfg))
    h = ctypes.c_void_p()
    assert lib.kvc_create(ctypes.byref(cfg), None, need, ctypes.byref(h)) == kv.KVC_E_INVAL
    assert lib.kvc_create(ctypes.byref(cfg), ctypes.c_void_p(BASE + 128), need,
                          ctypes.byref(h)) == kv.KVC_E_INVAL
    assert lib.kvc_create(ctypes.byref(cfg), ctypes.c_void_p(BASE), need - 1,
                          ctypes.byref(h)) == kv.KVC_E_NOMEM
    assert lib.kvc_create(None, ctypes.c_void_p(BASE), need, ctypes.byref(h)) == kv.KVC_E_INVAL
    assert lib.kvc_create(ctypes.byref(cfg), ctypes.c_void_p(BASE), need, None) == \
        kv.KVC_E_INVAL
    assert lib.kvc_create(ctypes.byref(cfg), ctypes.c_void_p(BASE), need,
                          ctypes.byref(h)) == kv.KVC_OK
    assert lib.kvc_destroy(h) == kv.KVC_OK
    assert lib.kvc_destroy(None) == kv.KVC_OK


@pytest.mark.parametrize("W", [0, 1, 2, 3, 6])
@pytest.mark.parametrize("m", [0, 40])
def test_stream_protocol_and_segment_tables(lib, W, m):
    r = FakeRing(lib, W=W, m=m)
    if m:
        assert r.attn() == kv.KVC_E_STATE            # nothing staged yet
        assert r.append(kv.KVC_COND) == kv.KVC_OK
    assert r.info()["phase"] == kv.KVC_PHASE_EMPTY
    n = 100
    for t in range(3 * W + 6):
        for step in range(2):
            assert r.append(kv.KVC_STAGE) == kv.KVC_OK
            segs = r.segments()
            # logical order: cond, sink, window oldest..newest, current
            ids = [s[0] for s in segs]
            exp = ([-1] if m else []) + O1.visible_chunks(t, W) + [t]
            assert ids == exp, (t, ids, exp)
            roles = [s[3] for s in segs]
            assert roles == ([0] if m else []) + ([1] if t else []) + \
                [2] * (len(exp) - (1 if m else 0) - (1 if t else 0) - 1) + [3]
            assert r.info()["kv_len"] == O1.kv_length(t, m, n, W)
            c0 = r.count()
            assert r.attn() == kv.KVC_OK
            assert r.count() == c0 + 1
            rec = r.last()
            assert rec.kind == 1 and rec.nseg == len(exp) and rec.rows == n
            assert [rec.seg_rows[i] for i in range(rec.nseg)] == [s[2] for s in segs]
            assert abs(rec.scale - 1 / math.sqrt(128)) < 1e-7
            assert rec.stream == 0x77
            # the current segment is the staging slot just written
            cur_slot_addr = r.slot(-2)[1].k
            assert rec.seg_k[rec.nseg - 1] == cur_slot_addr
        staged_slot = r.segments()[-1][1]
        assert r.append(kv.KVC_COMMIT) == kv.KVC_OK
        # COMMIT wrote into the staging slot and published it
        assert r.segments()[-1][1] == staged_slot
        st, v = r.slot(t)
        assert st == kv.KVC_OK
        if t == 0:
            assert r.info()["sink_valid"] == 1
        # clean-pass attention after COMMIT sees the same visible set
        assert [s[0] for s in r.segments()] == ([-1] if m else []) + \
            O1.visible_chunks(t, W) + [t]
        st, ev = r.evict()
        assert st == kv.KVC_OK
        expect_ev = t - W if (t >= 1 and t - W >= 1) else -1
        assert ev == expect_ev, (t, ev)
        info = r.info()
        assert info["phase"] == kv.KVC_PHASE_EMPTY and info["chunk"] == t + 1
        assert info["n_window"] == min(W, t)
        assert info["free_slots"] == (W + 2) - 1 - min(W, t)
    r.close()


def test_slot_recycling_and_pinned_sink(lib):
    W = 3
    r = FakeRing(lib, W=W)
    r.append(kv.KVC_COND)
    sink_addr = None
    freed_addr = {}
    for t in range(20):
        r.append(kv.KVC_STAGE)
        stage_addr = r.last().dst_k
        if t >= W + 2:
            # the staging slot of chunk t is the slot chunk t-W-1 occupied
            assert stage_addr == freed_addr[t - W - 1]
        r.append(kv.KVC_COMMIT)
        assert r.last().dst_k == stage_addr
        if t == 0:
            sink_addr = stage_addr
        else:
            assert stage_addr != sink_addr
            freed_addr[t] = stage_addr
        st, ev = r.evict()
        assert ev != 0
    st, v = r.slot(0)
    assert st == kv.KVC_OK and v.k == sink_addr
    r.close()


def test_state_errors(lib):
    r = FakeRing(lib, W=1, m=4)
    assert r.append(kv.KVC_STAGE) == kv.KVC_OK
    assert r.attn() == kv.KVC_E_STATE                # cond never written
    assert r.append(kv.KVC_COND) == kv.KVC_OK        # allowed in any phase
    assert r.attn() == kv.KVC_OK
    assert r.evict() == (kv.KVC_E_STATE, -7)          # cannot finish an uncommitted chunk
    assert r.append(kv.KVC_COMMIT) == kv.KVC_OK
    assert r.append(kv.KVC_COMMIT) == kv.KVC_E_STATE  # double commit
    assert r.append(kv.KVC_STAGE) == kv.KVC_E_STATE   # evict first
    assert r.evict() == (kv.KVC_OK, -1)
    assert r.attn() == kv.KVC_E_STATE                 # no current chunk
    assert r.evict() == (kv.KVC_OK, -1)               # no-op in EMPTY
    assert r.info()["chunk"] == 1
    assert r.append(99) == kv.KVC_E_INVAL
    assert r.append(kv.KVC_STAGE, k=0) == kv.KVC_E_INVAL
    assert r.append(kv.KVC_STAGE, v=0x2008) == kv.KVC_E_INVAL   # misaligned
    assert r.append(kv.KVC_STAGE) == kv.KVC_OK
    assert r.attn(q=0) == kv.KVC_E_INVAL
    assert r.attn(q=0x3004) == kv.KVC_E_INVAL
    assert r.attn(q=0x3000, o=0x3000) == kv.KVC_E_INVAL
    assert r.attn(lse=0x5002) == kv.KVC_E_INVAL
    assert r.attn(lse=0x5004) == kv.KVC_OK
    r.close()
    r0 = FakeRing(lib, m=0)
    assert r0.append(kv.KVC_COND) == kv.KVC_E_INVAL   # no condition tokens configured
    r0.close()


def test_no_free_slot_without_evict(lib):
    # W = 1: 3 chunk slots.  Committing chunks without evicting runs out of
    # slots once the window is over-full.
    r = FakeRing(lib, W=1, m=0)
    for t in range(2):
        assert r.append(kv.KVC_COMMIT) == kv.KVC_OK
        assert r.evict()[0] == kv.KVC_OK
    assert r.append(kv.KVC_COMMIT) == kv.KVC_OK          # chunk 2: window {1, 2}
    assert r.info()["n_window"] == 2
    st, ev = r.evict()
    assert ev == 1
    assert r.info()["free_slots"] == 1
    r.close()


def test_failed_launch_leaves_state_unchanged(lib):
    r = FakeRing(lib, W=2, m=4)
    assert r.append(kv.KVC_COND) == kv.KVC_OK
    for t in range(4):
        before = (r.info(), r.segments() if r.info()["phase"] else None)
        lib.kvcfake_fail_next(kv.KVC_E_DEVICE)
        assert r.append(kv.KVC_STAGE) == kv.KVC_E_DEVICE
        assert (r.info(), r.segments() if r.info()["phase"] else None) == before
        assert r.append(kv.KVC_STAGE) == kv.KVC_OK
        segs = r.segments()
        lib.kvcfake_fail_next(kv.KVC_E_DEVICE)
        assert r.attn() == kv.KVC_E_DEVICE
        assert r.segments() == segs
        info = r.info()
        lib.kvcfake_fail_next(kv.KVC_E_DEVICE)
        assert r.append(kv.KVC_COMMIT) == kv.KVC_E_DEVICE
        assert r.info() == info
        lib.kvcfake_fail_next(kv.KVC_E_DEVICE)
        assert r.append(kv.KVC_COND) == kv.KVC_E_DEVICE
        assert r.append(kv.KVC_COMMIT) == kv.KVC_OK
        assert r.evict()[0] == kv.KVC_OK
    r.close()


def test_resume_by_commits_only(lib):
    # a ring is fully determined by cond, the sink and the last W clean chunks:
    # re-creating it by COND + COMMIT (no STAGE) gives the same segment table.
    W = 2
    r = FakeRing(lib, W=W, m=8)
    r.append(kv.KVC_COND)
    for t in range(7):
        assert r.append(kv.KVC_COMMIT) == kv.KVC_OK
        assert r.evict()[0] == kv.KVC_OK
    assert r.append(kv.KVC_STAGE) == kv.KVC_OK
    assert [s[0] for s in r.segments()] == [-1, 0, 5, 6, 7]
    r.close()


def test_segment_addresses_follow_layout(lib):
    H, d, n, m, W = 3, 64, 70, 20, 1
    r = FakeRing(lib, H=H, d=d, n=n, m=m, W=W)
    r.append(kv.KVC_COND)
    rec = r.last()
    P = lambda x: (x + 63) // 64 * 64
    al = lambda x: (x + 255) // 256 * 256
    assert rec.dst_k == BASE and rec.rows == m and rec.pitch == P(m)
    assert rec.dst_vt == BASE + al(H * P(m) * d * 2)
    cond_bytes = 2 * al(H * P(m) * d * 2)
    slot_bytes = 2 * al(H * P(n) * d * 2)
    r.append(kv.KVC_STAGE)
    rec = r.last()
    assert rec.dst_k == BASE + cond_bytes          # first free chunk slot
    assert rec.pitch == P(n)
    st, v = r.slot(-1)
    assert st == kv.KVC_OK and v.k == BASE and v.pitch == P(m) and v.elem_bytes == 2
    r.append(kv.KVC_COMMIT)
    r.evict()
    r.append(kv.KVC_STAGE)
    assert r.last().dst_k == BASE + cond_bytes + slot_bytes
    r.close()


def test_fp8_ring_records_scales(lib):
    r = FakeRing(lib, H=4, d=128, n=64, m=0, W=1, dtype=kv.KVC_KV_FP8_E4M3)
    r.append(kv.KVC_STAGE)
    rec = r.last()
    assert rec.kv_dtype == kv.KVC_KV_FP8_E4M3 and rec.k_scale != 0
    st, v = r.slot(-2)
    assert v.elem_bytes == 1 and v.k_scale == rec.k_scale and v.v_scale == rec.k_scale + 16
    r.close()


def test_attention_epochs(lib):
    # Every attention call gets a new nonzero epoch (the kernel tells its own
    # arrival words and partial tags in the workspace from stale ones by it);
    # only the first call asks for the workspace to be zeroed; a failed call
    # consumes no epoch.
    r = FakeRing(lib, W=1)
    assert r.append(kv.KVC_COND) == kv.KVC_OK
    assert r.append(kv.KVC_STAGE) == kv.KVC_OK
    epochs = []
    for i in range(3):
        assert r.attn() == kv.KVC_OK
        rec = r.last()
        assert rec.kind == 1
        epochs.append(rec.epoch)
        assert rec.ws_ready == (0 if i == 0 else 1)
    assert epochs == [1, 2, 3]
    lib.kvcfake_fail_next(kv.KVC_E_DEVICE)
    assert r.attn() == kv.KVC_E_DEVICE
    assert r.attn() == kv.KVC_OK
    assert r.last().epoch == 4
    r.close()


def test_noalloc_call_uses_the_static_scratch(lib):
    # chunk_attn_fwd_noalloc: the same launch as chunk_attn_fwd but with the
    # library's static array as workspace, epochs of its own (shared by every
    # ring on the device), zeroing asked for only on its first use; a call
    # needing more than the array holds is refused before any launch.
    lib.chunk_attn_fwd_noalloc.argtypes = [ctypes.c_void_p] * 5
    r = FakeRing(lib, W=1)
    assert r.append(kv.KVC_COND) == kv.KVC_OK
    assert r.append(kv.KVC_STAGE) == kv.KVC_OK
    assert r.attn() == kv.KVC_OK
    plain = r.last()
    args = (r.h, ctypes.c_void_p(0x3000), ctypes.c_void_p(0x4000), None, ctypes.c_void_p(0x77))
    epochs = []
    for _ in range(2):
        assert lib.chunk_attn_fwd_noalloc(*args) == kv.KVC_OK
        rec = r.last()
        assert rec.kind == 1 and rec.nseg == plain.nseg and rec.rows == plain.rows
        assert rec.dst_k != plain.dst_k          # not the ring's workspace
        epochs.append((rec.epoch, rec.ws_ready))
    assert epochs[1][0] == epochs[0][0] + 1 and epochs[1][1] == 1
    # the ring's own epochs are untouched
    assert r.attn() == kv.KVC_OK and r.last().epoch == plain.epoch + 1
    r.close()
    # 41 heads x ceil(25600 / 128) = 8200 rows > KVC_NOALLOC_MAX_ROWS
    big = FakeRing(lib, H=41, n=25600, m=0, W=0)
    assert big.append(kv.KVC_STAGE) == kv.KVC_OK
    n0 = lib.kvcfake_count()
    st = lib.chunk_attn_fwd_noalloc(big.h, ctypes.c_void_p(0x3000), ctypes.c_void_p(0x4000),
                                    None, None)
    assert st == kv.KVC_E_SCRATCH
    assert lib.kvcfake_count() == n0
    assert b"static scratch" in lib.kvc_status_str(kv.KVC_E_SCRATCH)
    big.close()


def test_c_e4m3_rule_matches_oracle(lib):
    rng = np.random.default_rng(0)
    pos = O3.decode_table()[:127]
    mids = (pos[1:] + pos[:-1]) / 2
    x = np.concatenate([
        rng.standard_normal(200000) * 100, rng.uniform(-500, 500, 200000),
        rng.standard_normal(100000) * 1e-3, pos, -pos, mids, -mids,
        np.nextafter(mids.astype(np.float32), np.float32(0)),
        np.nextafter(mids.astype(np.float32), np.float32(1e9)),
        [448, 449, 463.9, 464, 480, 1e30, -1e30, np.inf, -np.inf, 0.0, -0.0, np.nan,
         2.0 ** -10, 3 * 2.0 ** -10, 2.0 ** -7 * 0.999, 1e-45, -1e-45],
    ]).astype(np.float32)
    out = np.empty(x.size, np.uint8)
    lib.kvcfake_e4m3_encode(x.ctypes.data, out.ctypes.data, x.size)
    np.testing.assert_array_equal(out, O3.encode(x))


@pytest.mark.parametrize("W", [0, 2, 3])
@pytest.mark.parametrize("m,rr,s", [(40, 30, 70), (0, 30, 0), (0, 0, 70), (40, 0, 70)])
def test_token_groups(lib, W, m, rr, s):
    # reference tokens: one always-visible segment after cond; source tokens:
    # written from rows n.. of each STAGE/COMMIT into their own slot, attended
    # by (and queried with) the current chunk only, never published as history
    H, d, n = 2, 128, 100
    r = FakeRing(lib, H=H, d=d, n=n, m=m, W=W, r=rr, s=s)
    row_bytes = H * d * 2
    if m:
        assert r.append(kv.KVC_COND) == kv.KVC_OK
    if not rr:
        assert r.append(kv.KVC_REF) == kv.KVC_E_INVAL
    st, _ = r.slot(-3)
    assert st == kv.KVC_E_STATE
    for t in range(W + 4):
        before = r.count()
        assert r.append(kv.KVC_STAGE, k=0x10000, v=0x20000) == kv.KVC_OK
        writes = r.count() - before
        assert writes == (2 if s else 1)
        if s:
            w = r.last()
            assert (w.kind, w.rows, w.src_k, w.src_v) == \
                (0, s, 0x10000 + n * row_bytes, 0x20000 + n * row_bytes)
            st, view = r.slot(-4)
            assert st == kv.KVC_OK and view.rows == s and w.dst_k == view.k
        if rr and t == 0:
            assert r.attn() == kv.KVC_E_STATE        # reference configured, not written
            assert r.append(kv.KVC_REF) == kv.KVC_OK
            st, view = r.slot(-3)
            assert st == kv.KVC_OK and view.rows == rr
            assert r.last().rows == rr and r.last().dst_k == view.k
        assert r.attn() == kv.KVC_OK
        a = r.last()
        assert a.kind == 1 and a.rows == n + s
        segs = r.segments()
        roles = [x[3] for x in segs]
        want = ([0] if m else []) + ([4] if rr else []) + ([1] if t >= 1 else []) + \
            [2] * min(W, max(t - 1, 0)) + [3] + ([5] if s else [])
        assert roles == want
        assert [x[2] for x in segs] == [{0: m, 4: rr, 5: s}.get(x, n) for x in roles]
        assert a.nseg == len(segs)
        assert list(a.seg_rows[:a.nseg]) == [x[2] for x in segs]
        assert r.info()["kv_len"] == O1.kv_length(t, m, n, W, rr, s)
        before = r.count()
        assert r.append(kv.KVC_COMMIT, k=0x30000, v=0x40000) == kv.KVC_OK
        assert r.count() - before == (2 if s else 1)
        assert r.evict()[0] == kv.KVC_OK
        if s:
            st, _ = r.slot(-4)
            assert st == kv.KVC_E_STATE                # no current chunk
    # the history holds chunk tokens only: every committed slot has n rows
    for cid in range(W + 4):
        st, view = r.slot(cid)
        if st == kv.KVC_OK:
            assert view.rows == n
    r.close()


def test_rope_tables_follow_the_rows(lib):
    # the K rotation table of a STAGE/COMMIT covers n + s rows: the source
    # write gets the table from row n on (n * d floats further); the
    # attention record carries q's table; misaligned tables and a rows map
    # without a count are rejected
    H, d, n, s = 2, 128, 100, 30
    r = FakeRing(lib, H=H, d=d, n=n, m=8, W=1, s=s)
    P = ctypes.c_void_p
    tab = 0x900000
    assert lib.kvc_append_chunk_rope(r.h, kv.KVC_COND, P(0x1000), P(0x2000), P(tab), P(0)) == 0
    assert r.last().rope == tab
    before = r.count()
    assert lib.kvc_append_chunk_rope(r.h, kv.KVC_STAGE, P(0x1000), P(0x2000), P(tab), P(0)) == 0
    assert r.count() - before == 2
    w0 = Record()
    lib.kvcfake_get(before, ctypes.byref(w0))
    assert w0.rope == tab and w0.rows == n
    assert r.last().rope == tab + n * d * 4 and r.last().rows == s
    assert lib.kvc_append_chunk_rope(r.h, kv.KVC_STAGE, P(0x1000), P(0x2000), P(tab + 4),
                                     P(0)) == kv.KVC_E_INVAL
    assert lib.kvc_append_chunk(r.h, kv.KVC_STAGE, P(0x1000), P(0x2000), P(0)) == 0
    assert r.last().rope == 0
    assert lib.chunk_attn_fwd_rope(r.h, P(0x3000), P(0x4000), None, P(tab), None, None,
                                   P(0)) == 0
    a = r.last()
    assert a.kind == 1 and a.rope == tab and a.qrows == 0 and a.rows == n + s
    assert lib.chunk_attn_fwd_rope(r.h, P(0x3000), P(0x4000), None, P(tab), P(0x5000), None,
                                   P(0)) == kv.KVC_E_INVAL
    assert lib.chunk_attn_fwd_rope(r.h, P(0x3000), P(0x4000), None, P(tab + 8), None, None,
                                   P(0)) == kv.KVC_E_INVAL
    assert lib.chunk_attn_fwd_rope(r.h, P(0x3000), P(0x4000), None, None, P(0x5000), P(0x6000),
                                   P(0)) == 0
    a = r.last()
    assert (a.rope, a.qrows, a.qcount) == (0, 0x5000, 0x6000)
    r.close()


def test_edit_mask_arguments(lib):
    P = ctypes.c_void_p
    ok = (P(0x1000), P(0x2000), 100, 16, ctypes.c_float(1.0), -1, P(0x3000), P(0x4000), P(0))
    lib.kvcfake_reset()
    assert lib.kvc_edit_mask(*ok) == 0
    r = Record()
    lib.kvcfake_get(0, ctypes.byref(r))
    assert (r.kind, r.rows, r.pitch, r.nseg, r.dst_k, r.dst_vt) == (2, 100, 16, -1, 0x3000, 0x4000)
    bad = [
        (P(0), P(0x2000), 100, 16, ctypes.c_float(1.0), -1, P(0x3000), P(0x4000), P(0)),
        (P(0x1000), P(0x2000), 0, 16, ctypes.c_float(1.0), -1, P(0x3000), P(0x4000), P(0)),
        (P(0x1000), P(0x2000), kv.KVC_MAX_MASK_TOKENS + 1, 16, ctypes.c_float(1.0), 3,
         P(0x3000), P(0x4000), P(0)),
        (P(0x1000), P(0x2000), 100, kv.KVC_MAX_MASK_CHANNELS + 1, ctypes.c_float(1.0), 3,
         P(0x3000), P(0x4000), P(0)),
        (P(0x1000), P(0x2000), 100, 16, ctypes.c_float(-1.0), -1, P(0x3000), P(0x4000), P(0)),
        (P(0x1000), P(0x2000), 100, 16, ctypes.c_float(float("nan")), -1, P(0x3000),
         P(0x4000), P(0)),
        (P(0x1000), P(0x2000), 100, 16, ctypes.c_float(1.0), -1, P(0x3002), P(0x4000), P(0)),
        (P(0x1001), P(0x2000), 100, 16, ctypes.c_float(1.0), -1, P(0x3000), P(0x4000), P(0)),
    ]
    for b in bad:
        assert lib.kvc_edit_mask(*b) == kv.KVC_E_INVAL
    # a negative tau is fine in top-k mode (ignored)
    assert lib.kvc_edit_mask(P(0x1000), P(0x2000), 100, 16, ctypes.c_float(-1.0), 5, P(0x3000),
                             P(0x4000), P(0)) == 0
    assert lib.kvcfake_count() == 2
