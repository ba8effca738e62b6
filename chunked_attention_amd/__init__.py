"""Python binding of libkvc.so: chunk-causal sink+window attention over a
bounded KV cache on MI355X (gfx950).

Argument marshalling only.  Every step of the path (cache writes, attention)
runs in the library's HIP kernels; PyTorch supplies device memory and
streams.  There is no fallback: if libkvc.so is missing or fails to load,
importing the library raises.

The C entry points keep their names here (``kvc_create``,
``kvc_append_chunk``, ``chunk_attn_fwd``, ``kvc_evict``, ...), taking torch
tensors where the C ABI takes device pointers.  :class:`Ring` wraps one ring
with its device buffer.
"""
from __future__ import annotations

import ctypes
import os

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libkvc.so")

KVC_OK = 0
KVC_E_INVAL = -1
KVC_E_STATE = -2
KVC_E_NOMEM = -3
KVC_E_DEVICE = -4
KVC_E_UNSUPPORTED = -5
KVC_E_SCRATCH = -6
KVC_NOALLOC_MAX_ROWS = 8192
KVC_NOALLOC_SCRATCH_BYTES = 65536 + 4096 + 1048576 + 67108864

KVC_KV_BF16 = 0
KVC_KV_FP8_E4M3 = 1
KVC_COND = 0
KVC_STAGE = 1
KVC_COMMIT = 2
KVC_REF = 3
KVC_PHASE_EMPTY = 0
KVC_PHASE_STAGED = 1
KVC_PHASE_COMMITTED = 2
KVC_MAX_WINDOW = 29
KVC_MAX_SEGMENTS = KVC_MAX_WINDOW + 5
KVC_TILE_KEYS = 64
KVC_ALIGN = 256
KVC_MAX_MASK_TOKENS = 16384
KVC_MAX_MASK_CHANNELS = 4096

_DTYPES = {"bf16": KVC_KV_BF16, "fp8_e4m3": KVC_KV_FP8_E4M3}


class kvc_config(ctypes.Structure):
    _fields_ = [("heads", ctypes.c_int32), ("head_dim", ctypes.c_int32),
                ("chunk_tokens", ctypes.c_int32), ("cond_tokens", ctypes.c_int32),
                ("window", ctypes.c_int32), ("kv_dtype", ctypes.c_int32),
                ("softmax_scale", ctypes.c_float), ("ref_tokens", ctypes.c_int32),
                ("source_tokens", ctypes.c_int32)]


class kvc_info(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in (
        "chunk", "phase", "cond_valid", "sink_valid", "n_window", "kv_len", "n_segments",
        "free_slots", "ref_valid")]


class kvc_segment(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in ("chunk", "slot", "rows", "role")]


class kvc_slot_view(ctypes.Structure):
    _fields_ = [("k", ctypes.c_void_p), ("vt", ctypes.c_void_p),
                ("k_scale", ctypes.c_void_p), ("v_scale", ctypes.c_void_p),
                ("rows", ctypes.c_int32), ("pitch", ctypes.c_int32),
                ("elem_bytes", ctypes.c_int32), ("reserved", ctypes.c_int32)]


EXPORTS = (
    "kvc_required_bytes", "kvc_create", "kvc_append_chunk", "chunk_attn_fwd", "kvc_evict",
    "kvc_destroy", "kvc_status_str", "kvc_get_info", "kvc_get_segments", "kvc_get_slot",
    "chunk_attn_fwd_rows", "kvc_edit_mask", "kvc_append_chunk_rope", "chunk_attn_fwd_rope",
    "chunk_attn_fwd_noalloc",
)


def declare(lib: ctypes.CDLL) -> ctypes.CDLL:
    """Attach C signatures (kvc.h) to a loaded library."""
    P = ctypes.c_void_p
    I = ctypes.c_int32
    lib.kvc_required_bytes.argtypes = [ctypes.POINTER(kvc_config)]
    lib.kvc_required_bytes.restype = ctypes.c_size_t
    lib.kvc_create.argtypes = [ctypes.POINTER(kvc_config), P, ctypes.c_size_t,
                               ctypes.POINTER(P)]
    lib.kvc_create.restype = I
    lib.kvc_append_chunk.argtypes = [P, I, P, P, P]
    lib.kvc_append_chunk.restype = I
    lib.chunk_attn_fwd.argtypes = [P, P, P, P, P]
    lib.chunk_attn_fwd.restype = I
    lib.chunk_attn_fwd_noalloc.argtypes = [P, P, P, P, P]
    lib.chunk_attn_fwd_noalloc.restype = I
    lib.chunk_attn_fwd_rows.argtypes = [P, P, P, P, P, P, P]
    lib.chunk_attn_fwd_rows.restype = I
    lib.kvc_edit_mask.argtypes = [P, P, I, I, ctypes.c_float, I, P, P, P]
    lib.kvc_edit_mask.restype = I
    lib.kvc_append_chunk_rope.argtypes = [P, I, P, P, P, P]
    lib.kvc_append_chunk_rope.restype = I
    lib.chunk_attn_fwd_rope.argtypes = [P, P, P, P, P, P, P, P]
    lib.chunk_attn_fwd_rope.restype = I
    lib.kvc_evict.argtypes = [P, ctypes.POINTER(I)]
    lib.kvc_evict.restype = I
    lib.kvc_destroy.argtypes = [P]
    lib.kvc_destroy.restype = I
    lib.kvc_status_str.argtypes = [I]
    lib.kvc_status_str.restype = ctypes.c_char_p
    lib.kvc_get_info.argtypes = [P, ctypes.POINTER(kvc_info)]
    lib.kvc_get_info.restype = I
    lib.kvc_get_segments.argtypes = [P, ctypes.POINTER(kvc_segment), I, ctypes.POINTER(I)]
    lib.kvc_get_segments.restype = I
    lib.kvc_get_slot.argtypes = [P, I, ctypes.POINTER(kvc_slot_view)]
    lib.kvc_get_slot.restype = I
    return lib


_lib: ctypes.CDLL | None = None


def lib() -> ctypes.CDLL:
    """The loaded libkvc.so (raises if it is not built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"{LIB_PATH} is not built; run `python -m chunked_attention_amd.build` "
                "(there is no fallback path)")
        _lib = declare(ctypes.CDLL(LIB_PATH))
    return _lib


class KvcError(RuntimeError):
    def __init__(self, status: int, what: str):
        self.status = status
        super().__init__(f"{what}: {status_str(status)}")


def status_str(status: int) -> str:
    return lib().kvc_status_str(status).decode()


def _check(status: int, what: str) -> None:
    if status != KVC_OK:
        raise KvcError(status, what)


def _stream_handle(stream) -> ctypes.c_void_p:
    import torch
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def make_config(heads: int, head_dim: int, chunk_tokens: int, cond_tokens: int, window: int,
                kv_dtype: str = "bf16", softmax_scale: float = 0.0, ref_tokens: int = 0,
                source_tokens: int = 0) -> kvc_config:
    return kvc_config(heads, head_dim, chunk_tokens, cond_tokens, window, _DTYPES[kv_dtype],
                      softmax_scale, ref_tokens, source_tokens)


def query_rows(cfg: kvc_config) -> int:
    """Rows of q / o / lse of an attention call: the chunk's own tokens
    followed by its source tokens."""
    return cfg.chunk_tokens + cfg.source_tokens


# ---- the C entry points, over torch tensors --------------------------------

def kvc_required_bytes(cfg: kvc_config) -> int:
    return lib().kvc_required_bytes(ctypes.byref(cfg))


def kvc_create(cfg: kvc_config, dev_buf) -> ctypes.c_void_p:
    handle = ctypes.c_void_p()
    _check(lib().kvc_create(ctypes.byref(cfg), ctypes.c_void_p(dev_buf.data_ptr()),
                            dev_buf.numel() * dev_buf.element_size(), ctypes.byref(handle)),
           "kvc_create")
    return handle


def _check_tokens(x, rows: int, cfg: kvc_config, what: str) -> None:
    import torch
    if x.dtype != torch.bfloat16 or not x.is_cuda or not x.is_contiguous():
        raise ValueError(f"{what} must be a contiguous bf16 CUDA tensor")
    if tuple(x.shape) != (rows, cfg.heads, cfg.head_dim):
        raise ValueError(f"{what} has shape {tuple(x.shape)}, expected "
                         f"{(rows, cfg.heads, cfg.head_dim)}")


def _check_rope(rope, rows: int, cfg: kvc_config) -> ctypes.c_void_p:
    import torch
    if rope is None:
        return ctypes.c_void_p(None)
    if rope.dtype != torch.float32 or not rope.is_cuda or not rope.is_contiguous() or \
            tuple(rope.shape) != (rows, cfg.head_dim // 2, 2):
        raise ValueError(f"rope must be a contiguous float32 CUDA tensor "
                         f"[{rows}, {cfg.head_dim // 2}, 2]")
    return ctypes.c_void_p(rope.data_ptr())


def kvc_append_chunk(handle, cfg: kvc_config, kind: int, k, v, stream=None, rope=None) -> None:
    """Cache write; with `rope` (float32 [rows, d/2, 2] of (cos, sin)) the
    keys are stored rotated (kvc_append_chunk_rope)."""
    rows = {KVC_COND: cfg.cond_tokens, KVC_REF: cfg.ref_tokens}.get(kind, query_rows(cfg))
    _check_tokens(k, rows, cfg, "k")
    _check_tokens(v, rows, cfg, "v")
    if rope is None:
        st = lib().kvc_append_chunk(handle, kind, ctypes.c_void_p(k.data_ptr()),
                                    ctypes.c_void_p(v.data_ptr()), _stream_handle(stream))
    else:
        st = lib().kvc_append_chunk_rope(handle, kind, ctypes.c_void_p(k.data_ptr()),
                                         ctypes.c_void_p(v.data_ptr()),
                                         _check_rope(rope, rows, cfg), _stream_handle(stream))
    _check(st, "kvc_append_chunk")


def _attn_args(cfg: kvc_config, q, o, lse):
    import torch
    nq = query_rows(cfg)
    _check_tokens(q, nq, cfg, "q")
    _check_tokens(o, nq, cfg, "o")
    if o.device != q.device:
        raise ValueError("q and o must be on the same device")
    lse_ptr = None
    if lse is not None:
        if lse.dtype != torch.float32 or not lse.is_cuda or not lse.is_contiguous() or \
                tuple(lse.shape) != (cfg.heads, nq):
            raise ValueError("lse must be a contiguous float32 CUDA tensor [heads, "
                             "chunk_tokens + source_tokens]")
        if lse.device != q.device:
            raise ValueError("lse must be on q's device")
        lse_ptr = lse.data_ptr()
    return ctypes.c_void_p(q.data_ptr()), ctypes.c_void_p(o.data_ptr()), ctypes.c_void_p(lse_ptr)


def _check_i32(x, what: str, numel: int | None = None) -> None:
    import torch
    if x.dtype != torch.int32 or not x.is_cuda or not x.is_contiguous():
        raise ValueError(f"{what} must be a contiguous int32 CUDA tensor")
    if numel is not None and x.numel() < numel:
        raise ValueError(f"{what} needs at least {numel} elements")


def chunk_attn_fwd(handle, cfg: kvc_config, q, o, lse=None, stream=None) -> None:
    _check(lib().chunk_attn_fwd(handle, *_attn_args(cfg, q, o, lse), _stream_handle(stream)),
           "chunk_attn_fwd")


def chunk_attn_fwd_noalloc(handle, cfg: kvc_config, q, o, lse=None, stream=None) -> None:
    """chunk_attn_fwd with the split-row scratch in the library's static
    device array (no allocation; calls on one device must not overlap)."""
    _check(lib().chunk_attn_fwd_noalloc(handle, *_attn_args(cfg, q, o, lse),
                                        _stream_handle(stream)), "chunk_attn_fwd_noalloc")


def chunk_attn_fwd_rows(handle, cfg: kvc_config, q, o, rows, count, lse=None,
                        stream=None) -> None:
    """Attention of rows[:count] of q only; the other rows of o (and lse) are
    left as they are.  rows/count are device int32 tensors (count: 1 element)."""
    _check_i32(rows, "rows", query_rows(cfg))
    _check_i32(count, "count", 1)
    _check(lib().chunk_attn_fwd_rows(handle, *_attn_args(cfg, q, o, lse),
                                     ctypes.c_void_p(rows.data_ptr()),
                                     ctypes.c_void_p(count.data_ptr()),
                                     _stream_handle(stream)), "chunk_attn_fwd_rows")


def chunk_attn_fwd_rope(handle, cfg: kvc_config, q, o, rope, lse=None, rows=None, count=None,
                        stream=None) -> None:
    """Attention with q rotated by `rope` (float32 [n+s, d/2, 2]) as it is
    loaded; rows/count optionally select active rows."""
    if (rows is None) != (count is None):
        raise ValueError("give both rows and count, or neither")
    rp = rc = ctypes.c_void_p(None)
    if rows is not None:
        _check_i32(rows, "rows", query_rows(cfg))
        _check_i32(count, "count", 1)
        rp, rc = ctypes.c_void_p(rows.data_ptr()), ctypes.c_void_p(count.data_ptr())
    _check(lib().chunk_attn_fwd_rope(handle, *_attn_args(cfg, q, o, lse),
                                     _check_rope(rope, query_rows(cfg), cfg), rp, rc,
                                     _stream_handle(stream)), "chunk_attn_fwd_rope")


def kvc_edit_mask(z_src, z_edit, tau: float | None = None, keep: int | None = None, rows=None,
                  count=None, stream=None):
    """LiveEdit's active rows: (rows [tokens] int32, count [1] int32), device
    tensors.  Give tau (threshold mode) or keep (top-k mode)."""
    import torch
    if (tau is None) == (keep is None):
        raise ValueError("give exactly one of tau and keep")
    for z, what in ((z_src, "z_src"), (z_edit, "z_edit")):
        if z.dtype != torch.bfloat16 or not z.is_cuda or not z.is_contiguous() or z.dim() != 2:
            raise ValueError(f"{what} must be a contiguous 2-d bf16 CUDA tensor")
    if z_src.shape != z_edit.shape:
        raise ValueError("z_src and z_edit differ in shape")
    tokens, channels = z_src.shape
    if rows is None:
        rows = torch.empty(tokens, dtype=torch.int32, device=z_src.device)
    if count is None:
        count = torch.empty(1, dtype=torch.int32, device=z_src.device)
    _check_i32(rows, "rows", tokens)
    _check_i32(count, "count", 1)
    _check(lib().kvc_edit_mask(ctypes.c_void_p(z_src.data_ptr()),
                               ctypes.c_void_p(z_edit.data_ptr()), tokens, channels,
                               0.0 if tau is None else float(tau),
                               -1 if keep is None else int(keep),
                               ctypes.c_void_p(rows.data_ptr()),
                               ctypes.c_void_p(count.data_ptr()), _stream_handle(stream)),
           "kvc_edit_mask")
    return rows, count


def kvc_evict(handle) -> int:
    ev = ctypes.c_int32(-1)
    _check(lib().kvc_evict(handle, ctypes.byref(ev)), "kvc_evict")
    return ev.value


def kvc_destroy(handle) -> None:
    lib().kvc_destroy(handle)


def kvc_get_info(handle) -> kvc_info:
    info = kvc_info()
    _check(lib().kvc_get_info(handle, ctypes.byref(info)), "kvc_get_info")
    return info


def kvc_get_segments(handle) -> list[tuple[int, int, int, int]]:
    buf = (kvc_segment * KVC_MAX_SEGMENTS)()
    count = ctypes.c_int32()
    _check(lib().kvc_get_segments(handle, buf, KVC_MAX_SEGMENTS, ctypes.byref(count)),
           "kvc_get_segments")
    return [(s.chunk, s.slot, s.rows, s.role) for s in buf[:count.value]]


def kvc_get_slot(handle, which: int) -> kvc_slot_view:
    view = kvc_slot_view()
    _check(lib().kvc_get_slot(handle, which, ctypes.byref(view)), "kvc_get_slot")
    return view


class Ring:
    """One KV ring (one layer) in a torch-allocated device buffer."""

    def __init__(self, heads: int, head_dim: int, chunk_tokens: int, cond_tokens: int,
                 window: int, kv_dtype: str = "bf16", softmax_scale: float = 0.0,
                 device="cuda", ref_tokens: int = 0, source_tokens: int = 0):
        import torch
        self.cfg = make_config(heads, head_dim, chunk_tokens, cond_tokens, window, kv_dtype,
                               softmax_scale, ref_tokens, source_tokens)
        nbytes = kvc_required_bytes(self.cfg)
        if nbytes == 0:
            raise KvcError(KVC_E_INVAL, "kvc_required_bytes")
        self.buf = torch.empty(nbytes, dtype=torch.uint8, device=device)
        self.handle = kvc_create(self.cfg, self.buf)

    def close(self) -> None:
        if self.handle is not None:
            kvc_destroy(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def cond(self, k, v, stream=None, rope=None) -> None:
        kvc_append_chunk(self.handle, self.cfg, KVC_COND, k, v, stream, rope)

    def ref(self, k, v, stream=None, rope=None) -> None:
        kvc_append_chunk(self.handle, self.cfg, KVC_REF, k, v, stream, rope)

    def stage(self, k, v, stream=None, rope=None) -> None:
        kvc_append_chunk(self.handle, self.cfg, KVC_STAGE, k, v, stream, rope)

    def commit(self, k, v, stream=None, rope=None) -> None:
        kvc_append_chunk(self.handle, self.cfg, KVC_COMMIT, k, v, stream, rope)

    def attention(self, q, out=None, lse=None, stream=None, rope=None):
        import torch
        if out is None:
            out = torch.empty_like(q)
        if rope is None:
            chunk_attn_fwd(self.handle, self.cfg, q, out, lse, stream)
        else:
            chunk_attn_fwd_rope(self.handle, self.cfg, q, out, rope, lse, stream=stream)
        return out

    def attention_rows(self, q, rows, count, out, lse=None, stream=None, rope=None):
        """Active-row attention: only rows[:count] of `out` are written."""
        if rope is None:
            chunk_attn_fwd_rows(self.handle, self.cfg, q, out, rows, count, lse, stream)
        else:
            chunk_attn_fwd_rope(self.handle, self.cfg, q, out, rope, lse, rows, count, stream)
        return out

    def evict(self) -> int:
        return kvc_evict(self.handle)

    def info(self) -> kvc_info:
        return kvc_get_info(self.handle)

    def segments(self):
        return kvc_get_segments(self.handle)

    def slot_tensors(self, which: int):
        """Views of a stored slot: K [H][pitch][d], Vt [H][pitch/T][d][T]
        (tiles of T = 32 keys for bf16, 64 for fp8; bf16 values or uint8
        codes) and, for fp8 rings, the float32 scales [H] of K and V."""
        import torch
        v = kvc_get_slot(self.handle, which)
        base = self.buf.data_ptr()
        H, d = self.cfg.heads, self.cfg.head_dim
        n = H * v.pitch * d * v.elem_bytes

        def part(ptr, nbytes):
            return self.buf[ptr - base: ptr - base + nbytes]
        dt = torch.bfloat16 if v.elem_bytes == 2 else torch.uint8
        k = part(v.k, n).view(dt).view(H, v.pitch, d)
        T = 32 if v.elem_bytes == 2 else 64
        vt = part(v.vt, n).view(dt).view(H, v.pitch // T, d, T)
        if v.k_scale:
            ks = part(v.k_scale, 4 * H).view(torch.float32)
            vs = part(v.v_scale, 4 * H).view(torch.float32)
            return k, vt, ks, vs, v.rows
        return k, vt, None, None, v.rows
