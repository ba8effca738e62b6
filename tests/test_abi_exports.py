"""The built HIP library loads on a host without a GPU and exports every
function include/kvc.h declares; host-only entry points work without a
device."""
import ctypes
import os
import re

import pytest

import chunked_attention_amd as kv

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def declared_functions():
    src = open(os.path.join(ROOT, "include", "kvc.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    names = re.findall(r"^\s*(?:const\s+)?[A-Za-z_][\w\s\*]*?\b(\w+)\s*\(", src, flags=re.M)
    return sorted(set(n for n in names if n.startswith(("kvc_", "chunk_"))))


def test_header_declares_the_boundary():
    names = declared_functions()
    for n in ("kvc_create", "kvc_append_chunk", "chunk_attn_fwd", "kvc_evict"):
        assert n in names
    assert set(names) == set(kv.EXPORTS)


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(kv.LIB_PATH):
        from chunked_attention_amd import build
        build.build()
    return kv.lib()


def test_library_exports_every_declared_symbol(lib):
    for name in declared_functions():
        assert hasattr(lib, name), name


def test_library_has_gfx950_code_object():
    data = open(kv.LIB_PATH, "rb").read()
    assert b"gfx950" in data


def test_host_only_calls_without_device(lib):
    cfg = kv.make_config(40, 128, 1620, 256, 3)
    need = lib.kvc_required_bytes(ctypes.byref(cfg))
    assert need == 2 * 40 * 128 * 2 * (256 + 5 * 1664) + 4352 + 4096 + 1048576 + 67108864
    h = ctypes.c_void_p()
    base = 0x7F0000000000
    assert lib.kvc_create(ctypes.byref(cfg), ctypes.c_void_p(base), need,
                          ctypes.byref(h)) == kv.KVC_OK
    info = kv.kvc_info()
    assert lib.kvc_get_info(h, ctypes.byref(info)) == kv.KVC_OK
    assert info.phase == kv.KVC_PHASE_EMPTY and info.free_slots == 5
    ev = ctypes.c_int32()
    assert lib.kvc_evict(h, ctypes.byref(ev)) == kv.KVC_OK and ev.value == -1
    assert lib.chunk_attn_fwd(h, ctypes.c_void_p(0x1000), ctypes.c_void_p(0x2000), None,
                              None) == kv.KVC_E_STATE
    assert b"KVC_E_STATE" in lib.kvc_status_str(kv.KVC_E_STATE)
    assert lib.kvc_destroy(h) == kv.KVC_OK
