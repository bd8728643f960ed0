"""The C-ABI library loads, exports every declared symbol, and rejects bad
arguments on the host before touching a GPU (CPU only: no compute calls)."""
from __future__ import annotations

import ctypes
import os
import re
import subprocess

import pytest

from mxfp4_routed_expert_route_amd import build as build_mod

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADERS = [os.path.join(ROOT, "include", h) for h in ("moe_mxfp4.h", "moe_mxfp4_profiling.h")]

OK, INVALID, UNSUPPORTED, MISALIGNED, WS_SMALL = 0, 1, 2, 3, 4


def declared_functions():
    text = "".join(open(h).read() for h in HEADERS)
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(moe_[a-z_0-9]+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(build_mod.LIB):
        build_mod.build_library()
    return ctypes.CDLL(build_mod.LIB)


def test_header_declares_the_five_calls():
    names = declared_functions()
    for n in ("moe_route", "moe_build_bitmatrix", "moe_expert_offsets", "moe_route_and_group",
              "moe_grouped_ffn_mxfp4", "moe_combine", "moe_workspace_bytes", "moe_status_string",
              "moe_grouped_ffn_mxfp4_timed", "moe_forward_mxfp4", "moe_forward_mxfp4_timed",
              "moe_read_probe"):
        assert n in names


def test_library_exports_every_declared_symbol(lib):
    out = subprocess.run(["nm", "-D", "--defined-only", build_mod.LIB], capture_output=True,
                         text=True, check=True).stdout
    exported = set(re.findall(r"\sT\s+(\S+)", out))
    missing = [n for n in declared_functions() if n not in exported]
    assert not missing, missing
    for n in declared_functions():
        getattr(lib, n)


def test_host_validation_driver():
    exe = build_mod.build_validate_check()
    r = subprocess.run([exe], capture_output=True, text=True)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "validate_check ok" in r.stdout


def test_error_codes_through_the_abi(lib):
    P, I64, I32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32
    lib.moe_route.argtypes = [P, I64, I32, I32, P, P, P]
    lib.moe_build_bitmatrix.argtypes = [P, I64, I32, I32, P, P]
    lib.moe_combine.argtypes = [P, P, P, I64, I32, I32, P, P]
    lib.moe_workspace_bytes.argtypes = [I64, I32, I32, I32, I32]
    lib.moe_workspace_bytes.restype = ctypes.c_size_t
    lib.moe_status_string.argtypes = [ctypes.c_int]
    lib.moe_status_string.restype = ctypes.c_char_p
    assert lib.moe_route(None, 16, 256, 6, None, None, None) == INVALID
    assert lib.moe_route(None, 0, 256, 6, None, None, None) == OK          # T = 0: nothing enqueued
    assert lib.moe_route(None, 16, 256, 9, None, None, None) == UNSUPPORTED
    assert lib.moe_route(None, 16, 2000, 6, None, None, None) == UNSUPPORTED
    assert lib.moe_route(None, -1, 256, 6, None, None, None) == INVALID
    assert lib.moe_route(1, 16, 256, 6, 8, 8, None) == MISALIGNED
    assert lib.moe_build_bitmatrix(None, 16, 256, 7, None, None) == INVALID
    assert lib.moe_combine(None, None, None, 0, 4096, 6, None, None) == OK
    assert lib.moe_combine(None, None, None, 4, 4100, 6, None, None) == UNSUPPORTED
    assert lib.moe_workspace_bytes(8191, 256, 6, 4096, 2048) >= 49146 * 2048 * 2
    assert lib.moe_workspace_bytes(-1, 256, 6, 4096, 2048) == 0
    assert lib.moe_status_string(WS_SMALL) == b"MOE_ERR_WORKSPACE_TOO_SMALL"
    lib.moe_read_probe.argtypes = [P, ctypes.c_size_t, P, P]
    assert lib.moe_read_probe(None, 0, 256, None) == OK        # nothing to read: nothing enqueued
    assert lib.moe_read_probe(256, 1 << 20, None, None) == INVALID   # no sink
    assert lib.moe_read_probe(None, 1 << 20, 256, None) == INVALID   # no buffer
    assert lib.moe_read_probe(256, 1000, 256, None) == MISALIGNED    # not a multiple of 16
    assert lib.moe_read_probe(264, 1 << 20, 256, None) == MISALIGNED  # buffer not 16-B aligned
    lib.moe_forward_mxfp4.argtypes = [P, P, I64, I32, I32, I32, I32, P, P, P, P, ctypes.c_float] + \
        [P] * 10 + [ctypes.c_size_t, P]
    fwd = lambda T, H, I, E, k, ptrs, ws_bytes: lib.moe_forward_mxfp4(
        *ptrs[:2], T, H, I, E, k, *ptrs[2:6], 10.0, *ptrs[6:16], ws_bytes, None)
    nulls = [None] * 16   # logits, x, 4 weight buffers, 9 outputs, workspace
    assert fwd(16, 4096, 2048, 256, 6, nulls, 0) == INVALID          # null pointers
    assert fwd(16, 4100, 2048, 256, 6, nulls, 0) == INVALID          # nulls are checked first
    assert fwd(-1, 4096, 2048, 256, 6, nulls, 0) == INVALID
    assert fwd(16, 4096, 2048, 256, 9, nulls, 0) == UNSUPPORTED      # k > 8
    big = [4096] * 16
    assert fwd(1, 65536, 65536, 4, 1, big, 1 << 40) == UNSUPPORTED   # a 4 GiB W1 slab per expert
    assert fwd(1, 65536, 65536 - 128, 4, 1, big, 0) == WS_SMALL      # just below: size checks pass
    # the timed one-call layer: the same checks, then its three events
    lib.moe_forward_mxfp4_timed.argtypes = lib.moe_forward_mxfp4.argtypes[:-1] + [P, P]
    ws = lib.moe_workspace_bytes(16, 256, 6, 4096, 2048)
    fake = [4096] * 16   # aligned stand-in device pointers: never dereferenced by the checks
    timed = lambda T, ptrs, ws_bytes, ev: lib.moe_forward_mxfp4_timed(
        *ptrs[:2], T, 4096, 2048, 256, 6, *ptrs[2:6], 10.0, *ptrs[6:16], ws_bytes, ev, None)
    no_events = (ctypes.c_void_p * 3)(None, None, None)
    assert timed(16, nulls, 0, None) == INVALID                       # null pointers first
    assert timed(16, fake, ws - 1, None) == WS_SMALL
    assert timed(16, fake, ws, None) == INVALID                       # no event array
    assert timed(16, fake, ws, no_events) == INVALID                  # null events


def test_noalloc_entry_point_host_checks(lib):
    # moe_forward_mxfp4_noalloc runs every host check before any HIP call: invalid
    # arguments and sizes beyond its static scratch return without touching a GPU
    P, I64, I32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32
    lib.moe_forward_mxfp4_noalloc.argtypes = [P, P, I64, I32, I32, I32, I32, P, P, P, P,
                                              ctypes.c_float] + [P] * 10
    lib.moe_workspace_bytes.argtypes = [I64, I32, I32, I32, I32]
    lib.moe_workspace_bytes.restype = ctypes.c_size_t
    fwd = lambda T, H, I, E, k, ptrs: lib.moe_forward_mxfp4_noalloc(
        *ptrs[:2], T, H, I, E, k, *ptrs[2:6], 10.0, *ptrs[6:15], None)
    scratch = 128 << 20   # MOE_NOALLOC_SCRATCH_BYTES
    fake = [4096] * 15   # aligned stand-in device pointers: never dereferenced by the checks
    assert fwd(16, 4096, 2048, 256, 6, [None] * 15) == INVALID
    assert fwd(16, 4096, 2048, 256, 9, fake) == UNSUPPORTED
    assert fwd(16, 4100, 2048, 256, 6, fake) == UNSUPPORTED
    assert lib.moe_workspace_bytes(4032, 256, 6, 4096, 2048) <= scratch
    assert lib.moe_workspace_bytes(4033, 256, 6, 4096, 2048) > scratch
    assert fwd(4033, 4096, 2048, 256, 6, fake) == WS_SMALL
    assert fwd(8191, 4096, 2048, 256, 6, fake) == WS_SMALL
    header = open(HEADERS[0]).read()
    assert re.search(r"#define MOE_NOALLOC_SCRATCH_BYTES \(\(size_t\)128 << 20\)", header)
