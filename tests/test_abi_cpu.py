"""The C-ABI library on the CPU: it loads, exports every symbol the header
declares, and every validation error is returned before any HIP call (the
pointers below are never dereferenced; nothing is launched)."""

import ctypes
import os
import re

import pytest

from deltanet_delta_rule_chunk_amd import binding

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "deltanet.h")

OK, NULL, SHAPE, UNSUP, ALIGN, ALIAS, WS, HIP = range(8)
F32, BF16 = 0, 1


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(binding.LIB_PATH):
        pytest.fail("libdeltanet.so not built (run python -m deltanet_delta_rule_chunk_amd.build)")
    return binding.load()


def test_header_declarations_are_exported(lib):
    text = open(HEADER).read()
    declared = set(re.findall(r"^\s*(?:int|size_t|const char\*)\s+(deltanet_\w+)\s*\(", text, re.M))
    assert declared == set(binding.EXPORTS)
    for name in declared:
        assert hasattr(lib, name), name


def test_version_and_status_strings(lib):
    assert lib.deltanet_version() == 200
    for s in range(8):
        assert lib.deltanet_status_string(s)
    assert lib.deltanet_status_string(99) == b"unknown status"
    assert lib.deltanet_last_hip_error() == 0


BASE = 1 << 40  # fake, 16-byte-aligned device addresses, never dereferenced
MB = 1 << 20


def _fwd(lib, q=BASE, k=BASE + 100 * MB, v=BASE + 200 * MB, beta=BASE + 300 * MB, S0=None,
         o=BASE + 400 * MB, Sf=BASE + 500 * MB, B=1, H=2, L=256, dk=64, dv=64, C=64,
         it=BF16, ot=F32, ws=BASE + 600 * MB, ws_bytes=1 << 40):
    return lib.deltanet_chunk_fwd(q, k, v, beta, S0, o, Sf, B, H, L, dk, dv, C, it, ot, ws,
                                  ws_bytes, None)


def test_chunk_fwd_validation(lib):
    assert _fwd(lib, q=None) == NULL
    assert _fwd(lib, beta=None) == NULL
    assert _fwd(lib, o=None) == NULL
    assert _fwd(lib, B=0) == SHAPE
    assert _fwd(lib, H=-1) == SHAPE
    assert _fwd(lib, L=-5) == SHAPE
    assert _fwd(lib, dk=96) == UNSUP
    assert _fwd(lib, dv=32) == UNSUP
    assert _fwd(lib, C=48) == UNSUP
    assert _fwd(lib, it=5) == UNSUP
    assert _fwd(lib, ot=2) == UNSUP
    assert _fwd(lib, B=300, H=300) == UNSUP
    assert _fwd(lib, q=BASE + 8) == ALIGN
    assert _fwd(lib, S0=BASE + 700 * MB + 4) == ALIGN
    assert _fwd(lib, o=BASE + 64) == ALIAS          # o overlaps q
    assert _fwd(lib, Sf=BASE + 200 * MB) == ALIAS   # S_final overlaps v
    assert _fwd(lib, S0=BASE + 700 * MB, Sf=BASE + 700 * MB + 16) == ALIAS  # partial overlap
    assert _fwd(lib, ws=BASE + 16) == ALIAS         # workspace overlaps q
    assert _fwd(lib, ws_bytes=16) == WS
    need = lib.deltanet_chunk_fwd_workspace_bytes(1, 2, 256, 64, 64, 64, BF16)
    assert need > 0
    assert _fwd(lib, ws_bytes=need - 1) == WS
    assert lib.deltanet_chunk_fwd_workspace_bytes(1, 2, 256, 96, 64, 64, BF16) == 0
    assert lib.deltanet_chunk_fwd_workspace_bytes(0, 2, 256, 64, 64, 64, BF16) == 0
    assert lib.deltanet_last_hip_error() == 0  # nothing reached HIP


def _dec(lib, q=BASE, k=BASE + 100 * MB, v=BASE + 200 * MB, beta=BASE + 300 * MB,
         S=BASE + 400 * MB, o=BASE + 900 * MB, B=2, H=3, dk=128, dv=128, it=BF16, ot=F32):
    return lib.deltanet_decode_step(q, k, v, beta, S, o, B, H, dk, dv, it, ot, None)


def test_decode_validation(lib):
    assert _dec(lib, S=None) == NULL
    assert _dec(lib, k=None) == NULL
    assert _dec(lib, B=0) == SHAPE
    assert _dec(lib, dk=100) == UNSUP
    assert _dec(lib, it=3) == UNSUP
    assert _dec(lib, v=BASE + 200 * MB + 2) == ALIGN
    assert _dec(lib, o=BASE + 400 * MB) == ALIAS   # o overlaps S
    assert _dec(lib, S=BASE + 32) == ALIAS         # S overlaps q
    assert lib.deltanet_last_hip_error() == 0


def test_binding_rejects_cpu_tensors():
    import torch
    x = torch.zeros(1, 1, 4, 64)
    with pytest.raises(ValueError):
        binding.chunk_fwd(x, x, x, torch.zeros(1, 1, 4))


def _gfwd(lib, alpha=BASE + 800 * MB, q=BASE, k=BASE + 100 * MB, v=BASE + 200 * MB,
          beta=BASE + 300 * MB, S0=None, o=BASE + 400 * MB, Sf=BASE + 500 * MB, B=1, H=2, L=256,
          dk=64, dv=64, C=64, it=BF16, ot=F32, ws=BASE + 600 * MB, ws_bytes=1 << 40):
    return lib.deltanet_gated_chunk_fwd(q, k, v, alpha, beta, S0, o, Sf, B, H, L, dk, dv, C, it,
                                        ot, ws, ws_bytes, None)


def test_gated_chunk_fwd_validation(lib):
    assert _gfwd(lib, alpha=None) == NULL
    assert _gfwd(lib, q=None) == NULL
    assert _gfwd(lib, B=0) == SHAPE
    assert _gfwd(lib, dk=96) == UNSUP
    assert _gfwd(lib, alpha=BASE + 800 * MB + 4) == ALIGN
    assert _gfwd(lib, o=BASE + 800 * MB) == ALIAS      # o overlaps alpha
    assert _gfwd(lib, Sf=BASE + 800 * MB) == ALIAS     # S_final overlaps alpha
    assert _gfwd(lib, ws=BASE + 800 * MB) == ALIAS     # workspace overlaps alpha
    plain = lib.deltanet_chunk_fwd_workspace_bytes(1, 2, 256, 64, 64, 64, BF16)
    need = lib.deltanet_gated_chunk_fwd_workspace_bytes(1, 2, 256, 64, 64, 64, BF16)
    assert need == plain + 1 * 2 * 256 * 4            # plus one log-decay per token
    assert _gfwd(lib, ws_bytes=need - 1) == WS
    assert lib.deltanet_gated_chunk_fwd_workspace_bytes(1, 2, 256, 64, 64, 48, BF16) == 0
    assert lib.deltanet_last_hip_error() == 0


def _gdec(lib, alpha=BASE + 800 * MB, q=BASE, k=BASE + 100 * MB, v=BASE + 200 * MB,
          beta=BASE + 300 * MB, S=BASE + 400 * MB, o=BASE + 900 * MB, B=2, H=3, dk=128, dv=128,
          it=BF16, ot=F32):
    return lib.deltanet_gated_decode_step(q, k, v, alpha, beta, S, o, B, H, dk, dv, it, ot, None)


def test_gated_decode_validation(lib):
    assert _gdec(lib, alpha=None) == NULL
    assert _gdec(lib, S=None) == NULL
    assert _gdec(lib, dk=100) == UNSUP
    assert _gdec(lib, alpha=BASE + 800 * MB + 8) == ALIGN
    assert _gdec(lib, o=BASE + 800 * MB) == ALIAS     # o overlaps alpha
    assert _gdec(lib, S=BASE + 800 * MB) == ALIAS     # S overlaps alpha
    assert lib.deltanet_last_hip_error() == 0
