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
    assert lib.deltanet_version() == 500
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


def _feat(lib, q=BASE, k=BASE + 100 * MB, bl=BASE + 200 * MB, qh=BASE + 300 * MB,
          kh=BASE + 400 * MB, b=BASE + 500 * MB, B=2, H=3, L=100, dk=128, dt=BF16):
    return lib.deltanet_feature_prep(q, k, bl, qh, kh, b, B, H, L, dk, dt, None)


def test_feature_prep_validation(lib):
    for name in ("q", "k", "bl", "qh", "kh", "b"):
        assert _feat(lib, **{name: None}) == NULL, name
    assert _feat(lib, q=None, L=0) == OK              # nothing to map: no pointer needed
    assert _feat(lib, B=0) == SHAPE
    assert _feat(lib, L=-1) == SHAPE
    assert _feat(lib, dk=96) == UNSUP
    assert _feat(lib, dt=2) == UNSUP
    assert _feat(lib, kh=BASE + 400 * MB + 2) == ALIGN
    assert _feat(lib, qh=BASE + 100 * MB) == ALIAS     # q_hat over k_raw
    assert _feat(lib, b=BASE + 400 * MB) == ALIAS      # beta over k_hat
    assert _feat(lib, qh=BASE + 16) == ALIAS           # partly over its own input
    assert _feat(lib, L=70000, B=65535, H=65535) == UNSUP  # more rows than one launch takes
    assert lib.deltanet_last_hip_error() == 0


def _ffwd(lib, alpha=None, q=BASE, k=BASE + 100 * MB, v=BASE + 200 * MB, bl=BASE + 300 * MB,
          S0=None, o=BASE + 400 * MB, Sf=BASE + 500 * MB, B=1, H=2, L=256, dk=64, dv=64, C=64,
          it=BF16, ot=F32, ws=BASE + 600 * MB, ws_bytes=1 << 40):
    return lib.deltanet_chunk_fwd_features(q, k, v, alpha, bl, S0, o, Sf, B, H, L, dk, dv, C, it,
                                           ot, ws, ws_bytes, None)


def test_chunk_fwd_features_validation(lib):
    assert _ffwd(lib, q=None) == NULL
    assert _ffwd(lib, bl=None) == NULL
    assert _ffwd(lib, dk=96) == UNSUP
    assert _ffwd(lib, C=32) == UNSUP
    assert _ffwd(lib, bl=BASE + 300 * MB + 4) == ALIGN
    assert _ffwd(lib, o=BASE + 100 * MB) == ALIAS      # o over k_raw
    assert _ffwd(lib, ws=BASE + 300 * MB) == ALIAS     # workspace over the logits
    for gated in (0, 1):
        core = (lib.deltanet_gated_chunk_fwd_workspace_bytes if gated
                else lib.deltanet_chunk_fwd_workspace_bytes)(1, 2, 256, 64, 64, 64, BF16)
        need = lib.deltanet_chunk_fwd_features_workspace_bytes(1, 2, 256, 64, 64, 64, BF16, gated)
        r = lambda n: (n + 255) // 256 * 256
        # the mapped q, k (bf16) and beta (fp32) follow the core's scratch
        assert need == r(core) + 2 * r(1 * 2 * 256 * 64 * 2) + r(1 * 2 * 256 * 4)
        alpha = BASE + 800 * MB if gated else None
        assert _ffwd(lib, alpha=alpha, ws_bytes=need - 1) == WS
    assert lib.deltanet_chunk_fwd_features_workspace_bytes(1, 2, 256, 64, 64, 48, BF16, 0) == 0
    assert lib.deltanet_last_hip_error() == 0


def test_decode_step_features_validation(lib):
    def d(**kw):
        a = dict(q=BASE, k=BASE + 100 * MB, v=BASE + 200 * MB, alpha=None, bl=BASE + 300 * MB,
                 S=BASE + 400 * MB, o=BASE + 900 * MB, B=2, H=3, dk=128, dv=128, it=BF16, ot=F32)
        a.update(kw)
        return lib.deltanet_decode_step_features(a["q"], a["k"], a["v"], a["alpha"], a["bl"],
                                                 a["S"], a["o"], a["B"], a["H"], a["dk"],
                                                 a["dv"], a["it"], a["ot"], None)
    assert d(bl=None) == NULL
    assert d(k=None) == NULL
    assert d(dv=32) == UNSUP
    assert d(alpha=BASE + 800 * MB + 4) == ALIGN
    assert d(o=BASE + 300 * MB) == ALIAS               # o over the logits
    assert d(S=BASE + 100 * MB) == ALIAS               # S over k_raw
    assert lib.deltanet_last_hip_error() == 0


def _kfwd(lib, alpha=BASE + 800 * MB, q=BASE, k=BASE + 100 * MB, v=BASE + 200 * MB,
          beta=BASE + 300 * MB, S0=None, o=BASE + 400 * MB, Sf=BASE + 500 * MB, B=1, H=2, L=256,
          dk=64, dv=64, C=64, it=BF16, ot=F32, ws=BASE + 600 * MB, ws_bytes=1 << 40):
    return lib.deltanet_kda_chunk_fwd(q, k, v, alpha, beta, S0, o, Sf, B, H, L, dk, dv, C, it, ot,
                                      ws, ws_bytes, None)


def test_kda_chunk_fwd_validation(lib):
    assert _kfwd(lib, alpha=None) == NULL
    # L = 0: no token to decay, alpha may be NULL (the later alignment check
    # is what stops this call, so the NULL alpha passed)
    assert _kfwd(lib, alpha=None, L=0, S0=BASE + 4) == ALIGN
    assert _kfwd(lib, v=None) == NULL
    assert _kfwd(lib, dk=32) == UNSUP
    assert _kfwd(lib, C=96) == UNSUP
    assert _kfwd(lib, alpha=BASE + 800 * MB + 4) == ALIGN
    # alpha is [B, H, L, d_k] fp32 = 128 KiB here: an output just past one
    # scalar per token still overlaps it
    assert _kfwd(lib, o=BASE + 800 * MB + 4096) == ALIAS
    assert _kfwd(lib, ws=BASE + 800 * MB + 64 * 1024) == ALIAS
    need = lib.deltanet_kda_chunk_fwd_workspace_bytes(1, 2, 256, 64, 64, 64, BF16)
    # o right after the gate does not overlap it (the workspace check after
    # the aliasing checks is what stops this call)
    assert _kfwd(lib, o=BASE + 800 * MB + 1 * 2 * 256 * 64 * 4, ws_bytes=need - 1) == WS
    # per 64-token chunk: T and P (64 x 64), three 64 x d_k decayed operands,
    # the d_k end-of-chunk decays, all fp32
    assert need == 1 * 2 * 4 * (2 * 64 * 64 + 3 * 64 * 64 + 64) * 4
    assert lib.deltanet_kda_chunk_fwd_workspace_bytes(1, 2, 256, 64, 64, 128, BF16) == need
    assert _kfwd(lib, ws_bytes=need - 1) == WS
    assert lib.deltanet_last_hip_error() == 0


def test_kda_decode_validation(lib):
    def d(**kw):
        a = dict(q=BASE, k=BASE + 100 * MB, v=BASE + 200 * MB, alpha=BASE + 800 * MB,
                 beta=BASE + 300 * MB, S=BASE + 400 * MB, o=BASE + 900 * MB, B=2, H=3, dk=128,
                 dv=128, it=BF16, ot=F32)
        a.update(kw)
        return lib.deltanet_kda_decode_step(a["q"], a["k"], a["v"], a["alpha"], a["beta"], a["S"],
                                            a["o"], a["B"], a["H"], a["dk"], a["dv"], a["it"],
                                            a["ot"], None)
    assert d(alpha=None) == NULL
    assert d(dk=100) == UNSUP
    assert d(alpha=BASE + 800 * MB + 8) == ALIGN
    assert d(o=BASE + 800 * MB + 2 * 3 * 4 * 64) == ALIAS   # inside the [B, H, d_k] gate
    assert d(S=BASE + 800 * MB + 1024) == ALIAS
    assert lib.deltanet_last_hip_error() == 0


def _bwd(lib, **kw):
    a = dict(q=BASE, k=BASE + 100 * MB, v=BASE + 200 * MB, beta=BASE + 300 * MB, S0=None,
             dO=BASE + 400 * MB, dSf=None, dq=BASE + 500 * MB, dk=BASE + 600 * MB,
             dv=BASE + 700 * MB, db=BASE + 800 * MB, dS0=BASE + 900 * MB, B=1, H=2, L=256, dk_=64,
             dv_=64, C=64, it=BF16, ws=BASE + 1000 * MB, wsb=1 << 40)
    a.update(kw)
    return lib.deltanet_chunk_bwd(a["q"], a["k"], a["v"], a["beta"], a["S0"], a["dO"], a["dSf"],
                                  a["dq"], a["dk"], a["dv"], a["db"], a["dS0"], a["B"], a["H"],
                                  a["L"], a["dk_"], a["dv_"], a["C"], a["it"], a["ws"], a["wsb"],
                                  None)


def test_chunk_bwd_validation(lib):
    for name in ("q", "k", "v", "beta", "dO", "dq", "dk", "dv", "db"):
        assert _bwd(lib, **{name: None}) == NULL, name
    assert _bwd(lib, B=0) == SHAPE
    assert _bwd(lib, dk_=80) == UNSUP
    assert _bwd(lib, C=32) == UNSUP
    assert _bwd(lib, dO=BASE + 400 * MB + 8) == ALIGN
    assert _bwd(lib, dS0=BASE + 900 * MB + 4) == ALIGN
    assert _bwd(lib, dq=BASE + 100 * MB) == ALIAS          # dq over k
    assert _bwd(lib, dv=BASE + 400 * MB) == ALIAS          # dv over dO
    assert _bwd(lib, db=BASE + 500 * MB + 64) == ALIAS     # dbeta inside dq
    assert _bwd(lib, dS0=BASE + 700 * MB) == ALIAS         # dS0 over dv
    assert _bwd(lib, ws=BASE + 800 * MB) == ALIAS          # workspace over dbeta
    need = lib.deltanet_chunk_bwd_workspace_bytes(1, 2, 256, 64, 64, 64, BF16)
    # per 64-token chunk: X, M, dM, W (64 x 64), the entering state and exit
    # gradient (d_k x d_v), R, Delta, dDelta (64 x d_v), all fp32; then, per
    # 128-token chunk of the forward pass, T's lower triangle: 20 blocks of
    # 32 x 32 (row tiles of 16 rows, blocks of 32 columns), hi and lo bf16
    assert need == (1 * 2 * 4 * (4 * 64 * 64 + 2 * 64 * 64 + 3 * 64 * 64) * 4
                    + 1 * 2 * 2 * 20 * 2 * 64 * 16)
    assert _bwd(lib, wsb=need - 1) == WS
    assert lib.deltanet_last_hip_error() == 0
