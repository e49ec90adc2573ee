"""deltanet_chunk_fwd_noalloc (the forward that allocates nothing: its scratch
is the library's fixed per-GPU area) against deltanet_chunk_fwd with a
caller-given workspace, both called through the C ABI."""

import ctypes
import sys

import pytest
import torch

from deltanet_delta_rule_chunk_amd import inputs as I
from oracle import delta_rule_forward
from parity import assert_parity, to64

DEV = "cuda:0"
NOALLOC_MAX = 64 << 20
DN_OK, DN_ERR_WORKSPACE = 0, 6


def _ptr(t):
    return None if t is None else t.data_ptr()


def _both(lib, w, seed, out_dtype):
    x = I.make_chunk_inputs(w, seed=seed)
    g = {k: (None if t is None else t.to(DEV)) for k, t in x.items()}
    code_in = 1 if w.dtype == "bf16" else 0
    code_out = 1 if out_dtype == torch.bfloat16 else 0
    need = lib.deltanet_chunk_fwd_workspace_bytes(w.B, w.H, w.L, w.d_k, w.d_v, w.C, code_in)
    assert 0 < need <= NOALLOC_MAX
    res = []
    for noalloc in (True, False):
        o = torch.empty(w.B, w.H, w.L, w.d_v, dtype=out_dtype, device=DEV)
        S = torch.empty(w.B, w.H, w.d_k, w.d_v, dtype=torch.float32, device=DEV)
        args = [_ptr(g["q"]), _ptr(g["k"]), _ptr(g["v"]), _ptr(g["beta"]), _ptr(g["S0"]),
                _ptr(o), _ptr(S), w.B, w.H, w.L, w.d_k, w.d_v, w.C, code_in, code_out]
        stream = torch.cuda.current_stream(DEV).cuda_stream
        if noalloc:
            st = lib.deltanet_chunk_fwd_noalloc(*args, stream)
        else:
            ws = torch.empty(need, dtype=torch.uint8, device=DEV)
            st = lib.deltanet_chunk_fwd(*args, _ptr(ws), need, stream)
        assert st == DN_OK, st
        torch.cuda.synchronize()
        res.append((o.cpu(), S.cpu()))
    return x, res


@pytest.mark.gpu
def test_noalloc_matches_workspace_entry_point(gpu_lib):
    """Two calls in a row, the second smaller (the area keeps the first call's
    contents), in both precisions of the chunk kernels."""
    cases = [
        # the mid-size workload (its 48 MiB workspace nearly fills the area)
        (I.WORKLOADS[2], 0, torch.float32),
        (I.ChunkWorkload("small_ragged", 1, 3, 333, 64, 128, 64, "bf16", s0_std=0.1), 3,
         torch.bfloat16),
        (I.ChunkWorkload("f32_ragged", 2, 2, 300, 128, 64, 128, "f32", s0_std=0.1), 4,
         torch.float32),
    ]
    for w, seed, od in cases:
        print(f"[noalloc] {w.name}", file=sys.stderr, flush=True)
        x, ((o1, S1), (o2, S2)) = _both(gpu_lib, w, seed, od)
        assert torch.equal(o1, o2) and torch.equal(S1, S2), w.name
        if w.B * w.H * w.L <= 4096:
            S0 = None if x["S0"] is None else to64(x["S0"])
            o_ref, S_ref = delta_rule_forward(to64(x["q"]), to64(x["k"]), to64(x["v"]),
                                              to64(x["beta"]), S0)
            assert_parity(o1, o_ref, w.dtype, f"{w.name} o")
            assert_parity(S1, S_ref, w.dtype, f"{w.name} S_final")


def test_noalloc_rejects_sizes_beyond_the_area():
    """Validated on the host before any HIP call (no GPU needed): a shape whose
    workspace exceeds the fixed area returns DN_ERR_WORKSPACE."""
    from deltanet_delta_rule_chunk_amd import binding

    lib = binding.load()
    B, H, L, d, C = 1, 32, 65536, 128, 128
    assert lib.deltanet_chunk_fwd_workspace_bytes(B, H, L, d, d, C, 1) > NOALLOC_MAX
    tok = B * H * L
    base, ptrs = 1 << 40, []
    for n in (tok * d * 2, tok * d * 2, tok * d * 2, tok * 4, tok * d * 4, B * H * d * d * 4):
        ptrs.append(base)
        base += (n + 4095) // 4096 * 4096
    q, k, v, beta, o, S = ptrs
    st = lib.deltanet_chunk_fwd_noalloc(q, k, v, beta, None, o, S, B, H, L, d, d, C, 1, 0, None)
    assert st == DN_ERR_WORKSPACE
