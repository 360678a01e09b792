"""The no-allocation entry point, intattn_forward_ex_noalloc, against
intattn_forward_ex with a caller workspace, through the C ABI.

It serves callers that cannot allocate device memory. Its split-decode shapes
use the library's static per-device scratch array: two calls in a row (the
second with a smaller input, so stale contents of the first sit in the
scratch) must each equal intattn_forward_ex with a workspace bit for bit, and
the oracle. Refusals of a caller workspace and of shapes beyond the scratch
size are checked on the host.
"""
import ctypes

import numpy as np
import pytest
import torch

from oracle import intattn_oracle as O

IA = pytest.importorskip("integer_only_quantized_amd._binding")


def _dev(x):
    return torch.from_numpy(np.ascontiguousarray(x)).cuda()


def _inputs(B, H, Skv, D, seed):
    rng = np.random.default_rng(seed)
    s = 1.0 / 32
    q = np.clip(np.rint(rng.standard_normal((B, H, 1, D)) * 32), -127, 127).astype(np.int8)
    k = np.clip(np.rint(rng.standard_normal((B, H, Skv, D)) * 32), -127, 127).astype(np.int8)
    v = np.clip(np.rint(rng.standard_normal((B, H, Skv, D)) * 32), -127, 127).astype(np.int8)
    return q, k, v, (s, s, s, s / 8)


@pytest.mark.gpu
def test_noalloc_equals_workspace_call_twice():
    # (B, H, Skv, D): a long cache past 16384 keys, then a smaller few-heads
    # shape (batch 1 from 4096 keys on) through the same scratch
    for i, (B, H, Skv, D) in enumerate(((2, 8, 40000, 128), (1, 4, 6000, 64))):
        q, k, v, scales = _inputs(B, H, Skv, D, 70 + i)
        need = IA.workspace_bytes(B, H, 1, Skv, D)
        assert 0 < need <= IA.NOALLOC_SCRATCH_BYTES
        print(f"case noalloc B={B} H={H} Skv={Skv} D={D} scratch={need}", flush=True)
        qd, kd, vd = _dev(q), _dev(k), _dev(v)
        ws = torch.empty(need, dtype=torch.uint8, device="cuda")
        ref_ws, rm_ws, rs_ws = IA.forward_ex(qd, kd, vd, scales, O.DEFAULT_CLIP, False, 32, stats=True, workspace=ws)
        got, rm, rs = IA.forward_ex_noalloc(qd, kd, vd, scales, O.DEFAULT_CLIP, False, 32, stats=True)
        torch.cuda.synchronize()
        assert torch.equal(got, ref_ws) and torch.equal(rm, rm_ws) and torch.equal(rs, rs_ws)
        ref = O.forward(q, k, v, scales, O.DEFAULT_CLIP, False)
        assert np.array_equal(got.cpu().numpy(), ref)


@pytest.mark.gpu
def test_noalloc_non_split_shape_equals_forward():
    """A shape that uses no scratch (prefill, short rows) runs the same
    kernels as intattn_forward_ex."""
    rng = np.random.default_rng(5)
    q, k, v = (rng.integers(-127, 128, (2, 3, 200, 64)).astype(np.int8) for _ in range(3))
    scales = (0.01, 0.01, 0.02, 0.01)
    a = IA.forward_ex(_dev(q), _dev(k), _dev(v), scales, O.DEFAULT_CLIP, True, 32)
    b = IA.forward_ex_noalloc(_dev(q), _dev(k), _dev(v), scales, O.DEFAULT_CLIP, True, 32)
    torch.cuda.synchronize()
    assert torch.equal(a, b)
    assert np.array_equal(b.cpu().numpy(), O.forward(q, k, v, scales, O.DEFAULT_CLIP, True))


def test_noalloc_refusals_before_any_device_call():
    E = {v: k for k, v in IA.STATUS_NAMES.items()}
    sc = IA.Scales(0.05, 0.05, 0.05, 0.05)
    P = (0x1000, 0x2000, 0x3000, 0x4000)
    # a caller workspace is refused: the scratch is the library's own
    sh = IA.Shape(1, 4, 1, 20000, 128)
    var = IA.Variant(32, 4, 0, 8, 16, 0x10000, 1 << 30)
    assert IA._lib.intattn_forward_ex_noalloc(*P, ctypes.byref(sh), ctypes.byref(sc), O.DEFAULT_CLIP, 0,
                                              ctypes.byref(var), None, None, None) == E["INTATTN_E_WORKSPACE"]
    # a split shape beyond the scratch size
    big = IA.Shape(2, 64, 1, 65535, 128)
    assert IA.workspace_bytes(2, 64, 1, 65535, 128) > IA.NOALLOC_SCRATCH_BYTES
    assert IA._lib.intattn_forward_ex_noalloc(*P, ctypes.byref(big), ctypes.byref(sc), O.DEFAULT_CLIP, 0,
                                              None, None, None, None) == E["INTATTN_E_SCRATCH"]
    # ordinary argument errors as intattn_forward_ex
    assert IA._lib.intattn_forward_ex_noalloc(0, *P[1:], ctypes.byref(sh), ctypes.byref(sc), O.DEFAULT_CLIP, 0,
                                              None, None, None, None) == E["INTATTN_E_NULL"]
    bad = IA.Scales(0.0, 0.05, 0.05, 0.05)
    assert IA._lib.intattn_forward_ex_noalloc(*P, ctypes.byref(sh), ctypes.byref(bad), O.DEFAULT_CLIP, 0,
                                              None, None, None, None) == E["INTATTN_E_SCALE"]
