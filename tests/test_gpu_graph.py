"""The forward pass captured in a HIP graph and replayed.

A serving loop that cannot afford one host launch per call captures the
calls once (torch.cuda.CUDAGraph records the library's kernel launches on the
capture stream) and replays them. The library's forward path allocates
nothing and records no memset, so a replay must reproduce the eager result
bit for bit. Each case: the eager output is checked against the oracle, three
calls are captured, and the graph is replayed three times with the test's
own eager work and a synchronisation between replays; every replay's output
must equal the eager one. Kernel families covered: short rows (ragged,
non-causal), long rows (causal), decode, decode with the keys split over
workgroups in a caller workspace (four launches a call) and the
no-allocation entry point (static per-device scratch).
"""
import numpy as np
import pytest
import torch

from oracle import intattn_oracle as O

pytestmark = pytest.mark.gpu

IA = pytest.importorskip("integer_only_quantized_amd._binding")

SCALES = (0.02, 0.02, 0.03, 0.01)


def _inputs(B, H, Sq, Skv, D, seed):
    rng = np.random.default_rng(seed)
    q = rng.integers(-127, 128, (B, H, Sq, D)).astype(np.int8)
    k = rng.integers(-127, 128, (B, H, Skv, D)).astype(np.int8)
    v = rng.integers(-127, 128, (B, H, Skv, D)).astype(np.int8)
    return q, k, v


def _replays_match(call, out, ref, other):
    """Capture three calls, replay three times with eager work between; every
    replay's output equals ref."""
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        call()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for _ in range(3):
            call()
    torch.cuda.synchronize()
    for r in range(3):
        out.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = out.cpu().numpy()
        assert np.array_equal(got, ref), f"replay {r}: {int((got != ref).sum())} outputs differ from eager"
        other()                              # eager work between replays
        torch.cuda.synchronize()
    del g


@pytest.mark.parametrize("B,H,Sq,Skv,D,causal", [
    (2, 3, 77, 150, 64, False),     # short-row kernel, ragged rows and keys
    (1, 2, 600, 1000, 128, True),   # long-row kernel, causal (bottom-right)
    (2, 4, 1, 3000, 128, False),    # decode kernel
])
def test_graph_replay_forward(B, H, Sq, Skv, D, causal):
    print(f"case forward B={B} H={H} Sq={Sq} Skv={Skv} D={D} causal={causal}", flush=True)
    q, k, v = _inputs(B, H, Sq, Skv, D, 900 + Sq)
    qd, kd, vd = (torch.from_numpy(x).cuda() for x in (q, k, v))
    out = torch.empty_like(qd)
    ref = IA.forward(qd, kd, vd, SCALES, IA.DEFAULT_CLIP, causal).cpu().numpy()
    assert np.array_equal(ref, O.forward(q, k, v, SCALES, O.DEFAULT_CLIP, causal))
    o2 = torch.empty_like(qd)
    _replays_match(lambda: IA.forward(qd, kd, vd, SCALES, IA.DEFAULT_CLIP, causal, out=out), out, ref,
                   lambda: IA.forward(qd, kd, vd, SCALES, IA.DEFAULT_CLIP, not causal and Sq <= Skv, out=o2))


def test_graph_replay_split_decode_and_no_alloc():
    """Decode over 20000 keys: the caller-workspace form (scores in the
    workspace, four kernels a call) and the no-allocation entry point."""
    B, H, Sq, Skv, D = 1, 4, 1, 20000, 128
    print(f"case split decode B={B} H={H} Skv={Skv} D={D}", flush=True)
    q, k, v = _inputs(B, H, Sq, Skv, D, 77)
    qd, kd, vd = (torch.from_numpy(x).cuda() for x in (q, k, v))
    ws = torch.empty(IA.workspace_bytes(B, H, Sq, Skv, D), dtype=torch.uint8, device="cuda")
    ref = IA.forward_ex(qd, kd, vd, SCALES, IA.DEFAULT_CLIP, False, workspace=ws).cpu().numpy()
    assert np.array_equal(ref, O.forward(q, k, v, SCALES, O.DEFAULT_CLIP, False))
    out = torch.empty_like(qd)
    other = lambda: IA.forward(qd, kd, vd, SCALES, IA.DEFAULT_CLIP, False)
    _replays_match(lambda: IA.forward_ex(qd, kd, vd, SCALES, IA.DEFAULT_CLIP, False, workspace=ws, out=out),
                   out, ref, other)
    print("case no-alloc split decode", flush=True)
    ref2 = IA.forward_ex_noalloc(qd, kd, vd, SCALES, IA.DEFAULT_CLIP, False).cpu().numpy()
    assert np.array_equal(ref2, ref)
    out2 = torch.empty_like(qd)
    _replays_match(lambda: IA.forward_ex_noalloc(qd, kd, vd, SCALES, IA.DEFAULT_CLIP, False, out=out2),
                   out2, ref, other)
