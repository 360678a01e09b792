"""Concurrent use of the library: two host threads, each with its own stream
(default priority), queue forward calls on the long-row, short-row and decode
kernels at once. The library keeps no per-call state beyond each kernel's
once-per-device launch setting, so every result must still equal the oracle
bit for bit.
"""
import threading

import numpy as np
import pytest
import torch

from oracle import intattn_oracle as O
from integer_only_quantized_amd import workloads as W

pytestmark = pytest.mark.gpu

IA = pytest.importorskip("integer_only_quantized_amd._binding")

SHAPES = [
    # (B, H, Sq, Skv, D, causal, seed): long rows, decode, short rows
    (1, 2, 300, 700, 64, True, 800),
    (2, 2, 1, 3000, 128, False, 801),
    (2, 2, 200, 256, 64, False, 802),
]


def test_two_threads_two_streams_bit_exact():
    cases = []
    for B, H, Sq, Skv, D, causal, seed in SHAPES:
        w = W.make_random(B, H, Sq, Skv, D, causal, seed, "normal", name="conc")
        ref = O.forward(w.q, w.k, w.v, w.scales, w.clip, causal)
        cases.append((w, causal, ref))
    print("case two threads x two streams, shapes", SHAPES, flush=True)
    errors = []

    def worker(tid):
        try:
            stream = torch.cuda.Stream()
            with torch.cuda.stream(stream):
                dev = [tuple(torch.from_numpy(x).cuda() for x in (w.q, w.k, w.v)) for w, _, _ in cases]
                outs = []
                for rep in range(20):
                    for (w, causal, _), (q, k, v) in zip(cases, dev):
                        outs.append(IA.forward(q, k, v, w.scales, w.clip, causal))
                stream.synchronize()
            for n, o in enumerate(outs):
                w, causal, ref = cases[n % len(cases)]
                if not np.array_equal(o.cpu().numpy(), ref):
                    errors.append(f"thread {tid} call {n}: differs from the oracle")
                    return
        except Exception as exc:          # reported below, in the main thread
            errors.append(f"thread {tid}: {exc!r}")

    threads = [threading.Thread(target=worker, args=(t,)) for t in range(2)]
    for t in threads:
        t.start()
    for t in threads:
        t.join(timeout=120)
    assert not any(t.is_alive() for t in threads), "a worker thread did not finish"
    assert not errors, errors
