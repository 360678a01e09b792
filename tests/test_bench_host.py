"""Host-side pieces of bench.py, on the CPU: the one-GPU contract and the
algorithmic work that every roofline fraction divides by.

The work per call is fixed by the shapes alone: 2*D operations per allowed
score for Q.K^T and 2*D for P.V; causal rows attend keys 0 .. i + Skv - Sq.
The expected counts below are closed forms (n(n+1)/2 for a square causal
head), not a re-run of the code under test.
"""
import types

import pytest

import bench
from integer_only_quantized_amd import workloads as W


def _w(name):
    B, H, Sq, Skv, D, causal, _, _ = W.CONFIGS[name]
    return types.SimpleNamespace(shape=(B, H, Sq, Skv, D), causal=causal)


@pytest.mark.parametrize("name,scores", [
    ("tiny", 128 * 128),
    ("bert", 8 * 12 * 512 * 512),                 # 25,165,824
    ("vit", 32 * 12 * 197 * 197),                 # 14,902,656
    ("llama_prefill", 32 * 4096 * 4097 // 2),     # 268,500,992: lower triangle with the diagonal
    ("decode", 16 * 32 * 8192),                   # 4,194,304
])
def test_algorithmic_work_closed_forms(name, scores):
    w = _w(name)
    B, H, Sq, Skv, D = w.shape
    ops, nbytes, got = bench.algorithmic_work(w)
    assert got == scores
    assert ops == 4 * D * scores
    assert nbytes == B * H * D * (2 * Sq + 2 * Skv)   # Q, K, V and O, int8


def test_causal_rectangular_rows_attend_their_prefix():
    # Sq < Skv: row i attends keys 0 .. i + (Skv - Sq), a cache prefix plus the new rows
    w = types.SimpleNamespace(shape=(1, 1, 3, 10, 64), causal=True)
    assert bench.algorithmic_work(w)[2] == 8 + 9 + 10


def test_more_than_one_gpu_is_refused_before_any_device_work(capsys):
    assert bench.main(["--gpus", "2"]) == 2
    assert "one GPU" in capsys.readouterr().err


def test_kernel_source_hash_covers_the_kernel_sources():
    for name, (kernel, srcs) in bench.KERNEL.items():
        h = bench.kernel_source_sha(srcs)
        assert len(h) == 64 and int(h, 16) >= 0, name
    # the short-row workloads share one source set, the others differ from it
    assert bench.kernel_source_sha(bench.KERNEL["bert"][1]) == bench.kernel_source_sha(bench.KERNEL["vit"][1])
    assert bench.kernel_source_sha(bench.KERNEL["bert"][1]) != bench.kernel_source_sha(bench.KERNEL["decode"][1])
