"""Seeded synthetic inputs for the five attention workloads and for edge cases.

This module only makes inputs: float activations drawn from seeded numpy
generators, per-tensor symmetric int8 quantisation, and the output scale. It
contains none of the integer attention arithmetic, and both the GPU path's
tests and the CPU oracle take their inputs from here.

The IntAttention digest pages evaluate BERT, GPT-2 and ViT on GLUE and
ImageNet (section "Results"), and one forum page adds LLaMA. Neither the
datasets nor trained weights are available, so these generators stand in for
them with the attention shapes of those models and activation statistics of
the stated kind (Gaussian, channel outliers, heavy tails).

Recipe (every workload):
  * numpy.random.default_rng(seed), draws in the order Q, K, V (float64
    N(0,1)), then any outlier masks;
  * per-tensor symmetric scale s = float32(absmax / 127); int8 value
    q = clip(rint(x / s), -127, 127) (round half to even);
  * output scale s_o = float32(absmax(O_ref) / 127) where O_ref is exact
    float64 softmax attention on the dequantised int8 inputs, with logits
    (s_q*s_k/sqrt(D)) * (q_int . k_int) and the same mask as the workload;
  * the sparsity-aware threshold is float32(ln 510).
"""
from __future__ import annotations

import math
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field

import numpy as np

DEFAULT_CLIP = float(np.float32(math.log(510.0)))


@dataclass
class Workload:
    name: str
    B: int
    H: int
    Sq: int
    Skv: int
    D: int
    causal: bool
    q: np.ndarray              # int8 [B, H, Sq, D]
    k: np.ndarray              # int8 [B, H, Skv, D]
    v: np.ndarray              # int8 [B, H, Skv, D]
    scales: tuple              # (s_q, s_k, s_v, s_o) as Python floats holding float32 values
    clip: float = DEFAULT_CLIP
    meta: dict = field(default_factory=dict)

    @property
    def shape(self):
        return (self.B, self.H, self.Sq, self.Skv, self.D)


# name -> (B, H, Sq, Skv, D, causal, seed, activation kind)
CONFIGS = {
    "tiny":          (1, 1, 128, 128, 64, False, 0, "normal"),
    "bert":          (8, 12, 512, 512, 64, False, 1, "channel_outliers"),
    "vit":           (32, 12, 197, 197, 64, False, 2, "normal"),
    "llama_prefill": (1, 32, 4096, 4096, 128, True, 3, "student_t_tail"),
    "decode":        (16, 32, 1, 8192, 128, False, 4, "normal"),
}

DESCRIPTIONS = {
    "tiny": "single head, B=1 H=1 S=128 d=64, N(0,1), non-causal",
    "bert": "BERT-base encoder attention, B=8 H=12 S=512 d=64, N(0,1) with 8 of 768 hidden channels x8, non-causal",
    "vit": "ViT-B/16 attention, B=32 H=12 S=197 d=64, N(0,1), non-causal",
    "llama_prefill": "LLaMA-7B-shaped causal prefill, B=1 H=32 S=4096 d=128, N(0,1) with 0.5% Student-t(3) entries",
    "decode": "LLaMA-7B-shaped batched decode, B=16 H=32 Sq=1 Skv=8192 d=128, N(0,1), non-causal",
}


def quant_scale(absmax: float) -> float:
    """Per-tensor symmetric scale float32(absmax/127)."""
    return float(np.float32(absmax / 127.0))


def quantise(x: np.ndarray, s: float) -> np.ndarray:
    """clip(rint(x / s), -127, 127) as int8 (numpy rint is half-to-even)."""
    y = np.rint(x / np.float64(s) if x.dtype == np.float64 else x / np.float32(s))
    return np.clip(y, -127, 127).astype(np.int8)


def reference_attention_absmax(q, k, v, s_q, s_k, s_v, causal, head_chunk=1):
    """max |O_ref| of float64 softmax attention on dequantised int8 tensors.

    Logits are (s_q*s_k/sqrt(D)) * (q_int . k_int); the integer dot products
    are exact in float64. Processed one (b, h) slice at a time.
    """
    B, H, Sq, D = q.shape
    Skv = k.shape[2]
    alpha = (float(s_q) * float(s_k)) / math.sqrt(float(D))
    if causal:
        allow = np.arange(Skv)[None, :] <= np.arange(Sq)[:, None] + (Skv - Sq)
    best = 0.0
    for b in range(B):
        for h in range(H):
            S = q[b, h].astype(np.float64) @ k[b, h].astype(np.float64).T
            L = alpha * S
            if causal:
                L = np.where(allow, L, -np.inf)
            L -= L.max(axis=1, keepdims=True)
            W = np.exp(L)
            W /= W.sum(axis=1, keepdims=True)
            O = (W @ v[b, h].astype(np.float64)) * float(s_v)
            best = max(best, float(np.abs(O).max()))
    return best


def _finish(name, B, H, Sq, Skv, D, causal, xq, xk, xv, meta, clip=DEFAULT_CLIP,
            s_o=None):
    s_q = quant_scale(float(np.abs(xq).max()))
    s_k = quant_scale(float(np.abs(xk).max()))
    s_v = quant_scale(float(np.abs(xv).max()))
    q = quantise(xq, s_q)
    k = quantise(xk, s_k)
    v = quantise(xv, s_v)
    if s_o is None:
        amax = reference_attention_absmax(q, k, v, s_q, s_k, s_v, causal)
        s_o = quant_scale(amax) if amax > 0 else s_v
    return Workload(name, B, H, Sq, Skv, D, causal, q, k, v,
                    (s_q, s_k, s_v, float(s_o)), clip, meta)


def make_random(B, H, Sq, Skv, D, causal=False, seed=0, kind="normal",
                name=None, s_o=None) -> Workload:
    """Generic seeded workload (used by the named configs and by edge-case tests)."""
    rng = np.random.default_rng(seed)
    xq = rng.standard_normal((B, H, Sq, D))
    xk = rng.standard_normal((B, H, Skv, D))
    xv = rng.standard_normal((B, H, Skv, D))
    meta = {"seed": seed, "kind": kind}
    if kind == "channel_outliers":
        # 1% of the H*D hidden channels scaled x8, chosen independently per tensor
        n_hidden = H * D
        n_out = int(round(0.01 * n_hidden))
        for name_t, x in (("q", xq), ("k", xk), ("v", xv)):
            ch = rng.choice(n_hidden, n_out, replace=False)
            meta["outlier_channels_" + name_t] = sorted(int(c) for c in ch)
            for c in ch:
                x[:, c // D, :, c % D] *= 8.0
    elif kind == "student_t_tail":
        # each element replaced with probability 0.005 by a Student-t(3) draw
        for x in (xq, xk, xv):
            sel = rng.random(x.shape) < 0.005
            x[sel] = rng.standard_t(3, size=int(sel.sum()))
    elif kind != "normal":
        raise ValueError("unknown activation kind " + kind)
    return _finish(name or "random", B, H, Sq, Skv, D, causal, xq, xk, xv, meta,
                   s_o=s_o)


def _make_decode(seed: int) -> Workload:
    """decode: float32 draws from per-(tensor, batch) spawned streams, in parallel.

    The K/V cache is 2 x 512 MiB of int8; float64 temporaries would need
    ~8.6 GB, so each batch slice b of tensor t is drawn in float32 from
    default_rng(SeedSequence(seed).spawn(3*B)[3*b + t]) with t = 0, 1, 2 for
    Q, K, V.
    """
    B, H, Sq, Skv, D, causal, _, _ = CONFIGS["decode"]
    kids = np.random.SeedSequence(seed).spawn(3 * B)
    xs = [np.empty((B, H, S, D), dtype=np.float32) for S in (Sq, Skv, Skv)]

    def job(b):
        for t in range(3):
            g = np.random.default_rng(kids[3 * b + t])
            xs[t][b] = g.standard_normal(xs[t][b].shape, dtype=np.float32)

    with ThreadPoolExecutor(max_workers=8) as ex:
        list(ex.map(job, range(B)))
    meta = {"seed": seed, "kind": "normal", "draw": "float32, spawned per (tensor, batch)"}
    return _finish("decode", B, H, Sq, Skv, D, causal, xs[0], xs[1], xs[2], meta)


_CACHE: dict = {}


def make_config(name: str, cache: bool = True) -> Workload:
    """One of the five named workloads, generated deterministically from its seed."""
    if cache and name in _CACHE:
        return _CACHE[name]
    if name not in CONFIGS:
        raise KeyError(name)
    B, H, Sq, Skv, D, causal, seed, kind = CONFIGS[name]
    if name == "decode":
        w = _make_decode(seed)
    else:
        w = make_random(B, H, Sq, Skv, D, causal, seed, kind, name=name)
    w.meta["description"] = DESCRIPTIONS[name]
    if cache:
        _CACHE[name] = w
    return w


def slice_heads(w: Workload, heads) -> Workload:
    """Sub-workload of selected (b, h) pairs (each attention head is independent)."""
    heads = list(heads)
    q = np.stack([w.q[b, h] for b, h in heads])[:, None]
    k = np.stack([w.k[b, h] for b, h in heads])[:, None]
    v = np.stack([w.v[b, h] for b, h in heads])[:, None]
    return Workload(w.name + "[heads]", len(heads), 1, w.Sq, w.Skv, w.D, w.causal,
                    q, k, v, w.scales, w.clip, dict(w.meta, heads=heads))
