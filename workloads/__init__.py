"""Seeded synthetic workloads for the DeepSeekMoE layer forward pass.

This module only *draws* inputs: token hidden states, gate vectors, biases and
expert weights.  It holds none of the layer's arithmetic (no gating, no top-K,
no FFN), so both the CPU oracle and the GPU path can be fed from it without
sharing any code of the method.

Recipe (every value is reproducible from ``(config, seed)``):

* Every tensor block has its own NumPy PCG64 stream,
  ``numpy.random.default_rng([seed, TAG, index])``.  Blocks are: 1024-token
  chunks of ``x``; the whole gate matrix; each bias vector; and one expert
  matrix (W1, W3 or W2 of one routed or shared expert).  Independent streams
  let the weights be drawn in parallel, and let a test regenerate only the
  experts it needs.
* ``x ~ N(0, 1)``; gate vectors ``~ N(0, 1/d)``; W1, W3 ``~ N(0, 1/d)``;
  W2 ``~ N(0, 1/inner)`` (each weight ``~ N(0, 1/fan_in)``).  Values are drawn
  in fp32 and rounded to nearest-even bf16 for bf16 workloads; the gate matrix
  and biases stay fp32 (the router runs in fp32).
* Selection bias (V3-style layer): ``U(-0.1, 0.1)`` per routed expert.
* Skewed small batch: a Zipf(s) log-bias ``b_e = -s * ln(r_e)`` added to the
  gate logits, where ``r`` is a seeded permutation of ``1..n_routed`` (the
  expert of rank ``r`` gets prior weight proportional to ``r**-s``).

The shapes follow the model descriptions on the pages: the 2B model (63
routed + 1 shared expert, 7 routed per token; DeepSeekMoE blog post,
"DeepSeekMoE 2B Model Example"), the 16B model (64 routed + 2 shared, 6 routed
per token, hidden 2048; same post, "Scaling Up to DeepSeekMoE 16B") and the V3
MoE layer (256 routed experts, 8 per token, group-limited routing and a
selection-only bias; DeepSeek-V3 Technical Report summary, sections
"2. Architecture" and "4. Pre-Training").  Real hidden states and trained
weights are not available; these draws stand in for them.
"""
from __future__ import annotations

import dataclasses
import os
from concurrent.futures import ThreadPoolExecutor
from typing import Optional

import numpy as np

# Stream tags (second word of every SeedSequence entropy list).
TAG_X = 1
TAG_GATE = 2
TAG_LOGIT_BIAS = 3
TAG_SELECT_BIAS = 4
TAG_ROUTED = (10, 11, 12)   # W1, W3, W2 of routed expert e
TAG_SHARED = (20, 21, 22)   # W1, W3, W2 of shared expert s
TAG_DOUT = 30               # gradient of the layer output (backward inputs)
X_CHUNK = 1024              # tokens per x stream


@dataclasses.dataclass(frozen=True)
class LayerConfig:
    """Shape and routing options of one MoE layer workload."""
    name: str
    T: int                   # tokens
    d: int                   # hidden size
    n_routed: int            # mN fine-grained routed experts
    inner: int               # routed expert SwiGLU inner size
    top_k: int               # mK routed experts kept per token
    n_shared: int            # K_s always-active shared experts
    shared_inner: int        # shared expert inner size
    score: str = "softmax"   # "softmax" | "sigmoid"
    norm_topk: bool = False  # renormalise the kept gate weights to sum 1
    n_groups: int = 1        # expert groups for group-limited routing
    topk_groups: int = 1     # groups kept per token
    select_bias_range: float = 0.0   # U(-r, r) selection-only bias (0 = none)
    zipf_s: float = 0.0      # Zipf exponent of the logit log-bias (0 = none)
    dtype: str = "bf16"      # "bf16" | "f32": x, out and expert weights; "fp8":
                             # generated as bf16 (the FP8 layer quantises them)
    routed_scale: float = 1.0
    seed: int = 0

    def replace(self, **kw) -> "LayerConfig":
        return dataclasses.replace(self, **kw)

    @property
    def has_logit_bias(self) -> bool:
        return self.zipf_s != 0.0

    @property
    def has_select_bias(self) -> bool:
        return self.select_bias_range != 0.0


# The five workloads.  Names say what each one is.
CONFIGS = {
    # Tiny fp32 layer: 4 base experts of inner 128 split m=4 into 16 routed
    # experts of inner 32, 4 kept, plus one shared expert of inner 32.
    "tiny-fp32": LayerConfig("tiny-fp32", T=64, d=64, n_routed=16, inner=32,
                             top_k=4, n_shared=1, shared_inner=32, dtype="f32"),
    # DeepSeekMoE-2B-shaped layer.
    "deepseekmoe-2b": LayerConfig("deepseekmoe-2b", T=8192, d=1280, n_routed=63,
                                  inner=1280, top_k=7, n_shared=1,
                                  shared_inner=1280),
    # DeepSeekMoE-16B-shaped layer (the throughput workload).
    "deepseekmoe-16b": LayerConfig("deepseekmoe-16b", T=16384, d=2048,
                                   n_routed=64, inner=1408, top_k=6, n_shared=2,
                                   shared_inner=1408),
    # DeepSeek-V3-style layer: sigmoid affinities, selection bias, 8 groups of
    # 32 experts with the best 4 kept, kept weights renormalised.
    "deepseek-v3": LayerConfig("deepseek-v3", T=4096, d=7168, n_routed=256,
                               inner=2048, top_k=8, n_shared=1,
                               shared_inner=2048, score="sigmoid",
                               norm_topk=True, n_groups=8, topk_groups=4,
                               select_bias_range=0.1),
    # The 16B-shaped layer with FP8 expert GEMMs (the same generated values;
    # the layer quantises the weights and activations to E4M3).
    "deepseekmoe-16b-fp8": LayerConfig("deepseekmoe-16b-fp8", T=16384, d=2048,
                                       n_routed=64, inner=1408, top_k=6, n_shared=2,
                                       shared_inner=1408, dtype="fp8"),
    # Skewed small batch on the 16B shapes: Zipf(1.2) logit log-bias.
    "skewed-16b-small": LayerConfig("skewed-16b-small", T=128, d=2048,
                                    n_routed=64, inner=1408, top_k=6,
                                    n_shared=2, shared_inner=1408, zipf_s=1.2),
}


def _threads() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def _round_bf16(a: np.ndarray) -> np.ndarray:
    """Round fp32 values to the nearest bf16 (ties to even); return fp32."""
    import torch
    return torch.from_numpy(np.ascontiguousarray(a, np.float32)).to(
        torch.bfloat16).float().numpy()


class Inputs:
    """Lazy, seeded access to one workload's tensors (host, fp32 values).

    Every accessor returns fp32 NumPy arrays whose values are exactly the ones
    the device receives (already rounded to bf16 where the workload is bf16).
    """

    def __init__(self, cfg: LayerConfig, seed: Optional[int] = None):
        self.cfg = cfg
        self.seed = cfg.seed if seed is None else seed
        self._cache = {}

    # -- primitives ------------------------------------------------------
    def _rng(self, *words) -> np.random.Generator:
        return np.random.default_rng([self.seed, *words])

    def _act(self, a: np.ndarray) -> np.ndarray:
        return _round_bf16(a) if self.cfg.dtype in ("bf16", "fp8") else a

    # -- token hidden states --------------------------------------------
    def x_rows(self, rows) -> np.ndarray:
        """Hidden states of the given token indices, [len(rows), d] fp32."""
        rows = np.asarray(rows, np.int64)
        out = np.empty((rows.size, self.cfg.d), np.float32)
        for c in np.unique(rows // X_CHUNK):
            chunk = self._x_chunk(int(c))
            sel = np.nonzero(rows // X_CHUNK == c)[0]
            out[sel] = chunk[rows[sel] - c * X_CHUNK]
        return out

    def _x_chunk(self, c: int) -> np.ndarray:
        key = ("x", c)
        if key not in self._cache:
            n = min(X_CHUNK, self.cfg.T - c * X_CHUNK)
            a = self._rng(TAG_X, c).standard_normal((n, self.cfg.d), np.float32)
            self._cache[key] = self._act(a)
        return self._cache[key]

    def x(self) -> np.ndarray:
        return self.x_rows(np.arange(self.cfg.T))

    def dout(self) -> np.ndarray:
        """Gradient of the layer output for the backward pass, [T, d] fp32
        values (N(0, 1), rounded like the activations)."""
        a = self._rng(TAG_DOUT).standard_normal((self.cfg.T, self.cfg.d), np.float32)
        return self._act(a)

    # -- router parameters ----------------------------------------------
    def w_gate(self) -> np.ndarray:
        cfg = self.cfg
        a = self._rng(TAG_GATE).standard_normal((cfg.n_routed, cfg.d), np.float32)
        return (a * np.float32(1.0 / np.sqrt(cfg.d))).astype(np.float32)

    def logit_bias(self) -> Optional[np.ndarray]:
        cfg = self.cfg
        if not cfg.has_logit_bias:
            return None
        rank = self._rng(TAG_LOGIT_BIAS).permutation(cfg.n_routed) + 1
        return (-cfg.zipf_s * np.log(rank.astype(np.float64))).astype(np.float32)

    def select_bias(self) -> Optional[np.ndarray]:
        cfg = self.cfg
        if not cfg.has_select_bias:
            return None
        r = cfg.select_bias_range
        return self._rng(TAG_SELECT_BIAS).uniform(-r, r, cfg.n_routed).astype(np.float32)

    # -- expert weights ---------------------------------------------------
    def _expert(self, tags, e: int, inner: int):
        d = self.cfg.d
        w1 = self._rng(tags[0], e).standard_normal((inner, d), np.float32)
        w3 = self._rng(tags[1], e).standard_normal((inner, d), np.float32)
        w2 = self._rng(tags[2], e).standard_normal((d, inner), np.float32)
        s_in = np.float32(1.0 / np.sqrt(d))
        s_out = np.float32(1.0 / np.sqrt(inner))
        return (self._act(w1 * s_in), self._act(w3 * s_in), self._act(w2 * s_out))

    def routed(self, e: int):
        """(W1 [inner, d], W3 [inner, d], W2 [d, inner]) of routed expert e."""
        return self._expert(TAG_ROUTED, e, self.cfg.inner)

    def shared(self, s: int):
        """(W1, W3, W2) of shared expert s."""
        return self._expert(TAG_SHARED, s, self.cfg.shared_inner)

    # -- device tensors -----------------------------------------------------
    def torch_tensors(self, device="cpu", progress=None):
        """All tensors as torch tensors on ``device`` (dtype bf16 or fp32).

        Returns a dict: x [T,d], w_gate [E,d] fp32, logit_bias / select_bias
        [E] fp32 or None, routed = (w1 [E,I,d], w3 [E,I,d], w2 [E,d,I]),
        shared = same with K_s experts (or None when K_s = 0).
        """
        import torch
        cfg = self.cfg
        tdt = torch.bfloat16 if cfg.dtype in ("bf16", "fp8") else torch.float32

        def stack(get, n, inner):
            w1 = torch.empty((n, inner, cfg.d), dtype=tdt)
            w3 = torch.empty((n, inner, cfg.d), dtype=tdt)
            w2 = torch.empty((n, cfg.d, inner), dtype=tdt)

            def fill(i):
                a, b, c = get(i)
                w1[i] = torch.from_numpy(a).to(tdt)
                w3[i] = torch.from_numpy(b).to(tdt)
                w2[i] = torch.from_numpy(c).to(tdt)
                if progress is not None and (i + 1) % 32 == 0:
                    progress(f"generated {i + 1}/{n} experts")
            with ThreadPoolExecutor(_threads()) as ex:
                list(ex.map(fill, range(n)))
            return tuple(t.to(device) for t in (w1, w3, w2))

        nchunks = (cfg.T + X_CHUNK - 1) // X_CHUNK
        with ThreadPoolExecutor(_threads()) as ex:
            list(ex.map(self._x_chunk, range(nchunks)))
        x = torch.from_numpy(np.concatenate(
            [self._x_chunk(c) for c in range(nchunks)], 0)).to(tdt)
        for c in range(nchunks):          # free host copies of large inputs
            self._cache.pop(("x", c), None)
        out = {
            "x": x.to(device),
            "w_gate": torch.from_numpy(self.w_gate()).to(device),
            "logit_bias": None, "select_bias": None,
            "routed": stack(self.routed, cfg.n_routed, cfg.inner),
            "shared": (stack(self.shared, cfg.n_shared, cfg.shared_inner)
                       if cfg.n_shared > 0 else None),
        }
        lb, sb = self.logit_bias(), self.select_bias()
        if lb is not None:
            out["logit_bias"] = torch.from_numpy(lb).to(device)
        if sb is not None:
            out["select_bias"] = torch.from_numpy(sb).to(device)
        return out


def make_inputs(cfg, seed: Optional[int] = None) -> Inputs:
    """Seeded inputs of a workload (``cfg`` is a LayerConfig or a name)."""
    if isinstance(cfg, str):
        cfg = CONFIGS[cfg]
    return Inputs(cfg, seed)
