"""Seeded synthetic workloads for the DFlash drafter block step.

This module only draws random numbers and stores them in the storage dtype a
workload names. It holds none of the drafter's arithmetic: no norm, no rope, no
projection, no quantisation. Both the HIP path and the CPU oracle consume the
arrays it returns, so the two sides always see the same inputs.

Workloads (shapes from the dflash-ops card, "Measured": 5 layers, n_embd 6656,
heads 32/8, head_dim 128, n_ff 19968, window 2048, block 16, vocab reduced to
8192; the fused feature width is 5 captured target layers times the target
hidden size, dflash_engine.py page, TargetContextFeatureFuser):

* ``tiny``  -- 1 layer, n_embd 256, 4/1 heads, head_dim 64, n_ff 768,
  window 64, vocab 512, target hidden 256: everything fits in cache; parity and
  invariants.
* ``real``  -- the card's dimensions above.

Distributions: every ``[out, in]`` matrix is N(0, 1/in); tok_embd and lm_head
``[V, E]`` are N(0, 1/E); norm weight vectors are 1 + N(0, 0.1); target
features are N(0, 1). The second argument of N is a variance throughout.

Storage: ``f32`` tensors are numpy float32; ``bf16`` tensors are numpy uint16
holding bfloat16 bit patterns (rounded to nearest even by torch); weights of
``fp8`` workloads are float32 masters, quantised later by whichever side uses
them.

Random streams: tensor ``name`` of a workload with seed ``s`` draws from
``numpy.random.SeedSequence(s, spawn_key=(crc32(name), chunk))`` in chunks of
``CHUNK`` elements, so the values do not depend on the number of threads that
generate them, nor on which other tensors are generated.
"""
from __future__ import annotations

import dataclasses
import os
import zlib
from concurrent.futures import ThreadPoolExecutor

import numpy as np

CHUNK = 1 << 22


@dataclasses.dataclass(frozen=True)
class Shape:
    n_layer: int
    n_embd: int
    n_head: int
    n_head_kv: int
    head_dim: int
    n_ff: int
    window: int
    block: int
    n_vocab: int
    n_capture: int
    target_hidden: int
    mask_id: int = 0
    rope_base: float = 10000.0
    rms_eps: float = 1e-6

    @property
    def q_dim(self) -> int:
        return self.n_head * self.head_dim

    @property
    def kv_dim(self) -> int:
        return self.n_head_kv * self.head_dim

    @property
    def feat_dim(self) -> int:
        return self.n_capture * self.target_hidden


TINY = Shape(n_layer=1, n_embd=256, n_head=4, n_head_kv=1, head_dim=64, n_ff=768,
             window=64, block=16, n_vocab=512, n_capture=5, target_hidden=256)
REAL = Shape(n_layer=5, n_embd=6656, n_head=32, n_head_kv=8, head_dim=128, n_ff=19968,
             window=2048, block=16, n_vocab=8192, n_capture=5, target_hidden=6656)

LAYER_MATS = ("wq", "wk", "wv", "wo", "w_gate", "w_up", "w_down")
LAYER_NORMS = ("attn_norm", "q_norm", "k_norm", "ffn_norm")


def _threads() -> int:
    return max(1, min(16, os.cpu_count() or 1))


def _key(name: str) -> int:
    return zlib.crc32(name.encode())


def normal(seed: int, name: str, shape, std: float = 1.0, mean: float = 0.0) -> np.ndarray:
    """float32 array of N(mean, std^2) drawn from the tensor's own chunked streams."""
    n = int(np.prod(shape))
    out = np.empty(n, dtype=np.float32)
    key = _key(name)

    def fill(c: int) -> None:
        lo, hi = c * CHUNK, min(n, (c + 1) * CHUNK)
        rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence(seed, spawn_key=(key, c))))
        v = rng.standard_normal(hi - lo, dtype=np.float32)
        if std != 1.0:
            v *= np.float32(std)
        if mean != 0.0:
            v += np.float32(mean)
        out[lo:hi] = v

    nchunks = (n + CHUNK - 1) // CHUNK
    if nchunks == 1:
        fill(0)
    else:
        with ThreadPoolExecutor(_threads()) as ex:
            list(ex.map(fill, range(nchunks)))
    return out.reshape(shape)


def integers(seed: int, name: str, shape, low: int, high: int) -> np.ndarray:
    """int32 array uniform in [low, high)."""
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence(seed, spawn_key=(_key(name), 0))))
    return rng.integers(low, high, size=shape, dtype=np.int64).astype(np.int32)


def to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """bfloat16 bit patterns (uint16) of a float32 array, via torch's round-to-nearest-even cast."""
    import torch

    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def store(a: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == "f32":
        return a
    if dtype == "bf16":
        return to_bf16_bits(a)
    raise ValueError(dtype)


def weights(shape: Shape, weight_dtype: str, seed: int = 0) -> dict:
    """Drafter weights in storage form.

    weight_dtype: "f32", "bf16" or "fp8". For "fp8" the seven layer matrices
    and lm_head are float32 masters (the consumer quantises them per output
    row); fc, tok_embd and the norm vectors are bf16.
    """
    aux = "f32" if weight_dtype == "f32" else "bf16"
    mat = weight_dtype if weight_dtype != "fp8" else "f32"
    E, F, V = shape.n_embd, shape.n_ff, shape.n_vocab
    w = {
        "tok_embd": store(normal(seed, "tok_embd", (V, E), std=E ** -0.5), aux),
        "lm_head": store(normal(seed, "lm_head", (V, E), std=E ** -0.5), mat),
        "fc": store(normal(seed, "fc", (E, shape.feat_dim), std=shape.feat_dim ** -0.5), aux),
        "hidden_norm": store(normal(seed, "hidden_norm", (E,), std=0.1 ** 0.5, mean=1.0), aux),
        "output_norm": store(normal(seed, "output_norm", (E,), std=0.1 ** 0.5, mean=1.0), aux),
        "layers": [],
    }
    dims = {
        "wq": (shape.q_dim, E), "wk": (shape.kv_dim, E), "wv": (shape.kv_dim, E),
        "wo": (E, shape.q_dim), "w_gate": (F, E), "w_up": (F, E), "w_down": (E, F),
    }
    norms = {"attn_norm": E, "q_norm": shape.head_dim, "k_norm": shape.head_dim, "ffn_norm": E}
    for l in range(shape.n_layer):
        lw = {}
        for nm in LAYER_MATS:
            o, i = dims[nm]
            lw[nm] = store(normal(seed, f"layer{l}.{nm}", (o, i), std=i ** -0.5), mat)
        for nm in LAYER_NORMS:
            lw[nm] = store(normal(seed, f"layer{l}.{nm}", (norms[nm],), std=0.1 ** 0.5, mean=1.0), aux)
        w["layers"].append(lw)
    return w


def features(shape: Shape, T: int, feature_dtype: str, seed: int = 0, tag: str = "feats") -> np.ndarray:
    """Fused target features ``[T, n_capture * target_hidden]`` drawn N(0, 1)."""
    return store(normal(seed, tag, (T, shape.feat_dim)), feature_dtype)


def hidden(shape: Shape, T: int, seed: int = 0, tag: str = "hidden") -> np.ndarray:
    """Encoded context rows ``[T, n_embd]`` float32 drawn N(0, 1): a direct input of the inject call (the
    scale of an RMS-normed row), for workloads whose subject is not the encoder."""
    return normal(seed, tag, (T, shape.n_embd))


def step_inputs(shape: Shape, B: int, seed: int = 0, tag: str = "step") -> dict:
    """Per-step draws: id_last ~ U[0, V) and a planted mismatch index m ~ U{0..block-1}."""
    return {
        "id_last": integers(seed, tag + ".id_last", (B,), 0, shape.n_vocab),
        "mismatch": integers(seed, tag + ".mismatch", (B,), 0, shape.block),
        "filler": integers(seed, tag + ".filler", (B, shape.block - 1), 0, shape.n_vocab),
    }


def planted_targets(drafts: np.ndarray, mismatch: np.ndarray, filler: np.ndarray, n_vocab: int) -> np.ndarray:
    """Target tokens that copy ``drafts`` up to the planted index m, differ at m, and are filler after.

    m == block-1 (== drafts.shape[1]) plants no mismatch. This is harness logic
    (it builds a test input), not a step of the drafter.
    """
    drafts = np.asarray(drafts, dtype=np.int64)
    B, n = drafts.shape
    tgt = np.array(filler, dtype=np.int64, copy=True)
    for b in range(B):
        m = int(mismatch[b])
        tgt[b, :m] = drafts[b, :m]
        if m < n:
            tgt[b, m] = (drafts[b, m] + 1) % n_vocab
    return tgt.astype(np.int32)


def batch_n_past(B: int, lo: int = 64, hi: int = 6000, seed: int = 0) -> np.ndarray:
    """Per-sequence context lengths uniform in [lo, hi] for the cross-sequence batch workload."""
    return integers(seed, "batch.n_past", (B,), lo, hi + 1)
