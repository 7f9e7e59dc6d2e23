"""Plain fp64 CPU oracle of the DFlash drafter block step.

TEST INFRASTRUCTURE ONLY. This module is the yardstick that the HIP library is
checked against; it is imported only by the tests, by the smoke check and by
the benchmark's CPU-baseline leg. It shares no code with the HIP path and does
not import it. It is meant to be slow and obviously correct: NumPy in float64,
straight loops or single library matmuls, no blocking, no fusion.

Sources (cited by page title and section):

* dflash-ops card (Hugging Face kernels hub), "Method": features are injected
  through wk/wv with no attention norm in front; K is RMS-normed per head and
  NEOX-roped, V is stored raw; the block attends non-causally; the window masks
  only the deep past (0 <= qpos - kpos < window); drafts are greedy at block
  positions 1..15; rope angles use a host fp64 inverse-frequency table;
  arithmetic is fp32 regardless of storage dtype.
* dflash-ops card, "Requirements and limits": ring slot = pos % window, at
  most window tokens per inject call, later calls overwrite.
* dflash-ops card, "Usage": the noise block is [id_last, mask x 15]; logits are
  [16, n_vocab]; acceptance counts leading matches on the device.
* metrale dflash_head.rs page, DflashLayer: per-layer tensors
  (input/post-attention layernorms, q/k/v/o projections, q_norm/k_norm,
  gate/up/down); BlockDiffusionDraftHead: fc, hidden_norm, norm, rotary_dim =
  head_dim, RMSNorm epsilon 1e-6; DflashQuantization: weight-only FP8 E4M3 with
  per-row f32 scales on the seven layer GEMM weights and the LM head, KV cache
  bf16.
* dflash_engine.py page: RMSNorm (x * rsqrt(mean(x^2) + eps) * w),
  TargetContextFeatureFuser (H_t = RMSNorm(W_c [H^(l1); ...; H^(l5)])),
  DFlashKVInjectionAttention (K = [W_K H_t; W_K H_d], V likewise, scale
  1/sqrt(head_dim)), DFlashDraftBlock (pre-norm residual, SwiGLU
  w2(silu(w1 x) * w3 x)), DFlashSpeculativeVerifier.verify_block (prefix
  agreement length).

Readings where the pages are silent (each is listed in the design notes):
block row i sits at position n_past + i; the window test applies to ring keys
only; kv head of q head h is h // (n_head / n_head_kv); argmax ties go to the
lowest index; fp8 scale = amax/448 computed in float32, code = nearest-even
saturating E4M3FN of float32(w / scale); block q/k/v are never rounded to
storage, ring K/V are.

Storage rounding S(.) is emulated exactly: float32 storage rounds fp64 to the
nearest float32; bf16 rounds to the nearest bfloat16 (ties to even); fp8
weights are dequantised exactly as code_value * scale.

Parity pins: every function below is pinned by tests/test_oracle_pins.py
against closed forms, invariants, brute force or library routines. The
composition of the full block step (logits at real dimensions) has no printed
values on the pages; it is pinned only through its parts and the structural
invariants.
"""
from __future__ import annotations

import dataclasses

import numpy as np

F64 = np.float64


# ---------------------------------------------------------------------------
# Storage formats
# ---------------------------------------------------------------------------

def bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    """Exact value of bfloat16 bit patterns: the high half of a float32."""
    b = np.asarray(bits).astype(np.uint32) << 16
    with np.errstate(invalid="ignore"):
        return b.view(np.float32).astype(F64)


def round_bf16(x) -> np.ndarray:
    """Nearest bfloat16 value of fp64 ``x`` (ties to even), returned as fp64.

    bfloat16 keeps 8 significant bits and float32's exponent range, so the
    quantum of a normal value 2^e * m (0.5 <= m < 1) is 2^(e - 8), and that
    of a subnormal is 2^-133.
    """
    x = np.asarray(x, dtype=F64)
    _, e = np.frexp(x)
    qe = np.maximum(e - 8, -133)
    return np.ldexp(np.rint(np.ldexp(x, -qe)), qe)


def round_f32(x) -> np.ndarray:
    """Nearest float32 value of fp64 ``x``, returned as fp64."""
    return np.asarray(x, dtype=F64).astype(np.float32).astype(F64)


E4M3_MAX = 448.0


def round_e4m3(v) -> np.ndarray:
    """Nearest E4M3FN value (ties to even), saturating at +-448, as fp64.

    E4M3FN: 1 sign, 4 exponent (bias 7), 3 mantissa bits; normals 2^(E-7) *
    (1 + m/8) for E in 1..15 except the all-ones NaN code, subnormals
    2^-6 * m/8. A normal 2^e * f (0.5 <= f < 1) has quantum 2^(e - 4);
    subnormals have quantum 2^-9.
    """
    v = np.asarray(v, dtype=F64)
    a = np.abs(v)
    _, e = np.frexp(a)
    qe = np.maximum(e - 4, -9)
    r = np.ldexp(np.rint(np.ldexp(a, -qe)), qe)
    r = np.minimum(r, E4M3_MAX)
    return np.copysign(r, v)


def e4m3_encode(q) -> np.ndarray:
    """Code bytes of values that are already exact E4M3FN values (sign from the input's sign bit)."""
    q = np.asarray(q, dtype=F64)
    sign = np.signbit(q).astype(np.uint32)
    a = np.abs(q)
    m, e = np.frexp(a)  # a = m * 2^e, 0.5 <= m < 1 ; unbiased exponent of a is e - 1
    normal = a >= 2.0 ** -6
    exp_field = np.where(normal, e - 1 + 7, 0)
    mant = np.where(normal, (2.0 * m - 1.0) * 8.0, a * 2.0 ** 9)
    code = (sign << 7) | (exp_field.astype(np.uint32) << 3) | mant.astype(np.uint32)
    return code.astype(np.uint8)


def e4m3_decode(codes) -> np.ndarray:
    """Exact value of E4M3FN code bytes (NaN for the two NaN codes)."""
    c = np.asarray(codes).astype(np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    ex = (c >> 3) & 0xF
    mt = c & 0x7
    val = np.where(ex == 0, mt / 8.0 * 2.0 ** -6, (1.0 + mt / 8.0) * np.ldexp(1.0, ex - 7))
    val = np.where((c & 0x7F) == 0x7F, np.nan, val)
    return sign * val


def quantize_fp8_rows(w32: np.ndarray):
    """Weight-only FP8 E4M3 with one float32 scale per output row.

    metrale dflash_head.rs page, DflashQuantization: E4M3 copies with per-row
    f32 scales. Reading: scale_r = float32(amax_r / 448) (1 for an all-zero
    row); code = nearest-even saturating E4M3FN of float32(w / scale_r). The
    division is done in float32 on both sides because it decides the code.
    Returns (codes uint8 [N, K], scales float32 [N]).
    """
    w32 = np.ascontiguousarray(w32, dtype=np.float32)
    amax = np.max(np.abs(w32), axis=1)
    scale = (amax / np.float32(E4M3_MAX)).astype(np.float32)
    scale = np.where(amax == 0, np.float32(1.0), scale).astype(np.float32)
    v = (w32 / scale[:, None]).astype(np.float32)
    q = round_e4m3(v.astype(F64))
    return e4m3_encode(q), scale


def fp8_dequant(codes: np.ndarray, scales: np.ndarray) -> np.ndarray:
    return e4m3_decode(codes) * np.asarray(scales, dtype=F64)[:, None]


# ---------------------------------------------------------------------------
# Elementary operations
# ---------------------------------------------------------------------------

def rmsnorm(x: np.ndarray, w: np.ndarray, eps: float) -> np.ndarray:
    """x * rsqrt(mean(x^2) + eps) * w over the last axis (dflash_engine.py page, RMSNorm)."""
    x = np.asarray(x, dtype=F64)
    ms = np.mean(x * x, axis=-1, keepdims=True)
    return x / np.sqrt(ms + eps) * np.asarray(w, dtype=F64)


def inv_freq(base: float, head_dim: int) -> np.ndarray:
    """Host fp64 inverse-frequency table base^(-2i/head_dim), i < head_dim/2 (dflash-ops card, Method)."""
    i = np.arange(head_dim // 2, dtype=F64)
    return np.power(F64(base), -2.0 * i / head_dim)


def rope(x: np.ndarray, pos, freqs: np.ndarray) -> np.ndarray:
    """NEOX rotary embedding over the whole head (rotary_dim = head_dim).

    x: [..., D] with positions ``pos`` broadcast against x[..., 0]. Pairs are
    (i, i + D/2): x'_i = x_i cos t - x_{i+D/2} sin t, x'_{i+D/2} = x_i sin t +
    x_{i+D/2} cos t, t = pos * inv_freq[i] in fp64.
    """
    x = np.asarray(x, dtype=F64)
    half = x.shape[-1] // 2
    theta = np.asarray(pos, dtype=F64)[..., None] * freqs
    c, s = np.cos(theta), np.sin(theta)
    x1, x2 = x[..., :half], x[..., half:]
    return np.concatenate([x1 * c - x2 * s, x1 * s + x2 * c], axis=-1)


def silu(z: np.ndarray) -> np.ndarray:
    return z / (1.0 + np.exp(-z))


def linear(x: np.ndarray, w: np.ndarray) -> np.ndarray:
    """y = x W^T for a row-major [out, in] weight."""
    return np.asarray(x, dtype=F64) @ np.asarray(w, dtype=F64).T


# ---------------------------------------------------------------------------
# Model description
# ---------------------------------------------------------------------------

@dataclasses.dataclass
class Config:
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
    ring_dtype: str = "f32"  # "f32" or "bf16"

    @classmethod
    def from_shape(cls, shape, ring_dtype: str) -> "Config":
        fields = {f.name: getattr(shape, f.name) for f in dataclasses.fields(cls) if hasattr(shape, f.name)}
        return cls(ring_dtype=ring_dtype, **fields)


class Weights:
    """Drafter weights as fp64 values, decoded lazily from their storage form.

    ``raw`` is the dict produced by the synthetic workload generator; ``dtype``
    names its storage ("f32", "bf16" or "fp8"). For "fp8" the seven layer
    matrices and lm_head arrive as float32 masters and are quantised here, per
    row, by :func:`quantize_fp8_rows`.
    """

    MATS = ("wq", "wk", "wv", "wo", "w_gate", "w_up", "w_down")

    def __init__(self, raw: dict, dtype: str):
        self.raw, self.dtype = raw, dtype
        self._fp8 = {}

    def _aux(self, a):
        return bf16_to_f64(a) if a.dtype == np.uint16 else np.asarray(a, dtype=F64)

    def _mat(self, key, a):
        if self.dtype == "fp8":
            if key not in self._fp8:
                self._fp8[key] = quantize_fp8_rows(a)
            return fp8_dequant(*self._fp8[key])
        return self._aux(a)

    def fp8_codes(self, key):
        """(codes, scales) of a quantised matrix; key is "lm_head" or (layer, name)."""
        if key == "lm_head":
            a = self.raw["lm_head"]
        else:
            a = self.raw["layers"][key[0]][key[1]]
        if key not in self._fp8:
            self._fp8[key] = quantize_fp8_rows(a)
        return self._fp8[key]

    def glob(self, name):
        if name == "lm_head":
            return self._mat("lm_head", self.raw["lm_head"])
        return self._aux(self.raw[name])

    def layer(self, l, name):
        a = self.raw["layers"][l][name]
        return self._mat((l, name), a) if name in self.MATS else self._aux(a)

    def embed_rows(self, ids):
        t = self.raw["tok_embd"]
        return self._aux(t[np.asarray(ids, dtype=np.int64)])


class Ring:
    """Per-sequence sliding-window KV ring: K and V [n_layer][n_kv][window][head_dim] plus slot_pos[window].

    Values are held in fp64 but are always storage-rounded (ring dtype) when
    written. slot_pos is -1 for a slot never written (dflash-ops card,
    "Requirements and limits": slot = pos % window; the explicit position
    table is the reading adopted for which position each slot holds).
    """

    def __init__(self, cfg: Config):
        shp = (cfg.n_layer, cfg.n_head_kv, cfg.window, cfg.head_dim)
        self.K = np.zeros(shp, dtype=F64)
        self.V = np.zeros(shp, dtype=F64)
        self.slot_pos = np.full(cfg.window, -1, dtype=np.int64)
        self.written = np.zeros(cfg.window, dtype=bool)

    def copy(self) -> "Ring":
        r = Ring.__new__(Ring)
        r.K, r.V, r.slot_pos, r.written = self.K.copy(), self.V.copy(), self.slot_pos.copy(), self.written.copy()
        return r


def storage_round(x, dtype: str):
    if dtype == "f32":
        return round_f32(x)
    if dtype == "bf16":
        return round_bf16(x)
    raise ValueError(dtype)


def feature_values(feats: np.ndarray) -> np.ndarray:
    return bf16_to_f64(feats) if feats.dtype == np.uint16 else np.asarray(feats, dtype=F64)


# ---------------------------------------------------------------------------
# Encode and inject
# ---------------------------------------------------------------------------

def encode(cfg: Config, w: Weights, feats: np.ndarray) -> np.ndarray:
    """Cross-layer feature fusion H_t = RMSNorm(W_c [H^(l1); ...; H^(l5)]).

    dflash_engine.py page, TargetContextFeatureFuser; metrale dflash_head.rs
    page, BlockDiffusionDraftHead (fc then hidden_norm). feats: [T, n_capture *
    target_hidden] in storage form. Returns h [T, n_embd] fp64 (activations are
    not rounded to storage).
    """
    y = linear(feature_values(feats), w.glob("fc"))
    return rmsnorm(y, w.glob("hidden_norm"), cfg.rms_eps)


def inject(cfg: Config, w: Weights, ring: Ring, h: np.ndarray, positions) -> None:
    """Write context K/V for every layer into the ring (dflash-ops card, Method and Requirements).

    For each layer l, position t and kv head j: k = rope(rmsnorm(h_t Wk_l^T)[j]
    * k_norm_l, pos_t), v = (h_t Wv_l^T)[j]; both rounded to the ring dtype and
    stored at slot pos_t % window; slot_pos[slot] = pos_t. No attention norm is
    applied to h before wk/wv. At most ``window`` positions per call, with
    distinct slots.
    """
    pos = np.asarray(positions, dtype=np.int64)
    T = pos.shape[0]
    assert T <= cfg.window, "at most window positions per inject call"
    slots = pos % cfg.window
    assert len(np.unique(slots)) == T, "positions of one call must map to distinct slots"
    freqs = inv_freq(cfg.rope_base, cfg.head_dim)
    D, Hkv = cfg.head_dim, cfg.n_head_kv
    for l in range(cfg.n_layer):
        k = linear(h, w.layer(l, "wk")).reshape(T, Hkv, D)
        v = linear(h, w.layer(l, "wv")).reshape(T, Hkv, D)
        k = rmsnorm(k, w.layer(l, "k_norm"), cfg.rms_eps)
        k = rope(k, pos[:, None], freqs)
        for t in range(T):
            ring.K[l, :, slots[t], :] = storage_round(k[t], cfg.ring_dtype)
            ring.V[l, :, slots[t], :] = storage_round(v[t], cfg.ring_dtype)
    ring.slot_pos[slots] = pos
    ring.written[slots] = True


# ---------------------------------------------------------------------------
# Block step
# ---------------------------------------------------------------------------

def visible_slots(cfg: Config, ring: Ring, qpos: int) -> np.ndarray:
    """Ring slots a query at ``qpos`` attends: written, and 0 <= qpos - slot_pos < window."""
    d = qpos - ring.slot_pos
    return np.nonzero((ring.slot_pos >= 0) & (d >= 0) & (d < cfg.window))[0]


def attention(cfg: Config, ring: Ring, l: int, q, kb, vb, n_past: int) -> np.ndarray:
    """Non-causal sliding-window GQA attention of the block against ring plus block.

    q: [block, n_head, D]; kb, vb: [block, n_kv, D] (the block's own keys and
    values, unrounded). Row i (position n_past + i), head h, kv head j = h // G
    sees the visible ring slots and all block rows; one softmax over both;
    scale 1/sqrt(D). Returns [block, n_head * D].
    """
    G = cfg.n_head // cfg.n_head_kv
    D = cfg.head_dim
    out = np.zeros((cfg.block, cfg.n_head, D), dtype=F64)
    for i in range(cfg.block):
        vis = visible_slots(cfg, ring, n_past + i)
        for h in range(cfg.n_head):
            j = h // G
            keys = np.concatenate([ring.K[l, j, vis, :], kb[:, j, :]], axis=0)
            vals = np.concatenate([ring.V[l, j, vis, :], vb[:, j, :]], axis=0)
            s = keys @ q[i, h] / np.sqrt(D)
            p = np.exp(s - s.max())
            p /= p.sum()
            out[i, h] = p @ vals
    return out.reshape(cfg.block, cfg.n_head * D)


def block_forward(cfg: Config, w: Weights, ring: Ring, block_ids, n_past: int, return_hidden: bool = False):
    """Logits [block, n_vocab] of one sequence's block through all drafter layers.

    Qwen3-style layer (metrale dflash_head.rs page, module doc and DflashLayer;
    dflash_engine.py page, DFlashDraftBlock): h = rmsnorm(x) * attn_norm;
    q/k/v projections; per-head rmsnorm with q_norm / k_norm and NEOX rope at
    position n_past + i; attention; x += o Wo^T; h2 = rmsnorm(x) * ffn_norm;
    x += (silu(h2 Wg^T) * (h2 Wu^T)) Wd^T. Output: rmsnorm(x) * output_norm
    times lm_head^T.
    """
    ids = np.asarray(block_ids, dtype=np.int64)
    assert ids.shape == (cfg.block,)
    freqs = inv_freq(cfg.rope_base, cfg.head_dim)
    qpos = n_past + np.arange(cfg.block)
    D, H, Hkv = cfg.head_dim, cfg.n_head, cfg.n_head_kv
    x = w.embed_rows(ids)
    for l in range(cfg.n_layer):
        h = rmsnorm(x, w.layer(l, "attn_norm"), cfg.rms_eps)
        q = linear(h, w.layer(l, "wq")).reshape(cfg.block, H, D)
        k = linear(h, w.layer(l, "wk")).reshape(cfg.block, Hkv, D)
        v = linear(h, w.layer(l, "wv")).reshape(cfg.block, Hkv, D)
        q = rope(rmsnorm(q, w.layer(l, "q_norm"), cfg.rms_eps), qpos[:, None], freqs)
        k = rope(rmsnorm(k, w.layer(l, "k_norm"), cfg.rms_eps), qpos[:, None], freqs)
        o = attention(cfg, ring, l, q, k, v, n_past)
        x = x + linear(o, w.layer(l, "wo"))
        h2 = rmsnorm(x, w.layer(l, "ffn_norm"), cfg.rms_eps)
        a = silu(linear(h2, w.layer(l, "w_gate"))) * linear(h2, w.layer(l, "w_up"))
        x = x + linear(a, w.layer(l, "w_down"))
    logits = linear(rmsnorm(x, w.glob("output_norm"), cfg.rms_eps), w.glob("lm_head"))
    return (logits, x) if return_hidden else logits


def block_forward_batch(cfg: Config, w: Weights, rings, ids, n_pasts) -> np.ndarray:
    """Logits [B, block, n_vocab] of B independent sequences.

    metrale dflash_head.rs page, DflashBatch: the rows of all sequences go
    through every weight projection together (sequence-major), while
    attention runs per sequence against that sequence's own ring at its own
    n_past. The operations are those of :func:`block_forward`; only the row
    count of each matmul differs, and each weight matrix is decoded from its
    storage form once for all rows.
    """
    ids = np.asarray(ids, dtype=np.int64)
    B = ids.shape[0]
    assert ids.shape == (B, cfg.block) and len(rings) == B and len(n_pasts) == B
    freqs = inv_freq(cfg.rope_base, cfg.head_dim)
    qpos = np.asarray(n_pasts, dtype=np.int64)[:, None] + np.arange(cfg.block)[None, :]  # [B, block]
    D, H, Hkv, R = cfg.head_dim, cfg.n_head, cfg.n_head_kv, B * cfg.block
    x = w.embed_rows(ids.reshape(-1))
    for l in range(cfg.n_layer):
        h = rmsnorm(x, w.layer(l, "attn_norm"), cfg.rms_eps)
        q = linear(h, w.layer(l, "wq")).reshape(B, cfg.block, H, D)
        k = linear(h, w.layer(l, "wk")).reshape(B, cfg.block, Hkv, D)
        v = linear(h, w.layer(l, "wv")).reshape(B, cfg.block, Hkv, D)
        q = rope(rmsnorm(q, w.layer(l, "q_norm"), cfg.rms_eps), qpos[:, :, None], freqs)
        k = rope(rmsnorm(k, w.layer(l, "k_norm"), cfg.rms_eps), qpos[:, :, None], freqs)
        o = np.concatenate([attention(cfg, rings[b], l, q[b], k[b], v[b], int(n_pasts[b])) for b in range(B)])
        x = x + linear(o.reshape(R, H * D), w.layer(l, "wo"))
        h2 = rmsnorm(x, w.layer(l, "ffn_norm"), cfg.rms_eps)
        a = silu(linear(h2, w.layer(l, "w_gate"))) * linear(h2, w.layer(l, "w_up"))
        x = x + linear(a, w.layer(l, "w_down"))
    logits = linear(rmsnorm(x, w.glob("output_norm"), cfg.rms_eps), w.glob("lm_head"))
    return logits.reshape(B, cfg.block, -1)


def block_ids(cfg: Config, id_last: int) -> np.ndarray:
    """The noise block [id_last, mask x (block-1)] (dflash-ops card, Usage and Method)."""
    ids = np.full(cfg.block, cfg.mask_id, dtype=np.int64)
    ids[0] = id_last
    return ids


def greedy_drafts(logits: np.ndarray) -> np.ndarray:
    """argmax over the vocabulary at block positions 1..block-1; position 0 is unused; ties to the lowest index."""
    return np.argmax(np.asarray(logits)[1:], axis=-1).astype(np.int32)


# --------------------------------------------------------------------------- sampling
PHILOX_M = (0xD2511F53, 0xCD9E8D57)   # round multipliers of Philox-4x32
PHILOX_W = (0x9E3779B9, 0xBB67AE85)   # key increments (Weyl sequence) between rounds
MASK32 = 0xFFFFFFFF


def philox4x32_10(counter, key):
    """Philox-4x32 with 10 rounds (Salmon, Moraes, Dror and Shaw, "Parallel random numbers: as easy as
    1, 2, 3", SC 2011), elementwise over arrays: counter = (c0, c1, c2, c3), key = (k0, k1), each an
    array (or scalar) of unsigned 32-bit values. Returns the four output words."""
    c = [np.asarray(x, dtype=np.uint64) & MASK32 for x in counter]
    k0 = np.asarray(key[0], dtype=np.uint64) & MASK32
    k1 = np.asarray(key[1], dtype=np.uint64) & MASK32
    for r in range(10):
        if r > 0:
            k0 = (k0 + PHILOX_W[0]) & MASK32
            k1 = (k1 + PHILOX_W[1]) & MASK32
        p0 = c[0] * np.uint64(PHILOX_M[0])  # exact: both factors < 2^32
        p1 = c[2] * np.uint64(PHILOX_M[1])
        hi0, lo0 = p0 >> np.uint64(32), p0 & MASK32
        hi1, lo1 = p1 >> np.uint64(32), p1 & MASK32
        c = [hi1 ^ c[1] ^ k0, lo1, hi0 ^ c[3] ^ k1, lo0]
    return [x.astype(np.uint32) for x in c]


def gumbel_noise(seed: int, b: int, positions, n_vocab: int) -> np.ndarray:
    """Gumbel(0, 1) noise [len(positions), n_vocab] for sequence b: u = (x0 >> 8) + 1/2 scaled by 2^-24,
    x0 the first Philox output word at counter (position, vocab id, b, 0) under key (seed low, seed high),
    and g = -log(-log(u)) in fp64. The 24-bit u is exact in fp32 and fp64 alike."""
    pos = np.asarray(positions, dtype=np.uint64)[:, None]
    n = np.arange(n_vocab, dtype=np.uint64)[None, :]
    x0 = philox4x32_10((pos + 0 * n, n + 0 * pos, np.uint64(b), np.uint64(0)),
                       (seed & MASK32, (seed >> 32) & MASK32))[0]
    u = ((x0 >> np.uint32(8)).astype(F64) + 0.5) * 2.0 ** -24
    return -np.log(-np.log(u))


def sampled_drafts(logits: np.ndarray, temperature: float, seed: int, b: int, n_past: int) -> np.ndarray:
    """Temperature sampling of the drafts (dflash_engine.py page, DFlashDraftModel.forward: a draw from
    softmax(logits / T) at block positions 1..block-1), by the Gumbel-max rule: the draft at row i is
    argmax over the vocabulary of logits[i] / T + g[i], g the Gumbel noise of position n_past + i
    (ties to the lowest index). T = 0 is the greedy draft."""
    logits = np.asarray(logits, dtype=F64)
    if temperature == 0.0:
        return greedy_drafts(logits)
    g = gumbel_noise(seed, b, n_past + np.arange(1, logits.shape[0]), logits.shape[1])
    return np.argmax(logits[1:] / temperature + g, axis=-1).astype(np.int32)


def block_step(cfg: Config, w: Weights, ring: Ring, id_last: int, n_past: int):
    """(logits [block, V], drafts [block-1]) of one sequence."""
    logits = block_forward(cfg, w, ring, block_ids(cfg, id_last), n_past)
    return logits, greedy_drafts(logits)


def accept(drafts, target) -> int:
    """First-mismatch acceptance: number of leading drafts equal to the target's tokens.

    dflash-ops card, Usage (``accept``); dflash_engine.py page,
    DFlashSpeculativeVerifier.verify_block (prefix agreement length k_match).
    The bonus token is not produced here.
    """
    n = 0
    for d, t in zip(drafts, target):
        if int(d) != int(t):
            break
        n += 1
    return n


def verify(drafts, target):
    """Acceptance with the bonus token: (k_match, bonus, accepted tokens).

    dflash_engine.py page, DFlashSpeculativeVerifier.verify_block: ``target``
    holds the target's tokens (its argmax) at the len(drafts) draft positions
    and at one more position; k_match drafts are accepted and the target's
    token at index k_match is appended, so tau = k_match + 1 tokens.
    """
    assert len(target) == len(drafts) + 1
    k = accept(drafts, target[:len(drafts)])
    bonus = int(target[k])
    return k, bonus, [int(d) for d in drafts[:k]] + [bonus]
