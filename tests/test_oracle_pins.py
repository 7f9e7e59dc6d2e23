"""Pins of the CPU oracle against what the pages and mathematics fix.

Nothing here re-types an oracle formula: each check compares the oracle with
a library routine (torch casts, torch rms_norm / silu / scaled_dot_product_
attention, numpy complex arithmetic), a closed form, an invariant, brute force
over a tiny input, or the pages' worked example.
"""
import json
import os

import numpy as np
import pytest
import torch

from block_diffusion_drafter_02_amd import synth
from oracle import dflash_oracle as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# --------------------------------------------------------------------------- storage formats

def test_bf16_round_matches_torch_cast():
    rng = np.random.default_rng(1)
    x = np.concatenate([
        rng.standard_normal(20000).astype(np.float32) * np.float32(10.0) ** rng.integers(-30, 30, 20000),
        np.array([0.0, -0.0, 1.0, -1.0, 3.0e38, 1e-40, -1e-42], np.float32),
    ]).astype(np.float32)
    # exact ties: a bf16 value plus half its ulp
    base = torch.from_numpy(rng.standard_normal(5000).astype(np.float32)).to(torch.bfloat16).float().numpy()
    ulp = np.abs(base) * 2.0 ** -7
    _, e = np.frexp(base)
    half = np.ldexp(1.0, e - 9).astype(np.float32)
    ties = (base + half).astype(np.float32)
    x = np.concatenate([x, ties])
    want = torch.from_numpy(x).to(torch.bfloat16).double().numpy()
    got = O.round_bf16(x.astype(np.float64))
    np.testing.assert_array_equal(got, want)
    assert ulp.size  # keep the ulp computation meaningful for readers


def test_bf16_decode_matches_torch():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    want = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).double().numpy()
    got = O.bf16_to_f64(bits)
    ok = ~np.isnan(want)
    np.testing.assert_array_equal(got[ok], want[ok])
    assert np.all(np.isnan(got[~ok]))


def test_e4m3_decode_all_codes_matches_torch():
    codes = np.arange(256, dtype=np.uint8)
    want = torch.from_numpy(codes).view(torch.float8_e4m3fn).double().numpy()
    got = O.e4m3_decode(codes)
    nan = np.isnan(want)
    assert nan.sum() == 2 and np.all(np.isnan(got[nan]))
    np.testing.assert_array_equal(got[~nan], want[~nan])


def test_e4m3_round_matches_torch_cast_in_range():
    rng = np.random.default_rng(2)
    x = (rng.standard_normal(50000) * 100.0).astype(np.float32)
    x = np.clip(x, -448, 448)
    x = np.concatenate([x, (rng.standard_normal(5000) * 1e-2).astype(np.float32)])
    # ties: midpoints between consecutive representable values
    vals = np.unique(np.abs(O.e4m3_decode(np.arange(0, 127, dtype=np.uint8))))
    mids = ((vals[1:] + vals[:-1]) / 2).astype(np.float32)
    x = np.concatenate([x, mids, -mids])
    want = torch.from_numpy(x).to(torch.float8_e4m3fn).double().numpy()
    got = O.round_e4m3(x.astype(np.float64))
    np.testing.assert_array_equal(got, want)


def test_e4m3_saturates_instead_of_nan():
    got = O.round_e4m3(np.array([448.0, 460.0, 470.0, 1e6, -1e6]))
    np.testing.assert_array_equal(got, [448.0, 448.0, 448.0, 448.0, -448.0])


def test_e4m3_encode_roundtrips_every_code():
    codes = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], dtype=np.uint8)
    vals = O.e4m3_decode(codes)
    vals = np.where(codes == 0x80, -0.0, vals)
    np.testing.assert_array_equal(O.e4m3_encode(vals), codes)


def test_quantize_fp8_rows_properties():
    rng = np.random.default_rng(3)
    w = (rng.standard_normal((64, 200)) / np.sqrt(200)).astype(np.float32)
    w[5] = 0.0
    codes, scale = O.quantize_fp8_rows(w)
    assert codes.dtype == np.uint8 and scale.dtype == np.float32
    amax = np.abs(w).max(axis=1)
    # scale is float32(amax / 448), 1 for an all-zero row
    expect = np.where(amax == 0, 1.0, (torch.from_numpy(amax) / 448.0).numpy()).astype(np.float32)
    np.testing.assert_array_equal(scale, expect)
    deq = O.fp8_dequant(codes, scale)
    np.testing.assert_array_equal(deq[5], 0.0)
    # the largest element of each non-zero row lands on +-448
    rows = [r for r in range(64) if r != 5]
    arg = np.abs(w[rows]).argmax(axis=1)
    np.testing.assert_array_equal(np.abs(O.e4m3_decode(codes[rows, arg])), 448.0)
    # error bound: half the E4M3 quantum at the value's binade (2^-9 for subnormals), times the scale
    v = np.abs(w.astype(np.float64) / scale[:, None].astype(np.float64))
    _, e = np.frexp(v)
    quantum = np.ldexp(1.0, np.maximum(e - 4, -9))
    err = np.abs(deq - w) / scale[:, None]
    assert np.all(err <= quantum / 2 * (1 + 1e-6) + 1e-12)
    # codes agree with torch's own E4M3 cast of float32(w / scale)
    v32 = (torch.from_numpy(w) / torch.from_numpy(scale)[:, None])
    tq = v32.to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    np.testing.assert_array_equal(codes, tq)


# --------------------------------------------------------------------------- elementary ops

def test_rmsnorm_constant_vector_closed_form():
    c, eps = 3.5, 1e-6
    w = np.linspace(0.5, 1.5, 32)
    got = O.rmsnorm(np.full(32, c), w, eps)
    np.testing.assert_allclose(got, c / np.sqrt(c * c + eps) * w, rtol=1e-15)


def test_rmsnorm_matches_torch():
    rng = np.random.default_rng(4)
    x = rng.standard_normal((7, 96)) * 3
    w = 1 + 0.3 * rng.standard_normal(96)
    want = torch.nn.functional.rms_norm(torch.from_numpy(x), (96,), torch.from_numpy(w), eps=1e-6).numpy()
    np.testing.assert_allclose(O.rmsnorm(x, w, 1e-6), want, rtol=1e-13, atol=1e-14)


def test_inv_freq_closed_forms():
    for base, D in [(10000.0, 64), (10000.0, 128), (500000.0, 128)]:
        f = O.inv_freq(base, D)
        assert f.shape == (D // 2,) and f[0] == 1.0
        np.testing.assert_allclose(f[D // 4], base ** -0.5, rtol=1e-15)
        np.testing.assert_allclose(f[1:] / f[:-1], base ** (-2.0 / D), rtol=1e-13)
        assert np.all(np.diff(f) < 0)


def _rope_complex(x, pos, base):
    """Textbook rotary embedding as a complex product (x_i + i x_{i+D/2}) e^{i pos w_i}, w_i = base^(-2i/D)."""
    D = x.shape[-1]
    w = np.array([base ** (-2.0 * i / D) for i in range(D // 2)])
    z = (x[..., : D // 2] + 1j * x[..., D // 2:]) * np.exp(1j * np.asarray(pos, np.float64)[..., None] * w)
    return np.concatenate([z.real, z.imag], axis=-1)


def test_rope_matches_complex_product_and_identities():
    rng = np.random.default_rng(5)
    D, base = 64, 10000.0
    f = O.inv_freq(base, D)
    x = rng.standard_normal((9, D))
    pos = np.array([0, 1, 2, 17, 79, 1000, 2047, 2300, 6015])
    got = O.rope(x, pos, f)
    np.testing.assert_allclose(got, _rope_complex(x, pos, base), rtol=1e-12, atol=1e-12)
    np.testing.assert_array_equal(O.rope(x, np.zeros(9), f), x)  # position 0 is the identity
    # pair norms preserved
    n0 = x[:, : D // 2] ** 2 + x[:, D // 2:] ** 2
    n1 = got[:, : D // 2] ** 2 + got[:, D // 2:] ** 2
    np.testing.assert_allclose(n1, n0, rtol=1e-12)
    # composition: rope(rope(x, a), b) == rope(x, a + b)
    a, b = pos, pos[::-1]
    np.testing.assert_allclose(O.rope(O.rope(x, a, f), b, f), O.rope(x, a + b, f), rtol=1e-9, atol=1e-10)
    # relative property: <rope(q, m), rope(k, n)> depends only on m - n
    q, k = rng.standard_normal(D), rng.standard_normal(D)
    d1 = O.rope(q, 2100, f) @ O.rope(k, 2000, f)
    d2 = O.rope(q, 100, f) @ O.rope(k, 0, f)
    np.testing.assert_allclose(d1, d2, rtol=1e-9)


def test_silu_matches_torch():
    z = np.linspace(-30, 30, 1001)
    np.testing.assert_allclose(O.silu(z), torch.nn.functional.silu(torch.from_numpy(z)).numpy(), rtol=1e-14, atol=1e-300)


def test_linear_orientation_and_exactness():
    rng = np.random.default_rng(6)
    x = rng.integers(-8, 8, (5, 12)).astype(np.float64)
    W = rng.integers(-8, 8, (7, 12)).astype(np.float64)
    want = np.array([[sum(x[i, k] * W[n, k] for k in range(12)) for n in range(7)] for i in range(5)])
    np.testing.assert_array_equal(O.linear(x, W), want)
    P = np.eye(12)[[3, 0, 11, 5]]  # a selection: y[:, r] = x[:, sel[r]]
    np.testing.assert_array_equal(O.linear(x, P), x[:, [3, 0, 11, 5]])


# --------------------------------------------------------------------------- small model helpers

PIN = synth.Shape(n_layer=1, n_embd=64, n_head=4, n_head_kv=2, head_dim=32, n_ff=64,
                  window=16, block=16, n_vocab=40, n_capture=2, target_hidden=32)


def _model(shape, wdtype="f32", ring="f32", seed=0):
    cfg = O.Config.from_shape(shape, ring)
    raw = synth.weights(shape, wdtype, seed=seed)
    return cfg, raw, O.Weights(raw, wdtype)


def _filled_ring(cfg, w, n_past, seed=0, base_pos=0, feats=None):
    """Ring after injecting positions base_pos .. base_pos + n_past - 1 in window-sized chunks."""
    ring = O.Ring(cfg)
    shape = synth.Shape(**{k: getattr(cfg, k) for k in ("n_layer", "n_embd", "n_head", "n_head_kv", "head_dim",
                                                         "n_ff", "window", "block", "n_vocab", "n_capture",
                                                         "target_hidden")})
    if feats is None:
        feats = synth.features(shape, n_past, "f32", seed=seed)
    h = O.encode(cfg, w, feats)
    for c0 in range(0, n_past, cfg.window):
        c1 = min(n_past, c0 + cfg.window)
        O.inject(cfg, w, ring, h[c0:c1], np.arange(c0, c1) + base_pos)
    return ring, feats


def test_encode_selector_reduces_to_rmsnorm_of_one_capture():
    cfg, raw, w = _model(PIN)
    E, Et = PIN.n_embd, PIN.target_hidden
    fc = np.zeros((E, PIN.feat_dim), np.float32)
    fc[:Et, :Et] = np.eye(Et)          # rows 0..Et-1 pick capture 0
    fc[Et:, Et:2 * Et] = np.eye(Et)    # rows Et.. pick capture 1
    raw["fc"] = fc
    X = synth.features(PIN, 5, "f32", seed=9)
    sel = np.concatenate([X[:, :Et], X[:, Et:2 * Et]], axis=1).astype(np.float64)
    want = torch.nn.functional.rms_norm(torch.from_numpy(sel), (E,), torch.from_numpy(raw["hidden_norm"].astype(np.float64)), eps=1e-6).numpy()
    np.testing.assert_allclose(O.encode(cfg, w, X), want, rtol=1e-12, atol=1e-14)


def test_inject_stores_raw_v_and_normed_roped_k():
    cfg, raw, w = _model(PIN)
    D, Hkv = PIN.head_dim, PIN.n_head_kv
    sel = np.zeros((Hkv * D, PIN.n_embd), np.float32)
    perm = np.random.default_rng(7).permutation(PIN.n_embd)[: Hkv * D]
    sel[np.arange(Hkv * D), perm] = 1.0
    raw["layers"][0]["wk"] = sel
    raw["layers"][0]["wv"] = sel[::-1].copy()
    h = np.random.default_rng(8).standard_normal((3, PIN.n_embd))
    ring = O.Ring(cfg)
    pos = np.array([5, 22, 40])  # slots 5, 6, 8
    O.inject(cfg, w, ring, h, pos)
    kn = raw["layers"][0]["k_norm"].astype(np.float64)
    for t, p in enumerate(pos):
        s = p % PIN.window
        k = h[t, perm].reshape(Hkv, D)
        k = torch.nn.functional.rms_norm(torch.from_numpy(k), (D,), torch.from_numpy(kn), eps=1e-6).numpy()
        k = _rope_complex(k, np.full(Hkv, p), PIN.rope_base)
        np.testing.assert_allclose(ring.K[0, :, s], np.float32(k).astype(np.float64), rtol=1e-6, atol=1e-7)
        v = h[t, perm[::-1]].reshape(Hkv, D)
        np.testing.assert_array_equal(ring.V[0, :, s], v.astype(np.float32).astype(np.float64))
    assert list(ring.slot_pos[[5, 6, 8]]) == [5, 22, 40]
    assert np.all(ring.slot_pos[[0, 1, 2, 3, 4, 7] + list(range(9, 16))] == -1)


def test_inject_ring_wraparound_tiny():
    cfg, raw, w = _model(synth.TINY)
    ring, feats = _filled_ring(cfg, w, 80)
    s = np.arange(64)
    np.testing.assert_array_equal(ring.slot_pos, np.where(s < 16, 64 + s, s))
    # the wrapped slots hold exactly what injecting that position alone would store
    h = O.encode(cfg, w, feats)
    for p in (64, 70, 79):
        solo = O.Ring(cfg)
        O.inject(cfg, w, solo, h[p:p + 1], [p])
        np.testing.assert_array_equal(ring.K[:, :, p % 64], solo.K[:, :, p % 64])
        np.testing.assert_array_equal(ring.V[:, :, p % 64], solo.V[:, :, p % 64])


def test_inject_rejects_oversized_and_colliding_calls():
    cfg, raw, w = _model(PIN)
    h = np.zeros((17, PIN.n_embd))
    with pytest.raises(AssertionError):
        O.inject(cfg, w, O.Ring(cfg), h, np.arange(17))
    with pytest.raises(AssertionError):
        O.inject(cfg, w, O.Ring(cfg), h[:2], [3, 19])


def test_bf16_ring_is_rounded():
    cfg, raw, w = _model(PIN, "bf16", "bf16")
    ring, _ = _filled_ring(cfg, w, 16)
    np.testing.assert_array_equal(O.round_bf16(ring.K), ring.K)
    np.testing.assert_array_equal(O.round_bf16(ring.V), ring.V)


# --------------------------------------------------------------------------- attention

def _visible_brute(n_past, window, qpos, slot_pos):
    """Visible slots by walking every position < n_past and asking where it lives."""
    out = []
    for s in range(window):
        p = slot_pos[s]
        if p >= 0 and qpos - window < p <= qpos:
            out.append(s)
    return out


def test_attention_with_zero_query_is_mean_of_visible_values():
    cfg, raw, w = _model(synth.TINY)
    ring, _ = _filled_ring(cfg, w, 80)
    rng = np.random.default_rng(10)
    q = np.zeros((16, 4, 64))
    kb, vb = rng.standard_normal((16, 1, 64)), rng.standard_normal((16, 1, 64))
    o = O.attention(cfg, ring, 0, q, kb, vb, 80).reshape(16, 4, 64)
    for i in range(16):
        # position p is visible to row i iff 80 + i - 64 < p <= 79, i.e. p >= 17 + i
        positions = list(range(17 + i, 80))
        assert len(positions) == 63 - i
        assert sorted(_visible_brute(80, 64, 80 + i, ring.slot_pos)) == sorted(p % 64 for p in positions)
        vals = np.concatenate([ring.V[0, 0, [p % 64 for p in positions]], vb[:, 0]], axis=0)
        for h in range(4):
            np.testing.assert_allclose(o[i, h], vals.mean(axis=0), rtol=1e-12, atol=1e-13)


def test_attention_without_window_matches_sdpa_with_gqa():
    shape = synth.Shape(n_layer=1, n_embd=64, n_head=4, n_head_kv=2, head_dim=32, n_ff=64,
                        window=64, block=16, n_vocab=40, n_capture=2, target_hidden=32)
    cfg, raw, w = _model(shape)
    ring, _ = _filled_ring(cfg, w, 40)  # W >= n_past + block: nothing is masked
    rng = np.random.default_rng(11)
    q = rng.standard_normal((16, 4, 32))
    kb, vb = rng.standard_normal((16, 2, 32)), rng.standard_normal((16, 2, 32))
    got = O.attention(cfg, ring, 0, q, kb, vb, 40).reshape(16, 4, 32)
    K = np.concatenate([ring.K[0][:, :40].transpose(1, 0, 2), kb], axis=0)  # [56, 2, 32]
    V = np.concatenate([ring.V[0][:, :40].transpose(1, 0, 2), vb], axis=0)
    Kt = torch.from_numpy(K).permute(1, 0, 2).repeat_interleave(2, dim=0)  # kv head of q head h is h // 2
    Vt = torch.from_numpy(V).permute(1, 0, 2).repeat_interleave(2, dim=0)
    Qt = torch.from_numpy(q).permute(1, 0, 2)
    want = torch.nn.functional.scaled_dot_product_attention(Qt, Kt, Vt).permute(1, 0, 2).numpy()
    np.testing.assert_allclose(got, want, rtol=1e-11, atol=1e-12)


def test_gqa_head_map_consecutive_heads_share_a_kv_head():
    cfg, raw, w = _model(PIN)
    ring = O.Ring(cfg)
    ring.slot_pos[:] = np.arange(16)
    ring.V[0, 0] = 1.0
    ring.V[0, 1] = -1.0
    o = O.attention(cfg, ring, 0, np.zeros((16, 4, 32)), np.zeros((16, 2, 32)), np.zeros((16, 2, 32)), 16)
    o = o.reshape(16, 4, 32)
    # row 0 sees 15 ring slots (positions 1..15) and 16 zero block values
    np.testing.assert_allclose(o[0, :2], 15 / 31)
    np.testing.assert_allclose(o[0, 2:], -15 / 31)


# --------------------------------------------------------------------------- whole block

def test_zero_attention_and_mlp_outputs_reduce_to_embedding_then_head():
    cfg, raw, w = _model(PIN)
    raw["layers"][0]["wo"][:] = 0
    raw["layers"][0]["w_down"][:] = 0
    ring, _ = _filled_ring(cfg, w, 20)
    ids = np.array([7] + [0] * 15)
    logits = O.block_forward(cfg, w, ring, ids, 20)
    x = torch.from_numpy(raw["tok_embd"][ids].astype(np.float64))
    h = torch.nn.functional.rms_norm(x, (PIN.n_embd,), torch.from_numpy(raw["output_norm"].astype(np.float64)), eps=1e-6)
    want = (h @ torch.from_numpy(raw["lm_head"].astype(np.float64)).T).numpy()
    np.testing.assert_allclose(logits, want, rtol=1e-12, atol=1e-13)


def test_swiglu_residual_structure():
    cfg, raw, w = _model(PIN)
    E = PIN.n_embd
    perm = np.random.default_rng(12).permutation(E)
    raw["layers"][0]["wo"][:] = 0
    raw["layers"][0]["w_gate"] = np.eye(E, dtype=np.float32)
    raw["layers"][0]["w_up"] = 2 * np.eye(E, dtype=np.float32)
    raw["layers"][0]["w_down"] = np.eye(E, dtype=np.float32)[perm]
    raw["lm_head"] = np.eye(PIN.n_vocab, E, dtype=np.float32)
    raw["output_norm"] = np.ones(E, np.float32)
    ring, _ = _filled_ring(cfg, w, 20)
    ids = np.array([3] + [0] * 15)
    logits, x = O.block_forward(cfg, w, ring, ids, 20, return_hidden=True)
    x0 = torch.from_numpy(raw["tok_embd"][ids].astype(np.float64))
    h2 = torch.nn.functional.rms_norm(x0, (E,), torch.from_numpy(raw["layers"][0]["ffn_norm"].astype(np.float64)), eps=1e-6)
    a = torch.nn.functional.silu(h2) * (2 * h2)  # silu(gate) times up
    want = x0 + a[:, perm]
    np.testing.assert_allclose(x, want.numpy(), rtol=1e-12, atol=1e-13)


def test_window_mask_perturbation_tiny():
    """Perturbing the slot of position p changes rows i <= p - 17 only; other rows stay bitwise equal."""
    cfg, raw, w = _model(synth.TINY)
    ring, _ = _filled_ring(cfg, w, 80)
    ids = O.block_ids(cfg, 123)
    base = O.block_forward(cfg, w, ring, ids, 80)
    for p in (20, 30, 79):
        r2 = ring.copy()
        r2.K[:, :, p % 64] += 0.5
        r2.V[:, :, p % 64] -= 0.5
        got = O.block_forward(cfg, w, r2, ids, 80)
        for i in range(16):
            if i <= p - 17:
                assert np.abs(got[i] - base[i]).max() > 1e-9, (p, i)
            else:
                np.testing.assert_array_equal(got[i], base[i])
    # a slot holding a position that no row can see (position 16, slot 16) changes nothing
    r3 = ring.copy()
    assert r3.slot_pos[16] == 16
    r3.K[:, :, 16] += 3.0
    np.testing.assert_array_equal(O.block_forward(cfg, w, r3, ids, 80), base)


def test_block_attention_is_non_causal():
    cfg, raw, w = _model(synth.TINY)
    ring, _ = _filled_ring(cfg, w, 80)
    ids = O.block_ids(cfg, 11)
    base = O.block_forward(cfg, w, ring, ids, 80)
    ids2 = ids.copy()
    ids2[15] = 77
    got = O.block_forward(cfg, w, ring, ids2, 80)
    assert np.all(np.abs(got[:15] - base[:15]).max(axis=1) > 1e-9)


def test_position_shift_invariance():
    cfg, raw, w = _model(synth.TINY)
    ring_a, feats = _filled_ring(cfg, w, 80)
    ring_b, _ = _filled_ring(cfg, w, 80, base_pos=1000, feats=feats)
    ids = O.block_ids(cfg, 400)
    la = O.block_forward(cfg, w, ring_a, ids, 80)
    lb = O.block_forward(cfg, w, ring_b, ids, 1080)
    # the fp32 ring rounds K at each position differently, so equality holds to fp32 storage level
    np.testing.assert_allclose(lb, la, rtol=1e-5, atol=2e-6)
    assert np.abs(lb - la).max() < 1e-3 * np.abs(la).max()


def test_block_forward_is_deterministic_and_fp8_uses_dequantised_weights():
    cfg, raw, w = _model(PIN, "fp8", "bf16")
    ring, _ = _filled_ring(cfg, w, 20)
    ids = np.array([9] + [0] * 15)
    np.testing.assert_array_equal(O.block_forward(cfg, w, ring, ids, 20), O.block_forward(cfg, w, ring, ids, 20))
    codes, scale = O.quantize_fp8_rows(raw["layers"][0]["w_up"])
    want = torch.from_numpy(codes).view(torch.float8_e4m3fn).double().numpy() * scale.astype(np.float64)[:, None]
    np.testing.assert_array_equal(w.layer(0, "w_up"), want)


def test_batched_forward_equals_independent_sequences():
    """Sequences of one batch are independent: each sequence's logits equal its own single-sequence forward,
    whatever the other sequences hold (different rings, n_past and block ids), in any batch order."""
    cfg, raw, w = _model(PIN, "bf16", "bf16")
    n_pasts = [20, 3, 0, 37]
    rings = [_filled_ring(cfg, w, n, seed=s)[0] if n else O.Ring(cfg) for s, n in enumerate(n_pasts)]
    ids = np.array([[5 + b] + [0] * 15 for b in range(4)])
    ids[3, 7] = 11  # a block with a non-mask id inside
    got = O.block_forward_batch(cfg, w, rings, ids, n_pasts)
    for b in range(4):
        want = O.block_forward(cfg, w, rings[b], ids[b], n_pasts[b])
        np.testing.assert_allclose(got[b], want, rtol=1e-12, atol=1e-12)
    perm = [2, 0, 3, 1]
    got_p = O.block_forward_batch(cfg, w, [rings[i] for i in perm], ids[perm], [n_pasts[i] for i in perm])
    np.testing.assert_allclose(got_p, got[perm], rtol=1e-12, atol=1e-12)


def test_greedy_drafts_skip_row_zero_and_break_ties_low():
    logits = np.zeros((16, 10))
    logits[0, 9] = 100  # row 0 is never drafted
    for i in range(1, 16):
        logits[i, (3 * i) % 10] = 1.0
        logits[i, (3 * i + 5) % 10] = 1.0  # tie
    got = O.greedy_drafts(logits)
    want = [min((3 * i) % 10, (3 * i + 5) % 10) for i in range(1, 16)]
    np.testing.assert_array_equal(got, want)


# --------------------------------------------------------------------------- acceptance

def test_accept_bruteforce_all_mismatch_indices():
    rng = np.random.default_rng(13)
    for trial in range(200):
        d = rng.integers(0, 50, 15)
        m = rng.integers(0, 16)
        t = d.copy()
        if m < 15:
            t[m] = (d[m] + 1 + rng.integers(0, 48)) % 50
            t[m + 1:] = rng.integers(0, 50, 15 - m - 1)
        assert O.accept(d, t) == m


def test_accept_worked_example_from_the_pages():
    ex = json.load(open(os.path.join(GOLDEN, "accept_worked_example.json")))
    d, t = np.array(ex["drafts"]), np.array(ex["target"])
    assert t[3] == (d[3] + 1) % ex["vocab"]
    n_ok = O.accept(d, t)
    assert n_ok == ex["expected_n_ok"]
    assert n_ok + 1 == ex["expected_tau"]  # tau counts the bonus token
    assert t[n_ok] == ex["expected_bonus"]


def test_verify_with_bonus_worked_example_from_the_pages():
    """The page's invariant 4: three matching drafts, a mismatch at index 3 -> tau = 4, accepted[3] is the
    mismatching target token; the fixture's target row gets one more (bonus) position appended."""
    ex = json.load(open(os.path.join(GOLDEN, "accept_worked_example.json")))
    d = np.array(ex["drafts"])
    t = np.array(ex["target"] + [77])
    k, bonus, acc = O.verify(d, t)
    assert k == ex["expected_n_ok"] and len(acc) == ex["expected_tau"] and acc[-1] == bonus == ex["expected_bonus"]
    assert acc[:k] == list(d[:k])


def test_verify_full_match_takes_the_bonus_after_the_last_draft():
    d = np.array([4, 4, 9, 1])
    k, bonus, acc = O.verify(d, np.array([4, 4, 9, 1, 23]))
    assert (k, bonus, acc) == (4, 23, [4, 4, 9, 1, 23])
    k, bonus, acc = O.verify(d, np.array([5, 4, 9, 1, 23]))
    assert (k, bonus, acc) == (0, 5, [5])


def test_planted_targets_round_trip_through_accept():
    st = synth.step_inputs(synth.TINY, 64, seed=5)
    drafts = synth.integers(5, "drafts", (64, 15), 0, 512)
    tgt = synth.planted_targets(drafts, st["mismatch"], st["filler"], 512)
    for b in range(64):
        assert O.accept(drafts[b], tgt[b]) == st["mismatch"][b]


def test_per_head_qk_norm_makes_step_invariant_to_projection_scale():
    """q and k are RMS-normed per head after projection, so scaling wq or wk (inject and block alike)
    leaves the logits unchanged up to eps; scaling the q_norm weight does change them."""
    cfg, raw, w = _model(synth.TINY)
    ring, feats = _filled_ring(cfg, w, 80)
    ids = O.block_ids(cfg, 5)
    base = O.block_forward(cfg, w, ring, ids, 80)
    raw["layers"][0]["wq"] = raw["layers"][0]["wq"] * np.float32(8.0)
    np.testing.assert_allclose(O.block_forward(cfg, w, ring, ids, 80), base, rtol=0, atol=2e-5)  # eps inside the root
    raw["layers"][0]["wk"] = raw["layers"][0]["wk"] * np.float32(8.0)
    ring2, _ = _filled_ring(cfg, w, 80, feats=feats)
    np.testing.assert_allclose(O.block_forward(cfg, w, ring2, ids, 80), base, rtol=0, atol=2e-5)
    raw["layers"][0]["q_norm"] = raw["layers"][0]["q_norm"] * np.float32(1.5)
    assert np.abs(O.block_forward(cfg, w, ring2, ids, 80) - base).max() > 1e-3


# --------------------------------------------------------------------------- sampling
def test_philox_known_answer_vectors():
    kat = json.load(open(os.path.join(GOLDEN, "philox4x32_10_kat.json")))
    for v in kat["vectors"]:
        ctr = [int(x, 16) for x in v["counter"]]
        key = [int(x, 16) for x in v["key"]]
        out = [int(x) for x in O.philox4x32_10(ctr, key)]
        assert out == [int(x, 16) for x in v["output"]]


def test_gumbel_max_draws_follow_softmax_over_temperature():
    """The sampling law: over many positions, the Gumbel-max draft frequencies match softmax(logits / T)
    (each within 5 standard deviations of the binomial count)."""
    logits = np.array([0.0, 1.0, -0.5, 2.0, 0.3, 1.7])
    n = 20000
    for T in (0.5, 1.0, 2.0):
        p = np.exp(logits / T - (logits / T).max())
        p /= p.sum()
        g = O.gumbel_noise(seed=0x1234ABCD5678, b=0, positions=np.arange(n), n_vocab=len(logits))
        draws = np.argmax(logits[None] / T + g, axis=1)
        counts = np.bincount(draws, minlength=len(logits))
        sd = np.sqrt(n * p * (1 - p))
        assert np.all(np.abs(counts - n * p) <= 5 * sd + 1), (T, counts, n * p)


def test_sampling_at_vanishing_temperature_is_greedy_and_zero_is_greedy():
    rng = np.random.default_rng(2)
    logits = rng.standard_normal((16, 64))
    greedy = O.greedy_drafts(logits)
    assert np.array_equal(O.sampled_drafts(logits, 0.0, 7, 0, 100), greedy)
    assert np.array_equal(O.sampled_drafts(logits, 1e-9, 7, 0, 100), greedy)
    # and a real temperature moves some drafts (the noise is not constant)
    assert not np.array_equal(O.sampled_drafts(logits, 5.0, 7, 0, 100), greedy)
