"""GPU parity of draft sampling (dflash_engine.py page, DFlashDraftModel.forward: a draw from
softmax(logits / T)) by the Gumbel-max rule over Philox-4x32-10 noise, against the oracle's
sampled_drafts on the same seed and positions.

A sampled draft is a float-decided integer: the HIP path takes the argmax of fp32 logit / T plus fp32
Gumbel noise, the oracle of fp64 ones. A draft must equal the oracle's, or score within the logit
tolerance (scaled by 1/T) plus the noise's fp32 rounding of the oracle's best score (a near tie).
The logits output stays unperturbed and is held to the usual bar."""
import dataclasses

import numpy as np
import pytest

from block_diffusion_drafter_02_amd import synth
from oracle import dflash_oracle as O
from tests import workload as WL
from tests.test_gpu_parity import _build, _check_logits, _spec_id, _step

pytestmark = pytest.mark.gpu

SEED = 0x5EED0123456789AB


def _torch():
    import torch

    return torch


def _check_sampled(ref_logits, drafts, T, seed, b, n_past, tol):
    """Rows 1..g-1: equal to the oracle's Gumbel-max draft or a near tie; returns the near-tie count."""
    g, V = ref_logits.shape
    noise = O.gumbel_noise(seed, b, n_past + np.arange(1, g), V)
    score = ref_logits[1:] / T + noise
    want = O.sampled_drafts(ref_logits, T, seed, b, n_past)
    ties = 0
    for i in range(g - 1):
        got = int(drafts[i])
        if got == int(want[i]):
            continue
        slack = tol / T + 1e-5 * (1.0 + np.abs(score[i]).max())
        assert score[i, got] >= score[i].max() - slack, (i, got, int(want[i]), score[i].max() - score[i, got])
        ties += 1
    return ties


SPECS = [WL.Spec(synth.TINY, "f32", "f32", "f32"), WL.Spec(WL.MEDIUM, "bf16", "bf16", "bf16")]


@pytest.mark.parametrize("T", [0.8, 2.0])
@pytest.mark.parametrize("g", [16, 6])
@pytest.mark.parametrize("spec", SPECS, ids=_spec_id)
def test_sampled_drafts_match_oracle_gumbel_max(gpu, spec, g, T):
    n_ctx = spec.shape.window + 16
    dr, ring, fdev, (ocfg, ow, oring), raw, feats = _build(spec, n_ctx)
    dr.set_block_width(g)
    dr.set_sampling(T, SEED)
    print(f"[case] {_spec_id(spec)} g={g} T={T}", flush=True)
    st = synth.step_inputs(spec.shape, 1, seed=17)
    logits, drafts = _step(dr, [ring], st["id_last"], [n_ctx])
    cfg_g = dataclasses.replace(ocfg, block=g)
    ref = O.block_forward(cfg_g, ow, oring, O.block_ids(cfg_g, int(st["id_last"][0])), n_ctx)
    tol = _check_logits(spec, ref, logits[:g])
    ties = _check_sampled(ref, drafts[0], T, SEED, 0, n_ctx, tol)
    assert ties <= 1, ties
    dr.set_sampling(0.0)
    dr.set_block_width(16)


def test_batched_sampling_matches_per_sequence_oracle(gpu):
    """B = 3 (the batched projection path) at T = 1: each sequence's noise is its own (counter b)."""
    from block_diffusion_drafter_02_amd.drafter import Drafter, to_device

    spec = WL.Spec(WL.MEDIUM, "bf16", "bf16", "bf16")
    shape = spec.shape
    raw = synth.weights(shape, "bf16", seed=0)
    dr = Drafter(shape, raw, "bf16", "bf16", "bf16", max_batch=3, max_inject=128)
    dr.set_sampling(1.0, SEED)
    n_pasts = [40, 256, 300]
    rings, orings = [], []
    for b, n in enumerate(n_pasts):
        feats = synth.features(shape, n, "bf16", seed=0, tag=f"feats{b}")
        pos = np.arange(n, dtype=np.int64)
        r = dr.new_ring()
        WL.gpu_inject(dr, r, to_device(feats, dr.device), pos, 128)
        rings.append(r)
        orings.append(WL.oracle_side(spec, raw, feats, pos, 128))
    st = synth.step_inputs(shape, 3, seed=19)
    print("[case] sampled batch B=3", flush=True)
    logits, drafts = _step(dr, rings, st["id_last"], n_pasts)
    total_ties = 0
    for b, n in enumerate(n_pasts):
        ocfg, ow, oring = orings[b]
        ref = O.block_forward(ocfg, ow, oring, O.block_ids(ocfg, int(st["id_last"][b])), n)
        tol = _check_logits(spec, ref, logits[16 * b:16 * (b + 1)], label=f"seq{b}")
        total_ties += _check_sampled(ref, drafts[b], 1.0, SEED, b, n, tol)
    assert total_ties <= 2, total_ties


def test_sampling_graph_replays_draw_at_the_fresh_positions(gpu):
    """A graph captured with sampling on replays like eager steps at the n_past written before each replay
    (the noise follows the positions), bitwise."""
    torch = _torch()
    spec = WL.Spec(WL.MEDIUM, "bf16", "bf16", "bf16")
    dr, ring, fdev, _, raw, feats = _build(spec, 300)
    dr.set_sampling(1.5, SEED)
    table = dr.ring_table([ring])
    il = torch.tensor([5], dtype=torch.int32, device=dr.device)
    npst = torch.tensor([300], dtype=torch.int32, device=dr.device)
    logits, drafts = dr.block_step(table, il, npst)
    torch.cuda.synchronize()
    stream = torch.cuda.Stream()
    g_logits, g_drafts = torch.empty_like(logits), torch.empty_like(drafts)
    gr = dr.capture_step(table, il, npst, g_logits, g_drafts, stream=stream)
    print("[case] sampling graph", flush=True)
    seen = set()
    for n in (300, 301, 290):
        npst.fill_(n)
        with torch.cuda.stream(stream):
            gr.launch(stream)
        stream.synchronize()
        e_logits, e_drafts = dr.block_step(table, il, npst)
        torch.cuda.synchronize()
        assert torch.equal(g_drafts, e_drafts) and torch.equal(g_logits, e_logits), n
        seen.add(tuple(e_drafts.cpu().numpy().ravel().tolist()))
    assert len(seen) > 1  # other positions, other draws
    gr.close()
    dr.set_sampling(0.0)
