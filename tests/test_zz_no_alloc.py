"""The allocation-free encode entry point (dflash_encode_static) against dflash_encode and the oracle.

Two calls in a row on one ctx, the second with fewer positions, at every combination of feature and fc
storage dtype that needs a different staging (bf16 features with bf16 fc: none; f32 features with bf16 fc:
the three-term split; bf16 features with f32 fc: an f32 copy; f32 with f32: none). Each call is made through
the C ABI and compared with dflash_encode on the same features (the same GEMM; the split-K counts may
differ, so the bar is fp32 summation order) and with the oracle's encode (the encode bar of the other
parity tests).
"""
import ctypes as C

import numpy as np
import pytest

from block_diffusion_drafter_02_amd import synth
from oracle import dflash_oracle as O
from tests import workload as WL

pytestmark = pytest.mark.gpu

CASES = [("bf16", "bf16"), ("bf16", "f32"), ("f32", "bf16"), ("f32", "f32")]  # (weight dtype, feature dtype)


@pytest.mark.parametrize("wdt,fdt", CASES, ids=[f"w{w}-f{f}" for w, f in CASES])
def test_static_scratch_encode_matches_workspace_encode(gpu, wdt, fdt):
    import torch

    from block_diffusion_drafter_02_amd import _lib
    from block_diffusion_drafter_02_amd.drafter import Drafter, to_device

    shape = WL.MEDIUM
    raw = synth.weights(shape, wdt, seed=0)
    dr = Drafter(shape, raw, wdt, "bf16" if wdt != "f32" else "f32", fdt, max_batch=1, max_inject=256)
    cfg = O.Config.from_shape(shape, "f32")
    ow = O.Weights(raw, wdt)
    L = _lib.lib()
    for T, tag in ((200, "noalloc.a"), (37, "noalloc.b")):
        print(f"[case] static encode {wdt}/{fdt} T={T}", flush=True)
        feats = synth.features(shape, T, fdt, seed=0, tag=tag)
        fdev = to_device(feats, dr.device)
        h_ws = dr.encode(fdev)
        h_st = torch.full_like(h_ws, float("nan"))
        rc = L.dflash_encode_static(dr._ctx, C.c_void_p(fdev.data_ptr()), T, C.c_void_p(h_st.data_ptr()),
                                    C.c_void_p(torch.cuda.current_stream().cuda_stream))
        _lib.check(rc)
        torch.cuda.synchronize()
        got, want = h_st.cpu().numpy().astype(np.float64), h_ws.cpu().numpy().astype(np.float64)
        scale = max(1.0, float(np.abs(want).max()))
        assert np.all(np.isfinite(got))
        assert np.abs(got - want).max() <= 1e-6 * scale, np.abs(got - want).max()
        ref = O.encode(cfg, ow, feats)
        assert np.abs(got - ref).max() <= 2e-5 * max(1.0, np.abs(ref).max())
