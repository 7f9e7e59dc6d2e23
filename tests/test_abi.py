"""CPU checks of the C ABI: the library loads, exports every function include/dflash.h declares, and
rejects bad arguments on the host before any GPU work (so these run without a GPU)."""
import ctypes as C
import dataclasses
import os
import re

import pytest

from block_diffusion_drafter_02_amd import _lib, synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "dflash.h")


@pytest.fixture(scope="module")
def L():
    src_dir = os.path.join(ROOT, "block_diffusion_drafter_02_amd", "csrc")
    newest = max(os.path.getmtime(os.path.join(src_dir, f)) for f in os.listdir(src_dir))
    if not os.path.exists(_lib.LIB_PATH) or os.path.getmtime(_lib.LIB_PATH) < newest:
        from block_diffusion_drafter_02_amd import build

        build.build()
    return _lib.lib()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(dflash_[a-z0-9_]+)\s*\(", text)))


def test_header_declares_the_boundary():
    names = declared_functions()
    for want in ("dflash_encode", "dflash_inject", "dflash_block_step", "dflash_accept", "dflash_step_graph_create",
                 "dflash_step_graph_launch", "dflash_create", "dflash_workspace_bytes"):
        assert want in names


def test_library_exports_every_declared_function(L):
    for name in declared_functions():
        assert hasattr(L, name), name
    assert set(declared_functions()) == set(_lib.SYMBOLS)


def _cfg(**kw):
    c = _lib.make_config(synth.TINY, "f32", "f32", "f32", max_batch=2, max_inject=64)
    for k, v in kw.items():
        setattr(c, k, v)
    return c


def test_ring_and_workspace_sizes(L):
    c = _cfg()
    ring = L.dflash_ring_bytes(C.byref(c))
    kv = synth.TINY.n_layer * synth.TINY.n_head_kv * synth.TINY.window * synth.TINY.head_dim * 4
    assert ring == 2 * ((kv + 255) // 256 * 256) + 256
    creal = _lib.make_config(synth.REAL, "bf16", "bf16", "bf16", max_batch=1, max_inject=512)
    ring_real = L.dflash_ring_bytes(C.byref(creal))
    assert ring_real == 2 * 5 * 8 * 2048 * 128 * 2 + 2048 * 4  # K + V of 5 layers at bf16: 41.9 MB
    ws = L.dflash_workspace_bytes(C.byref(creal))
    weights = 5 * (6144 * 6656 + 6656 * 4096 + 2 * 19968 * 6656 + 6656 * 19968) + 8192 * 6656
    assert ws > 2 * weights  # the re-tiled weight copies dominate


@pytest.mark.parametrize("field,value,msg", [
    ("head_dim", 96, "head_dim"),
    ("block", 8, "block"),
    ("n_head_kv", 3, "n_head"),
    ("n_head", 8, "query heads per kv head"),
    ("n_embd", 200, "multiples of 64"),
    ("window", 100, "multiples of 64"),
    ("max_batch", 9, "max_batch"),
    ("mask_id", 512, "mask_id"),
    ("weight_dtype", 7, "weight_dtype"),
    ("ring_dtype", 2, "ring_dtype"),
    ("aux_dtype", 2, "aux_dtype"),
])
def test_invalid_configs_are_rejected_with_a_message(L, field, value, msg):
    c = _cfg(**{field: value})
    assert L.dflash_workspace_bytes(C.byref(c)) == 0
    assert msg in L.dflash_last_error().decode()
    assert L.dflash_ring_bytes(C.byref(c)) == 0


def test_null_arguments_fail_before_any_gpu_work(L):
    h = C.c_void_p()
    assert L.dflash_create(None, None, None, 0, None, C.byref(h)) == _lib.EINVAL
    c = _cfg()
    assert L.dflash_create(C.byref(c), None, None, 0, None, C.byref(h)) == _lib.EINVAL
    assert "weights" in L.dflash_last_error().decode()
    w = _lib.Weights()
    assert L.dflash_create(C.byref(c), C.byref(w), None, 0, None, C.byref(h)) == _lib.EINVAL
    assert L.dflash_create(C.byref(c), None, None, 0, None, None) == _lib.EINVAL
    assert L.dflash_encode(None, None, 1, None, None) == _lib.EINVAL
    assert L.dflash_inject(None, None, None, None, 1, None) == _lib.EINVAL
    assert L.dflash_block_step(None, None, None, None, 1, None, None, None) == _lib.EINVAL
    assert L.dflash_block_step_accept(None, None, None, None, 1, None, None, None, None, None) == _lib.EINVAL
    assert L.dflash_block_forward(None, None, None, None, 1, None, None, None) == _lib.EINVAL
    assert L.dflash_accept(None, None, None, 1, None, None) == _lib.EINVAL
    assert L.dflash_step_graph_create(None, None, None, None, 1, None, None, None, None, None, C.byref(h)) == _lib.EINVAL
    assert L.dflash_step_graph_launch(None, None) == _lib.EINVAL
    assert L.dflash_quantize_fp8_rows(None, 1, 1, None, None, None) == _lib.EINVAL
    assert L.dflash_replay_stage(None, 0, 0, None) == _lib.EINVAL
    L.dflash_destroy(None)
    L.dflash_graph_destroy(None)


def test_fp8_config_requires_scales(L):
    c = _lib.make_config(synth.TINY, "fp8", "bf16", "bf16")
    layers = (_lib.LayerWeights * 1)()
    for f, _ in _lib.LayerWeights._fields_:
        if not f.startswith("s_"):
            setattr(layers[0], f, 256)  # non-NULL placeholders: validation fails before any use
    w = _lib.Weights(tok_embd=256, lm_head=256, fc=256, hidden_norm=256, output_norm=256, s_lm_head=None,
                     layers=C.cast(layers, C.POINTER(_lib.LayerWeights)))
    h = C.c_void_p()
    assert L.dflash_create(C.byref(c), C.byref(w), None, 0, None, C.byref(h)) == _lib.EINVAL
    assert "s_lm_head" in L.dflash_last_error().decode()


def test_oracle_and_library_share_no_code():
    """The oracle imports nothing from the package but the synthetic-input module, and vice versa."""
    oracle_src = open(os.path.join(ROOT, "oracle", "dflash_oracle.py")).read()
    assert "block_diffusion_drafter_02_amd" not in oracle_src
    pkg = os.path.join(ROOT, "block_diffusion_drafter_02_amd")
    for dirpath, _, files in os.walk(pkg):
        for f in files:
            if f.endswith(".py"):
                src = open(os.path.join(dirpath, f)).read()
                assert not re.search(r"^\s*(from\s+oracle|import\s+oracle)", src, flags=re.M), f
            if f.endswith((".hip", ".h", ".cpp")):
                assert "oracle/" not in open(os.path.join(dirpath, f)).read(), f
    assert dataclasses.is_dataclass(synth.Shape)
