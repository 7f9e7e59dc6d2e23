"""Thin torch-facing wrapper over the DFlash C ABI.

torch provides device memory and streams; every computation runs in
libdflash.so. Method names follow the dflash-ops card's Usage section:
encode, inject, the block step (eager or captured), accept.
"""
from __future__ import annotations

import ctypes as C

import numpy as np
import torch

from . import _lib
from ._lib import check, lib


def _stream(stream=None) -> int:
    s = stream if stream is not None else torch.cuda.current_stream()
    return s.cuda_stream


def _dev(t: torch.Tensor, dtype: torch.dtype, name: str) -> int:
    if not t.is_cuda or t.dtype != dtype or not t.is_contiguous():
        raise ValueError(f"{name} must be a contiguous {dtype} CUDA tensor")
    return t.data_ptr()


def to_device(a: np.ndarray, device) -> torch.Tensor:
    """Upload a storage array: float32 stays float32, uint16 bf16 bits travel as int16, uint8 as uint8."""
    if a.dtype == np.float32:
        t = torch.from_numpy(np.ascontiguousarray(a))
    elif a.dtype == np.uint16:
        t = torch.from_numpy(np.ascontiguousarray(a).view(np.int16))
    elif a.dtype == np.uint8:
        t = torch.from_numpy(np.ascontiguousarray(a))
    elif a.dtype == np.int32:
        t = torch.from_numpy(np.ascontiguousarray(a))
    else:
        raise TypeError(a.dtype)
    return t.to(device, non_blocking=False)


def quantize_fp8_rows(w: torch.Tensor, stream=None):
    """Per-row E4M3 quantisation on the GPU: returns (codes uint8 [R, K], scales float32 [R])."""
    R, K = w.shape
    codes = torch.empty((R, K), dtype=torch.uint8, device=w.device)
    scales = torch.empty((R,), dtype=torch.float32, device=w.device)
    check(lib().dflash_quantize_fp8_rows(_dev(w, torch.float32, "w"), R, K, codes.data_ptr(), scales.data_ptr(),
                                         _stream(stream)))
    return codes, scales


class StepGraph:
    def __init__(self, handle: int, keep: list):
        self._h = handle
        self._keep = keep

    def launch(self, stream=None) -> None:
        check(lib().dflash_step_graph_launch(self._h, _stream(stream)))

    def close(self) -> None:
        if self._h:
            lib().dflash_graph_destroy(self._h)
            self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


class Drafter:
    """One drafter context: re-tiled weights and workspace on one GPU.

    raw: weight dict from ``synth.weights`` (storage form). For weight_dtype
    "fp8" the float32 masters are uploaded and quantised on the GPU by
    dflash_quantize_fp8_rows.
    """

    def __init__(self, shape, raw: dict, weight_dtype: str, ring_dtype: str, feature_dtype: str,
                 max_batch: int = 1, max_inject: int = 64, device="cuda:0", stream=None):
        self.shape = shape
        self.device = torch.device(device)
        self.weight_dtype, self.ring_dtype, self.feature_dtype = weight_dtype, ring_dtype, feature_dtype
        self.cfg = _lib.make_config(shape, weight_dtype, ring_dtype, feature_dtype, max_batch, max_inject)
        L = lib()
        self.ws_bytes = L.dflash_workspace_bytes(C.byref(self.cfg))
        if self.ws_bytes == 0:
            raise _lib.DFlashError(_lib.EINVAL, L.dflash_last_error().decode())
        self.ring_bytes = L.dflash_ring_bytes(C.byref(self.cfg))
        keep = {}
        fp8 = weight_dtype == "fp8"

        def up(a):
            t = to_device(a, self.device)
            keep[id(t)] = t
            return t

        def mat(a):
            t = up(a)
            if fp8:
                codes, scales = quantize_fp8_rows(t, stream)
                keep[id(codes)], keep[id(scales)] = codes, scales
                return codes.data_ptr(), scales.data_ptr()
            return t.data_ptr(), None

        self.tok_embd = up(raw["tok_embd"])
        lm, s_lm = mat(raw["lm_head"])
        self._layers = (_lib.LayerWeights * shape.n_layer)()
        for l, lw in enumerate(raw["layers"]):
            d = self._layers[l]
            for nm in ("attn_norm", "q_norm", "k_norm", "ffn_norm"):
                setattr(d, nm, up(lw[nm]).data_ptr())
            for nm, sn in (("wq", "s_q"), ("wk", "s_k"), ("wv", "s_v"), ("wo", "s_o"), ("w_gate", "s_gate"),
                           ("w_up", "s_up"), ("w_down", "s_down")):
                p, sp = mat(lw[nm])
                setattr(d, nm, p)
                setattr(d, sn, sp)
        self._w = _lib.Weights(tok_embd=self.tok_embd.data_ptr(), lm_head=lm, fc=up(raw["fc"]).data_ptr(),
                               hidden_norm=up(raw["hidden_norm"]).data_ptr(),
                               output_norm=up(raw["output_norm"]).data_ptr(), s_lm_head=s_lm,
                               layers=C.cast(self._layers, C.POINTER(_lib.LayerWeights)))
        self.workspace = torch.empty(self.ws_bytes, dtype=torch.uint8, device=self.device)
        h = C.c_void_p()
        check(L.dflash_create(C.byref(self.cfg), C.byref(self._w), self.workspace.data_ptr(), self.ws_bytes,
                              _stream(stream), C.byref(h)))
        self._ctx = h.value
        torch.cuda.synchronize(self.device)
        # the library keeps reading only tok_embd; the other uploads can go
        keep.clear()

    # ------------------------------------------------------------------ rings
    def new_ring(self, stream=None) -> torch.Tensor:
        ring = torch.empty(self.ring_bytes, dtype=torch.uint8, device=self.device)
        self.ring_reset(ring, stream)
        return ring

    def ring_reset(self, ring: torch.Tensor, stream=None) -> None:
        check(lib().dflash_ring_reset(self._ctx, _dev(ring, torch.uint8, "ring"), _stream(stream)))

    # ------------------------------------------------------------------ paged drafter KV
    PAGE_SLOTS = 128

    def page_bytes(self) -> int:
        return int(lib().dflash_page_bytes(C.byref(self.cfg)))

    def set_paged_pool(self, pool: torch.Tensor | None, n_pages: int = 0) -> None:
        """Switch to paged KV over `pool` (uint8, n_pages * page_bytes()), or back to contiguous rings (None).
        In paged mode the `ring` of inject and the entries of ring_table are int32 block tables."""
        ptr = None if pool is None else _dev(pool, torch.uint8, "pool")
        check(lib().dflash_set_paged_pool(self._ctx, ptr, n_pages))
        self._paged = pool is not None

    def pages_reset(self, first: int, count: int, stream=None) -> None:
        check(lib().dflash_pages_reset(self._ctx, first, count, _stream(stream)))

    def new_pool(self, n_pages: int, stream=None) -> torch.Tensor:
        """A pool of n_pages pages, switched to and reset."""
        pool = torch.empty(n_pages * self.page_bytes(), dtype=torch.uint8, device=self.device)
        self.set_paged_pool(pool, n_pages)
        self.pages_reset(0, n_pages, stream)
        return pool

    def page_views(self, pool: torch.Tensor, page: int):
        """(K, V, slot_pos) of one page: K, V [L, Hkv, 128, D], slot_pos [128]."""
        s = self.shape
        es = 4 if self.ring_dtype == "f32" else 2
        P = self.PAGE_SLOTS
        kv = s.n_layer * s.n_head_kv * P * s.head_dim * es
        kv_al = (kv + 255) // 256 * 256
        pg = pool[page * self.page_bytes():(page + 1) * self.page_bytes()]
        dt = torch.float32 if es == 4 else torch.bfloat16
        shp = (s.n_layer, s.n_head_kv, P, s.head_dim)
        return pg[:kv].view(dt).view(shp), pg[kv_al:kv_al + kv].view(dt).view(shp), \
            pg[2 * kv_al:2 * kv_al + 4 * P].view(torch.int32)

    def gather_ring(self, pool: torch.Tensor, table: torch.Tensor):
        """The logical ring (K, V [L, Hkv, W, D], slot_pos [W]) a block table describes (entries outside the
        pool read as empty slots with zero K/V)."""
        s = self.shape
        ids = table.cpu().tolist()
        n_pages = pool.numel() // self.page_bytes()
        Ks, Vs, sps = [], [], []
        for pg in ids:
            if 0 <= pg < n_pages:
                K, V, sp = self.page_views(pool, pg)
            else:
                K0, V0, sp0 = self.page_views(pool, 0)
                K, V, sp = torch.zeros_like(K0), torch.zeros_like(V0), torch.full_like(sp0, -1)
            Ks.append(K), Vs.append(V), sps.append(sp)
        return torch.cat(Ks, dim=2), torch.cat(Vs, dim=2), torch.cat(sps)

    def _ring_geom(self):
        s = self.shape
        es = 4 if self.ring_dtype == "f32" else 2
        kv = s.n_layer * s.n_head_kv * s.window * s.head_dim * es
        kv_al = (kv + 255) // 256 * 256
        return es, kv, kv_al

    def ring_views(self, ring: torch.Tensor):
        """(K, V, slot_pos) views of a ring: K, V [L, Hkv, W, D] (float32 or bfloat16), slot_pos [W] int32."""
        s = self.shape
        es, kv, kv_al = self._ring_geom()
        dt = torch.float32 if es == 4 else torch.bfloat16
        shp = (s.n_layer, s.n_head_kv, s.window, s.head_dim)
        K = ring[:kv].view(dt).view(shp)
        V = ring[kv_al:kv_al + kv].view(dt).view(shp)
        sp = ring[2 * kv_al:2 * kv_al + 4 * s.window].view(torch.int32)
        return K, V, sp

    # ------------------------------------------------------------------ ops
    def encode(self, feats: torch.Tensor, h: torch.Tensor | None = None, stream=None) -> torch.Tensor:
        T = feats.shape[0]
        fdt = torch.float32 if self.feature_dtype == "f32" else torch.int16
        if h is None:
            h = torch.empty((T, self.shape.n_embd), dtype=torch.float32, device=self.device)
        check(lib().dflash_encode(self._ctx, _dev(feats, fdt, "feats"), T, _dev(h, torch.float32, "h"),
                                  _stream(stream)))
        return h

    def encode_static(self, feats: torch.Tensor, h: torch.Tensor | None = None, stream=None) -> torch.Tensor:
        """encode() whose scratch is the library's static per-GPU array (for callers that cannot allocate;
        calls on one GPU must not overlap)."""
        T = feats.shape[0]
        fdt = torch.float32 if self.feature_dtype == "f32" else torch.int16
        if h is None:
            h = torch.empty((T, self.shape.n_embd), dtype=torch.float32, device=self.device)
        check(lib().dflash_encode_static(self._ctx, _dev(feats, fdt, "feats"), T, _dev(h, torch.float32, "h"),
                                         _stream(stream)))
        return h

    def inject(self, ring: torch.Tensor, h: torch.Tensor, positions: torch.Tensor, stream=None) -> None:
        T = h.shape[0]
        rdt = torch.int32 if getattr(self, "_paged", False) else torch.uint8
        check(lib().dflash_inject(self._ctx, _dev(ring, rdt, "ring"), _dev(h, torch.float32, "h"),
                                  _dev(positions, torch.int32, "positions"), T, _stream(stream)))

    def inject_batch(self, ring_table: torch.Tensor, seq: torch.Tensor, h: torch.Tensor, positions: torch.Tensor,
                     stream=None) -> None:
        """One fused K/V projection over rows of several sequences: row t goes to ring_table[seq[t]]."""
        T = h.shape[0]
        check(lib().dflash_inject_batch(self._ctx, _dev(ring_table, torch.int64, "rings"), ring_table.shape[0],
                                        _dev(seq, torch.int32, "seq"), _dev(h, torch.float32, "h"),
                                        _dev(positions, torch.int32, "positions"), T, _stream(stream)))

    def ring_table(self, rings) -> torch.Tensor:
        return torch.tensor([r.data_ptr() for r in rings], dtype=torch.int64, device=self.device)

    def _outputs(self, B):
        s = self.shape
        logits = torch.empty((s.block * B, s.n_vocab), dtype=torch.float32, device=self.device)
        drafts = torch.empty((B, self.block_width() - 1), dtype=torch.int32, device=self.device)
        return logits, drafts

    def block_step(self, ring_table: torch.Tensor, id_last: torch.Tensor, n_past: torch.Tensor, out=None,
                   stream=None, target: torch.Tensor | None = None, n_ok: torch.Tensor | None = None):
        """The block step; with target [B, g-1] (and optionally n_ok [B]) also the acceptance scan, fused into
        the logits launch (dflash_block_step_accept). Returns (logits, drafts), plus n_ok when target is given."""
        B = id_last.shape[0]
        logits, drafts = out if out is not None else self._outputs(B)
        rings, il, npst = (_dev(ring_table, torch.int64, "rings"), _dev(id_last, torch.int32, "id_last"),
                           _dev(n_past, torch.int32, "n_past"))
        if target is None:
            check(lib().dflash_block_step(self._ctx, rings, il, npst, B, logits.data_ptr(), drafts.data_ptr(),
                                          _stream(stream)))
            return logits, drafts
        if n_ok is None:
            n_ok = torch.empty((B,), dtype=torch.int32, device=self.device)
        check(lib().dflash_block_step_accept(self._ctx, rings, il, npst, B, logits.data_ptr(), drafts.data_ptr(),
                                             _dev(target, torch.int32, "target"), _dev(n_ok, torch.int32, "n_ok"),
                                             _stream(stream)))
        return logits, drafts, n_ok

    def block_forward(self, ring_table: torch.Tensor, block_ids: torch.Tensor, n_past: torch.Tensor, stream=None):
        B = block_ids.shape[0]
        logits, drafts = self._outputs(B)
        check(lib().dflash_block_forward(self._ctx, _dev(ring_table, torch.int64, "rings"),
                                         _dev(block_ids, torch.int32, "block_ids"),
                                         _dev(n_past, torch.int32, "n_past"), B, logits.data_ptr(),
                                         drafts.data_ptr(), _stream(stream)))
        return logits, drafts

    def accept(self, drafts: torch.Tensor, target: torch.Tensor, n_ok: torch.Tensor | None = None, stream=None):
        B = drafts.shape[0]
        if n_ok is None:
            n_ok = torch.empty((B,), dtype=torch.int32, device=self.device)
        check(lib().dflash_accept(self._ctx, _dev(drafts, torch.int32, "drafts"), _dev(target, torch.int32, "target"),
                                  B, _dev(n_ok, torch.int32, "n_ok"), _stream(stream)))
        return n_ok

    def accept_bonus(self, drafts: torch.Tensor, target: torch.Tensor, stream=None):
        """(n_ok [B], bonus [B]): acceptance with the target's token at the first mismatch; target [B, g]."""
        B = drafts.shape[0]
        n_ok = torch.empty((B,), dtype=torch.int32, device=self.device)
        bonus = torch.empty((B,), dtype=torch.int32, device=self.device)
        check(lib().dflash_accept_bonus(self._ctx, _dev(drafts, torch.int32, "drafts"),
                                        _dev(target, torch.int32, "target"), B, _dev(n_ok, torch.int32, "n_ok"),
                                        _dev(bonus, torch.int32, "bonus"), _stream(stream)))
        return n_ok, bonus

    def capture_step(self, ring_table, id_last, n_past, logits, drafts, target=None, n_ok=None,
                     stream=None) -> StepGraph:
        """Capture the block step (plus accept when target/n_ok are given) on a non-default stream."""
        B = id_last.shape[0]
        s = stream if stream is not None else torch.cuda.Stream(self.device)
        h = C.c_void_p()
        check(lib().dflash_step_graph_create(
            self._ctx, _dev(ring_table, torch.int64, "rings"), _dev(id_last, torch.int32, "id_last"),
            _dev(n_past, torch.int32, "n_past"), B, _dev(logits, torch.float32, "logits"),
            _dev(drafts, torch.int32, "drafts"),
            None if target is None else _dev(target, torch.int32, "target"),
            None if n_ok is None else _dev(n_ok, torch.int32, "n_ok"), s.cuda_stream, C.byref(h)))
        return StepGraph(h.value, [ring_table, id_last, n_past, logits, drafts, target, n_ok, self])

    def set_block_width(self, g: int) -> int:
        """Block width of later steps and graph captures (clamped into 2..block); returns the width in use."""
        check(lib().dflash_set_block_width(self._ctx, g))
        return self.block_width()

    def block_width(self) -> int:
        return int(lib().dflash_block_width(self._ctx))

    def set_sampling(self, temperature: float, seed: int = 0) -> None:
        """Draft sampling of later steps: greedy at 0, else Gumbel-max draws from softmax(logits / T)."""
        check(lib().dflash_set_sampling(self._ctx, float(temperature), int(seed)))

    def set_path(self, path: int) -> None:
        """Route later block steps: _lib.PATH_AUTO, PATH_KERNELS or PATH_PERSISTENT."""
        check(lib().dflash_set_path(self._ctx, path))

    def step_path(self, B: int = 1) -> int:
        return int(lib().dflash_step_path(self._ctx, B))

    def check_device(self, stream=None) -> None:
        """Raise if a dataflow-chain wait gave up since the last check (the error is then cleared)."""
        check(lib().dflash_check_device(self._ctx, _stream(stream)))

    def set_wait_limit(self, microseconds: int, stream=None) -> None:
        """Wall-clock limit of each bounded wait of the dataflow chain (a test and tuning hook)."""
        check(lib().dflash_set_wait_limit(self._ctx, int(microseconds), _stream(stream)))

    def replay_stage(self, stage: int, layer: int = 0, stream=None) -> None:
        """Re-run one weight-streaming stage of the last block step (a single-kernel timing hook)."""
        check(lib().dflash_replay_stage(self._ctx, stage, layer, _stream(stream)))

    def close(self) -> None:
        if getattr(self, "_ctx", None):
            lib().dflash_destroy(self._ctx)
            self._ctx = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass
