"""Device buffers for a CSA2 workload and the calls that run it (torch = plumbing).

`DeviceCase` uploads a host case (pool, per-layer queries and windows) to HBM
as torch uint8 / uint16 / float32 / int32 tensors, allocates outputs and the
workspace, and drives the C ABI through the ctypes binding.  No arithmetic
of the method happens here.
"""
from __future__ import annotations

from typing import List, Optional

import numpy as np
import torch

from . import _lib as C
from .configs import FULL, REINDEX, REUSE
from .synth import HostCase


def _dev(a: np.ndarray, device) -> torch.Tensor:
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).to(device)
    return torch.from_numpy(a).to(device)


class DeviceCase:
    def __init__(self, case: HostCase, device: str = "cuda"):
        cfg = case.cfg
        self.cfg = cfg
        self.device = device
        p = case.pool
        self.latent = _dev(p.latent, device)
        self.scale = _dev(p.scale, device)
        self.idx_key = _dev(p.idx_key, device)
        self.pool = C.make_pool(self.latent, self.scale, self.idx_key, cfg.B, cfg.M, cfg.D,
                                cfg.HI, cfg.DI)
        B, Q, H, D, K = cfg.B, cfg.Q, cfg.H, cfg.D, cfg.K
        self.layers = []
        for L in case.layers:
            d = dict(mode=L.mode, q=_dev(L.q, device), swa=_dev(L.swa, device),
                     q_idx=None if L.q_idx is None else _dev(L.q_idx, device),
                     w_idx=None if L.w_idx is None else _dev(L.w_idx, device))
            d["o"] = torch.empty((B, Q, H, D), dtype=torch.float32, device=device)
            d["lse"] = torch.empty((B, Q, H), dtype=torch.float32, device=device)
            d["idx"] = torch.empty((B, Q, K), dtype=torch.int32, device=device)
            self.layers.append(d)
        self.ws = None
        self.ws_bytes = 0
        self.src_layer: Optional[List[int]] = None

    def use_lengths(self, lens) -> None:
        """Make the batch ragged: sequence b holds its first lens[b] entries."""
        cfg = self.cfg
        self.lens = torch.from_numpy(np.asarray(lens, dtype=np.int32)).to(self.device)
        self.pool = C.make_pool(self.latent, self.scale, self.idx_key, cfg.B, cfg.M, cfg.D,
                                cfg.HI, cfg.DI, len=self.lens, pages=getattr(self, "pages", None),
                                page_log2=getattr(self, "page_log2", 0))

    def use_pages(self, page_log2: int, seed: int = 0, spare_pages: int = 3) -> None:
        """Re-lay the pool out in pages of 2^page_log2 entries at shuffled
        physical positions (plus a few unused pages), with a page table."""
        cfg = self.cfg
        ps = 1 << page_log2
        assert cfg.M % ps == 0
        npg = cfg.M // ps
        total = cfg.B * npg + spare_pages
        perm = np.random.default_rng(seed).permutation(total)[:cfg.B * npg].astype(np.int32)
        table = torch.from_numpy(perm.reshape(cfg.B, npg)).to(self.device)
        dst = torch.from_numpy(np.repeat(perm, ps) * ps + np.tile(np.arange(ps), cfg.B * npg)
                               ).long().to(self.device)            # row of logical (b, e)
        arrays = []
        for t in (self.latent, self.scale, self.idx_key):
            flat = t.reshape(cfg.B * cfg.M, -1)
            phys = torch.zeros((total * ps, flat.shape[1]), dtype=t.dtype, device=self.device)
            phys[dst] = flat
            arrays.append(phys)
        self.latent, self.scale, self.idx_key = arrays
        self.pages, self.page_log2 = table, page_log2
        self.pool = C.make_pool(self.latent, self.scale, self.idx_key, cfg.B, cfg.M, cfg.D,
                                cfg.HI, cfg.DI, len=getattr(self, "lens", None), pages=table,
                                page_log2=page_log2)

    # -- workspace -----------------------------------------------------------
    def _workspace(self, nbytes: int) -> torch.Tensor:
        if self.ws is None or self.ws_bytes < nbytes:
            self.ws = torch.empty(max(nbytes, 256), dtype=torch.uint8, device=self.device)
            self.ws_bytes = nbytes
        return self.ws

    # -- decode step ---------------------------------------------------------
    def layer_structs(self, idx_for_reuse: bool = True):
        out = []
        for d in self.layers:
            reuse = d["mode"] == REUSE
            out.append(C.csa2_layer(d["mode"], C._p(d["q_idx"]), C._p(d["w_idx"]),
                                    C._p(d["q"]), C._p(d["swa"]), C._p(d["o"]),
                                    C._p(d["lse"]),
                                    C._p(d["idx"]) if (idx_for_reuse or not reuse) else None))
        return out

    def decode_workspace_bytes(self) -> int:
        cfg = self.cfg
        return C.csa2_workspace_bytes(C.CSA2_OP_DECODE_LAYERS, cfg.B, 1, cfg.M, cfg.K, cfg.P,
                                      cfg.W, cfg.H)

    def prepare_decode(self, idx_for_reuse: bool = True):
        assert self.cfg.Q == 1, "decode_layers runs one query token per sequence"
        nb = self.decode_workspace_bytes()
        assert nb > 0
        self._workspace(nb)
        self._structs = self.layer_structs(idx_for_reuse)

    def decode_layers(self, stream=None):
        if getattr(self, "_structs", None) is None:
            self.prepare_decode()
        cfg = self.cfg
        _, src = C.csa2_decode_layers(self.pool, self._structs, cfg.H, cfg.K, cfg.P, cfg.W,
                                      self.ws, self.ws_bytes, stream)
        self.src_layer = src
        return src

    def decode_layer(self, l: int, stream=None) -> int:
        """Layer l alone (csa2_decode_layer); layers before it must have run."""
        if getattr(self, "_structs", None) is None:
            self.prepare_decode()
        cfg = self.cfg
        if getattr(self, "_struct_arr", None) is None or self._struct_arr_src is not self._structs:
            self._struct_arr = (C.csa2_layer * len(self._structs))(*self._structs)
            self._struct_arr_src = self._structs
        _, src = C.csa2_decode_layer(self.pool, self._struct_arr, l, cfg.H, cfg.K, cfg.P, cfg.W,
                                     self.ws, self.ws_bytes, stream)
        return src

    # -- single-stage calls ----------------------------------------------------
    def index_scores(self, ell: int, cand=None, P: int = 0, hist=None, stream=None):
        cfg = self.cfg
        d = self.layers[ell]
        N = P if cand is not None else cfg.M
        scores = torch.empty((cfg.B, cfg.Q, N), dtype=torch.float32, device=self.device)
        C.csa2_index_score(self.pool, d["q_idx"], d["w_idx"], cfg.Q, cfg.pos0, cfg.ratio, cand,
                           P, scores, hist, stream)
        return scores

    def score_topk(self, ell: int, K: int = None, stream=None):
        """Layer ell's indexer score and Top-K in one pass (csa2_score_topk)."""
        cfg = self.cfg
        K = cfg.K if K is None else K
        d = self.layers[ell]
        nb = C.csa2_workspace_bytes(C.CSA2_OP_SCORE_TOPK, cfg.B, 1, cfg.M, K, 0, 0, 0)
        assert nb > 0, "shape not taken by the fused select"
        ws = torch.empty(nb, dtype=torch.uint8, device=self.device)
        idx = torch.empty((cfg.B, K), dtype=torch.int32, device=self.device)
        C.csa2_score_topk(self.pool, d["q_idx"], d["w_idx"], K, idx, ws, nb, stream)
        return idx

    def topk(self, scores: torch.Tensor, K: int, n_valid=None, cand=None, stream=None):
        R = scores.numel() // scores.shape[-1]
        N = scores.shape[-1]
        nb = C.csa2_workspace_bytes(C.CSA2_OP_TOPK, R, 1, N, K, 0, 0, 0)
        ws = torch.empty(max(nb, 256), dtype=torch.uint8, device=self.device)
        idx = torch.empty((R, K), dtype=torch.int32, device=self.device)
        C.csa2_topk(scores, R, N, n_valid, cand, K, idx, ws, nb, stream)
        return idx

    def sparse_attn(self, ell: int, idx: torch.Tensor, stream=None):
        cfg = self.cfg
        d = self.layers[ell]
        K = idx.shape[-1]
        nb = C.csa2_workspace_bytes(C.CSA2_OP_SPARSE_ATTN, cfg.B, cfg.Q, cfg.M, K, 0, 0, cfg.H)
        ws = torch.empty(max(nb, 256), dtype=torch.uint8, device=self.device)
        o = torch.empty((cfg.B, cfg.Q, cfg.H, cfg.D), dtype=torch.float32, device=self.device)
        lse = torch.empty((cfg.B, cfg.Q, cfg.H), dtype=torch.float32, device=self.device)
        C.csa2_sparse_attn(self.pool, d["q"], cfg.Q, cfg.H, idx.contiguous(), K, o, lse, ws, nb,
                           stream)
        return o, lse

    def swa_merge(self, ell: int, o: torch.Tensor, lse: torch.Tensor, stream=None):
        cfg = self.cfg
        d = self.layers[ell]
        nb = C.csa2_workspace_bytes(C.CSA2_OP_SWA_MERGE, cfg.B, cfg.Q, 0, 0, 0, cfg.W, cfg.H)
        ws = torch.empty(max(nb, 256), dtype=torch.uint8, device=self.device)
        C.csa2_swa_merge(d["q"], cfg.B, cfg.Q, cfg.H, cfg.D, d["swa"], cfg.W, o, lse, ws, nb,
                         stream)
        return o, lse

    # -- causal chunked prefill (one Full layer) ---------------------------------
    def visible_counts(self) -> torch.Tensor:
        cfg = self.cfg
        t = np.arange(cfg.Q, dtype=np.int64)
        vis = np.minimum(cfg.M, (cfg.pos0 + t + 1) // cfg.ratio) if cfg.pos0 >= 0 else \
            np.full(cfg.Q, cfg.M)
        return torch.from_numpy(np.tile(vis.astype(np.int32), cfg.B)).to(self.device)

    def prepare_prefill(self):
        """Allocate every buffer of a prefill step once (scores, indices, outputs, workspace)."""
        cfg = self.cfg
        dev = self.device
        R = cfg.B * cfg.Q
        self.pf_scores = torch.empty((cfg.B, cfg.Q, cfg.M), dtype=torch.float32, device=dev)
        self.pf_nvalid = self.visible_counts()
        self.pf_idx = torch.empty((R, cfg.K), dtype=torch.int32, device=dev)
        self.pf_o = torch.empty((cfg.B, cfg.Q, cfg.H, cfg.D), dtype=torch.float32, device=dev)
        self.pf_lse = torch.empty((cfg.B, cfg.Q, cfg.H), dtype=torch.float32, device=dev)
        nb = max(C.csa2_workspace_bytes(C.CSA2_OP_TOPK, R, 1, cfg.M, cfg.K, 0, 0, 0),
                 C.csa2_workspace_bytes(C.CSA2_OP_SPARSE_ATTN, cfg.B, cfg.Q, cfg.M, cfg.K, 0, 0,
                                        cfg.H),
                 C.csa2_workspace_bytes(C.CSA2_OP_SWA_MERGE, cfg.B, cfg.Q, 0, 0, 0, cfg.W, cfg.H))
        self.pf_ws = torch.empty(max(nb, 256), dtype=torch.uint8, device=dev)
        self.pf_ws_bytes = nb

    def prefill_stage(self, stage: int, stream=None):
        """One stage of the prefill step on the preallocated buffers:
        0 index score (Q rows, causal), 1 Top-K over the visible entries,
        2 sparse attention over the selected entries, 3 window merge."""
        cfg = self.cfg
        d = self.layers[0]
        R = cfg.B * cfg.Q
        if stage == 0:
            C.csa2_index_score(self.pool, d["q_idx"], d["w_idx"], cfg.Q, cfg.pos0, cfg.ratio, None,
                               0, self.pf_scores, None, stream)
        elif stage == 1:
            C.csa2_topk(self.pf_scores, R, cfg.M, self.pf_nvalid, None, cfg.K, self.pf_idx,
                        self.pf_ws, self.pf_ws_bytes, stream)
        elif stage == 2:
            C.csa2_sparse_attn(self.pool, d["q"], cfg.Q, cfg.H, self.pf_idx, cfg.K, self.pf_o,
                               self.pf_lse, self.pf_ws, self.pf_ws_bytes, stream)
        else:
            C.csa2_swa_merge(d["q"], cfg.B, cfg.Q, cfg.H, cfg.D, d["swa"], cfg.W, self.pf_o,
                             self.pf_lse, self.pf_ws, self.pf_ws_bytes, stream)

    def prefill(self, stream=None):
        """index_score (Q rows, causal) -> topk (n_valid = visible) -> sparse_attn -> swa_merge."""
        if getattr(self, "pf_scores", None) is None:
            self.prepare_prefill()
        for stage in range(4):
            self.prefill_stage(stage, stream)
        cfg = self.cfg
        return self.pf_idx.view(cfg.B, cfg.Q, cfg.K), self.pf_o, self.pf_lse

    # -- chunked prefill through the layer schedule -------------------------------
    def prefill_layers_workspace_bytes(self) -> int:
        cfg = self.cfg
        return C.csa2_workspace_bytes(C.CSA2_OP_PREFILL_LAYERS, cfg.B, cfg.Q, cfg.M, cfg.K, 0,
                                      cfg.W, cfg.H)

    def prepare_prefill_layers(self, idx_for_reuse: bool = True):
        nb = self.prefill_layers_workspace_bytes()
        assert nb > 0
        self._workspace(nb)
        self._pf_structs = self.layer_structs(idx_for_reuse)

    def prefill_layers(self, pos0: Optional[int] = None, stream=None):
        """Every layer of the schedule over the chunk (csa2_prefill_layers); outputs
        land in self.layers[l]["idx" / "o" / "lse"].  pos0 defaults to the config's."""
        cfg = self.cfg
        if getattr(self, "_pf_structs", None) is None:
            self.prepare_prefill_layers()
        _, self.src_layer = C.csa2_prefill_layers(
            self.pool, self._pf_structs, cfg.Q, cfg.pos0 if pos0 is None else pos0, cfg.ratio,
            cfg.H, cfg.K, cfg.W, self.ws, self.ws_bytes, stream)
        return self.layers

    # -- results -----------------------------------------------------------------
    def results(self):
        out = []
        for d in self.layers:
            out.append(dict(mode=d["mode"], idx=d["idx"].cpu().numpy(), o=d["o"].cpu().numpy(),
                            lse=d["lse"].cpu().numpy()))
        return out
