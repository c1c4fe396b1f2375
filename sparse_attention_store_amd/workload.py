"""Device-resident DSA layer state for a workload, and the layer steps through libdsa.

Allocates the paged caches (one index-K cache per full layer, one latent cache per
layer, one page table for all), fills them from the seeded device generator through the
library's own store kernels, prepares the per-step query tensors, and runs a full or
shared layer as a sequence of C-ABI calls on the current stream.  Plumbing only: every
step of the method runs in libdsa's kernels.
"""
from __future__ import annotations

import numpy as np
import torch

import dsa_inputs as gi

from . import dsa

LN_EPS = 1e-6
ROPE_THETA = 10000.0
SM_SCALE = 1.0 / 16.0      # 1 / sqrt(256), the MLA softmax scale
TOPK = 2048


def _runs(req: np.ndarray, pos: np.ndarray):
    """Split (req, pos) rows into runs of consecutive positions of one request."""
    start = 0
    n = len(pos)
    for i in range(1, n + 1):
        if i == n or req[i] != req[i - 1] or pos[i] != pos[i - 1] + 1:
            yield start, i
            start = i


class DeviceLayer:
    def __init__(self, w: gi.Workload, device="cuda", latent_layers=None, k_overrides=None,
                 populate_chunk_tokens: int = 1 << 18, logits_budget_bytes: int | None = None,
                 caches_from: "DeviceLayer | None" = None):
        self.w = w
        self.device = device
        self.seed = w.seed
        self.pages = dsa.Pages(torch.from_numpy(w.page_table).to(device), w.num_pages)
        self.token_base = w.token_base
        self.k_overrides = k_overrides or {}           # position (request 0) -> bf16[128] host
        R = w.R
        self.rows = dsa.Rows(torch.from_numpy(w.row_req).to(device), torch.from_numpy(w.row_pos).to(device),
                             w.max_pos, w.rows_per_req)
        self.layers = list(range(w.n_layers)) if latent_layers is None else list(latent_layers)
        self._chunk = populate_chunk_tokens
        if caches_from is not None:
            # another batch of the same request(s): same page table and caches, no re-population
            self.pages = caches_from.pages
            self.index_cache, self.latent_cache = caches_from.index_cache, caches_from.latent_cache
        else:
            self.index_cache = {l: torch.zeros((w.num_pages, dsa.INDEX_PAGE_BYTES), dtype=torch.uint8, device=device)
                                for l in w.full_layers}
            self.latent_cache = {l: torch.zeros((w.num_pages, dsa.LATENT_PAGE_BYTES), dtype=torch.uint8,
                                                device=device) for l in self.layers}
            self.populate()
        # per-step inputs (seeded by the rows' index in the whole workload)
        r0, rt = w.row0, w.rows_total
        self.k_new = self._gen_token_rows(gi.T_RAW_K, 128, w.row_req, w.row_pos, override=True)
        self.q_idx = self._gen(gi.T_IDX_Q, r0 * 32 * 128, R * 32 * 128).view(R, 32, 128)
        self.w_head = torch.empty((R, 32), dtype=torch.float32, device=device)
        gi.dev_uniform_f32(self.seed, gi.T_W, r0 * 32, R * 32, gi.w_scale(), self.w_head.data_ptr(), self._stream())
        self.q_mla = {l: self._gen(gi.T_MLA_Q, (l * rt + r0) * 64 * 576, R * 64 * 576).view(R, 64, 576)
                      for l in self.layers}
        # outputs and workspaces
        self.stride = dsa.dsa_logits_stride(w.max_pos)
        self._plan_row_chunks(logits_budget_bytes)
        self.q8 = torch.empty((R, 32, 128), dtype=torch.uint8, device=device)
        self.qs = torch.empty((R, 32), dtype=torch.float32, device=device)
        self.logits = torch.empty((self.rows_per_chunk, self.stride), dtype=torch.float32, device=device)
        self.idx = torch.empty((R, TOPK), dtype=torch.int32, device=device)
        self.out = {l: torch.empty((R, 64, 512), dtype=torch.int16, device=device) for l in self.layers}
        self.lse = {l: torch.empty((R, 64), dtype=torch.float32, device=device) for l in self.layers}
        nt = dsa.dsa_topk_workspace_size(self.rows_per_chunk, self.stride, TOPK)
        self.ws_topk = torch.empty(max(nt, 256), dtype=torch.uint8, device=device)
        nm = dsa.dsa_sparse_mla_workspace_size(R, TOPK)
        self.ws_mla = torch.empty(max(nm, 256), dtype=torch.uint8, device=device) if nm else None

    def _plan_row_chunks(self, budget):
        """Row chunks for the indexer when R x stride fp32 logits exceed `budget` bytes
        ("GLM-5.3 推理全链路(十一)", section on the logits temporary: rows_per_chunk =
        budget // row_bytes).  Chunks hold whole request groups, or lie inside one request."""
        w, R = self.w, self.w.R
        rpc = dsa.dsa_logits_rows_per_chunk(R, self.stride * 4, budget) if budget else 0
        if not rpc:
            self.rows_per_chunk, self.row_chunks = R, None
            return
        g = w.rows_per_req
        if g <= rpc:
            rpc -= rpc % g
        else:
            assert w.B == 1, "a chunk inside a request group needs a single request"
        self.rows_per_chunk = rpc
        self.row_chunks = []
        for a in range(0, R, rpc):
            b = min(R, a + rpc)
            rows = dsa.Rows(self.rows.req[a:b], self.rows.pos[a:b], int(w.row_pos[a:b].max()),
                            g if g <= rpc else b - a)
            self.row_chunks.append((a, b, rows))

    # ------------------------------------------------------------------ generation
    def _stream(self):
        return torch.cuda.current_stream().cuda_stream

    def _gen(self, tid: int, start: int, n: int) -> torch.Tensor:
        t = torch.empty(n, dtype=torch.int16, device=self.device)     # bf16 bit patterns
        gi.dev_normal_bf16(self.seed, tid, start, n, t.data_ptr(), self._stream())
        return t

    def _gen_token_rows(self, tid: int, width: int, req: np.ndarray, pos: np.ndarray, override=False):
        out = torch.empty((len(pos), width), dtype=torch.int16, device=self.device)
        for a, b in _runs(req, pos):
            start = (int(self.token_base[req[a]]) + int(pos[a])) * width
            gi.dev_normal_bf16(self.seed, tid, start, (b - a) * width, out[a:b].data_ptr(), self._stream())
        if override and self.k_overrides:
            for i in range(len(pos)):
                if req[i] == 0 and int(pos[i]) in self.k_overrides:
                    out[i] = torch.from_numpy(self.k_overrides[int(pos[i])].view(np.int16)).to(self.device)
        return out

    def _raw_keys(self, b: int, p0: int, p1: int) -> torch.Tensor:
        """Raw index keys of positions p0..p1-1 of request b, with the planted overrides."""
        n = p1 - p0
        k = self._gen(gi.T_RAW_K, (int(self.token_base[b]) + p0) * 128, n * 128).view(n, 128)
        if b == 0 and self.k_overrides:
            for p, v in self.k_overrides.items():
                if p0 <= p < p1:
                    k[p - p0] = torch.from_numpy(v.view(np.int16)).to(self.device)
        return k

    def populate(self):
        """Store every context position of every request into all caches."""
        w = self.w
        for b in range(w.B):
            L = int(w.ctx[b])
            for p0 in range(0, L, self._chunk):
                p1 = min(L, p0 + self._chunk)
                n = p1 - p0
                req = torch.full((n,), b, dtype=torch.int32, device=self.device)
                pos = torch.arange(p0, p1, dtype=torch.int32, device=self.device)
                rows = dsa.Rows(req, pos, p1 - 1)
                for l in w.full_layers:
                    k = self._raw_keys(b, p0, p1)
                    dsa.dsa_index_k_store(k, rows, self.pages, self.index_cache[l], LN_EPS, ROPE_THETA)
                for l in self.layers:
                    kv = self._gen(gi.T_LATENT0 + l, (int(self.token_base[b]) + p0) * 576, n * 576).view(n, 576)
                    dsa.dsa_latent_store(kv, rows, self.pages, self.latent_cache[l])
        torch.cuda.synchronize()

    def build_mxfp4_index(self, layer: int = 0) -> torch.Tensor:
        """An MXFP4 index-K cache (68 B per token) of the same keys as the layer's FP8 one."""
        w = self.w
        cache = torch.zeros((w.num_pages, dsa.INDEX_MXFP4_PAGE_BYTES), dtype=torch.uint8, device=self.device)
        for b in range(w.B):
            L = int(w.ctx[b])
            for p0 in range(0, L, self._chunk):
                p1 = min(L, p0 + self._chunk)
                n = p1 - p0
                req = torch.full((n,), b, dtype=torch.int32, device=self.device)
                pos = torch.arange(p0, p1, dtype=torch.int32, device=self.device)
                k = self._raw_keys(b, p0, p1)
                dsa.dsa_index_k_store_mxfp4(k, dsa.Rows(req, pos, p1 - 1), self.pages, cache, LN_EPS, ROPE_THETA)
        torch.cuda.synchronize()
        return cache

    # ------------------------------------------------------------------ layer steps
    def tok_rows(self) -> dsa.Rows:
        return self.rows

    def full_layer(self, layer: int = 0):
        """Index-K store of the step's tokens, q quantisation, indexer logits, top-k, sparse MLA."""
        dsa.dsa_index_k_store(self.k_new, self.rows, self.pages, self.index_cache[layer], LN_EPS, ROPE_THETA)
        dsa.dsa_quant_fp8(self.q_idx, self.q8, self.qs)
        self.indexer_topk(layer)
        self.mla(layer)

    def indexer_topk(self, layer: int = 0):
        if self.row_chunks is None:
            dsa.dsa_indexer_topk(self.q8, self.qs, self.w_head, self.rows, self.pages, self.index_cache[layer],
                                 self.logits, TOPK, self.idx, self.ws_topk)
            return
        for a, b, rows in self.row_chunks:
            dsa.dsa_indexer_topk(self.q8[a:b], self.qs[a:b], self.w_head[a:b], rows, self.pages,
                                 self.index_cache[layer], self.logits[:b - a], TOPK, self.idx[a:b], self.ws_topk)

    def mla(self, layer: int):
        fn = dsa.dsa_sparse_mla_prefill if self.w.rows_per_req > 64 else dsa.dsa_sparse_mla_decode
        fn(self.q_mla[layer], self.rows, self.pages, self.latent_cache[layer], self.idx, self.out[layer],
           self.lse[layer], self.ws_mla, SM_SCALE)

    def shared_layer(self, layer: int):
        """A shared layer reuses the last full layer's top-k tensor as is (same device pointer)."""
        self.mla(layer)

    # ------------------------------------------------------------------ MTP draft round
    def _mtp_setup(self, steps: int):
        """Per-step inputs of an MTP draft iteration: step s of request b is the request's row s
        (position p_b + s) as a one-row-per-request batch, with that row's queries."""
        m = getattr(self, "_mtp", None)
        if m is not None and m["steps"] == steps:
            return m
        w, dev = self.w, self.device
        g = w.rows_per_req
        assert steps <= g, "a draft step per row of the request"
        B = w.R // g
        reqs = torch.arange(B, dtype=torch.int32, device=dev)
        m = {"steps": steps, "B": B, "rows": [], "q_idx": [], "w": [], "q_mla": [], "out": [], "lse": [], "idx": []}
        for st in range(steps):
            sel = torch.arange(B, device=dev) * g + st
            pos = self.rows.pos[sel].contiguous()
            m["rows"].append(dsa.Rows(reqs, pos, int(w.row_pos.max()), 1))
            m["q_idx"].append(self.q_idx[sel].contiguous())
            m["w"].append(self.w_head[sel].contiguous())
            m["q_mla"].append(self.q_mla[self.layers[0]][sel].contiguous())
            m["out"].append(torch.empty((B, 64, 512), dtype=torch.int16, device=dev))
            m["lse"].append(torch.empty((B, 64), dtype=torch.float32, device=dev))
            m["idx"].append(torch.empty((B, TOPK), dtype=torch.int32, device=dev))
        m["q8"] = torch.empty((B, 32, 128), dtype=torch.uint8, device=dev)
        m["qs"] = torch.empty((B, 32), dtype=torch.float32, device=dev)
        m["logits"] = torch.empty((B, self.stride), dtype=torch.float32, device=dev)
        m["ws_topk"] = torch.empty(max(dsa.dsa_topk_workspace_size(B, self.stride, TOPK), 256), dtype=torch.uint8,
                                   device=dev)
        nm = dsa.dsa_sparse_mla_workspace_size(B, TOPK)
        m["ws_mla"] = torch.empty(max(nm, 256), dtype=torch.uint8, device=dev) if nm else None
        self._mtp = m
        return m

    def mtp_draft_round(self, carry: bool = True, steps: int = 5, layer: int = 0):
        """One MTP draft iteration over `layer`'s caches (standing in for the MTP layer's own):
        step 0 scores and selects; with the carry, steps 1.. reuse step 0's idx tensor as is
        (the same device pointer); without it, every step scores and selects again."""
        m = self._mtp_setup(steps)
        for st in range(steps):
            idx = m["idx"][0 if carry else st]
            if st == 0 or not carry:
                dsa.dsa_quant_fp8(m["q_idx"][st], m["q8"], m["qs"])
                dsa.dsa_indexer_topk(m["q8"], m["qs"], m["w"][st], m["rows"][st], self.pages, self.index_cache[layer],
                                     m["logits"], TOPK, idx, m["ws_topk"])
            dsa.dsa_sparse_mla_decode(m["q_mla"][st], m["rows"][st], self.pages, self.latent_cache[layer], idx,
                                      m["out"][st], m["lse"][st], m["ws_mla"], SM_SCALE)
        return m

    def group_step(self):
        for l in self.layers:
            if l in self.w.full_layers:
                self.full_layer(l)
            else:
                self.shared_layer(l)
