"""Layer chaining for one decode step (LycheeDecode summary page, method steps 1, 3, 4).

A decode step runs the layers in order on one stream: layer 0 is all retrieval and
seeds S; every later layer reads S^{l} and writes S^{l+1} in place (retrieval rows
replaced, sparse rows untouched). After layer 0 the workspace's membership bitmaps
track S, so later layers pass LD_FLAG_S_CHAINED and never re-read S.
HySparse-style stacks (section 3 of the HySparse page) pass the full layer's K/V
for the sparse layers; with window_len > 0 a sparse layer given its own window cache
and gate runs the gated block-sparse + sliding-window layer instead, on a workspace
whose leading part is the full layer's, so the chained bitmaps carry over.
"""
from __future__ import annotations

from typing import List, Optional, Sequence

import numpy as np

from . import (FLAG_BLOCK_SELECT, FLAG_S_CHAINED, HySparseWorkspace, Workspace, hybrid_layer, hybrid_layer_plan,
               hysparse_layer, make_shape)


class DecodeStep:
    """Buffers and launch sequence of one decode step over L layers."""

    def __init__(self, batch: int, num_q_heads: int, num_kv_heads: int, head_dim: int,
                 seq_lens: Sequence[int], k_per_seq: Sequence[int], retrieval_masks: Sequence[int],
                 csr: bool = False, device="cuda", split_flag: int = 0, window_len: int = 0):
        import torch
        self.torch = torch
        self.B, self.Hq, self.Hkv, self.d = batch, num_q_heads, num_kv_heads, head_dim
        self.seq_lens = [int(n) for n in seq_lens]
        self.N = max(self.seq_lens)
        self.k = [min(int(k), n) for k, n in zip(k_per_seq, self.seq_lens)]
        self.masks = [int(m) for m in retrieval_masks]
        all_heads = (1 << num_q_heads) - 1
        if self.masks[0] != all_heads:
            raise ValueError("every head of layer 0 must be a retrieval head")
        self.L = len(self.masks)
        self.device = device
        self.split_flag = split_flag
        self.window_len = int(window_len)
        ragged = len(set(self.seq_lens)) > 1 or csr
        offs = np.concatenate([[0], np.cumsum(self.seq_lens)]).astype(np.int64)
        self.kv_offsets = offs
        self.total_tokens = int(offs[-1])
        self.kv_indptr = torch.as_tensor(offs, device=device) if ragged else None
        if csr:
            rows = [self.k[b] for b in range(batch) for _ in range(num_q_heads)]
            self.s_indptr_host = np.concatenate([[0], np.cumsum(rows)]).astype(np.int64)
            self.s_indptr = torch.as_tensor(self.s_indptr_host, device=device)
            self.S = torch.zeros(int(self.s_indptr_host[-1]), dtype=torch.int32, device=device)
            self.k_arg = max(self.k)
        else:
            if len(set(self.k)) != 1:
                raise ValueError("dense S needs one k for every sequence (use csr=True)")
            self.s_indptr_host, self.s_indptr = None, None
            self.S = torch.zeros((batch, num_q_heads, self.k[0]), dtype=torch.int32, device=device)
            self.k_arg = self.k[0]
        self.outs = [torch.empty((batch, num_q_heads, head_dim), dtype=torch.bfloat16, device=device)
                     for _ in range(self.L)]
        self.workspace = None

    def _ws(self, q, kc):
        if self.workspace is None:
            shape = make_shape(q, kc, self.kv_indptr, self.N)
            if self.window_len:
                self.workspace = HySparseWorkspace(shape, self.k_arg, self.window_len, self.device)
            else:
                self.workspace = Workspace(shape, self.k_arg, self.device)
        return self.workspace

    def layer(self, l: int, q, kc, vc, extra_flags: int = 0, scores_out=None, block_table=None,
              page_size: int = 0, window=None):
        """Launch layer l (asynchronous). Paged KV: kc/vc are page pools and block_table
        maps each sequence's pages. window = (k_window, v_window, gate) runs a layer
        without retrieval heads as the gated block-sparse + window layer."""
        flags = (FLAG_S_CHAINED if l > 0 else 0) | self.split_flag | extra_flags
        if window is not None:
            if l == 0 or self.masks[l] or not self.window_len:
                raise ValueError("window branches need a sparse layer after the first and window_len")
            if self.s_indptr is not None:
                raise ValueError("window branches are set up for dense S")
            return hysparse_layer(q, kc, vc, self.k_arg, self.S, window[0], window[1], window[2],
                                  out=self.outs[l], flags=FLAG_S_CHAINED | (self.split_flag & FLAG_BLOCK_SELECT),
                                  workspace=self._ws(q, kc),
                                  kv_indptr=self.kv_indptr, seq_len=self.N, block_table=block_table,
                                  page_size=page_size)
        return hybrid_layer(q, kc, vc, self.masks[l], self.k_arg, self.S if l > 0 else None,
                            s_out=self.S, s_indptr=self.s_indptr, scores_out=scores_out,
                            out=self.outs[l], flags=flags, workspace=self._ws(q, kc),
                            kv_indptr=self.kv_indptr, seq_len=self.N, block_table=block_table,
                            page_size=page_size)

    def plan(self, l: int, q, kc, vc, extra_flags: int = 0, block_table=None, page_size: int = 0,
             window=None) -> Optional[dict]:
        """The launches layer(l, ...) makes with the same arguments (see hybrid_layer_plan);
        None for a window layer, which has its own entry point."""
        if window is not None:
            return None
        flags = (FLAG_S_CHAINED if l > 0 else 0) | self.split_flag | extra_flags
        return hybrid_layer_plan(q, kc, vc, self.masks[l], self.k_arg, self.S if l > 0 else None,
                                 s_out=self.S, s_indptr=self.s_indptr, out=self.outs[l], flags=flags,
                                 kv_indptr=self.kv_indptr, seq_len=self.N, block_table=block_table,
                                 page_size=page_size)

    def run(self, layers: List, events: Optional[list] = None, windows: Optional[list] = None):
        """One decode step. layers[l] = (q, k, v) device tensors, or (q, k_pool, v_pool,
        block_table, page_size) for paged KV. windows[l]: (k_window, v_window, gate) or
        None per layer. If `events` is a list of L+1 torch.cuda.Event (or None entries),
        events[l] is recorded right before layer l and events[L] after the last layer."""
        for l in range(self.L):
            if events is not None and events[l] is not None:
                events[l].record()
            q, kc, vc = layers[l][:3]
            win = windows[l] if windows is not None else None
            if len(layers[l]) > 3:
                self.layer(l, q, kc, vc, block_table=layers[l][3], page_size=layers[l][4], window=win)
            else:
                self.layer(l, q, kc, vc, window=win)
        if events is not None and events[self.L] is not None:
            events[self.L].record()
        return self.outs

    def s_rows(self):
        """Host copy of S as {(b, h): int64 indices}."""
        S = self.S.cpu().numpy()
        out = {}
        for b in range(self.B):
            for h in range(self.Hq):
                r = b * self.Hq + h
                if self.s_indptr_host is None:
                    out[(b, h)] = S[b, h].astype(np.int64)
                else:
                    out[(b, h)] = S[self.s_indptr_host[r]:self.s_indptr_host[r + 1]].astype(np.int64)
        return out
