"""One chunked-prefill step of a CSA layer, driven through the C ABI.

A chunk of T new tokens (positions P .. P+T-1) is appended to a sequence whose
first P tokens are already compressed.  The step is the same three calls as a
decode step, with T queries per sequence and causal visibility per query:

  csa_compress_many (main KV and index keys, T tokens) -> entries P/4 .. (P+T)/4 - 1
  csa_index_topk    (T queries; query i sees ids < (P+i+1)/4) -> top-k ids per query
  csa_sparse_attn_decode (T queries, LINEAR window of raw rows P-127 .. P+T-1)

This module owns the device buffers (torch tensors) and calls the entry points
in order; it computes nothing itself.
"""

import torch

from . import _lib
from . import synth
from .decode import Compressor, rope_tables


class CsaPrefillChunk:
    """Device state of one prefill chunk (batch 1) on a compressed prefix."""

    def __init__(self, w, device="cuda"):
        self.w = w
        P, T, N0, N = synth.prefill_shape(w)
        self.P, self.T, self.N0, self.N = P, T, N0, N
        dt = torch.bfloat16
        self.rope = rope_tables(P + T + 1, w.yarn, device)

        def up(a):
            return torch.from_numpy(a).to(device).to(dt)

        # cache: the prefix's entries and index keys; the chunk appends N - N0 rows
        self.ent = torch.empty((1, N, 512), dtype=dt, device=device)
        self.keys = torch.empty((1, N, 128), dtype=dt, device=device)
        step = 8192
        for lo in range(0, N0, step):
            hi = min(N0, lo + step)
            self.ent[0, lo:hi] = up(synth.prefill_entries(w, lo, hi))
            self.keys[0, lo:hi] = up(synth.prefill_index_keys(w, lo, hi))
        # raw window rows of positions P-127 .. P+T-1, addressed linearly
        self.win_rows = T + 127
        self.win = torch.empty((1, self.win_rows, 512), dtype=dt, device=device)
        self.q = torch.empty((1, T, w.H, 512), dtype=dt, device=device)
        self.qi = torch.empty((1, T, w.Hi, 128), dtype=dt, device=device)
        self.wi = torch.empty((1, T, w.Hi), dtype=torch.float32, device=device)
        self.x = torch.empty((1, T, w.dim), dtype=dt, device=device)
        step = 2048
        for lo in range(0, T, step):
            hi = min(T, lo + step)
            self.q[0, lo:hi] = up(synth.prefill_queries(w, lo, hi))
            qi, wi = synth.prefill_index_queries(w, lo, hi)
            self.qi[0, lo:hi] = up(qi)
            self.wi[0, lo:hi] = torch.from_numpy(wi).to(device)
            self.x[0, lo:hi] = up(synth.prefill_hidden(w, lo, hi))
        for lo in range(0, self.win_rows, step):
            hi = min(self.win_rows, lo + step)
            self.win[0, lo:hi] = up(synth.prefill_window(w, lo, hi))
        self.win_base = torch.tensor([P - 127], dtype=torch.int32, device=device)
        self.sink = torch.from_numpy(synth.prefill_sink(w)).to(device)
        self.pos = (torch.arange(T, dtype=torch.int32, device=device) + P).reshape(1, T)
        self.start = torch.tensor([P], dtype=torch.int32, device=device)

        # compressors; their state comes from the prefix's last block (positions
        # P-4 .. P-1): compressing it leaves those projections in the previous
        # slots and empty current slots.  entries_cap = N0 - 1 keeps the set-up
        # call from rewriting the prefix's last stored entry.
        self.cm = Compressor(w, 512, 4, 0, self.ent, "bf16", self.rope, device)
        self.ci = Compressor(w, 128, 4, 1, self.keys, "bf16", self.rope, device, indexer=True)
        tail = up(synth.prefill_tail(w)).reshape(1, 4, w.dim)
        st = torch.tensor([P - 4], dtype=torch.int32, device=device)
        for c, buf in ((self.cm, self.ent), (self.ci, self.keys)):
            c.entries = buf[:, :N0 - 1]
            c(tail, st)
            c.entries = buf
        # every step starts from this state
        self.state0 = [(c.kv.clone(), c.sc.clone()) for c in (self.cm, self.ci)]

        self.topk = torch.empty((1, T, w.topk), dtype=torch.int32, device=device)
        self.out = torch.empty((1, T, w.H, 512), dtype=dt, device=device)
        self.ws_idx = _lib.workspace(_lib.csa_index_topk_workspace_size(1, T, N, w.topk))
        self.ws_att = _lib.workspace(_lib.csa_sparse_attn_workspace_size(1, T, w.H, w.topk))
        args = [self.cm.args(self.x, self.start), self.ci.args(self.x, self.start)]
        self.ws_comp = _lib.workspace(_lib.csa_compress_many_workspace_size(args))
        self.step_no = 0

    def phases(self):
        w = self.w
        T, N = self.T, self.N

        def compress():
            for c, (kv, sc) in zip((self.cm, self.ci), self.state0):
                c.kv.copy_(kv)
                c.sc.copy_(sc)
            args = [self.cm.args(self.x, self.start), self.ci.args(self.x, self.start)]
            _lib.csa_compress_many(args, self.ws_comp)

        def index_topk():
            _lib.csa_index_topk(self.qi, "bf16", self.wi, self.keys, "bf16", self.pos, 4, 1, T,
                                w.Hi, N, w.topk, self.topk, None, self.ws_idx)

        def sparse_attn():
            _lib.csa_sparse_attn_decode(self.q, "bf16", self.win, "bf16", _lib.WIN_LINEAR,
                                        self.win_base, self.win_rows, self.ent, "bf16", N,
                                        self.topk, w.topk, self.pos, 1, T, w.H, self.sink,
                                        512 ** -0.5, self.rope[0], self.rope[1], self.out, "bf16",
                                        self.ws_att)

        return [("csa_compress", compress), ("csa_index_topk", index_topk),
                ("csa_sparse_attn_decode", sparse_attn)]

    def step(self):
        for _, f in self.phases():
            f()
        self.step_no += 1
