"""One decode step of a CSA or HCA layer, driven through the C ABI.

This module owns device buffers (torch tensors) and calls the library's entry
points in order; it computes nothing itself.  A CSA step at position t is:

  csa_compress_many (main KV: ratio 4, 512 wide;   -> maybe emits entry t//4
                     index keys: ratio 4, 128 wide, rotated)
  csa_index_topk                                   -> top-k entry ids
  csa_sparse_attn_decode                           -> [B, H, 512]

and an HCA step is csa_compress (ratio 128) followed by hca_attn_decode.

With a block cache (workload extra "paged") the same steps run through the
paged calls: entries and index keys sit in pools of blocks placed by a
seeded permutation and found through block tables, and the window rings and
compressor slots sit in a pool of state slots (csa_index_topk_paged,
csa_sparse_attn_decode_paged, hca_attn_decode_paged; the compressors take
the table and slot map in their arguments).

With a layer configuration (workload extra "layer") the CSA step also runs
the layer's steps on either side of the path: csa_layer_input first (query
path, index queries and head weights, window-entry write, all from the
token's hidden state) and csa_layer_output last (grouped output projection).
"""

import torch

from . import _lib
from . import synth


def _dev_rows(x, fmt, device):
    """float32 host values -> device rows in fmt (quantized by the library)."""
    src = torch.from_numpy(x).to(device)
    if fmt == "f32":
        return src
    if fmt == "bf16":
        return src.to(torch.bfloat16)
    D = x.shape[-1]
    rb = _lib.kv_row_bytes(fmt, D)
    out = torch.empty(x.shape[:-1] + (rb,), dtype=torch.uint8, device=device)
    _lib.kv_quantize(src, "f32", out, fmt, src.numel() // D, D)
    return out


class BlockCache:
    """Block tables and state slots of a paged workload: logical block j of
    sequence b sits in pool block table[b][j] (a seeded permutation of all
    blocks), and sequence b's window ring and compressor slots in state slot
    slot[b] of a pool of n_slots."""

    def __init__(self, w, device="cuda"):
        cfg = w.extra["paged"]
        self.bs = cfg["block_entries"]
        self.n_slots = cfg["slots"]
        assert w.n_entries % self.bs == 0
        self.nb = w.n_entries // self.bs
        g = torch.Generator().manual_seed(w.seed)
        self.perm = torch.randperm(w.B * self.nb, generator=g).to(device)
        self.table = self.perm.reshape(w.B, self.nb).to(torch.int32)
        self.slot = torch.randperm(self.n_slots, generator=g)[:w.B].to(torch.int32).to(device)
        self.bt = _lib.make_block_table(self.table, self.bs, w.B * self.nb)

    def pool(self, rows):
        """Logical rows [B, N, ...] -> the pool [blocks, bs, ...] they fill."""
        B = rows.shape[0]
        blocks = rows.reshape((B * self.nb, self.bs) + tuple(rows.shape[2:]))
        out = torch.empty_like(blocks)
        out[self.perm] = blocks
        return out

    def slots(self, rows):
        """Per-sequence state [B, ...] -> the slot pool [n_slots, ...]."""
        out = torch.zeros((self.n_slots,) + tuple(rows.shape[1:]), dtype=rows.dtype,
                          device=rows.device)
        out[self.slot.long()] = rows
        return out


class Compressor:
    """Weights, slot state and output rows of one compressor on the device
    (with a BlockCache: `entries` is a block pool and the state a slot pool)."""

    def __init__(self, w, head_dim, ratio, rotate, entries, entry_fmt, rope, device="cuda",
                 indexer=False, cache=None):
        wkv, wg, ape, norm = synth.compressor_weights(w, head_dim, ratio, indexer=indexer)
        dt = torch.bfloat16 if w.q_fmt == "bf16" else torch.float32
        self.wkv = torch.from_numpy(wkv).to(device).to(dt)
        self.wg = torch.from_numpy(wg).to(device).to(dt)
        self.ape = torch.from_numpy(ape).to(device)
        self.norm = torch.from_numpy(norm).to(device)
        self.cache = cache
        coff = 2 if ratio == 4 else 1
        shape = (w.B if cache is None else cache.n_slots, coff * ratio, coff * head_dim)
        self.kv = torch.zeros(shape, dtype=torch.float32, device=device)
        self.sc = torch.full(shape, float("-inf"), dtype=torch.float32, device=device)
        self.w, self.head_dim, self.ratio, self.rotate = w, head_dim, ratio, rotate
        self.entries, self.entry_fmt = entries, entry_fmt
        self.cos, self.sin = rope
        self.x_fmt = w.q_fmt
        self._ws = None

    def args(self, x, start_pos):
        B, T = x.shape[0], x.shape[1]
        kw = dict(B=B, T=T, dim=self.w.dim, ratio=self.ratio, head_dim=self.head_dim,
                  rotate=self.rotate, x=x, x_fmt=self.x_fmt, w_kv=self.wkv, w_gate=self.wg,
                  w_fmt=self.x_fmt, ape=self.ape, norm_w=self.norm, eps=1e-6, rope_cos=self.cos,
                  rope_sin=self.sin, start_pos=start_pos, kv_state=self.kv, score_state=self.sc,
                  entries=self.entries, entry_fmt=self.entry_fmt)
        c = self.cache
        if c is None:
            return _lib.make_compress_args(**kw, entries_cap=self.entries.shape[1])
        return _lib.make_compress_args(**kw, block_table=c.table, block_entries=c.bs,
                                       pool_blocks=self.entries.shape[0], state_slot=c.slot)

    def __call__(self, x, start_pos):
        a = self.args(x, start_pos)
        need = _lib.csa_compress_workspace_size(a)
        if self._ws is None or self._ws.numel() < need:
            self._ws = _lib.workspace(need)
        _lib.csa_compress(a, self._ws)


def rope_tables(rows, yarn, device="cuda"):
    cos = torch.empty((rows, 32), dtype=torch.float32, device=device)
    sin = torch.empty_like(cos)
    if yarn:
        _lib.csa_rope_table(160000.0, 16.0, 65536, 32.0, 1.0, rows, cos, sin)
    else:
        _lib.csa_rope_table(160000.0, 0.0, 0, 0.0, 0.0, rows, cos, sin)
    return cos, sin


class CsaDecodeLayer:
    """All device state of a CSA layer decoding one token per sequence."""

    def __init__(self, w, device="cuda", copies=1, hidden_tail=7):
        self.w = w
        B, N = w.B, w.n_entries
        self.rope = rope_tables(w.ctx + 1, w.yarn, device)
        # cache contents: N(0,1) rows stored in the workload's formats; `copies`
        # independent sets rotate between steps so no step reuses the last one's
        # lines from the 256 MB last-level cache
        ent = _dev_rows(synth.entries(w), w.ent_fmt, device)
        keys = _dev_rows(synth.index_keys(w), w.key_fmt, device)
        self.win = _dev_rows(synth.window_rows(w), w.win_fmt, device)
        self.cache = BlockCache(w, device) if w.extra.get("paged") else None
        if self.cache is not None:
            assert not w.extra.get("layer") and not w.extra.get("reuse"), \
                "the block cache serves the path's calls only"
            ent, keys = self.cache.pool(ent), self.cache.pool(keys)
            self.win = self.cache.slots(self.win)
        self.sets = [(ent, keys)] + [(ent.clone(), keys.clone()) for _ in range(copies - 1)]
        q, sink = synth.queries(w)
        qi, wi = synth.index_queries(w)
        qdt = torch.bfloat16 if w.q_fmt == "bf16" else torch.float32
        self.q = torch.from_numpy(q).to(device).to(qdt).reshape(B, 1, w.H, 512)
        self.sink = torch.from_numpy(sink).to(device)
        self.qi = torch.from_numpy(qi).to(device).to(qdt).reshape(B, 1, w.Hi, 128)
        # the index call's queries: bf16 values, or for the FP4 indexer the
        # MXFP4 rows themselves (scored by the block-scaled FP4 MFMA); self.qi
        # keeps their values in bf16 (exact)
        self.qi_arg = (self.qi, w.q_fmt)
        if w.key_fmt == "fp4_mx32":
            n = B * w.Hi
            rows = torch.empty((n, _lib.kv_row_bytes("fp4_mx32", 128)), dtype=torch.uint8,
                               device=device)
            _lib.kv_quantize(self.qi.reshape(n, 128), "bf16", rows, "fp4_mx32", n, 128)
            _lib.kv_dequantize(rows, "fp4_mx32", self.qi.reshape(n, 128), "bf16", n, 128)
            if not w.extra.get("layer"):  # the layer's input step writes bf16 queries
                self.qi_arg = (rows.reshape(B, 1, w.Hi, rows.shape[1]), "fp4_mx32")
        self.wi = torch.from_numpy(wi).to(device).reshape(B, 1, w.Hi)
        self.t = w.t
        self.pos = torch.full((B, 1), self.t, dtype=torch.int32, device=device)
        self.start = torch.full((B,), self.t, dtype=torch.int32, device=device)
        self.x = torch.from_numpy(
            synth.normal_batched(w.seed, synth.T_X, B, (1, w.dim))).to(device).to(qdt)
        self.topk = torch.empty((B, 1, w.topk), dtype=torch.int32, device=device)
        self.out = torch.empty((B, 1, w.H, 512), dtype=qdt, device=device)
        self.ws_idx = _lib.workspace(_lib.csa_index_topk_workspace_size(B, 1, N, w.topk))
        self.ws_att = _lib.workspace(_lib.csa_sparse_attn_workspace_size(B, 1, w.H, w.topk))
        self.comp = []
        for c in range(copies):
            ent, keys = self.sets[c]
            self.comp.append((
                Compressor(w, 512, w.ratio, 0, ent, w.ent_fmt, self.rope, device,
                           cache=self.cache),
                Compressor(w, 128, w.ratio, 1, keys, w.key_fmt, self.rope, device, indexer=True,
                           cache=self.cache)))
        # fill the compressor states from the tokens before t (positions t-7 .. t-1)
        if hidden_tail:
            tail = torch.from_numpy(synth.normal_batched(
                w.seed, synth.T_XTAIL, B, (hidden_tail, w.dim))).to(device).to(qdt)
            st = torch.full((B,), self.t - hidden_tail, dtype=torch.int32, device=device)
            for cm, ci in self.comp:
                cm(tail, st)
                ci(tail, st)
        self.ws_comp = [None] * copies
        self.step_no = 0
        self.lw = None
        if w.extra.get("layer"):
            self._init_layer(w.extra["layer"], copies, device)
        # reuse layers of a layer group: their own queries, sinks and windows,
        # the Full layer's entries and top-k ids; the whole group attends in
        # one csa_sparse_attn_decode_shared call (layer-major rows)
        self.reuse = []
        for layer in range(1, w.extra.get("reuse", 0) + 1):
            rq, rsink, rwin = synth.reuse_layer_inputs(w, layer)
            self.reuse.append((
                torch.from_numpy(rq).to(device).to(qdt).reshape(B, 1, w.H, 512),
                torch.from_numpy(rsink).to(device),
                _dev_rows(rwin, w.win_fmt, device),
                torch.empty((B, 1, w.H, 512), dtype=qdt, device=device)))
        if self.reuse:
            L = 1 + len(self.reuse)
            self.q_group = torch.cat([self.q] + [r[0] for r in self.reuse])
            self.win_group = torch.cat([self.win] + [r[2] for r in self.reuse])
            self.sink_group = torch.cat([self.sink] + [r[1] for r in self.reuse])
            self.pos_group = self.pos.repeat(L, 1)
            self.out_group = torch.empty((L * B, 1, w.H, 512), dtype=qdt, device=device)
            # the Full layer's buffers are views into the group's, so whatever
            # writes them (csa_layer_input included) is what the group reads
            self.q = self.q_group[:B]
            self.win = self.win_group[:B]
            self.out = self.out_group[:B]
            self.reuse = [(self.q_group[(i + 1) * B:(i + 2) * B], rs,
                           self.win_group[(i + 1) * B:(i + 2) * B],
                           self.out_group[(i + 1) * B:(i + 2) * B])
                          for i, (_, rs, _, _) in enumerate(self.reuse)]
            self.ws_group = _lib.workspace(
                _lib.csa_sparse_attn_workspace_size(L * B, 1, w.H, w.topk))

    def _init_layer(self, cfg, copies, device):
        w = self.w
        wn = synth.layer_weights(w.seed, w.dim, cfg["q_rank"], w.H, w.Hi, cfg["groups"],
                                 cfg["o_rank"])
        dev = {k: (torch.from_numpy(v).to(device) if k in ("q_norm", "kv_norm")
                   else torch.from_numpy(v).to(device).to(torch.bfloat16)) for k, v in wn.items()}
        # weight copies rotate with the cache copies, so a step does not find
        # the previous step's weights in the last-level cache
        self.lw_tensors = [dev] + [{k: v.clone() for k, v in dev.items()}
                                   for _ in range(copies - 1)]
        self.lw = [_lib.make_layer_weights(dim=w.dim, q_rank=cfg["q_rank"], H=w.H, Hi=w.Hi,
                                           groups=cfg["groups"], o_rank=cfg["o_rank"], **d)
                   for d in self.lw_tensors]
        self.y = torch.empty((w.B, w.dim), dtype=torch.bfloat16, device=device)
        self.ws_lin = _lib.workspace(_lib.csa_layer_input_workspace_size(self.lw[0], w.B))
        self.ws_lout = _lib.workspace(_lib.csa_layer_output_workspace_size(self.lw[0], w.B))

    def phases(self):
        """The step as a list of (name, callable) in stream order."""
        w = self.w
        c = self.step_no % len(self.sets)
        ent, keys = self.sets[c]
        cm, ci = self.comp[c]
        win_fmt, ent_fmt, key_fmt = w.win_fmt, w.ent_fmt, w.key_fmt
        B, N = w.B, w.n_entries

        def compress():
            args = [cm.args(self.x, self.start), ci.args(self.x, self.start)]
            need = _lib.csa_compress_many_workspace_size(args)
            if self.ws_comp[c] is None or self.ws_comp[c].numel() < need:
                self.ws_comp[c] = _lib.workspace(need)
            _lib.csa_compress_many(args, self.ws_comp[c])

        # the FP4 indexer ranks bf16 scores
        index_fn = _lib.csa_index_topk_bf16 if key_fmt == "fp4_mx32" else _lib.csa_index_topk

        def index_topk():
            index_fn(*self.qi_arg, self.wi, keys, key_fmt, self.pos, w.ratio, B, 1, w.Hi, N,
                     w.topk, self.topk, None, self.ws_idx)

        def sparse_attn():
            _lib.csa_sparse_attn_decode(self.q, w.q_fmt, self.win, win_fmt, _lib.WIN_RING128,
                                        None, 128, ent, ent_fmt, N, self.topk, w.topk, self.pos, B,
                                        1, w.H, self.sink, 512 ** -0.5, self.rope[0],
                                        self.rope[1], self.out, w.q_fmt, self.ws_att)

        pc = self.cache
        if pc is not None:
            def index_topk():  # noqa: F811 -- the block-cache form of the same call
                _lib.csa_index_topk_paged(*self.qi_arg, self.wi, keys, key_fmt, pc.bt,
                                          self.pos, w.ratio, B, 1, w.Hi, w.topk,
                                          int(key_fmt == "fp4_mx32"), self.topk, None,
                                          self.ws_idx)

            def sparse_attn():  # noqa: F811
                _lib.csa_sparse_attn_decode_paged(self.q, w.q_fmt, self.win, win_fmt, pc.slot,
                                                  pc.n_slots, ent, ent_fmt, pc.bt, self.topk,
                                                  w.topk, self.pos, B, 1, w.H, self.sink,
                                                  512 ** -0.5, self.rope[0], self.rope[1],
                                                  self.out, w.q_fmt, self.ws_att)

        core = [("csa_compress", compress), ("csa_index_topk", index_topk),
                ("csa_sparse_attn_decode", sparse_attn)]
        if self.reuse:
            L = 1 + len(self.reuse)

            def group_attn():
                _lib.csa_sparse_attn_decode_shared(
                    self.q_group, w.q_fmt, self.win_group, win_fmt, ent, ent_fmt, N, self.topk,
                    w.topk, self.pos_group, L * B, 1, w.H, B, self.sink_group, 512 ** -0.5,
                    self.rope[0], self.rope[1], self.out_group, w.q_fmt, self.ws_group)

            core[2] = ("csa_sparse_attn_group", group_attn)
        if self.lw is None:
            return core
        lw = self.lw[c]

        def layer_input():
            _lib.csa_layer_input(lw, self.x, self.pos, B, 1, self.rope[0], self.rope[1], self.q,
                                 self.qi, self.wi, self.win, win_fmt, self.ws_lin)

        def layer_output():
            _lib.csa_layer_output(lw, self.out, B, self.y, "bf16", self.ws_lout)

        return [("csa_layer_input", layer_input)] + core + [("csa_layer_output", layer_output)]

    def step(self):
        for _, f in self.phases():
            f()
        self.step_no += 1


class HcaDecodeLayer:
    """All device state of an HCA layer decoding one token per sequence."""

    def __init__(self, w, device="cuda", copies=1, hidden_tail=7):
        self.w = w
        B, N = w.B, w.n_entries
        self.rope = rope_tables(w.ctx + 1, w.yarn, device)
        ent = _dev_rows(synth.entries(w), w.ent_fmt, device)
        self.win = _dev_rows(synth.window_rows(w), w.win_fmt, device)
        self.cache = BlockCache(w, device) if w.extra.get("paged") else None
        if self.cache is not None:
            ent = self.cache.pool(ent)
            self.win = self.cache.slots(self.win)
        self.sets = [ent] + [ent.clone() for _ in range(copies - 1)]
        q, sink = synth.queries(w)
        qdt = torch.bfloat16 if w.q_fmt == "bf16" else torch.float32
        self.q = torch.from_numpy(q).to(device).to(qdt).reshape(B, 1, w.H, 512)
        self.sink = torch.from_numpy(sink).to(device)
        self.t = w.t
        self.pos = torch.full((B, 1), self.t, dtype=torch.int32, device=device)
        self.start = torch.full((B,), self.t, dtype=torch.int32, device=device)
        self.x = torch.from_numpy(
            synth.normal_batched(w.seed, synth.T_X, B, (1, w.dim))).to(device).to(qdt)
        self.out = torch.empty((B, 1, w.H, 512), dtype=qdt, device=device)
        self.ws_att = _lib.workspace(_lib.hca_attn_workspace_size(B, 1, w.H, N))
        self.comp = [Compressor(w, 512, w.ratio, 0, e, w.ent_fmt, self.rope, device,
                                cache=self.cache)
                     for e in self.sets]
        if hidden_tail:
            tail = torch.from_numpy(synth.normal_batched(
                w.seed, synth.T_XTAIL, B, (hidden_tail, w.dim))).to(device).to(qdt)
            st = torch.full((B,), self.t - hidden_tail, dtype=torch.int32, device=device)
            for cm in self.comp:
                cm(tail, st)
        self.step_no = 0

    def phases(self):
        w = self.w
        c = self.step_no % len(self.sets)
        ent = self.sets[c]
        cm = self.comp[c]

        def compress_main():
            cm(self.x, self.start)

        def hca_attn():
            pc = self.cache
            if pc is not None:
                _lib.hca_attn_decode_paged(self.q, w.q_fmt, self.win, w.win_fmt, pc.slot,
                                           pc.n_slots, ent, w.ent_fmt, pc.bt, w.ratio, self.pos,
                                           w.B, 1, w.H, self.sink, 512 ** -0.5, self.rope[0],
                                           self.rope[1], self.out, w.q_fmt, self.ws_att)
                return
            _lib.hca_attn_decode(self.q, w.q_fmt, self.win, w.win_fmt, _lib.WIN_RING128, None, 128,
                                 ent, w.ent_fmt, w.n_entries, w.ratio, self.pos, w.B, 1, w.H,
                                 self.sink, 512 ** -0.5, self.rope[0], self.rope[1], self.out,
                                 w.q_fmt, self.ws_att)

        return [("csa_compress", compress_main), ("hca_attn_decode", hca_attn)]

    def step(self):
        for _, f in self.phases():
            f()
        self.step_no += 1
