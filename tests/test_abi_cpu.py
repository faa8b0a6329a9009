"""The C-ABI library loads, exports every symbol include/csa.h declares, and
rejects bad arguments on the host before touching a GPU (CPU only)."""

import ctypes
import os
import re

import pytest

from kv_cache_decode_csa_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "csa.h")

if not os.path.exists(_lib.LIB_PATH):
    pytest.skip("libcsa.so not built (python -m kv_cache_decode_csa_amd.build)",
                allow_module_level=True)

EINVAL, EUNSUP, EWS = 1, 2, 3
A16 = 0x10000  # a fake, 16-byte aligned address: validation never dereferences it


def declared():
    text = open(HEADER).read()
    names = re.findall(r"^\s*(?:csa_status|size_t|const char\*)\s+(\w+)\s*\(", text, re.M)
    return sorted(set(names))


def test_header_symbols_exported():
    L = _lib.lib()
    names = declared()
    assert len(names) >= 16
    for n in names:
        assert hasattr(L, n), n
    # the binding wraps exactly the declared entry points
    assert sorted(_lib.EXPORTS) == names


def test_row_bytes_and_strings():
    L = _lib.lib()
    assert L.kv_row_bytes(_lib.FP8_MX32, 512) == 528
    assert L.kv_row_bytes(_lib.FP4_E4M3_16, 512) == 288
    assert L.kv_row_bytes(_lib.FP8_MX32, 128) == 132
    assert L.kv_row_bytes(_lib.BF16, 512) == 1024
    assert L.kv_row_bytes(_lib.FP8_MX32, 100) == 0
    assert L.kv_row_bytes(_lib.FP4_MX32, 128) == 68
    assert L.kv_row_bytes(_lib.MIX576, 512) == 592
    assert L.kv_row_bytes(_lib.MIX576, 128) == 0
    assert L.kv_row_bytes(9, 512) == 0
    assert L.csa_strerror(0) == b"ok"
    assert L.csa_strerror(3) == b"workspace too small"


def _detail():
    return _lib.lib().csa_last_error_detail().decode()


def test_codec_validation():
    L = _lib.lib()
    assert L.kv_quantize(None, 0, A16, 2, 4, 512, None) == EINVAL
    assert "src" in _detail()
    assert L.kv_quantize(A16, 0, A16, 2, 4, 500, None) == EINVAL       # dim % 32
    assert L.kv_quantize(A16, 2, A16, 2, 4, 512, None) == EUNSUP       # src must be F32/BF16
    assert L.kv_quantize(A16, 0, A16, 7, 4, 512, None) == EUNSUP
    assert L.kv_quantize(A16 + 4, 0, A16, 2, 4, 512, None) == EINVAL  # misaligned
    assert L.kv_quantize(None, 0, None, 2, 0, 512, None) == 0          # empty: no work
    assert L.kv_dequantize(A16, 2, A16, 2, 4, 512, None) == EUNSUP     # dst must be F32/BF16


def test_topk_validation():
    L = _lib.lib()
    assert L.csa_topk(A16, A16, 4, 100, 0, A16, A16, 1 << 30, None) == EUNSUP      # topk 0
    assert L.csa_topk(A16, A16, 4, 100, 4096, A16, A16, 1 << 30, None) == EUNSUP   # > max
    assert L.csa_topk(A16, A16, 4, 0, 8, A16, A16, 1 << 30, None) == EINVAL        # ld
    need = L.csa_topk_workspace_size(4, 100, 8)
    assert need > 0
    assert L.csa_topk(A16, A16, 4, 100, 8, A16, A16, need - 1, None) == EWS
    assert L.csa_topk(A16, A16, 4, 100, 8, A16, None, need, None) == EWS


def test_index_topk_validation():
    L = _lib.lib()
    ws = L.csa_index_topk_workspace_size(2, 1, 1000, 64)
    args = lambda **kw: dict(dict(q=A16, qf=1, w=A16, k=A16, kf=2, pos=A16, ratio=4, B=2, Q=1,
                                  Hi=64, N=1000, topk=64, out=A16, sc=None, ws=A16, wsb=ws), **kw)

    def call(d):
        return L.csa_index_topk(d["q"], d["qf"], d["w"], d["k"], d["kf"], d["pos"], d["ratio"],
                                d["B"], d["Q"], d["Hi"], d["N"], d["topk"], d["out"], d["sc"],
                                d["ws"], d["wsb"], None)

    assert call(args(Hi=24)) == EUNSUP          # multiple of 16 on the MFMA path
    assert call(args(Hi=256)) == EUNSUP
    assert call(args(kf=3)) == EUNSUP           # FP4 keys: not on this path
    assert call(args(qf=0)) == EUNSUP           # bf16/fp8 keys need bf16 queries
    assert call(args(qf=4)) == EUNSUP           # FP4 queries need FP4 keys
    assert call(args(qf=4, kf=1)) == EUNSUP
    assert call(args(qf=4, kf=4, Hi=24)) == EUNSUP
    assert call(args(qf=4, kf=4, q=None)) == EINVAL
    assert call(args(kf=0)) == EUNSUP           # f32 keys need f32 queries
    assert call(args(topk=0)) == EUNSUP
    assert call(args(N=0)) == EINVAL
    assert call(args(q=None)) == EINVAL
    assert call(args(wsb=ws - 1)) == EWS


def _attn_call(L, **kw):
    d = dict(q=A16, qf=1, win=A16, wf=1, wm=0, wb=None, wr=128, ent=A16, ef=2, N=1000, idx=A16,
             topk=64, pos=A16, B=1, Q=1, H=64, sink=A16, scale=0.044, cos=A16, sin=A16,
             rr=2048, out=A16, of=1)
    d.update(kw)
    ws = L.csa_sparse_attn_workspace_size(d["B"], d["Q"], d["H"], d["topk"])
    return L.csa_sparse_attn_decode(d["q"], d["qf"], d["win"], d["wf"], d["wm"], d["wb"], d["wr"],
                                    d["ent"], d["ef"], d["N"], d["idx"], d["topk"], d["pos"],
                                    d["B"], d["Q"], d["H"], d["sink"], d["scale"], d["cos"],
                                    d["sin"], d["rr"], d["out"], d["of"], kw.get("ws", A16),
                                    kw.get("wsb", ws), None)


def test_attention_validation():
    L = _lib.lib()
    assert _attn_call(L, H=40) == EUNSUP
    assert _attn_call(L, wr=64) == EINVAL            # ring needs 128 rows
    assert _attn_call(L, wm=1) == EINVAL             # linear mode needs win_base
    assert _attn_call(L, ef=0) == EUNSUP             # f32 rows need f32 queries
    assert _attn_call(L, of=2) == EUNSUP
    assert _attn_call(L, topk=10000) == EUNSUP
    assert _attn_call(L, idx=None) == EINVAL
    assert _attn_call(L, scale=float("nan")) == EINVAL
    assert _attn_call(L, ws=None) == EWS
    ws = L.hca_attn_workspace_size(16, 1, 64, 8192)
    assert ws > 0
    assert L.hca_attn_decode(A16, 1, A16, 1, 0, None, 128, A16, 1, 8192, 0, A16, 16, 1, 64, A16,
                             0.044, A16, A16, 100, A16, 1, A16, ws, None) == EINVAL  # ratio 0


def test_attention_workspace_follows_the_work_split():
    """Decode lists of at most 640 rows take one work-group per list from 256
    (unit, 16-head group) items on, with no partials (workspace 0); smaller
    batches split lists into 64-row chunks and need one partial per chunk;
    16+ queries per sequence take 640-row chunks (one chunk: no partials)."""
    L = _lib.lib()
    part = (16 + 16 + 16 * 512) * 4  # m, l, O of one (unit, head group, chunk)
    assert L.csa_sparse_attn_workspace_size(8, 1, 64, 512) == 8 * 4 * 10 * part
    assert L.csa_sparse_attn_workspace_size(63, 1, 64, 512) == 63 * 4 * 10 * part
    assert L.csa_sparse_attn_workspace_size(64, 1, 64, 512) == 0
    assert L.csa_sparse_attn_workspace_size(32, 1, 128, 512) == 0
    assert L.csa_sparse_attn_workspace_size(22, 3, 64, 300) == 0
    assert L.csa_sparse_attn_workspace_size(64, 1, 64, 600) > 0      # 728 rows: chunks
    assert L.csa_sparse_attn_workspace_size(2, 20, 64, 512) == 0     # one 640-row chunk


def test_compress_validation():
    L = _lib.lib()
    a = _lib.CompressArgs(1, 4, 1024, 4, 512, 0, A16, 0, A16, A16, 0, A16, A16, 1e-6, A16, A16,
                          100, A16, A16, A16, A16, 0, 16)
    assert L.csa_compress_workspace_size(ctypes.byref(a)) == 4 * 2 * 1024 * 4
    a.ratio = 8
    assert L.csa_compress(ctypes.byref(a), A16, 1 << 20, None) == EUNSUP
    a.ratio = 4
    a.rotate = 1
    assert L.csa_compress(ctypes.byref(a), A16, 1 << 20, None) == EUNSUP  # rotate needs d 128
    a.rotate = 0
    a.x = None
    assert L.csa_compress(ctypes.byref(a), A16, 1 << 20, None) == EINVAL
    a.x = A16
    assert L.csa_compress(ctypes.byref(a), A16, 10, None) == EWS
    assert L.csa_compress(None, A16, 10, None) == EINVAL


def test_rope_table_validation():
    L = _lib.lib()
    assert L.csa_rope_table(160000.0, 16.0, 65536, 32.0, 1.0, 0, A16, A16, None) == EINVAL
    assert L.csa_rope_table(1.0, 0.0, 0, 0.0, 0.0, 10, A16, A16, None) == EINVAL
    assert L.csa_rope_table(160000.0, 16.0, 0, 32.0, 1.0, 10, A16, A16, None) == EINVAL


def _layer_weights(**kw):
    d = dict(dim=4096, q_rank=1024, H=64, Hi=64, groups=8, o_rank=1024)
    d.update(kw)
    return _lib.LayerWeights(d["dim"], d["q_rank"], d["H"], d["Hi"], d["groups"], d["o_rank"],
                             A16, A16, A16, A16, A16, A16, A16, A16, A16, 1e-6)


def test_layer_validation():
    L = _lib.lib()
    w = _layer_weights()
    need = L.csa_layer_input_workspace_size(ctypes.byref(w), 8)
    assert need > 0 and L.csa_layer_output_workspace_size(ctypes.byref(w), 8) > 0

    def inp(w, B=8, T=1, win_fmt=2, ws=A16, wsb=1 << 30):
        return L.csa_layer_input(ctypes.byref(w), A16, A16, B, T, A16, A16, 100, A16, A16, A16,
                                 A16, win_fmt, ws, wsb, None)

    assert inp(w, B=65) == EUNSUP                     # M = B*T above 64
    assert inp(w, B=8, T=9) == EUNSUP
    assert inp(w, win_fmt=4) == EUNSUP                # FP4_MX32 is not a window format
    assert inp(w, ws=None) == EWS
    assert inp(w, wsb=need - 1) == EWS
    assert inp(_layer_weights(q_rank=3072)) == EINVAL  # q_rank above 2048
    assert inp(_layer_weights(dim=1000)) == EINVAL
    assert inp(_layer_weights(groups=7)) == EINVAL     # groups must divide H
    assert inp(_layer_weights(Hi=65)) == EUNSUP
    w0 = _layer_weights()
    w0.wq_b = None
    assert inp(w0) == EINVAL
    assert L.csa_layer_output(ctypes.byref(w), A16, 8, A16, 2, A16, 1 << 30, None) == EUNSUP
    assert L.csa_layer_output(ctypes.byref(_layer_weights(o_rank=48)), A16, 8, A16, 1, A16,
                              1 << 30, None) == EINVAL


def test_shared_attention_and_mixed_rows_validation():
    L = _lib.lib()

    def shared(B=12, ent_seqs=3, ef=2, qf=1):
        return L.csa_sparse_attn_decode_shared(A16, qf, A16, 2, A16, ef, 1000, A16, 512, A16, B, 1,
                                               64, ent_seqs, A16, 0.044, A16, A16, 100, A16, 1,
                                               A16, 1 << 30, None)

    assert shared(ent_seqs=5) == EINVAL               # must divide B
    assert shared(ent_seqs=0) == EINVAL
    assert shared(ef=4) == EUNSUP                     # FP4_MX32 is not an entry format
    assert shared(ef=5, qf=0) == EUNSUP               # mixed rows need bf16 queries
    assert L.kv_quantize(A16, 0, A16, 5, 4, 128, None) == EUNSUP   # mixed rows are 512-d
    assert L.kv_dequantize(A16, 5, A16, 0, 4, 256, None) == EUNSUP
    a = _lib.CompressArgs(1, 4, 1024, 4, 128, 1, A16, 0, A16, A16, 0, A16, A16, 1e-6, A16, A16,
                          100, A16, A16, A16, A16, 5, 16)
    assert L.csa_compress(ctypes.byref(a), A16, 1 << 20, None) == EUNSUP  # 128-d mixed rows


def test_index_topk_noalloc_rejects_oversize_on_host():
    """The fixed-scratch index call refuses a shape whose workspace exceeds its
    32 MiB before any device call."""
    L = _lib.lib()
    B, N, Hi, k = 64, 262144, 64, 512
    assert L.csa_index_topk_workspace_size(B, 1, N, k) > 32 << 20
    r = L.csa_index_topk_noalloc(A16, _lib.BF16, A16, A16, _lib.FP8_MX32, A16, 4, B, 1, Hi, N, k,
                                 A16, None, None)
    assert r == EWS and "scratch" in _detail()


def test_block_cache_validation():
    """Block-table descriptors and slot pools are checked on the host."""
    L = _lib.lib()
    ws = 1 << 30

    def topk(be=32, maxb=100, pool=50, table=A16, kt=True, bf16=0):
        t = _lib.BlockTable(table, maxb, be, pool)
        return L.csa_index_topk_paged(A16, _lib.BF16, A16, A16, _lib.FP8_MX32,
                                      ctypes.byref(t) if kt else None, A16, 4, 2, 1, 64, 512, bf16,
                                      A16, None, A16, ws, None)

    assert topk(kt=False) == EINVAL
    assert topk(table=None) == EINVAL
    assert topk(be=16) == EINVAL                      # index keys need >= 32 per block
    assert topk(be=48) == EINVAL                      # not a power of two
    assert topk(be=2048) == EINVAL
    assert topk(maxb=0) == EINVAL
    assert topk(pool=0) == EINVAL
    assert topk(maxb=(1 << 30) // 32 + 1) == EINVAL   # logical capacity above 2^30
    assert topk(bf16=2) == EINVAL
    assert "block_entries" in (topk(be=16) and _detail())

    def attn(be=32, pool=50, slot=A16, slots=16, B=8, hca=False):
        t = _lib.BlockTable(A16, 100, be, pool)
        if hca:
            return L.hca_attn_decode_paged(A16, 1, A16, 2, slot, slots, A16, 2, ctypes.byref(t),
                                           128, A16, B, 1, 64, A16, 0.044, A16, A16, 100, A16, 1,
                                           A16, ws, None)
        return L.csa_sparse_attn_decode_paged(A16, 1, A16, 2, slot, slots, A16, 2, ctypes.byref(t),
                                              A16, 512, A16, B, 1, 64, A16, 0.044, A16, A16, 100,
                                              A16, 1, A16, ws, None)

    assert attn(slots=0) == EINVAL
    assert attn(slot=None, slots=4, B=8) == EINVAL    # no slot map needs a slot per sequence
    assert attn(be=3) == EINVAL
    assert attn(be=1024, pool=(1 << 21) + 1) == EINVAL  # pool rows above 2^31 - 1
    assert attn(hca=True, be=0) == EINVAL

    a = _lib.CompressArgs(1, 4, 1024, 4, 512, 0, A16, 0, A16, A16, 0, A16, A16, 1e-6, A16, A16,
                          100, A16, A16, A16, A16, 0, 0, A16, 8, 33, 4, None, 0)
    assert L.csa_compress(ctypes.byref(a), A16, 1 << 20, None) == EINVAL  # 33 per block
    a.block_entries = 32
    a.entries = None
    assert L.csa_compress(ctypes.byref(a), A16, 1 << 20, None) == EINVAL  # pool pointer
    a.entries = A16
    a.state_slot = A16
    a.state_slots = 0
    assert L.csa_compress(ctypes.byref(a), A16, 1 << 20, None) == EINVAL


def test_arg_structs_keep_their_tensors_alive(monkeypatch):
    """The compress-args and block-table structs hold raw addresses, so they keep
    the tensors they were built from: a temporary passed to the builder stays
    allocated until the struct goes, and its memory cannot be handed to a
    later allocation (a workspace) before the library call reads it.  (Host
    tensors stand in for device tensors: only the references are checked.)"""
    import gc
    import weakref

    import torch

    def t(*shape, dtype=torch.float32):
        return torch.zeros(shape, dtype=dtype)

    monkeypatch.setattr(_lib, "_ptr", lambda x: 0 if x is None else x.data_ptr())
    refs = []

    def tracked(x):
        refs.append(weakref.ref(x))
        return x

    a = _lib.make_compress_args(
        B=1, T=4, dim=8, ratio=4, head_dim=128, rotate=0, x=tracked(t(1, 4, 8)), x_fmt="f32",
        w_kv=tracked(t(8, 512)), w_gate=tracked(t(8, 512)), w_fmt="f32", ape=tracked(t(4, 512)),
        norm_w=tracked(t(128)), eps=1e-6, rope_cos=tracked(t(8, 32)), rope_sin=tracked(t(8, 32)),
        start_pos=tracked(t(1, dtype=torch.int32)), kv_state=tracked(t(1, 8, 256)),
        score_state=tracked(t(1, 8, 256)), entries=tracked(t(1, 1, 128)), entry_fmt="f32")
    bt = _lib.make_block_table(tracked(t(1, 4, dtype=torch.int32)), 32, 4)
    gc.collect()
    assert all(r() is not None for r in refs)
    del a, bt
    gc.collect()
    assert all(r() is None for r in refs)
