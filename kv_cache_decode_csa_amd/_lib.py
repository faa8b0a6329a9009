"""ctypes binding of libcsa.so: argument marshalling only.

Every function here has the name of the C entry point it calls and takes
torch tensors that already live on the GPU.  It passes their data pointers and
torch's current HIP stream, checks the returned status and raises
``CsaError`` with the library's detail text.  All computation happens in the
library's HIP kernels; there is no fallback.  torch is imported before the
library is loaded so that both share one HIP runtime.
"""

import ctypes
import os

import torch

F32, BF16, FP8_MX32, FP4_E4M3_16, FP4_MX32, MIX576 = 0, 1, 2, 3, 4, 5
WIN_RING128, WIN_LINEAR = 0, 1
FMT_NAMES = {"f32": F32, "bf16": BF16, "fp8_mx32": FP8_MX32, "fp4_e4m3_16": FP4_E4M3_16,
             "fp4_mx32": FP4_MX32, "mix576": MIX576}

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libcsa.so")

_lib = None


class CsaError(RuntimeError):
    def __init__(self, status, detail, fn):
        super().__init__(f"{fn}: status {status}: {detail}")
        self.status = status
        self.detail = detail


class CompressArgs(ctypes.Structure):
    _fields_ = [
        ("B", ctypes.c_int), ("T", ctypes.c_int), ("dim", ctypes.c_int), ("ratio", ctypes.c_int),
        ("head_dim", ctypes.c_int), ("rotate", ctypes.c_int),
        ("x", ctypes.c_void_p), ("x_fmt", ctypes.c_int),
        ("w_kv", ctypes.c_void_p), ("w_gate", ctypes.c_void_p), ("w_fmt", ctypes.c_int),
        ("ape", ctypes.c_void_p), ("norm_w", ctypes.c_void_p), ("eps", ctypes.c_float),
        ("rope_cos", ctypes.c_void_p), ("rope_sin", ctypes.c_void_p), ("rope_rows", ctypes.c_int64),
        ("start_pos", ctypes.c_void_p), ("kv_state", ctypes.c_void_p),
        ("score_state", ctypes.c_void_p), ("entries", ctypes.c_void_p),
        ("entry_fmt", ctypes.c_int), ("entries_cap", ctypes.c_int64),
        ("block_table", ctypes.c_void_p), ("max_blocks", ctypes.c_int64),
        ("block_entries", ctypes.c_int), ("pool_blocks", ctypes.c_int64),
        ("state_slot", ctypes.c_void_p), ("state_slots", ctypes.c_int64),
    ]


class BlockTable(ctypes.Structure):
    _fields_ = [
        ("table", ctypes.c_void_p), ("max_blocks", ctypes.c_int64),
        ("block_entries", ctypes.c_int), ("pool_blocks", ctypes.c_int64),
    ]


class LayerWeights(ctypes.Structure):
    _fields_ = [
        ("dim", ctypes.c_int), ("q_rank", ctypes.c_int), ("H", ctypes.c_int), ("Hi", ctypes.c_int),
        ("groups", ctypes.c_int), ("o_rank", ctypes.c_int),
        ("wq_a", ctypes.c_void_p), ("q_norm", ctypes.c_void_p), ("wq_b", ctypes.c_void_p),
        ("wkv", ctypes.c_void_p), ("kv_norm", ctypes.c_void_p), ("wq_b_idx", ctypes.c_void_p),
        ("w_proj", ctypes.c_void_p), ("wo_a", ctypes.c_void_p), ("wo_b", ctypes.c_void_p),
        ("eps", ctypes.c_float),
    ]


_VP, _I, _I64, _SZ, _F, _D = (ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_size_t,
                              ctypes.c_float, ctypes.c_double)

_SIGS = {
    "csa_strerror": (ctypes.c_char_p, [_I]),
    "csa_last_error_detail": (ctypes.c_char_p, []),
    "kv_row_bytes": (_SZ, [_I, _I]),
    "csa_rope_table": (_I, [_D, _D, _I64, _D, _D, _I64, _VP, _VP, _VP]),
    "kv_quantize": (_I, [_VP, _I, _VP, _I, _I64, _I, _VP]),
    "kv_dequantize": (_I, [_VP, _I, _VP, _I, _I64, _I, _VP]),
    "csa_compress_workspace_size": (_SZ, [ctypes.POINTER(CompressArgs)]),
    "csa_compress": (_I, [ctypes.POINTER(CompressArgs), _VP, _SZ, _VP]),
    "csa_compress_many_workspace_size": (_SZ, [ctypes.POINTER(CompressArgs), _I]),
    "csa_compress_many": (_I, [ctypes.POINTER(CompressArgs), _I, _VP, _SZ, _VP]),
    "csa_index_topk_workspace_size": (_SZ, [_I, _I, _I64, _I]),
    "csa_index_topk": (_I, [_VP, _I, _VP, _VP, _I, _VP, _I, _I, _I, _I, _I64, _I, _VP, _VP, _VP,
                            _SZ, _VP]),
    "csa_index_topk_bf16": (_I, [_VP, _I, _VP, _VP, _I, _VP, _I, _I, _I, _I, _I64, _I, _VP, _VP,
                                 _VP, _SZ, _VP]),
    "csa_index_topk_noalloc": (_I, [_VP, _I, _VP, _VP, _I, _VP, _I, _I, _I, _I, _I64, _I, _VP,
                                    _VP, _VP]),
    "csa_topk_workspace_size": (_SZ, [_I64, _I64, _I]),
    "csa_topk": (_I, [_VP, _VP, _I64, _I64, _I, _VP, _VP, _SZ, _VP]),
    "csa_sparse_attn_workspace_size": (_SZ, [_I, _I, _I, _I]),
    "csa_sparse_attn_decode": (_I, [_VP, _I, _VP, _I, _I, _VP, _I64, _VP, _I, _I64, _VP, _I, _VP,
                                    _I, _I, _I, _VP, _F, _VP, _VP, _I64, _VP, _I, _VP, _SZ, _VP]),
    "csa_sparse_attn_decode_shared": (_I, [_VP, _I, _VP, _I, _VP, _I, _I64, _VP, _I, _VP, _I, _I,
                                           _I, _I, _VP, _F, _VP, _VP, _I64, _VP, _I, _VP, _SZ,
                                           _VP]),
    "hca_attn_workspace_size": (_SZ, [_I, _I, _I, _I64]),
    "hca_attn_decode": (_I, [_VP, _I, _VP, _I, _I, _VP, _I64, _VP, _I, _I64, _I, _VP, _I, _I, _I,
                             _VP, _F, _VP, _VP, _I64, _VP, _I, _VP, _SZ, _VP]),
    "csa_index_topk_paged": (_I, [_VP, _I, _VP, _VP, _I, ctypes.POINTER(BlockTable), _VP, _I, _I,
                                  _I, _I, _I, _I, _VP, _VP, _VP, _SZ, _VP]),
    "csa_sparse_attn_decode_paged": (_I, [_VP, _I, _VP, _I, _VP, _I64, _VP, _I,
                                          ctypes.POINTER(BlockTable), _VP, _I, _VP, _I, _I, _I,
                                          _VP, _F, _VP, _VP, _I64, _VP, _I, _VP, _SZ, _VP]),
    "hca_attn_decode_paged": (_I, [_VP, _I, _VP, _I, _VP, _I64, _VP, _I,
                                   ctypes.POINTER(BlockTable), _I, _VP, _I, _I, _I, _VP, _F, _VP,
                                   _VP, _I64, _VP, _I, _VP, _SZ, _VP]),
    "csa_layer_input_workspace_size": (_SZ, [ctypes.POINTER(LayerWeights), _I]),
    "csa_layer_input": (_I, [ctypes.POINTER(LayerWeights), _VP, _VP, _I, _I, _VP, _VP, _I64, _VP,
                             _VP, _VP, _VP, _I, _VP, _SZ, _VP]),
    "csa_layer_output_workspace_size": (_SZ, [ctypes.POINTER(LayerWeights), _I]),
    "csa_layer_output": (_I, [ctypes.POINTER(LayerWeights), _VP, _I, _VP, _I, _VP, _SZ, _VP]),
}

EXPORTS = tuple(_SIGS)


def lib():
    """Load libcsa.so once; raise if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"{LIB_PATH} is missing: build it with `python -m kv_cache_decode_csa_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIGS.items():
            fn = getattr(L, name)
            fn.restype = res
            fn.argtypes = args
        _lib = L
    return _lib


def _ptr(t):
    if t is None:
        return None
    if not isinstance(t, torch.Tensor):
        raise TypeError("expected a torch.Tensor")
    if not t.is_cuda:
        raise ValueError("tensor must live on the GPU")
    if not t.is_contiguous():
        raise ValueError("tensor must be contiguous")
    return t.data_ptr()


def _stream(stream):
    s = torch.cuda.current_stream() if stream is None else stream
    return s.cuda_stream


def _check(status, fn):
    if status != 0:
        L = lib()
        raise CsaError(status, L.csa_last_error_detail().decode(), fn)


def _fmt(f):
    return FMT_NAMES[f] if isinstance(f, str) else int(f)


def workspace(nbytes, device=None):
    """Device scratch buffer of at least nbytes (caller-owned, 256-B aligned)."""
    return torch.empty(max(int(nbytes), 1), dtype=torch.uint8, device=device or "cuda")


# ----------------------------------------------------------------------------- entry points

def kv_row_bytes(fmt, dim):
    return int(lib().kv_row_bytes(_fmt(fmt), int(dim)))


def csa_rope_table(theta, yarn_factor, yarn_orig_len, beta_fast, beta_slow, rows, cos_out,
                   sin_out, stream=None):
    _check(lib().csa_rope_table(float(theta), float(yarn_factor), int(yarn_orig_len),
                                float(beta_fast), float(beta_slow), int(rows), _ptr(cos_out),
                                _ptr(sin_out), _stream(stream)), "csa_rope_table")


def kv_quantize(src, src_fmt, dst, dst_fmt, rows, dim, stream=None):
    _check(lib().kv_quantize(_ptr(src), _fmt(src_fmt), _ptr(dst), _fmt(dst_fmt), int(rows),
                             int(dim), _stream(stream)), "kv_quantize")


def kv_dequantize(src, src_fmt, dst, dst_fmt, rows, dim, stream=None):
    _check(lib().kv_dequantize(_ptr(src), _fmt(src_fmt), _ptr(dst), _fmt(dst_fmt), int(rows),
                               int(dim), _stream(stream)), "kv_dequantize")


def make_compress_args(*, B, T, dim, ratio, head_dim, rotate, x, x_fmt, w_kv, w_gate, w_fmt,
                       ape, norm_w, eps, rope_cos, rope_sin, start_pos, kv_state, score_state,
                       entries, entry_fmt, entries_cap=0, block_table=None, block_entries=0,
                       pool_blocks=0, state_slot=None):
    """block_table ([B, max_blocks] int32) makes `entries` a pool of
    pool_blocks blocks of block_entries rows; state_slot ([B] int32) makes
    kv_state / score_state pools of slots (their first dimension).  The struct
    holds only addresses, so it keeps the tensors alive: a temporary passed
    here would otherwise be freed, and its memory handed to the next
    allocation (a workspace, say), before the call that reads it."""
    a = CompressArgs(int(B), int(T), int(dim), int(ratio), int(head_dim), int(rotate),
                        _ptr(x), _fmt(x_fmt), _ptr(w_kv), _ptr(w_gate), _fmt(w_fmt), _ptr(ape),
                        _ptr(norm_w), float(eps), _ptr(rope_cos), _ptr(rope_sin),
                        int(rope_cos.shape[0]), _ptr(start_pos), _ptr(kv_state),
                        _ptr(score_state), _ptr(entries), _fmt(entry_fmt), int(entries_cap),
                        _ptr(block_table),
                        int(block_table.shape[1]) if block_table is not None else 0,
                        int(block_entries), int(pool_blocks), _ptr(state_slot),
                        int(kv_state.shape[0]) if state_slot is not None else 0)
    a._tensors = (x, w_kv, w_gate, ape, norm_w, rope_cos, rope_sin, start_pos, kv_state,
                  score_state, entries, block_table, state_slot)
    return a


def make_block_table(table, block_entries, pool_blocks):
    """csa_block_table over a [B, max_blocks] int32 device tensor (the struct
    keeps it alive)."""
    bt = BlockTable(_ptr(table), int(table.shape[1]), int(block_entries), int(pool_blocks))
    bt._tensors = (table,)
    return bt


def csa_compress_workspace_size(args):
    return int(lib().csa_compress_workspace_size(ctypes.byref(args)))


def _args_array(args_list):
    arr = (CompressArgs * len(args_list))()
    for i, a in enumerate(args_list):
        arr[i] = a
    return arr


def csa_compress_many_workspace_size(args_list):
    arr = _args_array(args_list)
    return int(lib().csa_compress_many_workspace_size(arr, len(args_list)))


def csa_compress_many(args_list, ws, stream=None):
    arr = _args_array(args_list)
    _check(lib().csa_compress_many(arr, len(args_list), _ptr(ws),
                                   ws.numel() if ws is not None else 0, _stream(stream)),
           "csa_compress_many")


def csa_compress(args, ws, stream=None):
    _check(lib().csa_compress(ctypes.byref(args), _ptr(ws), ws.numel() if ws is not None else 0,
                              _stream(stream)), "csa_compress")


def csa_index_topk_workspace_size(B, Q, Nmax, topk):
    return int(lib().csa_index_topk_workspace_size(int(B), int(Q), int(Nmax), int(topk)))


def csa_index_topk(q_idx, q_fmt, w_idx, k_idx, k_fmt, pos, ratio, B, Q, Hi, Nmax, topk, out_idx,
                   out_scores, ws, stream=None):
    _check(lib().csa_index_topk(_ptr(q_idx), _fmt(q_fmt), _ptr(w_idx), _ptr(k_idx), _fmt(k_fmt),
                                _ptr(pos), int(ratio), int(B), int(Q), int(Hi), int(Nmax),
                                int(topk), _ptr(out_idx), _ptr(out_scores), _ptr(ws),
                                ws.numel() if ws is not None else 0, _stream(stream)),
           "csa_index_topk")


def csa_index_topk_bf16(q_idx, q_fmt, w_idx, k_idx, k_fmt, pos, ratio, B, Q, Hi, Nmax, topk,
                        out_idx, out_scores, ws, stream=None):
    _check(lib().csa_index_topk_bf16(_ptr(q_idx), _fmt(q_fmt), _ptr(w_idx), _ptr(k_idx),
                                     _fmt(k_fmt), _ptr(pos), int(ratio), int(B), int(Q), int(Hi),
                                     int(Nmax), int(topk), _ptr(out_idx), _ptr(out_scores),
                                     _ptr(ws), ws.numel() if ws is not None else 0,
                                     _stream(stream)), "csa_index_topk_bf16")


def csa_index_topk_noalloc(q_idx, q_fmt, w_idx, k_idx, k_fmt, pos, ratio, B, Q, Hi, Nmax, topk,
                           out_idx, out_scores, stream=None):
    _check(lib().csa_index_topk_noalloc(_ptr(q_idx), _fmt(q_fmt), _ptr(w_idx), _ptr(k_idx),
                                        _fmt(k_fmt), _ptr(pos), int(ratio), int(B), int(Q),
                                        int(Hi), int(Nmax), int(topk), _ptr(out_idx),
                                        _ptr(out_scores), _stream(stream)),
           "csa_index_topk_noalloc")


def csa_topk_workspace_size(R, ld, topk):
    return int(lib().csa_topk_workspace_size(int(R), int(ld), int(topk)))


def csa_topk(scores, n_valid, R, ld, topk, out_idx, ws, stream=None):
    _check(lib().csa_topk(_ptr(scores), _ptr(n_valid), int(R), int(ld), int(topk),
                          _ptr(out_idx), _ptr(ws), ws.numel() if ws is not None else 0,
                          _stream(stream)), "csa_topk")


def csa_sparse_attn_workspace_size(B, Q, H, topk):
    return int(lib().csa_sparse_attn_workspace_size(int(B), int(Q), int(H), int(topk)))


def csa_sparse_attn_decode(q, q_fmt, win, win_fmt, win_mode, win_base, win_rows, entries,
                           ent_fmt, Nmax, topk_idx, topk, pos, B, Q, H, sink, scale, rope_cos,
                           rope_sin, out, out_fmt, ws, stream=None):
    _check(lib().csa_sparse_attn_decode(
        _ptr(q), _fmt(q_fmt), _ptr(win), _fmt(win_fmt), int(win_mode), _ptr(win_base),
        int(win_rows), _ptr(entries), _fmt(ent_fmt), int(Nmax), _ptr(topk_idx), int(topk),
        _ptr(pos), int(B), int(Q), int(H), _ptr(sink), float(scale), _ptr(rope_cos),
        _ptr(rope_sin), int(rope_cos.shape[0]), _ptr(out), _fmt(out_fmt), _ptr(ws),
        ws.numel() if ws is not None else 0, _stream(stream)), "csa_sparse_attn_decode")


def csa_sparse_attn_decode_shared(q, q_fmt, win, win_fmt, entries, ent_fmt, Nmax, topk_idx, topk,
                                  pos, B, Q, H, ent_seqs, sink, scale, rope_cos, rope_sin, out,
                                  out_fmt, ws, stream=None):
    _check(lib().csa_sparse_attn_decode_shared(
        _ptr(q), _fmt(q_fmt), _ptr(win), _fmt(win_fmt), _ptr(entries), _fmt(ent_fmt), int(Nmax),
        _ptr(topk_idx), int(topk), _ptr(pos), int(B), int(Q), int(H), int(ent_seqs), _ptr(sink),
        float(scale), _ptr(rope_cos), _ptr(rope_sin), int(rope_cos.shape[0]), _ptr(out),
        _fmt(out_fmt), _ptr(ws), ws.numel() if ws is not None else 0, _stream(stream)),
        "csa_sparse_attn_decode_shared")


def csa_index_topk_paged(q_idx, q_fmt, w_idx, k_pool, k_fmt, kt, pos, ratio, B, Q, Hi, topk,
                         bf16_scores, out_idx, out_scores, ws, stream=None):
    _check(lib().csa_index_topk_paged(_ptr(q_idx), _fmt(q_fmt), _ptr(w_idx), _ptr(k_pool),
                                      _fmt(k_fmt), ctypes.byref(kt), _ptr(pos), int(ratio),
                                      int(B), int(Q), int(Hi), int(topk), int(bf16_scores),
                                      _ptr(out_idx), _ptr(out_scores), _ptr(ws),
                                      ws.numel() if ws is not None else 0, _stream(stream)),
           "csa_index_topk_paged")


def csa_sparse_attn_decode_paged(q, q_fmt, win_pool, win_fmt, win_slot, win_slots, ent_pool,
                                 ent_fmt, et, topk_idx, topk, pos, B, Q, H, sink, scale, rope_cos,
                                 rope_sin, out, out_fmt, ws, stream=None):
    _check(lib().csa_sparse_attn_decode_paged(
        _ptr(q), _fmt(q_fmt), _ptr(win_pool), _fmt(win_fmt), _ptr(win_slot), int(win_slots),
        _ptr(ent_pool), _fmt(ent_fmt), ctypes.byref(et), _ptr(topk_idx), int(topk), _ptr(pos),
        int(B), int(Q), int(H), _ptr(sink), float(scale), _ptr(rope_cos), _ptr(rope_sin),
        int(rope_cos.shape[0]), _ptr(out), _fmt(out_fmt), _ptr(ws),
        ws.numel() if ws is not None else 0, _stream(stream)), "csa_sparse_attn_decode_paged")


def hca_attn_decode_paged(q, q_fmt, win_pool, win_fmt, win_slot, win_slots, ent_pool, ent_fmt, et,
                          ratio, pos, B, Q, H, sink, scale, rope_cos, rope_sin, out, out_fmt, ws,
                          stream=None):
    _check(lib().hca_attn_decode_paged(
        _ptr(q), _fmt(q_fmt), _ptr(win_pool), _fmt(win_fmt), _ptr(win_slot), int(win_slots),
        _ptr(ent_pool), _fmt(ent_fmt), ctypes.byref(et), int(ratio), _ptr(pos), int(B), int(Q),
        int(H), _ptr(sink), float(scale), _ptr(rope_cos), _ptr(rope_sin), int(rope_cos.shape[0]),
        _ptr(out), _fmt(out_fmt), _ptr(ws), ws.numel() if ws is not None else 0, _stream(stream)),
        "hca_attn_decode_paged")


def hca_attn_workspace_size(B, Q, H, Nmax):
    return int(lib().hca_attn_workspace_size(int(B), int(Q), int(H), int(Nmax)))


def hca_attn_decode(q, q_fmt, win, win_fmt, win_mode, win_base, win_rows, entries, ent_fmt, Nmax,
                    ratio, pos, B, Q, H, sink, scale, rope_cos, rope_sin, out, out_fmt, ws,
                    stream=None):
    _check(lib().hca_attn_decode(
        _ptr(q), _fmt(q_fmt), _ptr(win), _fmt(win_fmt), int(win_mode), _ptr(win_base),
        int(win_rows), _ptr(entries), _fmt(ent_fmt), int(Nmax), int(ratio), _ptr(pos), int(B),
        int(Q), int(H), _ptr(sink), float(scale), _ptr(rope_cos), _ptr(rope_sin),
        int(rope_cos.shape[0]), _ptr(out), _fmt(out_fmt), _ptr(ws),
        ws.numel() if ws is not None else 0, _stream(stream)), "hca_attn_decode")


def make_layer_weights(*, dim, q_rank, H, Hi, groups, o_rank, wq_a=None, q_norm=None, wq_b=None,
                       wkv=None, kv_norm=None, wq_b_idx=None, w_proj=None, wo_a=None, wo_b=None,
                       eps=1e-6):
    """The C struct of device pointers; it keeps the tensors alive, since the
    struct holds only their addresses."""
    t = (wq_a, q_norm, wq_b, wkv, kv_norm, wq_b_idx, w_proj, wo_a, wo_b)
    lw = LayerWeights(int(dim), int(q_rank), int(H), int(Hi), int(groups), int(o_rank),
                      *[_ptr(x) for x in t], float(eps))
    lw._tensors = t
    return lw


def csa_layer_input_workspace_size(w, M):
    return int(lib().csa_layer_input_workspace_size(ctypes.byref(w), int(M)))


def csa_layer_input(w, x, pos, B, T, rope_cos, rope_sin, q, q_idx, w_idx, win, win_fmt, ws,
                    stream=None):
    _check(lib().csa_layer_input(ctypes.byref(w), _ptr(x), _ptr(pos), int(B), int(T),
                                 _ptr(rope_cos), _ptr(rope_sin), int(rope_cos.shape[0]), _ptr(q),
                                 _ptr(q_idx), _ptr(w_idx), _ptr(win), _fmt(win_fmt), _ptr(ws),
                                 ws.numel() if ws is not None else 0, _stream(stream)),
           "csa_layer_input")


def csa_layer_output_workspace_size(w, M):
    return int(lib().csa_layer_output_workspace_size(ctypes.byref(w), int(M)))


def csa_layer_output(w, o, M, y, y_fmt, ws, stream=None):
    _check(lib().csa_layer_output(ctypes.byref(w), _ptr(o), int(M), _ptr(y), _fmt(y_fmt), _ptr(ws),
                                  ws.numel() if ws is not None else 0, _stream(stream)),
           "csa_layer_output")
