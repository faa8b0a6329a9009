"""csa_index_topk_noalloc (GPU): the index + top-k call with the library's
fixed scratch instead of a caller workspace gives exactly csa_index_topk's
results, on two calls in a row (the second smaller, over the first call's
leftover scratch contents), with and without caller score buffers; a call
whose workspace would exceed the fixed scratch is rejected before anything
is enqueued."""

import numpy as np
import pytest
import torch

from kv_cache_decode_csa_amd import _lib

from gpu_util import need_gpu, say

pytestmark = pytest.mark.gpu


def _keys(B, N, fmt, seed):
    g = torch.Generator(device="cuda").manual_seed(seed)
    rows = B * N
    if fmt == "bf16":
        return torch.randn((B, N, 128), generator=g, device="cuda").to(torch.bfloat16)
    rb = _lib.kv_row_bytes(fmt, 128)
    out = torch.empty((B, N, rb), dtype=torch.uint8, device="cuda")
    step = 1 << 18
    flat = out.reshape(rows, rb)
    for lo in range(0, rows, step):
        hi = min(rows, lo + step)
        src = torch.randn((hi - lo, 128), generator=g, device="cuda")
        _lib.kv_quantize(src, "f32", flat[lo:hi], fmt, hi - lo, 128)
    return out


def _case(B, N, Hi, k, fmt, pos, seed):
    g = torch.Generator(device="cuda").manual_seed(seed + 1)
    qi = torch.randn((B, 1, Hi, 128), generator=g, device="cuda").to(torch.bfloat16)
    wi = torch.randn((B, 1, Hi), generator=g, device="cuda") * (128 * Hi) ** -0.5
    keys = _keys(B, N, fmt, seed)
    p = torch.tensor(pos, dtype=torch.int32, device="cuda").reshape(B, 1)
    return qi, wi, keys, p


def _compare(B, N, Hi, k, fmt, pos, seed, with_scores):
    qi, wi, keys, p = _case(B, N, Hi, k, fmt, pos, seed)
    ws = _lib.workspace(_lib.csa_index_topk_workspace_size(B, 1, N, k))
    ids_ref = torch.full((B, 1, k), -7, dtype=torch.int32, device="cuda")
    sc_ref = torch.zeros((B, 1, N), dtype=torch.float32, device="cuda")
    _lib.csa_index_topk(qi, "bf16", wi, keys, fmt, p, 4, B, 1, Hi, N, k, ids_ref, sc_ref, ws)
    ids = torch.full((B, 1, k), -7, dtype=torch.int32, device="cuda")
    sc = torch.zeros((B, 1, N), dtype=torch.float32, device="cuda") if with_scores else None
    say(f"noalloc B={B} N={N} Hi={Hi} k={k} {fmt} scores={'caller' if with_scores else 'scratch'}")
    _lib.csa_index_topk_noalloc(qi, "bf16", wi, keys, fmt, p, 4, B, 1, Hi, N, k, ids, sc)
    torch.cuda.synchronize()
    assert torch.equal(ids, ids_ref)
    if with_scores:
        nv = np.minimum((np.array(pos) + 1) // 4, N)
        a, b = sc.cpu().numpy()[:, 0], sc_ref.cpu().numpy()[:, 0]
        for r in range(B):
            assert np.array_equal(a[r, :nv[r]].view(np.uint32), b[r, :nv[r]].view(np.uint32))
    got = ids.cpu().numpy()[:, 0]
    for r in range(B):
        ke = min(k, (pos[r] + 1) // 4, N)
        assert np.all(got[r, ke:] == -1) and len(set(got[r, :ke].tolist())) == ke


def test_noalloc_matches_workspace_call_twice():
    need_gpu()
    # first call: the 1M-context shape (FP8 keys, 262,144 per sequence),
    # scores left in the scratch
    t = 4 * 262144 - 1
    _compare(8, 262144, 64, 512, "fp8_mx32", [t] * 8, 11, with_scores=False)
    # second call, smaller, over the first call's scratch contents: bf16 keys,
    # ragged visibility (one row sees fewer entries than k, one sees none)
    _compare(3, 40000, 32, 300, "bf16", [4 * 40000 - 1, 1001, 2], 12, with_scores=True)


def test_noalloc_rejects_oversize():
    need_gpu()
    B, N, Hi, k = 64, 262144, 64, 512
    need = _lib.csa_index_topk_workspace_size(B, 1, N, k)
    assert need > 32 << 20
    qi = torch.zeros((1, 1, Hi, 128), dtype=torch.bfloat16, device="cuda")
    wi = torch.zeros((1, 1, Hi), dtype=torch.float32, device="cuda")
    keys = torch.zeros((1, 1, 132), dtype=torch.uint8, device="cuda")
    p = torch.zeros((1, 1), dtype=torch.int32, device="cuda")
    ids = torch.full((1, 1, k), -7, dtype=torch.int32, device="cuda")
    with pytest.raises(_lib.CsaError) as ei:
        _lib.csa_index_topk_noalloc(qi, "bf16", wi, keys, "fp8_mx32", p, 4, B, 1, Hi, N, k, ids,
                                    None)
    assert ei.value.status == 3 and "scratch" in ei.value.detail
    torch.cuda.synchronize()
    assert bool((ids == -7).all())
