"""Top-k parity: given identical float32 scores the library's indices equal the
oracle's bit for bit (GPU)."""

import numpy as np
import pytest
import torch

from kv_cache_decode_csa_amd import _lib, synth
from oracle import topk as TK

from gpu_util import f32, i32, need_gpu, say

pytestmark = pytest.mark.gpu


def run_topk(S, n_valid, k):
    R, ld = S.shape
    ws = _lib.workspace(_lib.csa_topk_workspace_size(R, ld, k))
    out = torch.empty((R, k), dtype=torch.int32, device="cuda")
    _lib.csa_topk(f32(S), i32(n_valid), R, ld, k, out, ws)
    return out.cpu().numpy()


def check(S, n_valid, k):
    got = run_topk(S, n_valid, k)
    for r in range(S.shape[0]):
        want = TK.topk(S[r], k, n_valid[r])
        assert np.array_equal(got[r], want), (r, np.argwhere(got[r] != want)[:5].ravel())


def test_small_rows_edge_counts():
    need_gpu()
    rng = np.random.default_rng(1)
    ld = 1000
    S = np.stack([synth.random_scores(7, ld, idx=i) for i in range(8)])
    S[3, :10] = np.nan
    S[4] = np.float32(0.25)          # all equal: ties by index
    S[5, ::2] = -0.0
    S[5, 1::2] = 0.0
    n_valid = np.array([1000, 0, 5, 64, 1000, 700, 63, 65], np.int32)
    check(S, n_valid, 64)


@pytest.mark.parametrize("k", [1, 512, 2048])
def test_large_rows(k):
    need_gpu()
    ld = 262144
    S = np.stack([synth.random_scores(8, ld, idx=i) for i in range(4)])
    n_valid = np.array([ld, ld - 12345, 3 * 8192 + 7, k], np.int32)
    say(f"top-{k} over {ld}")
    check(S, n_valid, k)


def test_boundary_bin_overflow_falls_back():
    """More than the candidate capacity share the boundary bin (massive ties and
    a narrow distribution): the whole-row refinement must still be exact."""
    need_gpu()
    ld = 200000
    rng = np.random.default_rng(3)
    S = np.zeros((3, ld), np.float32)
    S[0] = np.float32(1.0)                                         # every score equal
    S[1] = (1.0 + rng.integers(0, 64, ld) * 2.0 ** -20).astype(np.float32)  # one 12-bit bin
    S[2] = (1.0 + rng.integers(0, 3, ld) * 2.0 ** -23).astype(np.float32)
    S[2, 12345] = 2.0
    check(S, np.array([ld, ld, ld - 1], np.int32), 512)


def test_boundary_bin_refinement_path():
    """Between 512 and the candidate capacity share the boundary bin: the
    two-digit refinement with index ties at the threshold decides; rows with a
    small boundary bin and ties inside it take the sort-only path."""
    need_gpu()
    ld = 6000
    rng = np.random.default_rng(4)
    S = np.zeros((4, ld), np.float32)
    S[0] = (1.0 + rng.integers(0, 4096, ld) * 2.0 ** -20).astype(np.float32)  # one 12-bit bin
    S[1] = (1.0 + rng.integers(0, 40, ld) * 2.0 ** -20).astype(np.float32)    # heavy ties
    S[2] = rng.standard_normal(ld).astype(np.float32)
    S[2, rng.choice(ld, 300, replace=False)] = np.float32(2.5)                 # ties in the tail
    S[3] = S[0]
    S[3, :700] = np.float32(3.0)                                               # hi list > 512
    check(S, np.array([ld, ld - 1, ld, ld], np.int32), 512)
    check(S, np.array([ld, 5000, 4000, ld], np.int32), 1024)


def test_boundary_bin_two_halves():
    """513..1024 entries share the boundary bin and at most 512 of them are
    taken: the two halves of the boundary list are sorted and merged."""
    need_gpu()
    ld = 5000
    rng = np.random.default_rng(6)
    S = (0.1 * rng.random((5, ld))).astype(np.float32)                 # far below the bin
    def fill(r, n_eq, n_above, distinct):
        pos = rng.choice(ld, n_eq + n_above, replace=False)
        S[r, pos[:n_eq]] = (1.0 + rng.integers(0, distinct, n_eq) * 2.0 ** -20).astype(np.float32)
        S[r, pos[n_eq:]] = (4.0 + rng.random(n_above)).astype(np.float32)
    fill(0, 800, 100, 4096)     # need 412 of 800
    fill(1, 1024, 0, 4096)      # need 512 of 1024
    fill(2, 513, 300, 8)        # heavy ties at the threshold: by index
    fill(3, 700, 0, 4096)       # k 1024 below: need > 512 takes the refinement
    fill(4, 1000, 511, 64)      # need 1
    check(S, np.full(5, ld, np.int32), 512)
    check(S, np.array([ld, ld, ld, ld, 4000], np.int32), 1024)


def test_run_to_run_bitwise():
    need_gpu()
    ld = 100000
    S = np.stack([synth.random_scores(9, ld, idx=i) for i in range(6)])
    nv = np.full(6, ld, np.int32)
    a = run_topk(S, nv, 512)
    b = run_topk(S, nv, 512)
    assert np.array_equal(a, b)
