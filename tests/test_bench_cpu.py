"""bench.py's host-side arithmetic and contract (CPU only): the algorithmic
bytes behind the roofline object reproduce the per-token figures of the
measurement plan (index keys, gathered rows, window, q + out, q_idx + w per
sequence), the prefill FLOP count is the sum over queries of the visible
keys, and a multi-GPU run is refused with a message."""

import os
import subprocess
import sys

import bench
from kv_cache_decode_csa_amd import synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def per_seq_read_bytes(w):
    ab = bench.algorithmic_bytes(w)
    if w.ratio == 4:
        # attention includes the sink once per call; index includes the ids written
        att = ab["csa_sparse_attn_decode"] - w.H * 4
        idx = ab["csa_index_topk"]
        return idx / w.B, att / w.B
    return None, (ab["hca_attn_decode"] - w.H * 4) / w.B


def test_fp8_1m_bytes_per_token():
    w = synth.WORKLOADS[5]
    idx, att = per_seq_read_bytes(w)
    # index keys 262,144 x 132 B; q_idx 64 x 128 x 2 B; w 64 x 4 B; ids 512 x 4 B
    assert idx == 262144 * 132 + 64 * 128 * 2 + 64 * 4 + 512 * 4
    # gathered 512 x 528 B (+ ids), window 128 x 528 B, q + out 2 x 64 x 512 x 2 B
    assert att == 512 * 528 + 512 * 4 + 128 * 528 + 2 * 64 * 512 * 2
    # the plan's total per token: 35,088,640 B (ids counted once there)
    assert idx + att - 2 * 512 * 4 == 35088640


def test_mxfp4_and_64k_and_hca_bytes_per_token():
    w = synth.mxfp4_variant(synth.WORKLOADS[5])
    idx, att = per_seq_read_bytes(w)
    # gathered rows 512 x 288 B; the window stays FP8-528 in this variant, so the
    # total is the FP8 one less 512 x (528 - 288) B.  (The plan prints 34,935,040,
    # which also counts the window at 288 B rows, against its own FP8-window rule.)
    assert idx + att - 2 * 512 * 4 == 35088640 - 512 * (528 - 288) == 34965760
    w = synth.WORKLOADS[2]
    idx, att = per_seq_read_bytes(w)
    # keys 16,384 x 256; gathered 512 x 1,024; window 128 x 1,024; q + out; q_idx + w (32 heads)
    assert idx + att - 2 * 512 * 4 == 4194304 + 524288 + 131072 + 131072 + 8320
    w = synth.WORKLOADS[3]
    _, att = per_seq_read_bytes(w)
    assert att == 8388608 + 131072 + 131072                # entries, window, q + out


def test_prefill_flops():
    w = synth.WORKLOADS[4]
    fl = bench.prefill_flops(w)
    P, T, N0, N = synth.prefill_shape(w)
    # query i sees floor((P + i + 1) / 4) entries: 65,536 + floor((i + 1) / 4)
    vis = T * N0 + sum((i + 1) // 4 for i in range(T))
    assert fl["csa_index_topk"] == 2.0 * vis * 64 * 128
    assert abs(fl["csa_index_topk"] / 1e12 - 37.38) < 0.01
    assert fl["csa_sparse_attn_decode"] == 2.0 * 2 * T * 64 * 512 * 640
    assert fl["csa_compress"] == 2.0 * T * 4096 * (2 * 512 * 2 + 2 * 128 * 2)


def test_csa2_and_layer_bytes():
    """CSA2 at m = 1: 262,144 FP4 index keys of 68 B per sequence (and 64 FP4
    query rows of 68 B), MXFP4 rows
    of 288 B read once for the group of 6 layers, each with its own window,
    q and output.
    The layer variant: every weight once (bf16) plus the token's inputs and
    outputs."""
    w = synth.WORKLOADS[6]
    ab = bench.algorithmic_bytes(w)
    assert ab["csa_index_topk"] == 8 * (262144 * 68 + 64 * 68 + 64 * 4 + 512 * 4)
    assert ab["csa_sparse_attn_group"] == (8 * (512 * 288 + 512 * 4)
                                           + 6 * 8 * (128 * 528 + 2 * 64 * 512 * 2) + 6 * 64 * 4)
    assert "csa_sparse_attn_decode" not in ab
    wl = synth.layer_variant(synth.WORKLOADS[5])
    ab = bench.algorithmic_bytes(wl)
    weights = 4096 * 1024 + 1024 * 64 * 512 + 4096 * 512 + 1024 * 64 * 128 + 4096 * 64
    assert ab["csa_layer_input"] == (2 * weights + 4 * (1024 + 512) + 8 * 4096 * 2
                                     + 8 * (64 * 512 * 2 + 64 * 128 * 2 + 64 * 4) + 8 * 528)
    assert ab["csa_layer_output"] == 2 * (1024 * 64 * 512 + 4096 * 8 * 1024) + 8 * 64 * 512 * 2 \
        + 8 * 4096 * 2


def test_batch_variant_scales_bytes_and_keeps_sequences():
    """The batch-128 variant of the 64K workload: the same per-sequence bytes,
    128 sequences, and the base workload's seeded data for its first ones."""
    base = synth.WORKLOADS[2]
    big = synth.batch_variant(base, 128)
    assert big.B == 128 and big.name == "csa_64k_bf16_b128" and big.seed == base.seed
    assert per_seq_read_bytes(big) == per_seq_read_bytes(base)
    assert "csa_64k_bf16_b128" in bench.WORKLOADS and big.name in bench.METRICS
    a = synth.normal_batched(base.seed, 3, base.B, (2, 4))
    b = synth.normal_batched(big.seed, 3, big.B, (2, 4))
    assert (a == b[:base.B]).all()


def test_multi_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_cpu_baseline_runs_whole_batch_and_single_thread():
    """The oracle baseline times the whole batch by default, including the
    compressors, and reports the BLAS thread count and a single-thread time
    for one sequence (tiny fp32 workload, CPU)."""
    import bench
    w = synth.WORKLOADS[1]
    r = bench.cpu_baseline(w, min_seconds=0.01)
    assert r["kind"] == "oracle" and r["value"] > 0
    assert r["blas_threads"] >= 1 and r["cores"] == r["blas_threads"]
    assert r["single_thread_seconds_one_sequence"] > 0
    assert "compressors" in r["sample"] and "the whole batch" in r["sample"]
