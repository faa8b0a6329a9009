"""GPU parity of the layer's steps around the decode path (csa_layer_input,
csa_layer_output) against the oracle, at small shapes with ragged tiles and at
the V4-Flash shapes the layer bench runs (dim 4096, q_rank 1024, 64 heads,
64 index heads, 8 output groups of rank 1024, 8 sequences)."""

import numpy as np
import pytest
import torch

from gpu_util import bf16, close_bf16, f32, i32, need_gpu, rope_tables, say, step_bound, to_np
from kv_cache_decode_csa_amd import _lib, synth
from oracle import codec as OC
from oracle import layer as OL
from oracle import rope as OR

pytestmark = pytest.mark.gpu

OMEGA = OR.frequencies(160000.0, OR.V4_YARN)
U = 2.0 ** -24


def _upload_weights(wn):
    dev = {}
    for k, v in wn.items():
        dev[k] = f32(v) if k in ("q_norm", "kv_norm") else bf16(v)
    return dev


def _make(dev, dim, q_rank, H, Hi, groups, o_rank):
    return _lib.make_layer_weights(dim=dim, q_rank=q_rank, H=H, Hi=Hi, groups=groups,
                                   o_rank=o_rank, **dev)


def _check_f32_bound(got, ref, terms_abs, name):
    """|got - ref| <= 256 u sum|terms| (float32 accumulation in slices) + tiny."""
    tol = 256 * U * terms_abs + 1e-30
    err = np.abs(np.asarray(got, np.float64) - ref)
    assert np.all(err <= tol), f"{name}: max err {err.max():.3e}, worst ratio {(err / tol).max():.2f}"


def run_input(seed, B, T, dim, q_rank, H, Hi, win_fmt, pos_list):
    wn = synth.layer_weights(seed, dim, q_rank, H, Hi, 2 if H % 2 == 0 else 1, 64)
    dev = _upload_weights(wn)
    LW = _make(dev, dim, q_rank, H, Hi, 2 if H % 2 == 0 else 1, 64)
    M = B * T
    x = synth.bf16_round(synth.normal(seed, synth.T_X, (M, dim)))
    pos = np.array(pos_list, dtype=np.int32).reshape(M)
    rows = int(max(pos.max(), 0)) + 1
    cos, sin = rope_tables(rows)
    rb = _lib.kv_row_bytes(win_fmt, 512)
    ring0 = synth.normal(seed, synth.T_WINDOW, (B * 128, 512))
    win = torch.empty((B, 128, rb // (4 if win_fmt == "f32" else 2 if win_fmt == "bf16" else 1)),
                      dtype={"f32": torch.float32, "bf16": torch.bfloat16}.get(win_fmt, torch.uint8),
                      device="cuda")
    if win_fmt in ("f32", "bf16"):
        win.copy_(f32(ring0).reshape(B, 128, 512).to(win.dtype))
    else:
        _lib.kv_quantize(f32(ring0), "f32", win.reshape(B * 128, rb), win_fmt, B * 128, 512)
    win_before = win.clone()
    q = torch.empty((M, H, 512), dtype=torch.bfloat16, device="cuda")
    qi = torch.empty((M, max(Hi, 1), 128), dtype=torch.bfloat16, device="cuda")
    wi = torch.empty((M, max(Hi, 1)), dtype=torch.float32, device="cuda")
    ws = _lib.workspace(_lib.csa_layer_input_workspace_size(LW, M))
    say(f"layer_input seed={seed} B={B} T={T} dim={dim} q_rank={q_rank} H={H} Hi={Hi} "
        f"win={win_fmt}")
    _lib.csa_layer_input(LW, bf16(x), i32(pos), B, T, cos, sin, q, qi, wi, win, win_fmt, ws)
    torch.cuda.synchronize()

    wts = dict(wn, H=H, Hi=Hi)
    pq = np.maximum(pos, 0)  # positions are clamped to the table
    q_ref, qi_ref, wi_ref, kv_ref = OL.layer_input(x.astype(np.float64), pq, wts, OMEGA,
                                                  rotate_q=False)
    close_bf16(to_np(q), q_ref)  # un-rotated: the attention call rotates q itself
    if Hi:
        close_bf16(to_np(qi), qi_ref)
        terms = np.abs(x.astype(np.float64)) @ np.abs(wn["w_proj"].astype(np.float64)).T
        _check_f32_bound(to_np(wi), wi_ref, terms * (128 * Hi) ** -0.5, "w_idx")
    # window ring: only slot p mod 128 of each written position changes
    got = win.reshape(B, 128, -1)
    before = win_before.reshape(B, 128, -1)
    written = set()
    for m in range(M):
        b, p = m // T, int(pos[m])
        if p < 0:
            continue
        written.add((b, p % 128))
        row = got[b, p % 128]
        if win_fmt in ("f32", "bf16"):
            vals = row.float().cpu().numpy()
        else:
            dq = torch.empty((1, 512), dtype=torch.float32, device="cuda")
            _lib.kv_dequantize(row.reshape(1, rb).contiguous(), win_fmt, dq, "f32", 1, 512)
            vals = dq.cpu().numpy()[0]
        # against the oracle's own storage rounding of its entry; a rounding
        # decision taken differently near a tie moves one step
        stored = OC.store(kv_ref[m], win_fmt)[1]
        tol = step_bound(kv_ref[m][None], win_fmt, 512)[0]
        if win_fmt == "bf16":
            tol = 2.0 ** -8 * np.abs(kv_ref[m]) + 1e-6
        err = np.abs(vals - stored)
        assert np.all(err <= tol), (m, err.max())
    for b in range(B):
        for s in range(128):
            if (b, s) not in written:
                assert torch.equal(got[b, s], before[b, s]), (b, s)


@pytest.mark.parametrize("B,T,H,Hi,win_fmt", [
    (3, 1, 16, 4, "fp8_mx32"),
    (2, 3, 6, 3, "bf16"),
    (1, 5, 3, 0, "f32"),
    (5, 1, 128, 64, "fp4_e4m3_16"),
])
def test_layer_input_small(B, T, H, Hi, win_fmt):
    need_gpu()
    M = B * T
    pos = [(37 + 129 * m) % 5000 for m in range(M)]
    if T > 1:  # consecutive tokens of one sequence
        pos = [1000 * (m // T) + 200 + (m % T) for m in range(M)]
    run_input(7 + B, B, T, 512, 256, H, Hi, win_fmt, pos)


def test_layer_input_negative_position():
    need_gpu()
    run_input(3, 2, 1, 256, 256, 4, 2, "bf16", [-1, 300])


def run_output(seed, M, dim, H, groups, o_rank, y_fmt):
    gw = H // groups * 512
    wn = synth.layer_weights(seed, dim, 256, H, 0, groups, o_rank)
    dev = {"wo_a": bf16(wn["wo_a"]), "wo_b": bf16(wn["wo_b"])}
    LW = _lib.make_layer_weights(dim=dim, q_rank=256, H=H, Hi=0, groups=groups, o_rank=o_rank,
                                 **dev)
    o = synth.bf16_round(synth.normal(seed, synth.T_O, (M, H, 512)))
    y = torch.empty((M, dim), dtype=torch.float32 if y_fmt == "f32" else torch.bfloat16,
                    device="cuda")
    ws = _lib.workspace(_lib.csa_layer_output_workspace_size(LW, M))
    say(f"layer_output seed={seed} M={M} dim={dim} H={H} groups={groups} o_rank={o_rank} {y_fmt}")
    _lib.csa_layer_output(LW, bf16(o), M, y, y_fmt, ws)
    torch.cuda.synchronize()
    ref = OL.output_projection(o.astype(np.float64), wn["wo_a"], wn["wo_b"])
    assert wn["wo_a"].shape == (groups, o_rank, gw)
    scale = np.sqrt(np.mean(ref ** 2))
    got = to_np(y).astype(np.float64)
    if y_fmt == "f32":
        err = np.abs(got - ref)
        assert np.all(err <= 2e-3 * scale + 1e-3 * np.abs(ref)), err.max() / scale
    else:
        close_bf16(got, ref, atol=2e-3 * scale, rtol=2.0 ** -7)


@pytest.mark.parametrize("M,dim,H,groups,o_rank,y_fmt", [
    (3, 512, 16, 2, 64, "f32"),
    (17, 256, 8, 1, 96, "bf16"),
    (64, 768, 24, 3, 32, "f32"),
])
def test_layer_output_small(M, dim, H, groups, o_rank, y_fmt):
    need_gpu()
    run_output(11 + M, M, dim, H, groups, o_rank, y_fmt)


def test_layer_batch_invariance():
    """A sequence's outputs do not depend on the rest of the batch."""
    need_gpu()
    dim, q_rank, H, Hi = 512, 256, 16, 4
    wn = synth.layer_weights(5, dim, q_rank, H, Hi, 2, 64)
    LW = _make(_upload_weights(wn), dim, q_rank, H, Hi, 2, 64)
    x = bf16(synth.bf16_round(synth.normal(5, synth.T_X, (20, dim))))
    pos = i32(np.arange(20, dtype=np.int32) * 7 + 100)
    cos, sin = rope_tables(300)
    outs = []
    for B in (20, 1):  # two row tiles, then one
        q = torch.empty((B, H, 512), dtype=torch.bfloat16, device="cuda")
        qi = torch.empty((B, Hi, 128), dtype=torch.bfloat16, device="cuda")
        wi = torch.empty((B, Hi), dtype=torch.float32, device="cuda")
        win = torch.zeros((B, 128, 512), dtype=torch.bfloat16, device="cuda")
        ws = _lib.workspace(_lib.csa_layer_input_workspace_size(LW, B))
        _lib.csa_layer_input(LW, x[:B].contiguous(), pos[:B].contiguous(), B, 1, cos, sin, q, qi,
                             wi, win, "bf16", ws)
        y = torch.empty((B, dim), dtype=torch.float32, device="cuda")
        wso = _lib.workspace(_lib.csa_layer_output_workspace_size(LW, B))
        _lib.csa_layer_output(LW, q, B, y, "f32", wso)
        outs.append((q[0], qi[0], wi[0], win[0], y[0]))
    torch.cuda.synchronize()
    for a, b in zip(*outs):
        assert torch.equal(a, b)


def test_layer_flash_full_size():
    """V4-Flash shapes at the bench's batch: every output against the oracle."""
    need_gpu()
    B, dim, q_rank, H, Hi, groups, o_rank = 8, 4096, 1024, 64, 64, 8, 1024
    seed = synth.WORKLOADS[5].seed
    wn = synth.layer_weights(seed, dim, q_rank, H, Hi, groups, o_rank)
    LW = _make(_upload_weights(wn), dim, q_rank, H, Hi, groups, o_rank)
    x = synth.bf16_round(synth.normal(seed, synth.T_X, (B, dim)))
    t = 1048575
    pos = np.full(B, t, dtype=np.int32)
    cos, sin = rope_tables(t + 1)
    q = torch.empty((B, H, 512), dtype=torch.bfloat16, device="cuda")
    qi = torch.empty((B, Hi, 128), dtype=torch.bfloat16, device="cuda")
    wi = torch.empty((B, Hi), dtype=torch.float32, device="cuda")
    rb = _lib.kv_row_bytes("fp8_mx32", 512)
    win = torch.zeros((B, 128, rb), dtype=torch.uint8, device="cuda")
    ws = _lib.workspace(_lib.csa_layer_input_workspace_size(LW, B))
    say("layer_input full size")
    _lib.csa_layer_input(LW, bf16(x), i32(pos), B, 1, cos, sin, q, qi, wi, win, "fp8_mx32", ws)
    o = synth.bf16_round(synth.normal(seed, synth.T_O, (B, H, 512)))
    y = torch.empty((B, dim), dtype=torch.bfloat16, device="cuda")
    wso = _lib.workspace(_lib.csa_layer_output_workspace_size(LW, B))
    say("layer_output full size")
    _lib.csa_layer_output(LW, bf16(o), B, y, "bf16", wso)
    torch.cuda.synchronize()
    wts = dict(wn, H=H, Hi=Hi)
    q_ref, qi_ref, wi_ref, kv_ref = OL.layer_input(x.astype(np.float64), pos, wts, OMEGA,
                                                  rotate_q=False)
    close_bf16(to_np(q), q_ref)
    close_bf16(to_np(qi), qi_ref)
    terms = np.abs(x.astype(np.float64)) @ np.abs(wn["w_proj"].astype(np.float64)).T
    _check_f32_bound(to_np(wi), wi_ref, terms * (128 * Hi) ** -0.5, "w_idx")
    dq = torch.empty((B, 512), dtype=torch.float32, device="cuda")
    _lib.kv_dequantize(win[:, t % 128].contiguous(), "fp8_mx32", dq, "f32", B, 512)
    err = np.abs(dq.cpu().numpy() - OC.store(kv_ref, "fp8_mx32")[1])
    assert np.all(err <= step_bound(kv_ref, "fp8_mx32", 512))
    y_ref = OL.output_projection(o.astype(np.float64), wn["wo_a"], wn["wo_b"])
    scale = np.sqrt(np.mean(y_ref ** 2))
    close_bf16(to_np(y), y_ref, atol=2e-3 * scale, rtol=2.0 ** -7)
