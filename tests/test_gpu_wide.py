"""GPU parity at the Flash-Next verifier's wide widths, 16 and 32 rows
(Flash-Next plan, "1. Target model and identity": verifier widths 1, 4, 8,
16, 32): every entry point against the oracle, and every row of a wide call
bit-identical to the same row computed narrow.  Units of the Q4 kernels take
at most 9 rows per pass, so experts with more rows than that (forced here by
small expert counts) and the shared expert run several passes."""

import numpy as np
import pytest
import torch

import oracle
import synth
from synth import device as sdev
from synth.inputs import DOWN, GATEUP, SHARED_DOWN, SHARED_GATEUP
from tests.gpu_helpers import DEV, assert_close, banner, q4_device_from_host, q4_host, to_np
from tests.test_gpu_moe import check_layer_vs_oracle, check_route, oracle_moe, run_layer, slot_outputs

pytestmark = pytest.mark.gpu

WIDE = [16, 32]


def _mods():
    from speculative_decode_verification_amd import ops, pipeline
    return ops, pipeline


@pytest.mark.parametrize("k", WIDE + [10, 27])
def test_dense_wide_rows_equal_narrow(k):
    """bf16 plain, fp32 plain and fp32 gate/up products at wide widths: row r
    of the width-k call equals row r of a width-1 call, and the oracle."""
    ops, _ = _mods()
    from synth.inputs import DENSE_W
    for mode, dt in (("plain", "bf16"), ("plain", "f32"), ("gateup", "f32")):
        banner(f"qmv wide k={k} {mode} {dt}")
        N, K = (1536, 1024) if mode == "plain" else (2 * 320, 640)
        codes, scales, biases = synth.dense_weight(11, DENSE_W if mode == "plain" else SHARED_GATEUP, 0, N, K)
        W = q4_device_from_host(codes, scales, biases).tiled(fused_gateup=mode == "gateup")
        if dt == "bf16":
            x = synth.activations(11, k, k, K)
            xd = sdev.upload_bf16(x, DEV)
            x64 = oracle.bf16_to_f64(x)
        else:
            x = np.random.default_rng(k).standard_normal((k, K)).astype(np.float32)
            xd = sdev.upload_f32(x, DEV)
            x64 = x.astype(np.float64)
        m = ops.MODE_PLAIN if mode == "plain" else ops.MODE_GATEUP_SWIGLU
        y = to_np(ops.qmv_k(W, xd, m))
        for r in (0, 8, 9, k - 1):
            y1 = to_np(ops.qmv_k(W, xd[r:r + 1].contiguous(), m))[0]
            assert np.array_equal(y[r], y1), f"k={k} row {r}"
        ref = oracle.qmv(codes, scales, biases, x64)
        if mode == "gateup":
            ref = oracle.swiglu(ref)
        assert_close(y, ref, f"qmv k={k} {mode} {dt}")


@pytest.mark.parametrize("N,K,mode,k", [(33, 64, "plain", 10), (4097, 192, "plain", 32), (2560, 5120, "plain", 32),
                                         (96, 5120, "gateup", 19), (2 * 320, 640, "gateup", 32), (1000, 576, "plain", 13)])
def test_dense_wide_form_shapes(N, K, mode, k):
    """The one-pass wide form of the dense product (bf16 rows beyond one
    narrow pass): ragged N, one K range (K = 64), an odd number of K ranges
    (K = 192, 576), the 5120 shape and the gate/up mode; every row against
    its width-1 call bit for bit and the oracle within tolerance."""
    ops, _ = _mods()
    from synth.inputs import DENSE_W
    banner(f"qmv wide form N={N} K={K} {mode} k={k}")
    codes, scales, biases = synth.dense_weight(12, DENSE_W if mode == "plain" else SHARED_GATEUP, 0, N, K)
    W = q4_device_from_host(codes, scales, biases).tiled(fused_gateup=mode == "gateup")
    x = synth.activations(12, k, k, K)
    xd = sdev.upload_bf16(x, DEV)
    m = ops.MODE_PLAIN if mode == "plain" else ops.MODE_GATEUP_SWIGLU
    y = to_np(ops.qmv_k(W, xd, m))
    for r in range(k):
        y1 = to_np(ops.qmv_k(W, xd[r:r + 1].contiguous(), m))[0]
        assert np.array_equal(y[r], y1), f"row {r}"
    ref = oracle.qmv(codes, scales, biases, oracle.bf16_to_f64(x))
    if mode == "gateup":
        ref = oracle.swiglu(ref)
    assert_close(y, ref, f"qmv wide form {N}x{K} {mode} k={k}")


@pytest.mark.parametrize("E,topk,mode,renorm", [(512, 10, "sigmoid", True), (256, 8, "softmax", False),
                                                (64, 16, "sigmoid", False), (4, 2, "softmax", True)])
def test_route_wide(E, topk, mode, renorm):
    ops, _ = _mods()
    rng = np.random.default_rng(E * 7 + topk)
    for k in WIDE + [17, 31]:
        banner(f"route wide E={E} topk={topk} k={k}")
        logits = rng.standard_normal((k, E)).astype(np.float32)
        logits[k - 1] = logits[0]                      # identical rows share every expert
        check_route(ops, logits, topk, mode, renorm)


@pytest.mark.parametrize("fused_experts", [False, True])
@pytest.mark.parametrize("k", WIDE)
def test_moe_expert_passes(k, fused_experts):
    """Four experts, top-2: every expert has far more than 9 rows, so each
    union expert and the shared expert run several passes.  Against the
    oracle, and each row against a width-1 layer bit for bit."""
    ops, pipeline = _mods()
    E, H, I, topk = 4, 256, 192, 2
    banner(f"moe expert passes k={k} fused_experts={fused_experts}")
    gu = q4_host(12, GATEUP, 0, E, 2 * I, H)
    dn = q4_host(12, DOWN, 0, E, H, I)
    inp = synth.moe_layer_inputs(12, 0, k, H, E)
    sgu = synth.dense_weight(12, SHARED_GATEUP, 0, 2 * I, H)
    sdn = synth.dense_weight(12, SHARED_DOWN, 0, H, I)
    layer, y = run_layer(ops, pipeline, gu, dn, inp, k, topk, "softmax", True, sgu, sdn, True, fused_experts)
    ref = oracle_moe(gu, dn, inp, topk, "softmax", True, sgu, sdn)
    counts = np.bincount(ref["idx"].ravel(), minlength=E)
    assert counts.max() > 9
    check_layer_vs_oracle(layer, y, ref, k, topk, True, f"moe k={k}")
    P = slot_outputs(layer) if fused_experts else None
    for r in (0, 9, 10, k - 1):
        one = {n: v[r:r + 1] for n, v in inp.items()}
        l1, y1 = run_layer(ops, pipeline, gu, dn, one, 1, topk, "softmax", True, sgu, sdn, True, fused_experts)
        assert np.array_equal(y1[0], y[r]), f"y row {r}"
        if fused_experts:
            assert np.array_equal(slot_outputs(l1)[0], P[r]), f"slot outputs row {r}"


def test_flash_next_layer_wide():
    """512 experts, hidden 2560, intermediate 640, sigmoid top-10 with the
    shared expert, at k = 16 and 32 on the fused expert path: routing exact,
    the output against the oracle, rows against the k = 9 call on the same
    rows bit for bit."""
    ops, pipeline = _mods()
    E, H, I, topk = 512, 2560, 640, 10
    cfg, layer_id = 4, 7
    banner("flash-next wide bank fill")
    gkeys = synth.bank_keys(cfg, GATEUP, layer_id)
    dkeys = synth.bank_keys(cfg, DOWN, layer_id)
    from speculative_decode_verification_amd.ops import Q4Weight
    gu_w = Q4Weight(*sdev.q4_bank(gkeys, E, 2 * I, H, DEV)).tiled(True)
    dn_w = Q4Weight(*sdev.q4_bank(dkeys, E, H, I, DEV)).tiled()
    sgu = synth.dense_weight(cfg, SHARED_GATEUP, layer_id, 2 * I, H)
    sdn = synth.dense_weight(cfg, SHARED_DOWN, layer_id, H, I)
    sgu_w, sdn_w = q4_device_from_host(*sgu).tiled(True), q4_device_from_host(*sdn).tiled()
    for k in WIDE:
        banner(f"flash-next layer k={k}")
        inp = synth.moe_layer_inputs(cfg, layer_id, k, H, E)
        args = (sdev.upload_bf16(inp["x"], DEV), sdev.upload_f32(inp["logits"], DEV),
                sdev.upload_f32(inp["z"], DEV))
        fused = pipeline.MoeLayer(gu_w, dn_w, k, topk, ops.ROUTE_SIGMOID, True, sgu_w, sdn_w)
        assert fused.fused_experts
        y = to_np(fused(*args))
        narrow = pipeline.MoeLayer(gu_w, dn_w, 9, topk, ops.ROUTE_SIGMOID, True, sgu_w, sdn_w)
        y9 = to_np(narrow(*(a[k - 9:].clone() for a in args)))
        assert np.array_equal(y[k - 9:], y9)
        idx, _ = oracle.route(inp["logits"], topk, "sigmoid", True)
        used = sorted(set(idx.ravel().tolist()))
        gmat = {e: oracle.dequant(*synth.q4_rows(gkeys, E, 2 * I, H, expert=e)) for e in used}
        dmat = {e: oracle.dequant(*synth.q4_rows(dkeys, E, H, I, expert=e)) for e in used}
        ref = oracle.moe_verify(oracle.bf16_to_f64(inp["x"]), inp["logits"], gmat.__getitem__,
                                dmat.__getitem__, topk, "sigmoid", True, z=inp["z"],
                                shared_gate_up=oracle.dequant(*sgu), shared_down=oracle.dequant(*sdn))
        assert np.array_equal(to_np(fused.route.idx), ref["idx"])
        assert int(to_np(fused.route.n_union)[0]) == ref["n_union"]
        assert_close(y, ref["y"], f"flash-next y k={k}")


@pytest.mark.parametrize("k", WIDE)
def test_gdn_wide_rows(k):
    """The recurrence over k rows against the oracle and against chained
    width-1 calls bit for bit; rollback selects every prefix's snapshot."""
    ops, _ = _mods()
    hv, hk, d = 48, 16, 128
    banner(f"gdn wide k={k}")
    S = synth.gdn_state(13, 0, hv, d, d)
    inp = synth.gdn_layer_inputs(13, 0, k, hv, hk, d, d)
    Sd = sdev.upload_f32(S, DEV)
    dd = {n: sdev.upload_f32(v, DEV) for n, v in inp.items()}
    snaps = [torch.empty_like(Sd) for _ in range(k)]
    y = to_np(ops.gdn_verify_k(Sd, dd["q"], dd["k"], dd["v"], dd["g"], dd["beta"], snaps))
    ry, rs = oracle.gdn_verify(S, inp["q"], inp["k"], inp["v"], inp["g"], inp["beta"])
    assert_close(y, ry, "gdn y")
    assert_close(np.stack([to_np(s) for s in snaps]), np.stack(rs), "gdn snapshots")
    cur = Sd
    for t in (0, 9, 10, k - 1):
        # width-1 from the snapshot before row t
        prev = Sd if t == 0 else snaps[t - 1]
        one = [torch.empty_like(Sd)]
        y1 = to_np(ops.gdn_verify_k(prev, *(dd[n][t:t + 1].contiguous() for n in ("q", "k", "v", "g", "beta")), one))
        assert np.array_equal(y1[0], y[t]), t
        assert torch.equal(one[0], snaps[t]), t
    for j in range(k + 1):
        assert ops.gdn_rollback(k, j) == j
    del cur


@pytest.mark.parametrize("k", WIDE)
@pytest.mark.parametrize("act", ["none", "silu"])
def test_gdn_prep_wide(k, act):
    """Preparation and the one-launch preparation + recurrence at wide
    widths: the two paths bit for bit, the oracle within tolerance, the
    conv window exact."""
    ops, _ = _mods()
    hv, hk, d = 48, 16, 128
    a = {"none": 0, "silu": 1}[act]
    banner(f"gdn prep wide k={k} act={act}")
    raw = synth.gdn_raw_inputs(14, 0, k, hv, hk, d, d)
    S = synth.gdn_state(14, 0, hv, d, d)
    dd = {n: sdev.upload_f32(v, DEV) for n, v in raw.items()}
    Sd = sdev.upload_f32(S, DEV)
    p = ops.gdn_prepare_k(dd["qkv"], dd["hist"], dd["conv_w"], dd["a"], dd["b"], dd["A_log"], dd["dt_bias"], hk, d, a)
    snaps_a = [torch.empty_like(Sd) for _ in range(k)]
    y_a = ops.gdn_verify_k(Sd, p["q"], p["k"], p["v"], p["g"], p["beta"], snaps_a)
    snaps_b = [torch.empty_like(Sd) for _ in range(k)]
    win_b = torch.empty_like(p["window"])
    y_b = ops.gdn_verify_prep_k(Sd, dd["qkv"], dd["hist"], dd["conv_w"], dd["a"], dd["b"], dd["A_log"],
                                dd["dt_bias"], hk, snaps_b, win_b, conv_act=a)
    out = ops.gdn_gated_norm_k(y_b, dd["z"], dd["norm_w"])
    torch.cuda.synchronize()
    assert torch.equal(y_a, y_b)
    assert torch.equal(p["window"], win_b)
    for t in range(k):
        assert torch.equal(snaps_a[t], snaps_b[t]), t
    ref = oracle.gdn_prepare(raw["qkv"], raw["hist"], raw["conv_w"], raw["a"], raw["b"], raw["A_log"],
                             raw["dt_bias"], hk, hv, d, d, act)
    assert np.array_equal(to_np(win_b), ref["window"].astype(np.float32))
    for n in ("q", "k", "v", "g", "beta"):
        assert_close(to_np(p[n]), ref[n], n)
    y_ref, s_ref = oracle.gdn_verify(S, ref["q"], ref["k"], ref["v"], ref["g"], ref["beta"])
    assert_close(to_np(y_b), y_ref, "y")
    assert_close(to_np(snaps_b[-1])[None], s_ref[-1][None], "last snapshot")
    assert_close(to_np(out), oracle.gdn_gated_norm(y_ref, raw["z"], raw["norm_w"]), "gated norm")
    # rows of the wide preparation equal a narrow call on the same history
    for t in (9, k - 1):
        one = ops.gdn_prepare_k(dd["qkv"][t:t + 1].contiguous(), win_b[t:t + 3], dd["conv_w"],
                                dd["a"][t:t + 1].contiguous(), dd["b"][t:t + 1].contiguous(), dd["A_log"],
                                dd["dt_bias"], hk, d, a)
        torch.cuda.synchronize()
        for n in ("q", "k", "v", "g", "beta"):
            assert torch.equal(one[n][0], p[n][t]), (n, t)


@pytest.mark.parametrize("k", WIDE)
def test_accept_wide(k):
    ops, _ = _mods()
    V = 248320
    banner(f"accept wide k={k}")
    for planted in (0, 9, 15, k - 1):
        logits, drafts, _ = synth.verify_block(36, k * 100 + planted, k, V, accepted=planted)
        tok, acc = ops.verify_accept_k(sdev.upload_f32(logits, DEV), torch.from_numpy(drafts).to(DEV))
        torch.cuda.synchronize()
        ref = oracle.verify_cycle(logits, drafts)
        assert np.array_equal(to_np(tok), ref["tokens"])
        assert int(to_np(acc)[0]) == ref["accepted"] == planted
    logits, _, _ = synth.verify_block(36, 1, k, 5000, accepted=0)
    noise = synth.gumbel_noise(36, 1, k, 5000)
    toks = oracle.sample_tokens(logits, noise, 0.8)
    drafts = toks[:k - 1].copy()
    tok, acc = ops.verify_accept_k(sdev.upload_f32(logits, DEV), torch.from_numpy(drafts).to(DEV),
                                   sdev.upload_f32(noise, DEV), 0.8)
    torch.cuda.synchronize()
    assert np.array_equal(to_np(tok), toks)
    assert int(to_np(acc)[0]) == k - 1
