"""GPU parity of sdv_moe_route_experts_k, the router dispatch and the fused
expert kernel as one call (Red Lite dev45, "What it is": one router dispatch,
then all of the union's (expert, row) pairs in one dispatch).  Its route outputs
equal the oracle's selection and union bit for bit, and every output equals
that of sdv_moe_route_k followed by sdv_moe_experts_k bit for bit: on the
one-launch path (k <= 9, E <= 512) and on the two-launch path it takes
beyond (wide k, E = 1024)."""

import numpy as np
import pytest
import torch

import oracle
import synth
from synth import device as sdev
from synth.inputs import DOWN, GATEUP, SHARED_DOWN, SHARED_GATEUP
from tests.gpu_helpers import DEV, assert_close, banner, q4_device_from_host, q4_host, to_np

pytestmark = pytest.mark.gpu


def _ops():
    from speculative_decode_verification_amd import ops
    return ops


def bank(cfg, E, H, I, shared):
    gu = q4_device_from_host(*q4_host(cfg, GATEUP, 2, E, 2 * I, H)).tiled(True)
    dn = q4_device_from_host(*q4_host(cfg, DOWN, 2, E, H, I)).tiled()
    sgu = sdn = None
    if shared:
        sgu = q4_device_from_host(*synth.dense_weight(cfg, SHARED_GATEUP, 2, 2 * I, H)).tiled(True)
        sdn = q4_device_from_host(*synth.dense_weight(cfg, SHARED_DOWN, 2, H, I)).tiled()
    return gu, dn, sgu, sdn


def poisoned_route(ops, k, topk):
    r = ops.route_buffers(k, topk, DEV)
    for t in r:
        t.fill_(-7)
    return r


def used_slots(partial, topk, shared):
    return partial if shared else partial[:, :, :topk]


def check_against_two_calls(ops, logits, mode, renorm, gu, dn, x, topk, sgu, sdn, label):
    k, E = logits.shape
    H, I = gu.K, gu.N // 2
    ld = sdev.upload_f32(logits, DEV)
    xd = sdev.upload_bf16(x, DEV)
    smode = ops.ROUTE_SOFTMAX if mode == "softmax" else ops.ROUTE_SIGMOID
    r2 = ops.moe_route_k(ld, topk, smode, renorm)
    p2 = ops.moe_experts_k(gu, dn, xd, r2, k, topk, sgu, sdn)
    r1 = poisoned_route(ops, k, topk)
    p1 = ops.experts_partial(k, topk, H, I, DEV)
    p1.fill_(float("nan"))
    ops.moe_route_experts_k(ld, smode, renorm, gu, dn, xd, topk, sgu, sdn, route=r1, partial=p1)
    torch.cuda.synchronize()
    # the selection and the union against the oracle
    idx, w = oracle.route(logits, topk, mode, renorm)
    uid, off, prow, pslot = oracle.union_pairs(idx)
    assert np.array_equal(to_np(r1.idx), idx), label
    nu = int(to_np(r1.n_union)[0])
    assert nu == len(uid), label
    assert np.array_equal(to_np(r1.union_ids)[:nu], uid), label
    assert np.array_equal(to_np(r1.pair_off)[:nu + 1], off), label
    assert np.array_equal(to_np(r1.pair_row), prow), label
    assert np.array_equal(to_np(r1.pair_slot), pslot), label
    assert_close(to_np(r1.w), w, f"{label} weights")
    # every output equals the two calls' bit for bit
    for name in ("idx", "w", "pair_row", "pair_slot"):
        assert np.array_equal(to_np(getattr(r1, name)), to_np(getattr(r2, name))), f"{label} {name}"
    assert np.array_equal(to_np(r1.union_ids)[:nu], to_np(r2.union_ids)[:nu]), label
    assert np.array_equal(to_np(r1.pair_off)[:nu + 1], to_np(r2.pair_off)[:nu + 1]), label
    shared = sgu is not None
    a, b = used_slots(to_np(p1), topk, shared), used_slots(to_np(p2), topk, shared)
    assert not np.isnan(a).any(), f"{label}: a used slot was not written"
    assert np.array_equal(a, b), f"{label} partial"
    return r1, p1


@pytest.mark.parametrize("E,H,I,topk,k,mode,renorm,shared", [
    (16, 256, 192, 4, 9, "softmax", False, True),
    (8, 192, 64, 2, 5, "sigmoid", True, True),
    (64, 256, 128, 8, 9, "sigmoid", True, False),
    (128, 128, 64, 10, 7, "softmax", True, True),
    (256, 256, 128, 8, 9, "softmax", False, False),
    (512, 256, 128, 10, 9, "sigmoid", True, True),
    (16, 256, 128, 1, 1, "softmax", False, False),
    (3, 128, 64, 3, 2, "sigmoid", False, True),
])
def test_route_experts_one_launch(E, H, I, topk, k, mode, renorm, shared):
    ops = _ops()
    banner(f"route+experts E={E} H={H} I={I} topk={topk} k={k} {mode} renorm={renorm} shared={shared}")
    gu, dn, sgu, sdn = bank(31, E, H, I, shared)
    inp = synth.moe_layer_inputs(31, E + k, k, H, E)
    check_against_two_calls(ops, inp["logits"], mode, renorm, gu, dn, inp["x"], topk, sgu, sdn, "one launch")


def test_route_experts_ties():
    """Tied and signed-zero logits (lowest index first among equals), a row
    whose experts all lie outside every other row's, and every row equal."""
    ops = _ops()
    banner("route+experts ties")
    E, H, I, topk, k = 64, 128, 64, 6, 9
    gu, dn, sgu, sdn = bank(32, E, H, I, True)
    inp = synth.moe_layer_inputs(32, 0, k, H, E)
    lg = inp["logits"].copy()
    lg[0, :] = np.float32(0.5)
    lg[1, [3, 1, 7, 40]] = np.float32(5.0)
    lg[2, [9, 5]] = np.float32(-0.0)
    lg[2, [10, 6]] = np.float32(0.0)
    lg[3, :] = -np.abs(lg[3, :]) - 10.0
    lg[3, 58:] = np.float32(30.0)
    check_against_two_calls(ops, lg, "softmax", False, gu, dn, inp["x"], topk, sgu, sdn, "ties softmax")
    same = np.repeat(lg[4:5], k, axis=0)
    check_against_two_calls(ops, same, "sigmoid", True, gu, dn, inp["x"], topk, sgu, sdn, "equal rows")


def test_route_experts_two_launch_fallback():
    """Beyond one pass of rows (k = 16, 32) and beyond 512 experts (E = 1024)
    the call runs the router dispatch as a launch of its own; the results are
    the same as the two calls'."""
    ops = _ops()
    for E, k, topk in ((64, 16, 8), (64, 32, 4), (1024, 9, 8)):
        banner(f"route+experts fallback E={E} k={k} topk={topk}")
        gu, dn, sgu, sdn = bank(33, E, 128, 64, True)
        inp = synth.moe_layer_inputs(33, E + k, k, 128, E)
        check_against_two_calls(ops, inp["logits"], "sigmoid", True, gu, dn, inp["x"], topk, sgu, sdn, "fallback")


def test_route_experts_back_to_back_and_width1():
    """Two calls in a row on the same buffers with different logits and
    widths leave no state behind; each row equals its width-1 call."""
    ops = _ops()
    banner("route+experts back to back")
    E, H, I, topk = 32, 256, 128, 4
    gu, dn, sgu, sdn = bank(34, E, H, I, True)
    inp = synth.moe_layer_inputs(34, 1, 9, H, E)
    r9, p9 = check_against_two_calls(ops, inp["logits"], "softmax", True, gu, dn, inp["x"], topk, sgu, sdn, "k=9")
    p9 = to_np(p9)
    inp2 = synth.moe_layer_inputs(34, 2, 4, H, E)
    check_against_two_calls(ops, inp2["logits"], "softmax", True, gu, dn, inp2["x"], topk, sgu, sdn, "k=4")
    for r in (0, 8):
        _, p1 = check_against_two_calls(ops, inp["logits"][r:r + 1], "softmax", True, gu, dn, inp["x"][r:r + 1],
                                        topk, sgu, sdn, f"row {r}")
        assert np.array_equal(to_np(p1)[:, 0], p9[:, r]), f"row {r} against the width-9 call"


def test_layer_routes_inside_the_expert_call():
    """The layer with the fused expert kernel issues the router dispatch
    inside the expert call when asked; against the oracle and against the
    layer with a separate router launch, bit for bit."""
    from speculative_decode_verification_amd import pipeline
    ops = _ops()
    banner("layer route in experts")
    E, H, I, topk, k = 64, 256, 192, 8, 9
    gu_h = q4_host(35, GATEUP, 0, E, 2 * I, H)
    dn_h = q4_host(35, DOWN, 0, E, H, I)
    sgu_h = synth.dense_weight(35, SHARED_GATEUP, 0, 2 * I, H)
    sdn_h = synth.dense_weight(35, SHARED_DOWN, 0, H, I)
    gu = q4_device_from_host(*gu_h).tiled(True)
    dn = q4_device_from_host(*dn_h).tiled()
    sgu = q4_device_from_host(*sgu_h).tiled(True)
    sdn = q4_device_from_host(*sdn_h).tiled()
    inp = synth.moe_layer_inputs(35, 0, k, H, E)
    args = (sdev.upload_bf16(inp["x"], DEV), sdev.upload_f32(inp["logits"], DEV), sdev.upload_f32(inp["z"], DEV))
    a = pipeline.MoeLayer(gu, dn, k, topk, ops.ROUTE_SIGMOID, True, sgu, sdn, route_in_experts=True)
    b = pipeline.MoeLayer(gu, dn, k, topk, ops.ROUTE_SIGMOID, True, sgu, sdn)
    assert a.route_in_experts and not b.route_in_experts
    assert [n for n, _ in a.bind(*args)] == ["experts", "combine"]
    ya, yb = to_np(a(*args)).copy(), to_np(b(*args))
    assert np.array_equal(ya, yb)
    ref = oracle.moe_verify(oracle.bf16_to_f64(inp["x"]), inp["logits"],
                            lambda e: oracle.dequant(gu_h[0][e], gu_h[1][e], gu_h[2][e]),
                            lambda e: oracle.dequant(dn_h[0][e], dn_h[1][e], dn_h[2][e]), topk, "sigmoid", True,
                            z=inp["z"], shared_gate_up=oracle.dequant(*sgu_h), shared_down=oracle.dequant(*sdn_h))
    assert np.array_equal(to_np(a.route.idx), ref["idx"])
    assert_close(ya, ref["y"], "layer y")
    # the bound calls give the same
    a.y.fill_(0.0)
    for _, call in a.bind(*args):
        call()
    torch.cuda.synchronize()
    assert np.array_equal(to_np(a.y), ya)


def test_route_experts_rejects_bad_arguments():
    ops = _ops()
    banner("route+experts argument errors")
    E, H, I, topk, k = 8, 128, 64, 2, 3
    gu, dn, sgu, sdn = bank(36, E, H, I, False)
    x = torch.zeros((k, H), dtype=torch.int16, device=DEV)
    logits = torch.zeros((k, E), dtype=torch.float32, device=DEV)
    with pytest.raises(ops.SdvError, match="score mode"):
        ops.moe_route_experts_k(logits, 7, False, gu, dn, x, topk)
    with pytest.raises(ops.SdvError, match="topk"):
        ops.moe_route_experts_k(logits, ops.ROUTE_SOFTMAX, False, gu, dn, x, E + 1)
    r = ops.route_buffers(k, topk, DEV)
    with pytest.raises(ops.SdvError, match="overlap"):
        ops.moe_route_experts_k(logits, ops.ROUTE_SOFTMAX, False, gu, dn, x, topk,
                                route=r._replace(w=logits.view(-1)[:k * topk]))
    q8 = q8_bank(E, H, I)
    with pytest.raises(ops.SdvError, match="Q8_0"):
        ops.moe_route_experts_k(logits, ops.ROUTE_SOFTMAX, False, q8[0], q8[1], x, topk)


def q8_bank(E, H, I):
    from speculative_decode_verification_amd.ops import Q8Weight
    out = []
    for kind, N, K, fused in ((GATEUP, 2 * I, H, True), (DOWN, H, I, False)):
        qs, d = synth.q8_0_weight(36, kind, 0, E, N, K)
        W = Q8Weight(torch.from_numpy(np.ascontiguousarray(qs)).to(DEV),
                     torch.from_numpy(np.ascontiguousarray(d).view(np.int16)).to(DEV))
        out.append(W.tiled(fused_gateup=fused))
    return out
