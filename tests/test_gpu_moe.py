"""GPU parity of the MoE half of the verify step: router dispatch and union
(bit-exact), gathered gate/up + down (oracle within tolerance; each row
bit-identical to a width-1 run) and the combine, from tiny banks up to the
256-expert and 512-expert layer shapes."""

import numpy as np
import pytest
import torch

import oracle
import synth
from synth import device as sdev
from synth.inputs import DOWN, GATEUP, SHARED_DOWN, SHARED_GATEUP
from tests.gpu_helpers import DEV, assert_close, banner, q4_device_from_host, q4_host, to_np

pytestmark = pytest.mark.gpu


def _mods():
    from speculative_decode_verification_amd import ops, pipeline
    return ops, pipeline


def check_route(ops, logits, topk, mode, renorm):
    k = logits.shape[0]
    r = ops.moe_route_k(sdev.upload_f32(logits, DEV), topk,
                        ops.ROUTE_SOFTMAX if mode == "softmax" else ops.ROUTE_SIGMOID, renorm)
    idx, w = oracle.route(logits, topk, mode, renorm)
    uid, off, prow, pslot = oracle.union_pairs(idx)
    assert np.array_equal(to_np(r.idx), idx)
    nu = int(to_np(r.n_union)[0])
    assert nu == len(uid)
    assert np.array_equal(to_np(r.union_ids)[:nu], uid)
    assert np.array_equal(to_np(r.pair_off)[:nu + 1], off)
    assert np.array_equal(to_np(r.pair_row), prow)
    assert np.array_equal(to_np(r.pair_slot), pslot)
    assert_close(to_np(r.w), w, f"route weights {mode}")
    return r


@pytest.mark.parametrize("E,topk,mode,renorm", [(256, 8, "softmax", False), (512, 10, "sigmoid", True),
                                                (256, 8, "softmax", True), (64, 16, "sigmoid", False),
                                                (1024, 4, "softmax", False), (3, 3, "sigmoid", True)])
def test_route_bit_exact(E, topk, mode, renorm):
    banner(f"route E={E} topk={topk} {mode} renorm={renorm}")
    ops, _ = _mods()
    rng = np.random.default_rng(E + topk)
    for k in range(1, 10):
        logits = rng.standard_normal((k, E)).astype(np.float32)
        check_route(ops, logits, topk, mode, renorm)


def test_route_ties_and_shared_experts():
    banner("route ties")
    ops, _ = _mods()
    rng = np.random.default_rng(1)
    logits = rng.standard_normal((9, 256)).astype(np.float32)
    logits[0, :] = np.float32(0.5)                       # all tied: lowest indices win
    logits[1, [3, 1, 7, 200]] = np.float32(5.0)          # tie at the top
    logits[2, [9, 5]] = np.float32(-0.0)
    logits[2, 6] = np.float32(0.0)
    logits[3] = logits[4]                                # identical rows share all experts
    logits[5, 250:] = np.float32(9.0)
    check_route(ops, logits, 8, "softmax", False)
    check_route(ops, logits, 8, "sigmoid", True)


def small_moe(k, E=16, H=256, I=128, topk=4, cfg=9, shared=False):
    gu = q4_host(cfg, GATEUP, 0, E, 2 * I, H)
    dn = q4_host(cfg, DOWN, 0, E, H, I)
    inp = synth.moe_layer_inputs(cfg, 0, k, H, E)
    sgu = synth.dense_weight(cfg, SHARED_GATEUP, 0, 2 * I, H) if shared else None
    sdn = synth.dense_weight(cfg, SHARED_DOWN, 0, H, I) if shared else None
    return gu, dn, inp, sgu, sdn


def oracle_moe(gu, dn, inp, topk, mode, renorm, sgu=None, sdn=None):
    x = oracle.bf16_to_f64(inp["x"])
    return oracle.moe_verify(x, inp["logits"], lambda e: oracle.dequant(gu[0][e], gu[1][e], gu[2][e]),
                             lambda e: oracle.dequant(dn[0][e], dn[1][e], dn[2][e]), topk, mode, renorm,
                             z=inp["z"] if sgu is not None else None,
                             shared_gate_up=oracle.dequant(*sgu) if sgu is not None else None,
                             shared_down=oracle.dequant(*sdn) if sdn is not None else None)


def run_layer(ops, pipeline, gu, dn, inp, k, topk, mode, renorm, sgu=None, sdn=None, fuse_shared=True):
    layer = pipeline.MoeLayer(q4_device_from_host(*gu).tiled(True), q4_device_from_host(*dn).tiled(), k, topk,
                              ops.ROUTE_SOFTMAX if mode == "softmax" else ops.ROUTE_SIGMOID, renorm,
                              q4_device_from_host(*sgu).tiled(True) if sgu is not None else None,
                              q4_device_from_host(*sdn).tiled() if sdn is not None else None,
                              fuse_shared=fuse_shared)
    assert layer.fused_shared == (fuse_shared and sgu is not None)
    y = layer(sdev.upload_bf16(inp["x"], DEV), sdev.upload_f32(inp["logits"], DEV),
              sdev.upload_f32(inp["z"], DEV))
    torch.cuda.synchronize()
    return layer, to_np(y)


@pytest.mark.parametrize("shared,fuse", [(False, True), (True, True), (True, False)])
def test_small_moe_matches_oracle_and_width1(shared, fuse):
    ops, pipeline = _mods()
    k, topk = 9, 4
    gu, dn, inp, sgu, sdn = small_moe(k, shared=shared)
    banner(f"small moe shared={shared} fused={fuse}")
    layer, y = run_layer(ops, pipeline, gu, dn, inp, k, topk, "softmax", False, sgu, sdn, fuse)
    ref = oracle_moe(gu, dn, inp, topk, "softmax", False, sgu, sdn)
    assert int(to_np(layer.route.n_union)[0]) == ref["n_union"]
    assert_close(to_np(layer.h), ref["h"], "h")
    assert_close(to_np(layer.partial), ref["partial"], "partial")
    if shared:
        assert_close(to_np(layer.sh_out), ref["shared"], "shared expert")
    assert_close(y, ref["y"], "y")
    h9, p9 = to_np(layer.h), to_np(layer.partial)
    for r in range(k):
        one = {n: (v[r:r + 1] if n != "z" else v[r:r + 1]) for n, v in inp.items()}
        l1, y1 = run_layer(ops, pipeline, gu, dn, one, 1, topk, "softmax", False, sgu, sdn, fuse)
        assert np.array_equal(to_np(l1.h)[0], h9[r]), f"h row {r}"
        assert np.array_equal(to_np(l1.partial)[0], p9[r]), f"partial row {r}"
        assert np.array_equal(y1[0], y[r]), f"y row {r}"


def test_ornith_shaped_layer():
    """256 experts, hidden 2048, intermediate 512, softmax top-8, k = 2..9;
    the bank is generated on the device and spot-checked against the host
    generator."""
    ops, pipeline = _mods()
    E, H, I, topk = 256, 2048, 512, 8
    cfg, layer_id = 2, 0
    banner("ornith layer bank fill")
    gkeys = synth.bank_keys(cfg, GATEUP, layer_id)
    dkeys = synth.bank_keys(cfg, DOWN, layer_id)
    gu_d = sdev.q4_bank(gkeys, E, 2 * I, H, DEV)
    dn_d = sdev.q4_bank(dkeys, E, H, I, DEV)
    for e in (0, 77, 255):
        host = synth.q4_rows(gkeys, E, 2 * I, H, expert=e, row_start=1000, row_count=24)
        for a, b in zip(host, gu_d):
            dev_rows = to_np(b[e, 1000:1024])
            assert np.array_equal(dev_rows.view(a.dtype), a), f"bank fill mismatch expert {e}"
    from speculative_decode_verification_amd.ops import Q4Weight
    gu_w, dn_w = Q4Weight(*gu_d).tiled(True), Q4Weight(*dn_d).tiled()
    for k in (2, 5, 9):
        banner(f"ornith layer k={k}")
        inp = synth.moe_layer_inputs(cfg, layer_id, k, H, E)
        layer = pipeline.MoeLayer(gu_w, dn_w, k, topk, ops.ROUTE_SOFTMAX, False)
        y = to_np(layer(sdev.upload_bf16(inp["x"], DEV), sdev.upload_f32(inp["logits"], DEV)))
        idx, _ = oracle.route(inp["logits"], topk, "softmax", False)
        used = sorted(set(idx.ravel().tolist()))
        gmat = {e: oracle.dequant(*synth.q4_rows(gkeys, E, 2 * I, H, expert=e)) for e in used}
        dmat = {e: oracle.dequant(*synth.q4_rows(dkeys, E, H, I, expert=e)) for e in used}
        ref = oracle.moe_verify(oracle.bf16_to_f64(inp["x"]), inp["logits"], gmat.__getitem__,
                                dmat.__getitem__, topk, "softmax", False)
        assert np.array_equal(to_np(layer.route.idx), ref["idx"])
        assert_close(to_np(layer.h), ref["h"], "h")
        assert_close(y, ref["y"], "y")


def test_flash_next_shaped_layer():
    """512 experts, hidden 2560, intermediate 640, sigmoid top-10 renormalised,
    one sigmoid-gated shared expert, k = 9."""
    ops, pipeline = _mods()
    E, H, I, topk, k = 512, 2560, 640, 10, 9
    cfg, layer_id = 4, 5
    banner("flash-next layer bank fill")
    gkeys = synth.bank_keys(cfg, GATEUP, layer_id)
    dkeys = synth.bank_keys(cfg, DOWN, layer_id)
    from speculative_decode_verification_amd.ops import Q4Weight
    gu_w = Q4Weight(*sdev.q4_bank(gkeys, E, 2 * I, H, DEV)).tiled(True)
    dn_w = Q4Weight(*sdev.q4_bank(dkeys, E, H, I, DEV)).tiled()
    sgu = synth.dense_weight(cfg, SHARED_GATEUP, layer_id, 2 * I, H)
    sdn = synth.dense_weight(cfg, SHARED_DOWN, layer_id, H, I)
    sgu_w, sdn_w = q4_device_from_host(*sgu).tiled(True), q4_device_from_host(*sdn).tiled()
    layer = pipeline.MoeLayer(gu_w, dn_w, k, topk, ops.ROUTE_SIGMOID, True, sgu_w, sdn_w)
    assert layer.fused_shared
    inp = synth.moe_layer_inputs(cfg, layer_id, k, H, E)
    banner("flash-next layer k=9")
    args = (sdev.upload_bf16(inp["x"], DEV), sdev.upload_f32(inp["logits"], DEV), sdev.upload_f32(inp["z"], DEV))
    y = to_np(layer(*args))
    # the same layer with the shared expert as two dense launches
    split = pipeline.MoeLayer(gu_w, dn_w, k, topk, ops.ROUTE_SIGMOID, True, sgu_w, sdn_w, fuse_shared=False)
    y_split = to_np(split(*args))
    # the bound (marshalled-once) launches give the fused layer's result bit for bit
    layer.y.zero_()
    for _, call in layer.bind(*args):
        call()
    torch.cuda.synchronize()
    assert np.array_equal(to_np(layer.y), y)
    idx, _ = oracle.route(inp["logits"], topk, "sigmoid", True)
    used = sorted(set(idx.ravel().tolist()))
    gmat = {e: oracle.dequant(*synth.q4_rows(gkeys, E, 2 * I, H, expert=e)) for e in used}
    dmat = {e: oracle.dequant(*synth.q4_rows(dkeys, E, H, I, expert=e)) for e in used}
    ref = oracle.moe_verify(oracle.bf16_to_f64(inp["x"]), inp["logits"], gmat.__getitem__, dmat.__getitem__,
                            topk, "sigmoid", True, z=inp["z"], shared_gate_up=oracle.dequant(*sgu),
                            shared_down=oracle.dequant(*sdn))
    assert np.array_equal(to_np(layer.route.idx), ref["idx"])
    assert int(to_np(layer.route.n_union)[0]) == ref["n_union"]
    assert_close(to_np(layer.h), ref["h"], "h")
    assert_close(to_np(layer.partial), ref["partial"], "partial")
    assert_close(to_np(layer.sh_out), ref["shared"], "shared expert")
    assert_close(to_np(split.sh_out), ref["shared"], "shared expert (dense launches)")
    assert_close(y, ref["y"], "y")
    assert_close(y_split, ref["y"], "y (dense shared launches)")


def test_combine_matches_oracle_order():
    banner("combine")
    ops, _ = _mods()
    rng = np.random.default_rng(3)
    k, topk, H = 9, 10, 2560
    partial = rng.standard_normal((k, topk, H)).astype(np.float32)
    w = rng.uniform(0, 1, (k, topk)).astype(np.float32)
    sh = rng.standard_normal((k, H)).astype(np.float32)
    z = rng.standard_normal(k).astype(np.float32)
    y = to_np(ops.moe_combine_k(sdev.upload_f32(partial, DEV), sdev.upload_f32(w, DEV), sdev.upload_f32(sh, DEV),
                                sdev.upload_f32(z, DEV)))
    assert_close(y, oracle.combine(partial, w, sh, z), "combine")
    y2 = to_np(ops.moe_combine_k(sdev.upload_f32(partial, DEV), sdev.upload_f32(w, DEV)))
    assert_close(y2, oracle.combine(partial, w), "combine (no shared)")
