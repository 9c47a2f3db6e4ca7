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


def run_layer(ops, pipeline, gu, dn, inp, k, topk, mode, renorm, sgu=None, sdn=None, fuse_shared=True,
              fused_experts=False):
    layer = pipeline.MoeLayer(q4_device_from_host(*gu).tiled(True), q4_device_from_host(*dn).tiled(), k, topk,
                              ops.ROUTE_SOFTMAX if mode == "softmax" else ops.ROUTE_SIGMOID, renorm,
                              q4_device_from_host(*sgu).tiled(True) if sgu is not None else None,
                              q4_device_from_host(*sdn).tiled() if sdn is not None else None,
                              fuse_shared=fuse_shared, fused_experts=fused_experts)
    assert layer.fused_shared == (fuse_shared and sgu is not None)
    y = layer(sdev.upload_bf16(inp["x"], DEV), sdev.upload_f32(inp["logits"], DEV),
              sdev.upload_f32(inp["z"], DEV))
    torch.cuda.synchronize()
    return layer, to_np(y)


def slot_outputs(layer):
    """Per-slot expert outputs of a fused-path layer: the slices of
    sdv_moe_experts_k summed in slice order (fp32), [k, topk (+ 1), H]; the
    shared slot only when the layer has a shared expert (else it is never
    written)."""
    xp = to_np(layer.xpartial)
    if layer.shared_gate_up is None:
        xp = xp[:, :, :layer.topk]
    acc = xp[0].copy()
    for j in range(1, xp.shape[0]):
        acc = acc + xp[j]
    return acc


def check_layer_vs_oracle(layer, y, ref, k, topk, shared, label):
    if layer.fused_experts:
        P = slot_outputs(layer)
        idx = to_np(layer.route.idx)
        assert (idx >= 0).all()
        assert_close(P[:, :topk], ref["partial"], f"{label} slot outputs")
        if shared:
            assert_close(P[:, topk], ref["shared"], f"{label} shared expert")
    else:
        assert_close(to_np(layer.h), ref["h"], f"{label} h")
        assert_close(to_np(layer.partial), ref["partial"], f"{label} partial")
        if shared:
            assert_close(to_np(layer.sh_out), ref["shared"], f"{label} shared expert")
    assert_close(y, ref["y"], f"{label} y")


PATHS = [(False, True, False), (True, True, False), (True, False, False), (False, True, True), (True, True, True)]


@pytest.mark.parametrize("shared,fuse,fused_experts", PATHS)
def test_small_moe_matches_oracle_and_width1(shared, fuse, fused_experts):
    ops, pipeline = _mods()
    k, topk = 9, 4
    gu, dn, inp, sgu, sdn = small_moe(k, shared=shared)
    banner(f"small moe shared={shared} fused_shared={fuse} fused_experts={fused_experts}")
    layer, y = run_layer(ops, pipeline, gu, dn, inp, k, topk, "softmax", False, sgu, sdn, fuse, fused_experts)
    ref = oracle_moe(gu, dn, inp, topk, "softmax", False, sgu, sdn)
    assert int(to_np(layer.route.n_union)[0]) == ref["n_union"]
    check_layer_vs_oracle(layer, y, ref, k, topk, shared, "small moe")
    if fused_experts:
        P9 = slot_outputs(layer)
    else:
        h9, p9 = to_np(layer.h), to_np(layer.partial)
    for r in range(k):
        one = {n: v[r:r + 1] for n, v in inp.items()}
        l1, y1 = run_layer(ops, pipeline, gu, dn, one, 1, topk, "softmax", False, sgu, sdn, fuse, fused_experts)
        if fused_experts:
            assert np.array_equal(slot_outputs(l1)[0], P9[r]), f"slot outputs row {r}"
        else:
            assert np.array_equal(to_np(l1.h)[0], h9[r]), f"h row {r}"
            assert np.array_equal(to_np(l1.partial)[0], p9[r]), f"partial row {r}"
        assert np.array_equal(y1[0], y[r]), f"y row {r}"


@pytest.mark.parametrize("E,H,I,topk,k,shared", [(16, 256, 192, 4, 9, True), (8, 192, 64, 2, 5, True),
                                                 (32, 320, 384, 6, 7, False), (4, 128, 128, 4, 9, True),
                                                 (64, 1024, 256, 8, 3, True), (16, 256, 128, 1, 1, False)])
def test_fused_experts_shapes(E, H, I, topk, k, shared):
    """Ragged geometry of the fused expert path: a 64-wide last slice, fewer
    down tiles than waves, a hidden size that is not a multiple of 256, top-1
    and one row, every expert in the union (topk = E)."""
    ops, pipeline = _mods()
    banner(f"fused experts E={E} H={H} I={I} topk={topk} k={k} shared={shared}")
    cfg = 9
    gu = q4_host(cfg, GATEUP, 1, E, 2 * I, H)
    dn = q4_host(cfg, DOWN, 1, E, H, I)
    inp = synth.moe_layer_inputs(cfg, 1, k, H, E)
    sgu = synth.dense_weight(cfg, SHARED_GATEUP, 1, 2 * I, H) if shared else None
    sdn = synth.dense_weight(cfg, SHARED_DOWN, 1, H, I) if shared else None
    layer, y = run_layer(ops, pipeline, gu, dn, inp, k, topk, "sigmoid", True, sgu, sdn, True, True)
    ref = oracle_moe(gu, dn, inp, topk, "sigmoid", True, sgu, sdn)
    assert np.array_equal(to_np(layer.route.idx), ref["idx"])
    check_layer_vs_oracle(layer, y, ref, k, topk, shared, "fused experts")
    # the gathered path computes the same layer
    _, y_g = run_layer(ops, pipeline, gu, dn, inp, k, topk, "sigmoid", True, sgu, sdn, True, False)
    assert_close(y_g, ref["y"], "gathered path y")


def test_fused_experts_unused_slots_untouched():
    """Slices and slots the layer does not use are not written: a sentinel
    in the shared slot survives a layer without a shared expert."""
    ops, pipeline = _mods()
    banner("fused experts sentinel")
    k, topk = 3, 2
    gu, dn, inp, _, _ = small_moe(k)
    layer = pipeline.MoeLayer(q4_device_from_host(*gu).tiled(True), q4_device_from_host(*dn).tiled(), k, topk,
                              ops.ROUTE_SOFTMAX, False, fused_experts=True)
    layer.xpartial.fill_(12345.0)
    layer(sdev.upload_bf16(inp["x"], DEV), sdev.upload_f32(inp["logits"], DEV))
    torch.cuda.synchronize()
    xp = to_np(layer.xpartial)
    assert (xp[:, :, topk] == 12345.0).all()
    assert not (xp[:, :, :topk] == 12345.0).any()


class _Bank:
    """One layer's expert bank: generated on the device, with the host
    generator's experts dequantised for the oracle on demand (cached, so the
    widths of one test module share them)."""

    def __init__(self, cfg, layer_id, E, H, I):
        from speculative_decode_verification_amd.ops import Q4Weight
        self.cfg, self.E, self.H, self.I = cfg, E, H, I
        self.gkeys = synth.bank_keys(cfg, GATEUP, layer_id)
        self.dkeys = synth.bank_keys(cfg, DOWN, layer_id)
        self.gu_d = sdev.q4_bank(self.gkeys, E, 2 * I, H, DEV)
        self.dn_d = sdev.q4_bank(self.dkeys, E, H, I, DEV)
        self.gu_w, self.dn_w = Q4Weight(*self.gu_d).tiled(True), Q4Weight(*self.dn_d).tiled()
        self._g, self._d = {}, {}

    def gmat(self, e):
        if e not in self._g:
            self._g[e] = oracle.dequant(*synth.q4_rows(self.gkeys, self.E, 2 * self.I, self.H, expert=e))
        return self._g[e]

    def dmat(self, e):
        if e not in self._d:
            self._d[e] = oracle.dequant(*synth.q4_rows(self.dkeys, self.E, self.H, self.I, expert=e))
        return self._d[e]


ORNITH = dict(E=256, H=2048, I=512, topk=8, cfg=2, layer=0)


@pytest.fixture(scope="module")
def ornith_bank():
    banner("ornith layer bank fill")
    o = ORNITH
    b = _Bank(o["cfg"], o["layer"], o["E"], o["H"], o["I"])
    for e in (0, 77, 255):
        host = synth.q4_rows(b.gkeys, b.E, 2 * b.I, b.H, expert=e, row_start=1000, row_count=24)
        for a, d in zip(host, b.gu_d):
            dev_rows = to_np(d[e, 1000:1024])
            assert np.array_equal(dev_rows.view(a.dtype), a), f"bank fill mismatch expert {e}"
    return b


@pytest.mark.parametrize("k", list(range(2, 10)))
def test_ornith_shaped_layer(ornith_bank, k):
    """256 experts, hidden 2048, intermediate 512, softmax top-8, every width
    k = 2..9, on the gathered launches and on the fused expert kernel; the
    bank is generated on the device and spot-checked against the host
    generator."""
    ops, pipeline = _mods()
    b, o = ornith_bank, ORNITH
    topk = o["topk"]
    banner(f"ornith layer k={k}")
    inp = synth.moe_layer_inputs(o["cfg"], o["layer"], k, b.H, b.E)
    layer = pipeline.MoeLayer(b.gu_w, b.dn_w, k, topk, ops.ROUTE_SOFTMAX, False, fused_experts=False)
    fused = pipeline.MoeLayer(b.gu_w, b.dn_w, k, topk, ops.ROUTE_SOFTMAX, False, fused_experts=True)
    args = (sdev.upload_bf16(inp["x"], DEV), sdev.upload_f32(inp["logits"], DEV))
    y = to_np(layer(*args))
    y_f = to_np(fused(*args))
    ref = oracle.moe_verify(oracle.bf16_to_f64(inp["x"]), inp["logits"], b.gmat, b.dmat, topk, "softmax", False)
    assert np.array_equal(to_np(layer.route.idx), ref["idx"])
    assert np.array_equal(to_np(fused.route.idx), ref["idx"])
    assert int(to_np(fused.route.n_union)[0]) == ref["n_union"]
    assert_close(to_np(layer.h), ref["h"], "h")
    assert_close(to_np(layer.partial), ref["partial"], "partial")
    assert_close(y, ref["y"], "y")
    assert_close(slot_outputs(fused)[:, :topk], ref["partial"], "fused slot outputs")
    assert_close(y_f, ref["y"], "fused y")


def _width1_rows(ops, pipeline, gu_w, dn_w, inp, k, topk, mode, renorm, sgu_w=None, sdn_w=None, fused=True):
    """Each row of a k-row layer against its own one-row layer, bit for bit:
    y, and the slot outputs (with the shared slot) or h and the partials."""
    sm = ops.ROUTE_SOFTMAX if mode == "softmax" else ops.ROUTE_SIGMOID
    has_z = sgu_w is not None
    layer = pipeline.MoeLayer(gu_w, dn_w, k, topk, sm, renorm, sgu_w, sdn_w, fused_experts=fused)
    args = (sdev.upload_bf16(inp["x"], DEV), sdev.upload_f32(inp["logits"], DEV),
            sdev.upload_f32(inp["z"], DEV) if has_z else None)
    y = to_np(layer(*args))
    if fused:
        P = slot_outputs(layer)
    else:
        h, part = to_np(layer.h), to_np(layer.partial)
        sh = to_np(layer.sh_out) if has_z else None
    one = pipeline.MoeLayer(gu_w, dn_w, 1, topk, sm, renorm, sgu_w, sdn_w, fused_experts=fused)
    for r in range(k):
        a1 = (sdev.upload_bf16(inp["x"][r:r + 1], DEV), sdev.upload_f32(inp["logits"][r:r + 1], DEV),
              sdev.upload_f32(inp["z"][r:r + 1], DEV) if has_z else None)
        y1 = to_np(one(*a1))
        assert np.array_equal(y1[0], y[r]), f"y row {r}"
        if fused:
            P1 = slot_outputs(one)
            assert np.array_equal(P1[0, :topk], P[r, :topk]), f"slot outputs row {r}"
            if has_z:
                assert np.array_equal(P1[0, topk], P[r, topk]), f"shared slot row {r}"
        else:
            assert np.array_equal(to_np(one.h)[0], h[r]), f"h row {r}"
            assert np.array_equal(to_np(one.partial)[0], part[r]), f"partial row {r}"
            if has_z:
                assert np.array_equal(to_np(one.sh_out)[0], sh[r]), f"shared output row {r}"


@pytest.mark.parametrize("fused", [True, False])
def test_ornith_width9_equals_width1(ornith_bank, fused):
    """At the 256-expert, 2048 / 512 geometry every row of a nine-row layer
    equals the same row run alone, bit for bit."""
    ops, pipeline = _mods()
    b, o = ornith_bank, ORNITH
    banner(f"ornith width 9 vs width 1 fused={fused}")
    inp = synth.moe_layer_inputs(o["cfg"], o["layer"], 9, b.H, b.E)
    _width1_rows(ops, pipeline, b.gu_w, b.dn_w, inp, 9, o["topk"], "softmax", False, fused=fused)


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
    layer = pipeline.MoeLayer(gu_w, dn_w, k, topk, ops.ROUTE_SIGMOID, True, sgu_w, sdn_w, fused_experts=False)
    assert layer.fused_shared
    inp = synth.moe_layer_inputs(cfg, layer_id, k, H, E)
    banner("flash-next layer k=9")
    args = (sdev.upload_bf16(inp["x"], DEV), sdev.upload_f32(inp["logits"], DEV), sdev.upload_f32(inp["z"], DEV))
    y = to_np(layer(*args))
    # the same layer with the shared expert as two dense launches
    split = pipeline.MoeLayer(gu_w, dn_w, k, topk, ops.ROUTE_SIGMOID, True, sgu_w, sdn_w, fuse_shared=False,
                              fused_experts=False)
    y_split = to_np(split(*args))
    # the fused expert path (the step's hot path), marshalled once like the bench
    fused = pipeline.MoeLayer(gu_w, dn_w, k, topk, ops.ROUTE_SIGMOID, True, sgu_w, sdn_w)
    assert fused.fused_experts
    y_f = to_np(fused(*args))
    fused.y.zero_()
    for _, call in fused.bind(*args):
        call()
    torch.cuda.synchronize()
    assert np.array_equal(to_np(fused.y), y_f)
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
    P = slot_outputs(fused)
    assert_close(P[:, :topk], ref["partial"], "fused slot outputs")
    assert_close(P[:, topk], ref["shared"], "fused shared expert")
    assert_close(y_f, ref["y"], "fused y")


@pytest.mark.parametrize("fused", [True, False])
def test_flash_next_width9_equals_width1(fused):
    """At the 512-expert, 2560 / 640 geometry with the sigmoid-gated shared
    expert (five 128-wide slices, 40-group gate/up streams) every row of a
    nine-row layer equals the same row run alone, bit for bit: y, the slot
    outputs and the shared slot."""
    ops, pipeline = _mods()
    E, H, I, topk, k = 512, 2560, 640, 10, 9
    cfg, layer_id = 4, 7
    banner(f"flash-next width 9 vs width 1 fused={fused}")
    from speculative_decode_verification_amd.ops import Q4Weight
    gu_w = Q4Weight(*sdev.q4_bank(synth.bank_keys(cfg, GATEUP, layer_id), E, 2 * I, H, DEV)).tiled(True)
    dn_w = Q4Weight(*sdev.q4_bank(synth.bank_keys(cfg, DOWN, layer_id), E, H, I, DEV)).tiled()
    sgu = synth.dense_weight(cfg, SHARED_GATEUP, layer_id, 2 * I, H)
    sdn = synth.dense_weight(cfg, SHARED_DOWN, layer_id, H, I)
    sgu_w, sdn_w = q4_device_from_host(*sgu).tiled(True), q4_device_from_host(*sdn).tiled()
    inp = synth.moe_layer_inputs(cfg, layer_id, k, H, E)
    _width1_rows(ops, pipeline, gu_w, dn_w, inp, k, topk, "sigmoid", True, sgu_w, sdn_w, fused=fused)


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
