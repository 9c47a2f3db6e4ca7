"""GPU parity of the Q8_0 weight format (Red Lite dev45, "What it is": the
MTP block's Q8_0 experts; mere.run transfer report, "Shared architecture and
implemented paths": Q8 router and shared-gate weights) in the dense and
gathered products and the fused expert kernel: against the oracle within
tolerance, bit-exact on an integer-exact case, every row bit-identical to its
width-1 run, at narrow and wide widths."""

import numpy as np
import pytest
import torch

import oracle
import synth
from synth import device as sdev
from synth.inputs import DENSE_W, DOWN, GATEUP, SHARED_DOWN, SHARED_GATEUP
from tests.gpu_helpers import DEV, assert_close, banner, to_np

pytestmark = pytest.mark.gpu


def _mods():
    from speculative_decode_verification_amd import ops, pipeline
    return ops, pipeline


def q8_device(qs, d, fused=False):
    from speculative_decode_verification_amd.ops import Q8Weight
    W = Q8Weight(torch.from_numpy(np.ascontiguousarray(qs)).to(DEV),
                 torch.from_numpy(np.ascontiguousarray(d).view(np.int16)).to(DEV))
    return W.tiled(fused_gateup=fused)


@pytest.mark.parametrize("N,K", [(1024, 1024), (33, 64), (4097, 192), (96, 5120), (2560, 640)])
def test_dense_q8_matches_oracle_and_width1(N, K):
    ops, _ = _mods()
    banner(f"q8 dense N={N} K={K}")
    qs, d = synth.q8_0_weight(20, DENSE_W, N + K, 1, N, K)
    qs, d = qs[0], d[0]
    W = q8_device(qs, d)
    assert W.fmt == ops.FMT_Q8_0
    x = synth.activations(20, N, 9, K)
    xd = sdev.upload_bf16(x, DEV)
    y = to_np(ops.qmv_k(W, xd))
    assert_close(y, oracle.qmv_q8_0(qs, d, oracle.bf16_to_f64(x)), "q8 dense bf16")
    for r in (0, 4, 8):
        assert np.array_equal(to_np(ops.qmv_k(W, xd[r:r + 1].contiguous()))[0], y[r])
    h = np.random.default_rng(N * K).standard_normal((9, K)).astype(np.float32)
    if K > 2048:
        # nine fp32 rows are staged as 27 bf16 part rows: at K = 5120 they do
        # not fit the LDS, and the call is refused before any launch
        with pytest.raises(ops.SdvError, match="LDS"):
            ops.qmv_k(W, sdev.upload_f32(h, DEV))
        return
    yh = to_np(ops.qmv_k(W, sdev.upload_f32(h, DEV)))
    assert_close(yh, oracle.qmv_q8_0(qs, d, h.astype(np.float64)), "q8 dense fp32")


def test_dense_q8_gate_up_and_wide():
    ops, _ = _mods()
    I, H = 320, 640
    banner("q8 gate/up k=9 and k=32")
    qs, d = synth.q8_0_weight(21, SHARED_GATEUP, 0, 1, 2 * I, H)
    qs, d = qs[0], d[0]
    W = q8_device(qs, d, fused=True)
    for k in (9, 32):
        x = synth.activations(21, k, k, H)
        xd = sdev.upload_bf16(x, DEV)
        y = to_np(ops.qmv_k(W, xd, ops.MODE_GATEUP_SWIGLU))
        ref = oracle.swiglu(oracle.qmv_q8_0(qs, d, oracle.bf16_to_f64(x)))
        assert_close(y, ref, f"q8 gate/up k={k}")
        for r in (0, k - 1):
            y1 = to_np(ops.qmv_k(W, xd[r:r + 1].contiguous(), ops.MODE_GATEUP_SWIGLU))[0]
            assert np.array_equal(y1, y[r])


def test_q8_integer_exact_is_bit_exact():
    """Scales that are powers of two and small integer activations: every
    partial sum is exact, so the product equals the oracle bit for bit, and
    the codes' full range (-128..127) is exercised."""
    ops, _ = _mods()
    banner("q8 integer-exact")
    N, K, k = 256, 1024, 9
    rng = np.random.default_rng(5)
    qs = rng.integers(-128, 128, size=(N, K), dtype=np.int64).astype(np.int8)
    d = (2.0 ** rng.integers(-9, -4, size=(N, K // 32))).astype(np.float16).view(np.uint16)
    x = rng.integers(-6, 7, size=(k, K)).astype(np.float32)
    W = q8_device(qs, d)
    y = to_np(ops.qmv_k(W, sdev.upload_bf16(synth.bf16_bits_from_f32(x), DEV)))
    ref = oracle.qmv_q8_0(qs, d, x.astype(np.float64)).astype(np.float32)
    assert np.array_equal(y, ref)


def q8_bank(cfg, kind, layer, E, N, K, fused):
    qs, d = synth.q8_0_weight(cfg, kind, layer, E, N, K)
    return (qs, d), q8_device(qs, d, fused)


def _slots(layer):
    """Per-slot outputs of the fused expert kernel: slices added in order."""
    xp = to_np(layer.xpartial)
    acc = xp[0].copy()
    for j in range(1, xp.shape[0]):
        acc = acc + xp[j]
    return acc


@pytest.mark.parametrize("k", [9, 32])
@pytest.mark.parametrize("fused", [False, True])
def test_q8_moe_layer(k, fused):
    """A Q8_0 MoE layer (routed experts and the shared expert in Q8_0) on the
    gathered launches and on the fused expert kernel: against the oracle, and
    rows against width-1 layers bit for bit."""
    ops, pipeline = _mods()
    E, H, I, topk = 16, 256, 128, 4
    banner(f"q8 moe layer k={k} fused={fused}")
    (gq, gd), gu = q8_bank(22, GATEUP, 0, E, 2 * I, H, True)
    (dq, dd), dn = q8_bank(22, DOWN, 0, E, H, I, False)
    (sgq, sgd), sgu = q8_bank(22, SHARED_GATEUP, 0, 1, 2 * I, H, True)
    (sdq, sdd), sdn = q8_bank(22, SHARED_DOWN, 0, 1, H, I, False)
    inp = synth.moe_layer_inputs(22, 0, k, H, E)

    def run(rows):
        layer = pipeline.MoeLayer(gu, dn, rows["x"].shape[0], topk, ops.ROUTE_SIGMOID, True, sgu, sdn,
                                  fused_experts=fused)
        assert layer.fused_experts == fused and layer.fused_shared
        y = layer(sdev.upload_bf16(rows["x"], DEV), sdev.upload_f32(rows["logits"], DEV),
                  sdev.upload_f32(rows["z"], DEV))
        torch.cuda.synchronize()
        return layer, to_np(y)

    layer, y = run(inp)
    ref = oracle.moe_verify(oracle.bf16_to_f64(inp["x"]), inp["logits"],
                            lambda e: oracle.dequant_q8_0(gq[e], gd[e]), lambda e: oracle.dequant_q8_0(dq[e], dd[e]),
                            topk, "sigmoid", True, z=inp["z"], shared_gate_up=oracle.dequant_q8_0(sgq[0], sgd[0]),
                            shared_down=oracle.dequant_q8_0(sdq[0], sdd[0]))
    assert np.array_equal(to_np(layer.route.idx), ref["idx"])
    if fused:
        P = _slots(layer)
        assert_close(P[:, :topk], ref["partial"], "q8 fused slot outputs")
        assert_close(P[:, topk], ref["shared"], "q8 fused shared expert")
    else:
        assert_close(to_np(layer.h), ref["h"], "q8 h")
        assert_close(to_np(layer.partial), ref["partial"], "q8 partial")
        assert_close(to_np(layer.sh_out), ref["shared"], "q8 shared expert")
    assert_close(y, ref["y"], "q8 y")
    for r in (0, k - 1):
        l1, y1 = run({n: v[r:r + 1] for n, v in inp.items()})
        assert np.array_equal(y1[0], y[r]), r
        if fused:
            assert np.array_equal(_slots(l1)[0], _slots(layer)[r]), r


@pytest.mark.parametrize("k", [9, 3])
def test_q8_fused_flash_next_geometry(k):
    """The fused expert kernel on Q8_0 weights of the Flash-Next expert
    geometry (hidden 2560, intermediate 640: five slices, 40-group gate/up
    streams) with 16 experts, top-10 sigmoid and the shared expert: against
    the oracle and the gathered launches."""
    ops, pipeline = _mods()
    E, H, I, topk = 16, 2560, 640, 10
    banner(f"q8 fused flash-next geometry k={k}")
    (gq, gd), gu = q8_bank(25, GATEUP, 0, E, 2 * I, H, True)
    (dq, dd), dn = q8_bank(25, DOWN, 0, E, H, I, False)
    (sgq, sgd), sgu = q8_bank(25, SHARED_GATEUP, 0, 1, 2 * I, H, True)
    (sdq, sdd), sdn = q8_bank(25, SHARED_DOWN, 0, 1, H, I, False)
    inp = synth.moe_layer_inputs(25, k, k, H, E)
    args = (sdev.upload_bf16(inp["x"], DEV), sdev.upload_f32(inp["logits"], DEV), sdev.upload_f32(inp["z"], DEV))
    fused = pipeline.MoeLayer(gu, dn, k, topk, ops.ROUTE_SIGMOID, True, sgu, sdn)
    assert fused.fused_experts
    y = to_np(fused(*args))
    gathered = pipeline.MoeLayer(gu, dn, k, topk, ops.ROUTE_SIGMOID, True, sgu, sdn, fused_experts=False)
    yg = to_np(gathered(*args))
    ref = oracle.moe_verify(oracle.bf16_to_f64(inp["x"]), inp["logits"],
                            lambda e: oracle.dequant_q8_0(gq[e], gd[e]), lambda e: oracle.dequant_q8_0(dq[e], dd[e]),
                            topk, "sigmoid", True, z=inp["z"], shared_gate_up=oracle.dequant_q8_0(sgq[0], sgd[0]),
                            shared_down=oracle.dequant_q8_0(sdq[0], sdd[0]))
    P = _slots(fused)
    assert_close(P[:, :topk], ref["partial"], "q8 fused slot outputs")
    assert_close(P[:, topk], ref["shared"], "q8 fused shared expert")
    assert_close(y, ref["y"], "q8 fused y")
    assert_close(yg, ref["y"], "q8 gathered y")


def test_q8_mtp_block_geometry():
    """The MTP block's expert geometry (hidden 2048, intermediate 512, top-10
    sigmoid), 64 Q8_0 experts, k = 9 and 4."""
    ops, pipeline = _mods()
    E, H, I, topk = 64, 2048, 512, 10
    (gq, gd), gu = q8_bank(23, GATEUP, 0, E, 2 * I, H, True)
    (dq, dd), dn = q8_bank(23, DOWN, 0, E, H, I, False)
    for k in (9, 4):
        banner(f"q8 mtp geometry k={k}")
        inp = synth.moe_layer_inputs(23, k, k, H, E)
        layer = pipeline.MoeLayer(gu, dn, k, topk, ops.ROUTE_SIGMOID, True)
        y = to_np(layer(sdev.upload_bf16(inp["x"], DEV), sdev.upload_f32(inp["logits"], DEV)))
        ref = oracle.moe_verify(oracle.bf16_to_f64(inp["x"]), inp["logits"],
                                lambda e: oracle.dequant_q8_0(gq[e], gd[e]),
                                lambda e: oracle.dequant_q8_0(dq[e], dd[e]), topk, "sigmoid", True)
        assert_close(y, ref["y"], f"q8 mtp y k={k}")


def test_route_in_experts_rejects_q8():
    """The router dispatch inside the expert kernel is built for affine Q4
    only; Q8_0 layers route with their own launch."""
    ops, pipeline = _mods()
    banner("q8 route+experts rejected")
    E, H, I = 4, 128, 64
    _, gu = q8_bank(24, GATEUP, 0, E, 2 * I, H, True)
    _, dn = q8_bank(24, DOWN, 0, E, H, I, False)
    x = torch.zeros((2, H), dtype=torch.int16, device=DEV)
    logits = torch.zeros((2, E), dtype=torch.float32, device=DEV)
    with pytest.raises(ops.SdvError, match="affine Q4"):
        ops.moe_route_experts_k(logits, ops.ROUTE_SOFTMAX, False, gu, dn, x, 2)
    with pytest.raises(ValueError, match="affine-Q4"):
        pipeline.MoeLayer(gu, dn, 2, 2, ops.ROUTE_SOFTMAX, False, route_in_experts=True)
