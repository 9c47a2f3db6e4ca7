"""GPU parity of the affine-Q3/g64 format (mere.run transfer report, "Shared
architecture and implemented paths": the gathered expert kernel's Q3
specialization) in the dense, gathered and fused-expert products: against the oracle
within tolerance, bit-exact on an integer-exact case, every row
bit-identical to its width-1 run, at narrow and wide widths."""

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


def q3_device(codes, scales, biases, fused=False):
    from speculative_decode_verification_amd.ops import Q3Weight
    up = lambda a, dt: torch.from_numpy(np.ascontiguousarray(a).view(dt)).to(DEV)
    return Q3Weight(up(codes, np.uint8), up(scales, np.int16), up(biases, np.int16)).tiled(fused_gateup=fused)


@pytest.mark.parametrize("N,K", [(1024, 1024), (33, 64), (4097, 192), (96, 5120), (2560, 640)])
def test_dense_q3_matches_oracle_and_width1(N, K):
    ops, _ = _mods()
    banner(f"q3 dense N={N} K={K}")
    codes, sc, bi, _ = synth.q3_weight(25, DENSE_W, N + K, 1, N, K)
    codes, sc, bi = codes[0], sc[0], bi[0]
    W = q3_device(codes, sc, bi)
    assert W.fmt == ops.FMT_AFFINE_Q3
    x = synth.activations(25, N, 9, K)
    xd = sdev.upload_bf16(x, DEV)
    y = to_np(ops.qmv_k(W, xd))
    assert_close(y, oracle.qmv_q3(codes, sc, bi, oracle.bf16_to_f64(x)), "q3 dense bf16")
    for r in (0, 4, 8):
        assert np.array_equal(to_np(ops.qmv_k(W, xd[r:r + 1].contiguous()))[0], y[r])
    if K <= 2048:
        h = np.random.default_rng(N * K).standard_normal((9, K)).astype(np.float32)
        yh = to_np(ops.qmv_k(W, sdev.upload_f32(h, DEV)))
        assert_close(yh, oracle.qmv_q3(codes, sc, bi, h.astype(np.float64)), "q3 dense fp32")


def test_q3_integer_exact_is_bit_exact():
    """Scales 2^-6, biases multiples of 2^-6 and integer activations: every
    partial sum is exact, so the product equals the oracle bit for bit over
    all eight codes."""
    ops, _ = _mods()
    banner("q3 integer-exact")
    N, K, k = 256, 1024, 9
    rng = np.random.default_rng(6)
    q = rng.integers(0, 8, size=(N, K))
    bits = np.stack([(q >> i) & 1 for i in range(3)], axis=-1).reshape(N, 3 * K).astype(np.uint8)
    codes = np.packbits(bits, axis=-1, bitorder="little")
    sc = synth.bf16_bits_from_f32(np.full((N, K // 64), 2.0 ** -6, dtype=np.float32))
    bi = synth.bf16_bits_from_f32((rng.integers(-8, 9, size=(N, K // 64)) * 2.0 ** -6).astype(np.float32))
    x = rng.integers(-8, 9, size=(k, K)).astype(np.float32)
    W = q3_device(codes, sc, bi)
    y = to_np(ops.qmv_k(W, sdev.upload_bf16(synth.bf16_bits_from_f32(x), DEV)))
    ref = oracle.qmv_q3(codes, sc, bi, x.astype(np.float64)).astype(np.float32)
    assert np.array_equal(y, ref)


def test_dense_q3_gate_up_wide():
    ops, _ = _mods()
    I, H = 320, 640
    banner("q3 gate/up k=9 and k=32")
    codes, sc, bi, _ = synth.q3_weight(26, SHARED_GATEUP, 0, 1, 2 * I, H)
    codes, sc, bi = codes[0], sc[0], bi[0]
    W = q3_device(codes, sc, bi, fused=True)
    for k in (9, 32):
        x = synth.activations(26, k, k, H)
        xd = sdev.upload_bf16(x, DEV)
        y = to_np(ops.qmv_k(W, xd, ops.MODE_GATEUP_SWIGLU))
        ref = oracle.swiglu(oracle.qmv_q3(codes, sc, bi, oracle.bf16_to_f64(x)))
        assert_close(y, ref, f"q3 gate/up k={k}")
        y1 = to_np(ops.qmv_k(W, xd[k - 1:].contiguous(), ops.MODE_GATEUP_SWIGLU))[0]
        assert np.array_equal(y1, y[k - 1])


def _slots(layer):
    """Per-slot outputs of the fused expert kernel: slices added in order."""
    xp = to_np(layer.xpartial)
    acc = xp[0].copy()
    for j in range(1, xp.shape[0]):
        acc = acc + xp[j]
    return acc


def _q3_bank(seed, E, H, I):
    w = {}
    for name, kind, e, n, kk, fused in (("gu", GATEUP, E, 2 * I, H, True), ("dn", DOWN, E, H, I, False),
                                         ("sgu", SHARED_GATEUP, 1, 2 * I, H, True),
                                         ("sdn", SHARED_DOWN, 1, H, I, False)):
        codes, sc, bi, _ = synth.q3_weight(seed, kind, 0, e, n, kk)
        w[name] = ((codes, sc, bi), q3_device(codes, sc, bi, fused))
    return w


@pytest.mark.parametrize("k", [9, 32])
@pytest.mark.parametrize("fused", [False, True])
def test_q3_moe_layer(k, fused):
    """A Q3 MoE layer (routed and shared experts in Q3) on the gathered
    launches and on the fused expert kernel: against the oracle, rows
    against width-1 layers bit for bit."""
    ops, pipeline = _mods()
    E, H, I, topk = 16, 256, 128, 4
    banner(f"q3 moe layer k={k} fused={fused}")
    w = _q3_bank(27, E, H, I)
    inp = synth.moe_layer_inputs(27, 0, k, H, E)
    deq = lambda nm, e: oracle.dequant_q3(*(a[e] for a in w[nm][0]))

    def run(rows):
        layer = pipeline.MoeLayer(w["gu"][1], w["dn"][1], rows["x"].shape[0], topk, ops.ROUTE_SOFTMAX, False,
                                  w["sgu"][1], w["sdn"][1], fused_experts=fused)
        assert layer.fused_experts == fused and layer.fused_shared
        y = layer(sdev.upload_bf16(rows["x"], DEV), sdev.upload_f32(rows["logits"], DEV),
                  sdev.upload_f32(rows["z"], DEV))
        torch.cuda.synchronize()
        return layer, to_np(y)

    layer, y = run(inp)
    ref = oracle.moe_verify(oracle.bf16_to_f64(inp["x"]), inp["logits"], lambda e: deq("gu", e),
                            lambda e: deq("dn", e), topk, "softmax", False, z=inp["z"],
                            shared_gate_up=deq("sgu", 0), shared_down=deq("sdn", 0))
    assert np.array_equal(to_np(layer.route.idx), ref["idx"])
    if fused:
        P = _slots(layer)
        assert_close(P[:, :topk], ref["partial"], "q3 fused slot outputs")
        assert_close(P[:, topk], ref["shared"], "q3 fused shared expert")
    else:
        assert_close(to_np(layer.h), ref["h"], "q3 h")
        assert_close(to_np(layer.partial), ref["partial"], "q3 partial")
    assert_close(y, ref["y"], "q3 y")
    for r in (0, k - 1):
        l1, y1 = run({n: v[r:r + 1] for n, v in inp.items()})
        assert np.array_equal(y1[0], y[r]), r
        if fused:
            assert np.array_equal(_slots(l1)[0], _slots(layer)[r]), r


@pytest.mark.parametrize("k", [9, 2])
def test_q3_fused_flash_next_geometry(k):
    """The fused expert kernel on affine-Q3 weights of the Flash-Next expert
    geometry (hidden 2560, intermediate 640) with 16 experts, top-10 sigmoid
    and the shared expert: against the oracle and the gathered launches."""
    ops, pipeline = _mods()
    E, H, I, topk = 16, 2560, 640, 10
    banner(f"q3 fused flash-next geometry k={k}")
    w = _q3_bank(28, E, H, I)
    inp = synth.moe_layer_inputs(28, k, k, H, E)
    deq = lambda nm, e: oracle.dequant_q3(*(a[e] for a in w[nm][0]))
    args = (sdev.upload_bf16(inp["x"], DEV), sdev.upload_f32(inp["logits"], DEV), sdev.upload_f32(inp["z"], DEV))
    fused = pipeline.MoeLayer(w["gu"][1], w["dn"][1], k, topk, ops.ROUTE_SIGMOID, True, w["sgu"][1], w["sdn"][1])
    assert fused.fused_experts
    y = to_np(fused(*args))
    gathered = pipeline.MoeLayer(w["gu"][1], w["dn"][1], k, topk, ops.ROUTE_SIGMOID, True, w["sgu"][1],
                                 w["sdn"][1], fused_experts=False)
    yg = to_np(gathered(*args))
    ref = oracle.moe_verify(oracle.bf16_to_f64(inp["x"]), inp["logits"], lambda e: deq("gu", e),
                            lambda e: deq("dn", e), topk, "sigmoid", True, z=inp["z"],
                            shared_gate_up=deq("sgu", 0), shared_down=deq("sdn", 0))
    P = _slots(fused)
    assert_close(P[:, :topk], ref["partial"], "q3 fused slot outputs")
    assert_close(P[:, topk], ref["shared"], "q3 fused shared expert")
    assert_close(y, ref["y"], "q3 fused y")
    assert_close(yg, ref["y"], "q3 gathered y")
