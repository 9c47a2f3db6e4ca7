"""GPU parity of the dense multi-row affine-Q4 product (sdv_qmv_k) against
the CPU oracle, plus bitwise width-k == width-1 and integer-exact cases."""

import numpy as np
import pytest
import torch

import oracle
import synth
from synth import device as sdev
from synth.inputs import DENSE_W, SHARED_GATEUP
from tests.gpu_helpers import DEV, assert_close, banner, q4_device_from_host, to_np

pytestmark = pytest.mark.gpu


def _ops():
    from speculative_decode_verification_amd import ops
    return ops


def dense_case(cfg, layer, N, K, rows, kind=DENSE_W):
    codes, scales, biases = synth.dense_weight(cfg, kind, layer, N, K)
    x = synth.activations(cfg, layer, rows, K)
    return codes, scales, biases, x


def test_tiny_projection_matches_oracle():
    banner("qmv tiny N=K=1024 k=2")
    ops = _ops()
    codes, scales, biases, x = dense_case(0, 0, 1024, 1024, 2)
    W = q4_device_from_host(codes, scales, biases).tiled()
    y = ops.qmv_k(W, sdev.upload_bf16(x, DEV))
    ref = oracle.qmv(codes, scales, biases, oracle.bf16_to_f64(x))
    assert_close(to_np(y), ref, "tiny projection")


def test_integer_exact_is_bit_exact():
    banner("qmv integer-exact N=256 K=1024 k=9")
    ops = _ops()
    codes, scales, biases, x = synth.integer_exact_weight(3, 256, 1024, 9)
    W = q4_device_from_host(codes, scales, biases).tiled()
    y = to_np(ops.qmv_k(W, sdev.upload_bf16(x, DEV)))
    ref = oracle.qmv(codes, scales, biases, oracle.bf16_to_f64(x)).astype(np.float32)
    assert np.array_equal(y, ref)


def test_dense_5120_widths_bitwise_and_parity():
    banner("qmv 5120x5120 widths 1,4,8,9")
    ops = _ops()
    codes, scales, biases, x = dense_case(1, 0, 5120, 5120, 9)
    W = q4_device_from_host(codes, scales, biases).tiled()
    xd = sdev.upload_bf16(x, DEV)
    singles = [to_np(ops.qmv_k(W, xd[r:r + 1].contiguous()))[0] for r in range(9)]
    for k in (1, 4, 8, 9):
        y = to_np(ops.qmv_k(W, xd[:k].contiguous()))
        for r in range(k):
            assert np.array_equal(y[r], singles[r]), f"width {k} row {r} differs from width 1"
    ref = oracle.qmv(codes, scales, biases, oracle.bf16_to_f64(x))
    assert_close(np.stack(singles), ref, "5120x5120 projection")


@pytest.mark.parametrize("N,K", [(1000, 576), (33, 64), (1, 64), (4097, 192), (96, 5120)])
def test_ragged_shapes(N, K):
    banner(f"qmv ragged N={N} K={K}")
    ops = _ops()
    codes, scales, biases, x = dense_case(0, 7, N, K, 9)
    W = q4_device_from_host(codes, scales, biases).tiled()
    xd = sdev.upload_bf16(x, DEV)
    ref = oracle.qmv(codes, scales, biases, oracle.bf16_to_f64(x))
    for k in (1, 3, 9):
        y = to_np(ops.qmv_k(W, xd[:k].contiguous()))
        assert_close(y, ref[:k], f"N={N} K={K} k={k}")


@pytest.mark.parametrize("I,H", [(640, 2560), (40, 128), (17, 192)])
def test_gate_up_swiglu(I, H):
    banner(f"qmv gate/up I={I} H={H}")
    ops = _ops()
    codes, scales, biases, x = dense_case(4, 3, 2 * I, H, 9, kind=SHARED_GATEUP)
    W = q4_device_from_host(codes, scales, biases).tiled(fused_gateup=True)
    xd = sdev.upload_bf16(x, DEV)
    ref = oracle.swiglu(oracle.qmv(codes, scales, biases, oracle.bf16_to_f64(x)))
    y9 = to_np(ops.qmv_k(W, xd, mode=ops.MODE_GATEUP_SWIGLU))
    assert_close(y9, ref, "gate/up swiglu")
    for r in range(9):
        y1 = to_np(ops.qmv_k(W, xd[r:r + 1].contiguous(), mode=ops.MODE_GATEUP_SWIGLU))[0]
        assert np.array_equal(y9[r], y1)


@pytest.mark.parametrize("N,K", [(2560, 640), (300, 512), (64, 2048)])
def test_fp32_activations(N, K):
    banner(f"qmv fp32 act N={N} K={K}")
    ops = _ops()
    codes, scales, biases = synth.dense_weight(4, 4, 5, N, K)
    h = np.random.default_rng(N + K).standard_normal((9, K)).astype(np.float32) * np.float32(0.3)
    W = q4_device_from_host(codes, scales, biases).tiled()
    hd = sdev.upload_f32(h, DEV)
    ref = oracle.qmv(codes, scales, biases, h.astype(np.float64))
    y9 = to_np(ops.qmv_k(W, hd))
    assert_close(y9, ref, "fp32 activations")
    for r in (0, 4, 8):
        y1 = to_np(ops.qmv_k(W, hd[r:r + 1].contiguous()))[0]
        assert np.array_equal(y9[r], y1)


def test_mfma_row_position_independence():
    """A row's result must not depend on where it sits among the activation
    rows: permuting the rows permutes the outputs bit for bit."""
    banner("qmv row permutation")
    ops = _ops()
    codes, scales, biases, x = dense_case(1, 3, 512, 1024, 9)
    W = q4_device_from_host(codes, scales, biases).tiled()
    y = to_np(ops.qmv_k(W, sdev.upload_bf16(x, DEV)))
    perm = np.array([8, 3, 0, 5, 1, 7, 2, 6, 4])
    yp = to_np(ops.qmv_k(W, sdev.upload_bf16(np.ascontiguousarray(x[perm]), DEV)))
    assert np.array_equal(yp, y[perm])


def test_repeat_is_deterministic():
    banner("qmv determinism")
    ops = _ops()
    codes, scales, biases, x = dense_case(1, 4, 2048, 2048, 9)
    W = q4_device_from_host(codes, scales, biases).tiled()
    xd = sdev.upload_bf16(x, DEV)
    a = to_np(ops.qmv_k(W, xd))
    b = to_np(ops.qmv_k(W, xd))
    assert np.array_equal(a, b)


def tile_host(codes, scales, biases, fused):
    """The tiled layout written out from its definition in numpy (layout only)."""
    n, kw = codes.shape
    k = kw * 8
    g = k // 64
    T = (n // 2 + 15) // 16 if fused else (n + 31) // 32
    tc = np.zeros((T, g, 64, 4), dtype=np.uint32)
    tsb = np.zeros((T, g, 32), dtype=np.uint32)
    for t in range(T):
        for c in range(32):
            if fused:
                i = 16 * t + (c % 16)
                if i >= n // 2:
                    continue
                row = i if c < 16 else n // 2 + i
            else:
                row = 32 * t + c
                if row >= n:
                    continue
            for gg in range(g):
                for h in range(2):
                    tc[t, gg, 32 * h + c] = codes[row, 8 * gg + 4 * h: 8 * gg + 4 * h + 4]
                tsb[t, gg, c] = int(scales[row, gg]) | (int(biases[row, gg]) << 16)
    return tc, tsb


@pytest.mark.parametrize("N,K,fused", [(64, 128, False), (70, 192, False), (2 * 40, 128, True), (2 * 17, 64, True)])
def test_repack_layout(N, K, fused):
    banner(f"repack N={N} K={K} fused={fused}")
    codes, scales, biases = synth.dense_weight(0, 9, 1, N, K)
    W = q4_device_from_host(codes, scales, biases)
    Wt = W.tiled(fused_gateup=fused)
    tc, tsb = tile_host(codes, scales, biases, fused)
    got_c = to_np(Wt.codes).view(np.uint32).reshape(tc.shape)
    got_s = to_np(Wt.sb).view(np.uint32).reshape(tsb.shape)
    assert np.array_equal(got_c, tc)
    assert np.array_equal(got_s, tsb)


def test_mode_must_match_layout():
    banner("qmv layout/mode mismatch")
    ops = _ops()
    codes, scales, biases, x = dense_case(0, 8, 64, 128, 2)
    W = q4_device_from_host(codes, scales, biases)
    xd = sdev.upload_bf16(x, DEV)
    with pytest.raises(ops.SdvError, match="fused_gateup=1"):
        ops.qmv_k(W.tiled(False), xd, mode=ops.MODE_GATEUP_SWIGLU)
    with pytest.raises(ops.SdvError, match="fused_gateup=0"):
        ops.qmv_k(W.tiled(True), xd)


MULTI_CASES = [("q4", 0, False, 9, 336, 1024, 5), ("q4", 0, True, 5, 336, 1024, 5), ("q4", 1, False, 9, 320, 1024, 5),
               ("q4", 0, False, 32, 336, 1024, 5), ("q8", 0, False, 9, 336, 1024, 5), ("q3", 0, False, 4, 336, 1024, 5),
               ("q3", 1, False, 20, 320, 1024, 5), ("q8", 0, False, 16, 336, 1024, 5),
               # several (tile, weight) items per workgroup (one staging of the rows for all of them)
               ("q4", 0, False, 9, 2560, 5120, 12), ("q4", 1, False, 7, 5120, 1024, 9),
               ("q4", 0, True, 5, 10240, 512, 5), ("q8", 0, False, 9, 2560, 1024, 12),
               ("q3", 0, False, 9, 2560, 1024, 12),
               # K = 1088: 17 groups over 16 waves, so one wave's K range has two
               # groups and the others one (the step cursors of the several-item form)
               ("q4", 0, False, 9, 2560, 1088, 12), ("q8", 1, False, 5, 2560, 1088, 12),
               # 2560 items: ten per workgroup, as in the 16-weight launches of 5120 x 5120
               ("q4", 0, False, 9, 5120, 1024, 16), ("q4", 0, False, 1, 5120, 1024, 16),
               ("q4", 1, False, 9, 5120, 1024, 16), ("q8", 0, False, 5, 5120, 1024, 16),
               ("q3", 0, False, 9, 5120, 1088, 16)]


@pytest.mark.parametrize("fmt_name,mode,act_f32,k,N,K,nw", MULTI_CASES)
def test_multi_weight_launch_equals_single_calls(fmt_name, mode, act_f32, k, N, K, nw):
    """sdv_qmv_k_multi over several weights of one shape that share the
    activation rows: every output equals its own sdv_qmv_k call bit for bit
    (ragged N, the gate/up mode, fp32 rows, 32 rows, Q8_0, Q3, and launches
    whose workgroups take several (tile, weight) items, in shares that differ
    by one: 2560 x 5120 x 12, 5120 x 1024 x 9, 10240 x 512 x 5, and K ranges
    of different lengths: K = 1088; ten items per workgroup), and the first
    and last weights match the oracle."""
    ops = _ops()
    from speculative_decode_verification_amd.ops import Q3Weight, Q8Weight
    banner(f"qmv multi {fmt_name} mode={mode} f32={act_f32} k={k} N={N} K={K} nw={nw}")
    Ws, refs = [], {}
    x = synth.activations(40, 0, k, K)
    x64 = oracle.bf16_to_f64(x)
    if act_f32:
        x64 = (oracle.bf16_to_f64(x).astype(np.float32) * np.float32(1.25)).astype(np.float64)
    for m in range(nw):
        if fmt_name == "q8":
            qs, d = synth.q8_0_weight(40, DENSE_W, m, 1, N, K)
            W = Q8Weight(torch.from_numpy(np.ascontiguousarray(qs[0])).to(DEV),
                         torch.from_numpy(np.ascontiguousarray(d[0]).view(np.int16)).to(DEV))
            ref = (lambda qs=qs, d=d: oracle.qmv_q8_0(qs[0], d[0], x64))
        elif fmt_name == "q3":
            c, sc, bi, _ = synth.q3_weight(40, DENSE_W, m, 1, N, K)
            W = Q3Weight(torch.from_numpy(np.ascontiguousarray(c[0])).to(DEV),
                         torch.from_numpy(np.ascontiguousarray(sc[0]).view(np.int16)).to(DEV),
                         torch.from_numpy(np.ascontiguousarray(bi[0]).view(np.int16)).to(DEV))
            ref = (lambda c=c, sc=sc, bi=bi: oracle.qmv_q3(c[0], sc[0], bi[0], x64))
        else:
            host = synth.dense_weight(40, DENSE_W, m, N, K)
            W = q4_device_from_host(*host)
            ref = (lambda host=host: oracle.qmv(*host, x64))
        if m in (0, nw - 1):
            refs[m] = ref
        Ws.append(W.tiled(fused_gateup=(mode == 1)))
    xd = sdev.upload_bf16(x, DEV)
    if act_f32:
        xd = torch.from_numpy(x64.astype(np.float32)).to(DEV)
    outs = ops.qmv_k_multi(Ws, xd, mode)
    for m, W in enumerate(Ws):
        single = to_np(ops.qmv_k(W, xd, mode))
        assert np.array_equal(to_np(outs[m]), single), f"weight {m}"
    for m, ref in refs.items():
        r = ref()
        assert_close(to_np(outs[m]), oracle.swiglu(r) if mode == 1 else r, f"multi weight {m}")
    # the bound form gives the same
    for o in outs:
        o.fill_(0.0)
    ops.bind_qmv_k_multi(Ws, xd, mode, outs)()
    torch.cuda.synchronize()
    for m, W in enumerate(Ws):
        assert np.array_equal(to_np(outs[m]), to_np(ops.qmv_k(W, xd, mode))), f"bound, weight {m}"
