"""GPU parity of sdv_gdn_verify_prep_norm_k: the preparation, the recurrence
and the gated output norm of one GDN layer in one launch (Flash-Next plan,
"2.1 Gated DeltaNet": conv, q/k norm and gates, the delta-rule recurrence,
then the gated RMSNorm).  y, the snapshots, the window and the normed output
equal sdv_gdn_verify_prep_k followed by sdv_gdn_gated_norm_k bit for bit,
and the output matches the oracle within tolerance.  The per-head counters
are zero after every call, so calls in a row (also at a smaller width) need
no reset."""

import numpy as np
import pytest
import torch

import oracle
import synth
from synth import device as sdev
from tests.gpu_helpers import DEV, assert_close, banner, to_np

pytestmark = pytest.mark.gpu

ACTS = {"none": 0, "silu": 1}
GATES = {"sigmoid": 0, "silu": 1}


def _ops():
    from speculative_decode_verification_amd import ops
    return ops


def separate_and_fused(ops, raw, S_d, hk, d, act, gate, counters):
    dd = {n: sdev.upload_f32(v, DEV) for n, v in raw.items()}
    k = raw["qkv"].shape[0]
    snaps_a = [torch.empty_like(S_d) for _ in range(k)]
    win_a = torch.empty((k + 3, raw["qkv"].shape[1]), dtype=torch.float32, device=DEV)
    y_a = ops.gdn_verify_prep_k(S_d, dd["qkv"], dd["hist"], dd["conv_w"], dd["a"], dd["b"], dd["A_log"],
                                dd["dt_bias"], hk, snaps_a, win_a, conv_act=ACTS[act])
    out_a = ops.gdn_gated_norm_k(y_a, dd["z"], dd["norm_w"], GATES[gate])
    snaps_b = [torch.full_like(S_d, float("nan")) for _ in range(k)]
    win_b = torch.full_like(win_a, float("nan"))
    out_b = torch.full_like(out_a, float("nan"))
    y_b, _ = ops.gdn_verify_prep_norm_k(S_d, dd["qkv"], dd["hist"], dd["conv_w"], dd["a"], dd["b"], dd["A_log"],
                                        dd["dt_bias"], hk, snaps_b, win_b, dd["z"], dd["norm_w"], counters,
                                        out=out_b, conv_act=ACTS[act], gate_act=GATES[gate])
    torch.cuda.synchronize()
    assert torch.equal(y_a, y_b)
    assert torch.equal(win_a, win_b)
    for t in range(k):
        assert torch.equal(snaps_a[t], snaps_b[t]), t
    assert torch.equal(out_a, out_b)
    assert not counters.any(), "the counters must be left zero"
    return out_b


@pytest.mark.parametrize("hv,hk,d", [(48, 16, 128), (4, 4, 64), (8, 2, 64), (6, 2, 128)])
@pytest.mark.parametrize("act,gate", [("none", "sigmoid"), ("silu", "silu")])
@pytest.mark.parametrize("k", [1, 4, 9])
def test_prep_norm_equals_separate_calls(hv, hk, d, act, gate, k):
    ops = _ops()
    banner(f"gdn verify+prep+norm hv={hv} hk={hk} d={d} act={act} gate={gate} k={k}")
    raw = synth.gdn_raw_inputs(47, hv, k, hv, hk, d, d)
    S = synth.gdn_state(47, hv, hv, d, d)
    counters = ops.gdn_norm_counters(hv, DEV)
    out = separate_and_fused(ops, raw, sdev.upload_f32(S, DEV), hk, d, act, gate, counters)
    ref = oracle.gdn_prepare(raw["qkv"], raw["hist"], raw["conv_w"], raw["a"], raw["b"], raw["A_log"],
                             raw["dt_bias"], hk, hv, d, d, act)
    y_ref, _ = oracle.gdn_verify(S, ref["q"], ref["k"], ref["v"], ref["g"], ref["beta"])
    assert_close(to_np(out), oracle.gdn_gated_norm(y_ref, raw["z"], raw["norm_w"], gate), "normed output")


def test_prep_norm_wide_and_back_to_back():
    """Widths 16 and 32 (the wide instantiation), then 9 and 1 on the same
    counters: every call equals the separate calls and leaves them zero."""
    ops = _ops()
    hv, hk, d = 48, 16, 128
    S_d = sdev.upload_f32(synth.gdn_state(48, hv, hv, d, d), DEV)
    counters = ops.gdn_norm_counters(hv, DEV)
    for k in (16, 32, 9, 1):
        banner(f"gdn verify+prep+norm k={k}")
        raw = synth.gdn_raw_inputs(48, k, k, hv, hk, d, d)
        separate_and_fused(ops, raw, S_d, hk, d, "none", "sigmoid", counters)


def test_layer_from_proj_norm_bound_steps():
    """GdnLayer.bind_from_proj_norm over steps with rollback: each step's
    output equals a layer run with the separate norm launch."""
    from speculative_decode_verification_amd import pipeline
    ops = _ops()
    hv, hk, d, k = 8, 2, 64, 9
    banner("gdn layer bound prep+norm steps")
    S0 = sdev.upload_f32(synth.gdn_state(49, 0, hv, d, d), DEV)
    raw = synth.gdn_raw_inputs(49, 0, k, hv, hk, d, d)
    dd = {n: sdev.upload_f32(v, DEV) for n, v in raw.items()}
    la = pipeline.GdnLayer(S0, k).attach_prep(dd["hist"], dd["conv_w"], dd["A_log"], dd["dt_bias"], hk)
    lb = pipeline.GdnLayer(S0, k).attach_prep(dd["hist"], dd["conv_w"], dd["A_log"], dd["dt_bias"], hk)
    out_a = torch.empty((k, hv, d), dtype=torch.float32, device=DEV)
    out_b = torch.empty_like(out_a)
    lb.bind_from_proj_norm(dd["qkv"], dd["a"], dd["b"], dd["z"], dd["norm_w"], out_b)
    for step, j in enumerate((3, 9, 0, 5)):
        ya = la.verify_from_proj(dd["qkv"], dd["a"], dd["b"])
        ops.gdn_gated_norm_k(ya, dd["z"], dd["norm_w"], out=out_a)
        lb.run_from_proj_bound()
        torch.cuda.synchronize()
        assert torch.equal(out_a, out_b), step
        assert torch.equal(la.state, lb.state), step
        la.rollback(j)
        lb.rollback(j)
