"""GPU parity of the layered GDN launch (sdv_gdn_verify_prep_k_layers): a
measurement form that runs several independent GDN layers of one shape, each
preparation + recurrence with snapshots (Flash-Next plan, "2.1 Gated
DeltaNet"), in one launch.  Every layer's y, snapshots and window must equal
its own sdv_gdn_verify_prep_k call's bit for bit."""

import pytest
import torch

import synth
from synth import device as sdev
from tests.gpu_helpers import DEV, banner

pytestmark = pytest.mark.gpu


def _mods():
    from speculative_decode_verification_amd import ops, pipeline
    return ops, pipeline


def _layer(seed, hv, hk, d, k):
    raw = synth.gdn_raw_inputs(seed, hv, k, hv, hk, d, d)
    dd = {n: sdev.upload_f32(v, DEV) for n, v in raw.items()}
    return dd, sdev.upload_f32(synth.gdn_state(seed, hv, hv, d, d), DEV)


def _outputs(S, k, hv, hk, d, fill):
    C = 2 * hk * d + hv * d
    return (torch.full((k, hv, d), fill, device=DEV), [torch.full_like(S, fill) for _ in range(k)],
            torch.full((k + 3, C), fill, device=DEV))


@pytest.mark.parametrize("hv,hk,d", [(48, 16, 128), (3, 1, 128), (8, 2, 64)])
@pytest.mark.parametrize("k", [1, 9, 16])
def test_layers_equal_single_calls(hv, hk, d, k):
    """Three layers (block counts that are and are not multiples of 8, both
    block sizes, narrow and wide widths): the layered launch against each
    layer's own call, and against itself when issued again."""
    ops, _ = _mods()
    banner(f"gdn layers hv={hv} hk={hk} d={d} k={k}")
    layers = [_layer(60 + l, hv, hk, d, k) for l in range(3)]
    ref, got, calls = [], [], []
    for dd, S in layers:
        y, snaps, win = _outputs(S, k, hv, hk, d, 0.0)
        ops.gdn_verify_prep_k(S, dd["qkv"], dd["hist"], dd["conv_w"], dd["a"], dd["b"], dd["A_log"], dd["dt_bias"],
                              hk, snaps, win, y, conv_act=ops.CONV_SILU)
        ref.append((y, snaps, win))
        out = _outputs(S, k, hv, hk, d, float("nan"))
        calls.append(ops.bind_gdn_verify_prep_k(S, dd["qkv"], dd["hist"], dd["conv_w"], dd["a"], dd["b"], dd["A_log"],
                                                dd["dt_bias"], hk, out[1], out[2], out[0], ops.CONV_SILU))
        got.append(out)
    launch = ops.GdnLayersLaunch(calls, DEV)
    for rep in range(2):
        launch()
        torch.cuda.synchronize()
        for l, ((y0, s0, w0), (y1, s1, w1)) in enumerate(zip(ref, got)):
            assert torch.equal(y0, y1), (rep, l)
            assert torch.equal(w0, w1), (rep, l)
            for t in range(k):
                assert torch.equal(s0[t], s1[t]), (rep, l, t)


def test_layers_from_bound_gdn_layers():
    """The step's GDN layers (GdnLayer bound from their projections) in one
    launch through their prepared calls: the same y, snapshots and window as
    running each layer."""
    ops, pipeline = _mods()
    hv, hk, d, k = 48, 16, 128, 9
    banner("gdn layers from bound GdnLayer objects")
    gls = []
    for l in range(4):
        dd, S = _layer(70 + l, hv, hk, d, k)
        gl = pipeline.GdnLayer(S, k).attach_prep(dd["hist"], dd["conv_w"], dd["A_log"], dd["dt_bias"], hk)
        gl.bind_from_proj(dd["qkv"], dd["a"], dd["b"])
        gls.append(gl)
    ref = []
    for gl in gls:
        y = gl.run_from_proj_bound().clone()
        ref.append((y, [gl.slots[i].clone() for i in gl.snap_ids], gl.windows[gl.win][:k + 3].clone()))
        for i in gl.snap_ids:
            gl.slots[i].fill_(float("nan"))
        gl.windows[gl.win].fill_(float("nan"))
        gl.y.fill_(float("nan"))
    launch = ops.GdnLayersLaunch([gl.prep_call() for gl in gls], DEV)
    launch()
    torch.cuda.synchronize()
    for gl, (y, snaps, win) in zip(gls, ref):
        assert torch.equal(gl.y[:k], y)
        assert torch.equal(gl.windows[gl.win][:k + 3], win)
        for i, s in zip(gl.snap_ids, snaps):
            assert torch.equal(gl.slots[i], s)


def test_layers_reject_mixed_shapes():
    ops, _ = _mods()
    a = _layer(80, 8, 2, 64, 2)
    b = _layer(81, 8, 2, 64, 3)
    calls = []
    for (dd, S), k in ((a, 2), (b, 3)):
        y, snaps, win = _outputs(S, k, 8, 2, 64, 0.0)
        calls.append(ops.bind_gdn_verify_prep_k(S, dd["qkv"], dd["hist"], dd["conv_w"], dd["a"], dd["b"], dd["A_log"],
                                                dd["dt_bias"], 2, snaps, win, y))
    with pytest.raises(ValueError):
        ops.GdnLayersLaunch(calls, DEV)
