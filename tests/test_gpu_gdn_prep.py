"""GPU parity of the GDN preparation and output norm (sdv_gdn_prepare_k,
sdv_gdn_gated_norm_k) against the oracle: the window bit-exact (it is a copy
of the inputs), q, k, v, g, beta and the normed output within the per-row
normwise tolerance; every width-k row bit-identical to the width-1 call on
the same inputs; the conv history carried across verify steps by selecting
rows of the window; and a whole layer (prepare, recurrence, output norm)
over several steps with rollback, against the oracle run on the accepted
stream."""

import numpy as np
import pytest
import torch

import oracle
import synth
from synth import device as sdev
from tests.gpu_helpers import DEV, assert_close, banner, to_np

pytestmark = pytest.mark.gpu

# (hv, hk, d): the 48/16/128 heads of the hybrid model's GDN layers
# (Flash-Next plan, "5.1 Gated DeltaNet"), a 1:1 head map, and 64-wide heads.
SHAPES = [(48, 16, 128), (4, 4, 64), (8, 2, 64)]
ACTS = {"none": 0, "silu": 1}


def _ops():
    from speculative_decode_verification_amd import ops
    return ops


def upload(raw):
    return {n: sdev.upload_f32(v, DEV) for n, v in raw.items()}


def run_prepare(ops, d, hk, dk, act, eps=1e-6, hist=None):
    out = ops.gdn_prepare_k(d["qkv"], d["hist"] if hist is None else hist, d["conv_w"], d["a"], d["b"],
                            d["A_log"], d["dt_bias"], hk, dk, ACTS[act], eps)
    torch.cuda.synchronize()
    return {n: to_np(t) for n, t in out.items()}


def check_prepare(got, raw, hv, hk, d, act, eps=1e-6, hist=None):
    ref = oracle.gdn_prepare(raw["qkv"], raw["hist"] if hist is None else hist, raw["conv_w"], raw["a"], raw["b"],
                             raw["A_log"], raw["dt_bias"], hk, hv, d, d, act, eps)
    assert np.array_equal(got["window"], ref["window"].astype(np.float32))
    for n in ("q", "k", "v", "g", "beta"):
        assert_close(got[n], ref[n], n)
    return ref


@pytest.mark.parametrize("hv,hk,d", SHAPES)
@pytest.mark.parametrize("act", ["none", "silu"])
@pytest.mark.parametrize("k", [1, 2, 5, 9])
def test_prepare_parity(hv, hk, d, act, k):
    ops = _ops()
    banner(f"gdn prepare hv={hv} hk={hk} d={d} act={act} k={k}")
    raw = synth.gdn_raw_inputs(40, hv, k, hv, hk, d, d)
    got = run_prepare(ops, upload(raw), hk, d, act)
    check_prepare(got, raw, hv, hk, d, act)


@pytest.mark.parametrize("hv,hk,d", SHAPES[:2])
def test_prepare_width_rows_match_width_one(hv, hk, d):
    """Row t of a width-9 call equals the width-1 call whose history is
    window rows t..t+2 and whose input is row t, bit for bit."""
    ops = _ops()
    banner(f"gdn prepare width invariance hv={hv} d={d}")
    k = 9
    raw = synth.gdn_raw_inputs(41, 0, k, hv, hk, d, d)
    dd = upload(raw)
    full = run_prepare(ops, dd, hk, d, "silu")
    win = dd["qkv"].new_empty((k + 3, dd["qkv"].shape[1]))
    win.copy_(torch.from_numpy(full["window"]).to(DEV))
    for t in range(k):
        one = dict(dd, qkv=dd["qkv"][t:t + 1].contiguous(), a=dd["a"][t:t + 1].contiguous(),
                   b=dd["b"][t:t + 1].contiguous())
        got = run_prepare(ops, one, hk, d, "silu", hist=win[t:t + 3])
        for n in ("q", "k", "v", "g", "beta"):
            assert np.array_equal(got[n][0], full[n][t]), (n, t)


def test_prepare_degenerate_rows():
    """A zero row gives zero q and k (0 / sqrt(eps)); eps = 0 still divides
    a nonzero row by its norm; large inputs stay finite."""
    ops = _ops()
    banner("gdn prepare degenerate rows")
    hv, hk, d, k = 4, 4, 64, 4
    raw = synth.gdn_raw_inputs(42, 0, k, hv, hk, d, d)
    raw["hist"][:] = 0.0
    raw["qkv"][0] = 0.0
    raw["qkv"][2] *= np.float32(1e15)
    raw["a"][1] = np.float32(80.0)     # softplus ~ a: g underflows toward 0
    raw["a"][3] = np.float32(-80.0)    # softplus ~ e^a: g ~ 1
    raw["b"][1] = np.float32(-60.0)    # beta ~ 1e-26
    for eps in (1e-6, 0.0):
        got = run_prepare(ops, upload(raw), hk, d, "none", eps=eps)
        if eps > 0:
            assert not got["q"][0].any() and not got["k"][0].any()
        else:
            assert np.isnan(got["q"][0]).all()   # 0 / 0, as the oracle computes it
        rows = [1, 2, 3] if eps == 0.0 else [0, 1, 2, 3]
        ref = oracle.gdn_prepare(raw["qkv"], raw["hist"], raw["conv_w"], raw["a"], raw["b"], raw["A_log"],
                                 raw["dt_bias"], hk, hv, d, d, "none", eps)
        for n in ("q", "k", "v", "g", "beta"):
            assert_close(got[n][rows], ref[n][rows], f"{n} eps={eps}")
        assert np.isfinite(got["q"][2]).all()


@pytest.mark.parametrize("hv,hk,d", SHAPES)
def test_conv_history_carried_by_selection(hv, hk, d):
    """Three verify steps; after each, j rows are accepted and rows j..j+2 of
    the window become the next step's history (a view, no copy).  Every step
    matches the oracle run with the history of the accepted stream."""
    ops = _ops()
    banner(f"gdn prepare history chain hv={hv} d={d}")
    k = 9
    hist_dev = None
    stream = None
    wins = []
    for step, j in enumerate([4, 1, 9]):
        raw = synth.gdn_raw_inputs(43, 0, k, hv, hk, d, d, step=step)
        if stream is None:
            stream = raw["hist"].astype(np.float64)
        dd = upload(raw)
        out = ops.gdn_prepare_k(dd["qkv"], dd["hist"] if hist_dev is None else hist_dev, dd["conv_w"], dd["a"],
                                dd["b"], dd["A_log"], dd["dt_bias"], hk, d, 1)
        torch.cuda.synchronize()
        got = {n: to_np(t) for n, t in out.items()}
        check_prepare(got, raw, hv, hk, d, "silu", hist=stream[-3:].astype(np.float32))
        stream = np.concatenate([stream, raw["qkv"][:j].astype(np.float64)])
        wins.append(out["window"])             # keep the window alive while its rows are the history
        hist_dev = out["window"][j:j + 3]


@pytest.mark.parametrize("hv,d", [(48, 128), (4, 64)])
@pytest.mark.parametrize("act", ["sigmoid", "silu"])
@pytest.mark.parametrize("k", [1, 9])
def test_gated_norm_parity(hv, d, act, k):
    ops = _ops()
    banner(f"gdn gated norm hv={hv} d={d} act={act} k={k}")
    raw = synth.gdn_raw_inputs(44, 0, k, hv, hv, d, d)
    y = synth.gdn_layer_inputs(44, 0, k, hv, hv, d, d)["v"]
    y[0, 0] = 0.0                                        # a zero head: output zero
    out = ops.gdn_gated_norm_k(sdev.upload_f32(y, DEV), sdev.upload_f32(raw["z"], DEV),
                               sdev.upload_f32(raw["norm_w"], DEV), {"sigmoid": 0, "silu": 1}[act])
    torch.cuda.synchronize()
    got = to_np(out)
    ref = oracle.gdn_gated_norm(y, raw["z"], raw["norm_w"], act)
    assert_close(got, ref, "gated norm")
    assert not got[0, 0].any()
    # every row equals its width-1 call, bit for bit
    if k > 1:
        for t in (0, k - 1):
            one = ops.gdn_gated_norm_k(sdev.upload_f32(y[t:t + 1], DEV), sdev.upload_f32(raw["z"][t:t + 1], DEV),
                                       sdev.upload_f32(raw["norm_w"], DEV), {"sigmoid": 0, "silu": 1}[act])
            torch.cuda.synchronize()
            assert np.array_equal(to_np(one)[0], got[t])


def test_layer_steps_with_rollback():
    """A whole GDN layer from its projections over four verify steps:
    prepare, recurrence with snapshots, output norm; after each step the
    accepted prefix becomes the state and the conv history.  Outputs of the
    rows of each step and the live state after it match the oracle run over
    the accepted stream."""
    from speculative_decode_verification_amd import pipeline
    banner("gdn layer steps with rollback")
    hv, hk, d, k = 48, 16, 128, 9
    S = synth.gdn_state(45, 0, hv, d, d)
    raw0 = synth.gdn_raw_inputs(45, 0, k, hv, hk, d, d)
    layer = pipeline.GdnLayer(sdev.upload_f32(S, DEV), k)
    layer.attach_prep(sdev.upload_f32(raw0["hist"], DEV), sdev.upload_f32(raw0["conv_w"], DEV),
                      sdev.upload_f32(raw0["A_log"], DEV), sdev.upload_f32(raw0["dt_bias"], DEV), hk,
                      conv_act=1)
    ops = _ops()
    norm_w = sdev.upload_f32(raw0["norm_w"], DEV)
    S_ref = S.astype(np.float64)
    hist_ref = raw0["hist"].astype(np.float64)
    for step, (rows, j) in enumerate([(9, 3), (5, 5), (9, 0), (1, 1)]):
        raw = synth.gdn_raw_inputs(45, 0, rows, hv, hk, d, d, step=step + 1)
        dd = upload(raw)
        p = layer.prepare(dd["qkv"], dd["a"], dd["b"])
        y = layer.verify(p["q"], p["k"], p["v"], p["g"], p["beta"])
        o = ops.gdn_gated_norm_k(y, dd["z"], norm_w, 0)
        torch.cuda.synchronize()
        ref = oracle.gdn_prepare(raw["qkv"], hist_ref, raw["conv_w"], raw["a"], raw["b"], raw["A_log"],
                                 raw["dt_bias"], hk, hv, d, d, "silu")
        y_ref, snaps = oracle.gdn_verify(S_ref, ref["q"], ref["k"], ref["v"], ref["g"], ref["beta"])
        assert_close(to_np(y), y_ref, f"step {step} y")
        assert_close(to_np(o), oracle.gdn_gated_norm(y_ref, raw["z"], raw["norm_w"]), f"step {step} out")
        live = layer.rollback(j)
        if j > 0:
            S_ref = snaps[j - 1]
        hist_ref = ref["window"][j:j + 3]
        assert_close(to_np(live)[None], S_ref[None], f"step {step} state after {j} rows")
        assert np.array_equal(to_np(layer.hist), hist_ref.astype(np.float32))


@pytest.mark.parametrize("hv,hk,d", SHAPES + [(3, 1, 64), (6, 2, 128)])
@pytest.mark.parametrize("act", ["none", "silu"])
@pytest.mark.parametrize("k", [1, 4, 9])
def test_fused_prep_equals_separate_calls(hv, hk, d, act, k):
    """sdv_gdn_verify_prep_k: y, every snapshot and the window equal the
    preparation followed by the recurrence, bit for bit, and the oracle
    within tolerance (head counts whose block count is and is not a multiple
    of 8, so both block placements run)."""
    ops = _ops()
    banner(f"gdn verify+prep hv={hv} hk={hk} d={d} act={act} k={k}")
    raw = synth.gdn_raw_inputs(46, hv, k, hv, hk, d, d)
    S = synth.gdn_state(46, hv, hv, d, d)
    dd = upload(raw)
    S_d = sdev.upload_f32(S, DEV)
    p = ops.gdn_prepare_k(dd["qkv"], dd["hist"], dd["conv_w"], dd["a"], dd["b"], dd["A_log"], dd["dt_bias"], hk, d,
                          ACTS[act])
    snaps_a = [torch.empty_like(S_d) for _ in range(k)]
    y_a = ops.gdn_verify_k(S_d, p["q"], p["k"], p["v"], p["g"], p["beta"], snaps_a)
    snaps_b = [torch.full_like(S_d, float("nan")) for _ in range(k)]
    win_b = torch.full_like(p["window"], float("nan"))
    y_b = ops.gdn_verify_prep_k(S_d, dd["qkv"], dd["hist"], dd["conv_w"], dd["a"], dd["b"], dd["A_log"],
                                dd["dt_bias"], hk, snaps_b, win_b, conv_act=ACTS[act])
    torch.cuda.synchronize()
    assert torch.equal(y_a, y_b)
    assert torch.equal(p["window"], win_b)
    for t in range(k):
        assert torch.equal(snaps_a[t], snaps_b[t]), t
    ref = oracle.gdn_prepare(raw["qkv"], raw["hist"], raw["conv_w"], raw["a"], raw["b"], raw["A_log"],
                             raw["dt_bias"], hk, hv, d, d, act)
    y_ref, s_ref = oracle.gdn_verify(S, ref["q"], ref["k"], ref["v"], ref["g"], ref["beta"])
    assert_close(to_np(y_b), y_ref, "y")
    assert_close(np.stack([to_np(s) for s in snaps_b]), np.stack(s_ref), "snapshots")


def test_fused_layer_steps_with_rollback():
    """The layer's one-launch path over four steps (bound calls), against the
    oracle run on the accepted stream, and against the two-launch path bit
    for bit."""
    from speculative_decode_verification_amd import pipeline
    banner("gdn fused layer steps with rollback")
    hv, hk, d, k = 48, 16, 128, 9
    S = synth.gdn_state(47, 0, hv, d, d)
    raw0 = synth.gdn_raw_inputs(47, 0, k, hv, hk, d, d)
    mk = lambda: pipeline.GdnLayer(sdev.upload_f32(S, DEV), k).attach_prep(
        sdev.upload_f32(raw0["hist"], DEV), sdev.upload_f32(raw0["conv_w"], DEV), sdev.upload_f32(raw0["A_log"], DEV),
        sdev.upload_f32(raw0["dt_bias"], DEV), hk)
    fused, split = mk(), mk()
    S_ref = S.astype(np.float64)
    hist_ref = raw0["hist"].astype(np.float64)
    bufs = {n: torch.empty_like(t) for n, t in upload(raw0).items()}
    fused.bind_from_proj(bufs["qkv"], bufs["a"], bufs["b"])
    for step, j in enumerate([3, 9, 0, 6, 1]):
        raw = synth.gdn_raw_inputs(47, 0, k, hv, hk, d, d, step=step + 1)
        for n, t in upload(raw).items():
            bufs[n].copy_(t)
        y = fused.run_from_proj_bound()
        p = split.prepare(bufs["qkv"], bufs["a"], bufs["b"])
        y2 = split.verify(p["q"], p["k"], p["v"], p["g"], p["beta"])
        torch.cuda.synchronize()
        assert torch.equal(y, y2), step
        ref = oracle.gdn_prepare(raw["qkv"], hist_ref, raw["conv_w"], raw["a"], raw["b"], raw["A_log"],
                                 raw["dt_bias"], hk, hv, d, d)
        y_ref, snaps = oracle.gdn_verify(S_ref, ref["q"], ref["k"], ref["v"], ref["g"], ref["beta"])
        assert_close(to_np(y), y_ref, f"step {step} y")
        live, live2 = fused.rollback(j), split.rollback(j)
        assert torch.equal(live, live2)
        assert torch.equal(fused.hist, split.hist)
        if j > 0:
            S_ref = snaps[j - 1]
        hist_ref = ref["window"][j:j + 3]
        assert_close(to_np(live)[None], S_ref[None], f"step {step} state after {j} rows")
        assert np.array_equal(to_np(fused.hist), hist_ref.astype(np.float32))
