"""GPU parity of the k-row Gated DeltaNet verify (sdv_gdn_verify_k) and of
rollback by selection: oracle tolerance on y and every snapshot, width-k ==
chained width-1 bit for bit, rollback to every accepted prefix at widths 4,
8 and 9 equal to a fresh j-row run bit for bit, snapshot isolation with guard
bands, and a 16-step chain with random accepted prefixes."""

import numpy as np
import pytest
import torch

import oracle
import synth
from synth import device as sdev
from tests.gpu_helpers import DEV, assert_close, banner, to_np

pytestmark = pytest.mark.gpu


def _ops():
    from speculative_decode_verification_amd import ops
    return ops


def layer_inputs(cfg, layer, k, hv, hk, d, step=0, dv=None):
    dv = d if dv is None else dv
    S = synth.gdn_state(cfg, layer, hv, dv, d)
    inp = synth.gdn_layer_inputs(cfg, layer, k, hv, hk, d, dv, step=step)
    return S, inp


def upload(inp):
    return {n: sdev.upload_f32(v, DEV) for n, v in inp.items()}


def run(ops, S_d, d, rows=None):
    rows = rows or d["q"].shape[0]
    snaps = [torch.empty_like(S_d) for _ in range(rows)]
    y = ops.gdn_verify_k(S_d, *(d[n][:rows].contiguous() for n in ("q", "k", "v", "g", "beta")), snaps)
    return y, snaps


def oracle_run(S, inp, rows=None):
    rows = rows or inp["q"].shape[0]
    return oracle.gdn_verify(S, *(inp[n][:rows] for n in ("q", "k", "v", "g", "beta")))


def compare(y, snaps, ref_y, ref_snaps, what):
    k = ref_y.shape[0]
    for t in range(k):
        assert_close(to_np(y[t]), ref_y[t], f"{what} y row {t}")
        assert_close(to_np(snaps[t]), ref_snaps[t], f"{what} snapshot {t}")


def test_tiny_layer_and_rollback_to_prefix_1():
    banner("gdn tiny Hv=Hk=4 D=64 k=2")
    ops = _ops()
    S, inp = layer_inputs(0, 0, 2, 4, 4, 64)
    S_d, d = sdev.upload_f32(S, DEV), upload(inp)
    y, snaps = run(ops, S_d, d)
    ref_y, ref_s = oracle_run(S, inp)
    compare(y, snaps, ref_y, ref_s, "tiny")
    slot = ops.gdn_rollback(2, 1)
    assert slot == 1
    st = torch.empty_like(S_d)
    ops.gdn_rollback_copy(st, S_d, snaps, 1)
    assert_close(to_np(st), oracle.rollback(S, ref_s, 1), "rollback to prefix 1")


@pytest.mark.parametrize("hv,hk,d,dv", [(48, 16, 128, 128), (4, 1, 64, 64), (6, 2, 128, 128), (5, 5, 64, 64),
                                        (3, 1, 64, 40), (2, 2, 128, 7)])
def test_layer_matches_oracle(hv, hk, d, dv):
    banner(f"gdn layer Hv={hv} Hk={hk} Dk={d} Dv={dv} k=9")
    ops = _ops()
    S, inp = layer_inputs(3, 1, 9, hv, hk, d, dv=dv)
    S_d, dd = sdev.upload_f32(S, DEV), upload(inp)
    y, snaps = run(ops, S_d, dd)
    ref_y, ref_s = oracle_run(S, inp)
    compare(y, snaps, ref_y, ref_s, f"Hv={hv}")
    for t in range(9):
        err = np.abs(to_np(snaps[t]).astype(np.float64) - ref_s[t]).reshape(hv, -1).max(axis=1) / \
            np.abs(ref_s[t]).reshape(hv, -1).max(axis=1)
        assert np.all(err <= 1e-5), f"per-head snapshot error {err.max():.2e} at row {t}"


def test_width_k_equals_chained_width_1():
    banner("gdn width-k vs chained width-1")
    ops = _ops()
    S, inp = layer_inputs(3, 2, 9, 48, 16, 128)
    S_d, d = sdev.upload_f32(S, DEV), upload(inp)
    y9, s9 = run(ops, S_d, d)
    state = S_d
    for t in range(9):
        one = {n: v[t:t + 1].contiguous() for n, v in d.items()}
        y1, s1 = run(ops, state, one)
        assert torch.equal(y1[0], y9[t]), f"y row {t}"
        assert torch.equal(s1[0], s9[t]), f"snapshot {t}"
        state = s1[0]
    for k in range(1, 9):
        yk, sk = run(ops, S_d, d, rows=k)
        assert torch.equal(yk, y9[:k])
        assert torch.equal(sk[-1], s9[k - 1])


@pytest.mark.parametrize("k", [4, 8, 9])
def test_rollback_every_prefix(k):
    banner(f"gdn rollback every prefix k={k}")
    ops = _ops()
    S, inp = layer_inputs(3, 10 + k, k, 48, 16, 128)
    S_d, d = sdev.upload_f32(S, DEV), upload(inp)
    S_before = S_d.clone()
    # snapshots inside guard bands
    n = S_d.numel()
    pad = 4096
    guards = [torch.full((n + 2 * pad,), 1234.5, dtype=torch.float32, device=DEV) for _ in range(k)]
    snaps = [g[pad:pad + n].view_as(S_d) for g in guards]
    y = ops.gdn_verify_k(S_d, d["q"], d["k"], d["v"], d["g"], d["beta"], snaps)
    assert torch.equal(S_d, S_before), "input state modified"
    for g in guards:
        assert torch.all(g[:pad] == 1234.5) and torch.all(g[pad + n:] == 1234.5), "guard band written"
    for j in range(k + 1):
        dst = torch.empty_like(S_d)
        ops.gdn_rollback_copy(dst, S_d, snaps, j)
        if j == 0:
            assert torch.equal(dst, S_before)
            continue
        _, fresh = run(ops, S_d, d, rows=j)
        assert torch.equal(dst, fresh[-1]), f"rollback to {j} differs from a fresh {j}-row run"
    ref_y, ref_s = oracle_run(S, inp)
    compare(y, snaps, ref_y, ref_s, f"k={k}")


def test_sixteen_step_chain_with_rollback():
    """Per step: verify k rows, draw the accepted prefix j, roll back by
    selection.  The oracle runs the same chain in fp64 from the same inputs."""
    ops = _ops()
    from speculative_decode_verification_amd.pipeline import GdnLayer
    hv, hk, dd = 48, 16, 128
    S = synth.gdn_state(3, 20, hv, dd, dd)
    ref_state = S.astype(np.float64)
    for k in (1, 5, 9):
        banner(f"gdn 16-step chain k={k}")
        layer = GdnLayer(sdev.upload_f32(S, DEV), k)
        ref_state = S.astype(np.float64)
        for step in range(16):
            inp = synth.gdn_layer_inputs(3, 20, k, hv, hk, dd, dd, step=step)
            d = upload(inp)
            y = layer.verify(d["q"], d["k"], d["v"], d["g"], d["beta"])
            ry, rs = oracle.gdn_verify(ref_state, inp["q"], inp["k"], inp["v"], inp["g"], inp["beta"])
            assert_close(to_np(y), ry, f"chain k={k} step {step} y")
            j = synth.accepted_prefix(3, step, k)
            layer.rollback(j)
            ref_state = oracle.rollback(ref_state, rs, j)
        assert_close(to_np(layer.state)[None], ref_state[None], f"chain k={k} final state")


def test_device_fill_matches_host_generator():
    banner("synth device fill")
    keys = synth.bank_keys(4, 1, 3)
    c, s, b = sdev.q4_bank(keys, 3, 40, 256, DEV)
    for e in range(3):
        hc, hs, hb = synth.q4_rows(keys, 3, 40, 256, expert=e)
        assert np.array_equal(to_np(c[e]).view(np.uint32), hc)
        assert np.array_equal(to_np(s[e]).view(np.uint16), hs)
        assert np.array_equal(to_np(b[e]).view(np.uint16), hb)
