"""GPU parity of the acceptance of a verified block (sdv_verify_accept_k):
sampled tokens and the accepted draft count bit-exact against the oracle for
greedy and Gumbel sampling, over ragged and full vocabulary sizes, ties,
NaN, signed zeros and infinities, the end-of-answer rule, every width, and a
verify cycle that rolls GDN layers back to the accepted prefix."""

import numpy as np
import pytest
import torch

import oracle
import synth
from synth import device as sdev
from tests.gpu_helpers import DEV, banner, to_np

pytestmark = pytest.mark.gpu

VOCAB = 248320  # Flash-Next plan, "1. Target model and identity": vocab 248,320 (padded)


def _ops():
    from speculative_decode_verification_amd import ops
    return ops


def run(ops, logits, drafts, noise=None, inv_temp=1.0, eos=-1):
    k = logits.shape[0]
    l = sdev.upload_f32(logits, DEV)
    d = torch.from_numpy(np.ascontiguousarray(drafts, dtype=np.int32)).to(DEV) if k > 1 else \
        torch.zeros(1, dtype=torch.int32, device=DEV)
    n = sdev.upload_f32(noise, DEV) if noise is not None else None
    tok, acc = ops.verify_accept_k(l, d, n, inv_temp, eos)
    torch.cuda.synchronize()
    return to_np(tok), int(to_np(acc)[0])


def check(ops, logits, drafts, noise=None, inv_temp=1.0, eos=-1):
    tok, n = run(ops, logits, drafts, noise, inv_temp, eos)
    ref_tok = oracle.sample_tokens(logits, noise, inv_temp)
    ref_n = oracle.accept(ref_tok, drafts, eos)
    assert np.array_equal(tok, ref_tok), (tok, ref_tok)
    assert n == ref_n, (n, ref_n)
    return n


@pytest.mark.parametrize("k", [1, 2, 4, 8, 9])
@pytest.mark.parametrize("V", [1, 37, 4095, 4096, 4097, 100003])
def test_greedy_every_prefix(k, V):
    ops = _ops()
    banner(f"accept greedy k={k} V={V}")
    seen = set()
    for planted in range(k):
        logits, drafts, _ = synth.verify_block(30, 100 * V + planted, k, V, accepted=planted)
        n = check(ops, logits, drafts)
        if V > 1:
            assert n == planted
        seen.add(n)
    assert V == 1 or seen == set(range(k))


def test_full_vocabulary():
    ops = _ops()
    banner(f"accept greedy k=9 V={VOCAB}")
    for step in range(4):
        logits, drafts, planted = synth.verify_block(31, step, 9, VOCAB)
        assert check(ops, logits, drafts) == planted


@pytest.mark.parametrize("V", [64, 5000, VOCAB])
def test_gumbel_sampling(V):
    """Drafts follow the oracle's sampled tokens for a prefix, then differ."""
    ops = _ops()
    banner(f"accept gumbel V={V}")
    k = 9
    for step, inv_temp in enumerate([1.0, 0.6, 1.7]):
        logits, _, _ = synth.verify_block(32, step, k, V, accepted=0)
        noise = synth.gumbel_noise(32, step, k, V)
        toks = oracle.sample_tokens(logits, noise, inv_temp)
        for planted in (0, 3, 8):
            drafts = toks[:k - 1].copy()
            if planted < k - 1:
                drafts[planted] = (drafts[planted] + 1) % V
            assert check(ops, logits, drafts, noise, inv_temp) == planted


def test_ties_nan_signed_zero_inf():
    ops = _ops()
    banner("accept ties / NaN / signed zero / inf")
    nan, inf = np.float32("nan"), np.float32("inf")
    V = 9000
    rng = np.random.default_rng(3)
    logits = rng.integers(-2, 3, size=(9, V)).astype(np.float32)  # massive ties
    logits[1, :] = nan
    logits[2, :] = -0.0
    logits[2, 5000] = 0.0
    logits[3, 4096:] = nan
    logits[4, [100, 8000]] = inf
    logits[5, :] = -inf
    logits[6, 4095:4097] = 50.0                                    # tie across chunks
    logits[7, ::2] = nan
    toks = oracle.sample_tokens(logits)
    assert toks[1] == -1 and toks[2] == 0 and toks[4] == 100 and toks[5] == 0 and toks[6] == 4095
    drafts = toks[:8].copy()
    assert check(ops, logits, drafts) == 8
    drafts[1] = 0                       # row 1 sampled -1 (no number): a real token never matches
    assert check(ops, logits, drafts) == 1


def test_end_of_answer_rejected():
    ops = _ops()
    banner("accept end-of-answer")
    V, k = 5000, 6
    logits, drafts, _ = synth.verify_block(33, 0, k, V, accepted=k - 1)
    eos = int(drafts[2])
    assert check(ops, logits, drafts, eos=eos) == 2
    assert check(ops, logits, drafts, eos=-1) == k - 1
    eos0 = int(drafts[0])
    assert check(ops, logits, drafts, eos=eos0) == 0


def test_bound_call_repeats():
    ops = _ops()
    banner("accept bound call")
    k, V = 9, 30000
    logits, drafts, planted = synth.verify_block(34, 0, k, V, accepted=5)
    l = sdev.upload_f32(logits, DEV)
    d = torch.from_numpy(drafts).to(DEV)
    tok = torch.full((k,), -7, dtype=torch.int32, device=DEV)
    acc = torch.full((1,), -7, dtype=torch.int32, device=DEV)
    ws = ops.verify_accept_workspace(k, V, DEV)
    call = ops.bind_verify_accept_k(l, d, tok, acc, ws)
    for _ in range(3):
        call()
    torch.cuda.synchronize()
    assert np.array_equal(to_np(tok), oracle.sample_tokens(logits))
    assert int(to_np(acc)[0]) == planted == 5


def test_verify_cycle_rolls_gdn_back():
    """A verify step of two GDN layers, then the cycle: every layer's live
    state equals the state after the accepted prefix (the GPU snapshot of row
    n, and within tolerance of the oracle's run over rows 0..n)."""
    from speculative_decode_verification_amd import pipeline
    from tests.gpu_helpers import assert_close
    banner("verify cycle with GDN rollback")
    k, V, hv, hk, d = 9, 20000, 8, 4, 64
    layers, inputs, states = [], [], []
    for li in range(2):
        S = synth.gdn_state(35, li, hv, d, d)
        inp = synth.gdn_layer_inputs(35, li, k, hv, hk, d, d)
        layers.append(pipeline.GdnLayer(sdev.upload_f32(S, DEV), k))
        inputs.append({n: sdev.upload_f32(v, DEV) for n, v in inp.items()})
        states.append((S, inp))
    cycle = pipeline.VerifyCycle(layers, k, V, DEV)
    for step, planted in enumerate([4, 0, 8]):
        starts = [to_np(layer.state).copy() for layer in layers]
        for layer, dd in zip(layers, inputs):
            layer.verify(dd["q"], dd["k"], dd["v"], dd["g"], dd["beta"])
        snaps = [[to_np(layer.slots[i]).copy() for i in layer.snap_ids] for layer in layers]
        logits, drafts, _ = synth.verify_block(35, step, k, V, accepted=planted)
        n, emitted = cycle(sdev.upload_f32(logits, DEV), torch.from_numpy(drafts).to(DEV))
        ref = oracle.verify_cycle(logits, drafts)
        assert n == ref["accepted"] == planted
        assert emitted == ref["emitted"]
        for li, layer in enumerate(layers):
            live = to_np(layer.state)
            assert np.array_equal(live, snaps[li][n])
            _, inp = states[li]
            _, rs = oracle.gdn_verify(starts[li], *(inp[m][:n + 1] for m in ("q", "k", "v", "g", "beta")))
            assert_close(live[None], rs[-1][None], f"layer {li} state after prefix {n + 1}")


def test_verify_cycle_deferred_rollback_equals_eager():
    """``VerifyCycle(..., defer=True)`` leaves each layer's rollback to its
    next run: over a chain of steps with varied accepted counts, from the
    projections (conv history rolled back with the state), every output and
    live state equals the eager cycle's bit for bit."""
    from speculative_decode_verification_amd import pipeline
    banner("verify cycle, deferred rollback")
    k, V, hv, hk, d = 9, 20000, 8, 4, 64
    C = 2 * hk * d + hv * d
    rng = np.random.default_rng(77)
    S0 = synth.gdn_state(36, 0, hv, d, d)
    hist = rng.standard_normal((3, C)).astype(np.float32)
    conv_w = (0.5 * rng.standard_normal((C, 4))).astype(np.float32)
    A_log = rng.standard_normal(hv).astype(np.float32)
    dt_bias = rng.standard_normal(hv).astype(np.float32)
    up = lambda a: sdev.upload_f32(a, DEV)
    runs = {}
    for defer in (False, True):
        layers = [pipeline.GdnLayer(up(S0), k).attach_prep(up(hist), up(conv_w), up(A_log), up(dt_bias), hk)
                  for _ in range(2)]
        cycle = pipeline.VerifyCycle(layers, k, V, DEV)
        ys, states = [], []
        for step, planted in enumerate([3, 0, 8, 5, 1]):
            srng = np.random.default_rng(100 + step)
            for layer in layers:
                qkv = up(srng.standard_normal((k, C)).astype(np.float32))
                a = up(srng.standard_normal((k, hv)).astype(np.float32))
                b = up(srng.standard_normal((k, hv)).astype(np.float32))
                ys.append(to_np(layer.verify_from_proj(qkv, a, b)).copy())
            logits, drafts, _ = synth.verify_block(36, step, k, V, accepted=planted)
            n, _ = cycle(sdev.upload_f32(logits, DEV), torch.from_numpy(drafts).to(DEV), defer=defer)
            assert n == planted
        states = [to_np(layer.state).copy() for layer in layers]
        runs[defer] = (ys, states)
    for a, b in zip(runs[False][0], runs[True][0]):
        assert np.array_equal(a, b)
    for a, b in zip(runs[False][1], runs[True][1]):
        assert np.array_equal(a, b)
