"""The allocation-free acceptance (sdv_verify_accept_k_noalloc) against the
workspace form (sdv_verify_accept_k), through the C ABI: sampled tokens and
the accepted count bit for bit, on two calls in a row, the second with a
smaller input (the built-in scratch keeps the first call's keys), for greedy
and Gumbel sampling, then the workspace form once more."""

import numpy as np
import pytest
import torch

import synth
from synth import device as sdev
from tests.gpu_helpers import DEV, banner, to_np

pytestmark = pytest.mark.gpu


def _upload(logits, drafts, noise):
    l = sdev.upload_f32(logits, DEV)
    d = torch.from_numpy(np.ascontiguousarray(drafts, dtype=np.int32)).to(DEV)
    n = sdev.upload_f32(noise, DEV) if noise is not None else None
    return l, d, n


def _both(ops, logits, drafts, noise=None, inv_temp=1.0, eos=-1):
    l, d, n = _upload(logits, drafts, noise)
    k = logits.shape[0]
    tok_a = torch.full((k,), -7, dtype=torch.int32, device=DEV)
    acc_a = torch.full((1,), -7, dtype=torch.int32, device=DEV)
    ops.verify_accept_k_noalloc(l, d, tok_a, acc_a, n, inv_temp, eos)
    tok_w, acc_w = ops.verify_accept_k(l, d, n, inv_temp, eos)
    torch.cuda.synchronize()
    return (to_np(tok_a), int(to_np(acc_a)[0])), (to_np(tok_w), int(to_np(acc_w)[0]))


@pytest.mark.parametrize("sampled", [False, True])
def test_noalloc_equals_workspace_form(sampled):
    from speculative_decode_verification_amd import ops
    vocab = 248320
    # a large call, then a smaller one (fewer rows and chunks than the scratch now holds)
    for step, (k, V, planted) in enumerate(((32, vocab, 20), (9, vocab, 5), (3, 5000, 1))):
        banner(f"accept noalloc sampled={sampled} k={k} V={V} call {step}")
        logits, drafts, _ = synth.verify_block(31, 1000 * step + int(sampled), k, V, accepted=planted)
        noise = synth.gumbel_noise(31, step, k, V) if sampled else None
        (ta, na), (tw, nw) = _both(ops, logits, drafts, noise, 0.8 if sampled else 1.0)
        assert np.array_equal(ta, tw), (ta, tw)
        assert na == nw
        if not sampled:
            assert na == planted
    # the workspace form is unaffected by the scratch's last contents
    logits, drafts, _ = synth.verify_block(31, 77, 4, 9000, accepted=2)
    (ta, na), (tw, nw) = _both(ops, logits, drafts)
    assert np.array_equal(ta, tw) and na == nw == 2


def test_noalloc_rejects_oversize_before_launch():
    from speculative_decode_verification_amd import ops
    from speculative_decode_verification_amd._lib import SDV_ERANGE, SdvError
    banner("accept noalloc oversize")
    k, V = 32, 4096 * 4096 + 1
    # only host validation runs: the buffers are never touched
    l = torch.empty(16, dtype=torch.float32, device=DEV)
    tok = torch.full((k,), -7, dtype=torch.int32, device=DEV)
    acc = torch.full((1,), -7, dtype=torch.int32, device=DEV)
    from speculative_decode_verification_amd._lib import lib
    import ctypes
    st = lib().sdv_verify_accept_k_noalloc(ctypes.c_void_p(l.data_ptr()), None, ctypes.c_float(1.0),
                                           ctypes.c_void_p(l.data_ptr()), k, V, -1, ctypes.c_void_p(tok.data_ptr()),
                                           ctypes.c_void_p(acc.data_ptr()), None)
    assert st == SDV_ERANGE
    torch.cuda.synchronize()
    assert (to_np(tok) == -7).all() and int(to_np(acc)[0]) == -7
