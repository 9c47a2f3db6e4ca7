"""Shared helpers for the GPU parity tests (inputs from synth, expected values
from the oracle; nothing here computes the method's results)."""

import numpy as np
import torch

import synth
from synth import device as sdev

DEV = "cuda:0"
TOL = 1e-5  # max |G - R| / max |R| per verified row


def normwise(G, R):
    """Per-row normwise relative error over the trailing axes."""
    G = np.asarray(G, dtype=np.float64)
    R = np.asarray(R, dtype=np.float64)
    d = np.abs(G - R).reshape(G.shape[0], -1).max(axis=1)
    m = np.abs(R).reshape(R.shape[0], -1).max(axis=1)
    return d / np.where(m > 0, m, 1.0)


def assert_close(G, R, what, tol=TOL):
    err = normwise(G, R)
    assert np.all(err <= tol), f"{what}: max normwise error {err.max():.3e} (tol {tol:.0e}), per row {err}"


def to_np(t):
    return t.detach().cpu().numpy()


def q4_host(cfg, kind, layer, E, N, K):
    """Host arrays of a whole (small) bank."""
    keys = synth.bank_keys(cfg, kind, layer)
    parts = [synth.q4_rows(keys, E, N, K, expert=e) for e in range(E)]
    return tuple(np.stack([p[i] for p in parts]) for i in range(3))


def q4_device_from_host(codes, scales, biases):
    from speculative_decode_verification_amd.ops import Q4Weight
    return Q4Weight(*sdev.upload_q4(codes, scales, biases, DEV))


def banner(msg):
    print(f"[gpu-case] {msg}", flush=True)
