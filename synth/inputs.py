"""Host-side generators for every input of the five workloads.

Distributions (the workloads' recipe): activations x ~ N(0,1) rounded to bf16;
router logits ~ N(0,1) fp32; shared-expert gate logit z ~ N(0,1) fp32;
codes ~ U{0..15}; scales ~ U(0.005, 0.02) bf16; biases ~ U(-0.1, 0.1) bf16;
GDN state S ~ N(0, 0.1^2) fp32; q, k ~ N(0,1) then L2-normalised per (row,
head); v ~ N(0,1); beta = sigmoid(N(0,1)); g = exp(-softplus(N(0,1)));
accepted prefix j ~ U{0..k}.  Verify-block next-token logits ~ N(0,1) fp32
over the vocabulary, with a planted number of accepted drafts ~ U{0..k-1}
(the planted tokens are raised a fixed margin above their row's maximum);
Gumbel noise g = -log(-log(u)), u ~ U(0,1), for sampled acceptance.  GDN
preparation inputs: projections qkv ~ N(0,1), conv history ~ N(0,1), conv
weights ~ U(-0.5, 0.5), a, b ~ N(0,1), A_log, dt_bias ~ U(-1, 1); output
gate z ~ N(0,1) and norm weight ~ U(0.5, 1.5).
"""

from collections import namedtuple

import numpy as np

from .counter import SEED, derive_key, q4_rows, bf16_bits_from_f32

BankKeys = namedtuple("BankKeys", "codes scales biases")

# bank kinds (part of the stream keys)
DENSE_W, GATEUP, DOWN, SHARED_GATEUP, SHARED_DOWN = 0, 1, 2, 3, 4
# tensor ids (part of the numpy seeds)
T_X, T_LOGITS, T_Z, T_S, T_Q, T_K, T_V, T_G, T_BETA, T_J = 10, 11, 12, 20, 21, 22, 23, 24, 25, 30
T_VLOGITS, T_GUMBEL, T_DRAFTS = 40, 41, 42
T_QKV, T_HIST, T_CONVW, T_A, T_B, T_ALOG, T_DTB, T_GATEZ, T_NORMW = 50, 51, 52, 53, 54, 55, 56, 57, 58
T_Q8, T_Q3 = 60, 61


def bank_keys(cfg_id, kind, layer):
    return BankKeys(*(derive_key(cfg_id, kind, layer, part) for part in (1, 2, 3)))


def _rng(*ids):
    return np.random.default_rng([SEED, *[int(i) for i in ids]])


def dense_weight(cfg_id, kind, layer, n, k):
    """A full dense Q4 matrix ``[N, K]`` (E = 1) as host arrays."""
    return q4_rows(bank_keys(cfg_id, kind, layer), 1, n, k, expert=0)


def bf16_normal(rng, shape):
    return bf16_bits_from_f32(rng.standard_normal(shape, dtype=np.float32))


def activations(cfg_id, layer, rows, k, step=0, tensor=T_X):
    """bf16 activation rows [rows, k] ~ N(0,1) (bit patterns)."""
    return bf16_normal(_rng(cfg_id, tensor, layer, step), (rows, k))


def moe_layer_inputs(cfg_id, layer, rows, hidden, experts, step=0):
    """x (bf16 bits [rows, hidden]), router logits (fp32 [rows, E]) and the
    shared-expert gate logit z (fp32 [rows]) of one MoE layer."""
    x = bf16_normal(_rng(cfg_id, T_X, layer, step), (rows, hidden))
    logits = _rng(cfg_id, T_LOGITS, layer, step).standard_normal((rows, experts), dtype=np.float32)
    z = _rng(cfg_id, T_Z, layer, step).standard_normal((rows,), dtype=np.float32)
    return {"x": x, "logits": logits, "z": z}


def gdn_state(cfg_id, layer, hv, dv, dk):
    s = 0.1 * _rng(cfg_id, T_S, layer).standard_normal((hv, dv, dk))
    return s.astype(np.float32)


def _l2n(a):
    return a / np.sqrt(np.sum(a * a, axis=-1, keepdims=True))


def gdn_layer_inputs(cfg_id, layer, rows, hv, hk, dk, dv, step=0):
    """Per-row GDN inputs of one layer: q, k fp32 [rows, Hk, Dk] (unit norm per
    head), v fp32 [rows, Hv, Dv], g and beta fp32 [rows, Hv]."""
    q = _l2n(_rng(cfg_id, T_Q, layer, step).standard_normal((rows, hk, dk))).astype(np.float32)
    k = _l2n(_rng(cfg_id, T_K, layer, step).standard_normal((rows, hk, dk))).astype(np.float32)
    v = _rng(cfg_id, T_V, layer, step).standard_normal((rows, hv, dv)).astype(np.float32)
    a = _rng(cfg_id, T_G, layer, step).standard_normal((rows, hv))
    g = np.exp(-np.logaddexp(0.0, a)).astype(np.float32)
    b = _rng(cfg_id, T_BETA, layer, step).standard_normal((rows, hv))
    beta = (1.0 / (1.0 + np.exp(-b))).astype(np.float32)
    return {"q": q, "k": k, "v": v, "g": g, "beta": beta}


def accepted_prefix(cfg_id, step, rows):
    """Accepted-prefix length j ~ U{0..rows} for one verify step."""
    return int(_rng(cfg_id, T_J, step).integers(0, rows + 1))


def q3_weight(cfg_id, kind, layer, E, N, K):
    """An affine-Q3/g64 weight in its interchange form: codes uint8
    [E, N, 3K/8] (a little-endian bit stream of 3-bit codes ~ U{0..7}),
    scales ~ U(0.01, 0.04) and biases ~ U(-0.1, 0.1) as bf16 bits
    [E, N, K/64].  Returns (codes, scales, biases, q) with q the codes
    unpacked, for generators' own checks."""
    rng = _rng(cfg_id, T_Q3, kind, layer)
    q = rng.integers(0, 8, size=(E, N, K), dtype=np.int64)
    bits = np.stack([(q >> i) & 1 for i in range(3)], axis=-1).reshape(E, N, 3 * K).astype(np.uint8)
    codes = np.packbits(bits, axis=-1, bitorder="little")
    sc = bf16_bits_from_f32(rng.uniform(0.01, 0.04, size=(E, N, K // 64)).astype(np.float32))
    bi = bf16_bits_from_f32(rng.uniform(-0.1, 0.1, size=(E, N, K // 64)).astype(np.float32))
    return codes, sc, bi, q.astype(np.uint8)


def q8_0_weight(cfg_id, kind, layer, E, N, K):
    """A Q8_0 weight in the GGUF interchange form: signed codes int8
    [E, N, K] ~ U{-127..127} (a Q8_0 quantiser never emits -128) and half
    scales [E, N, K/32] ~ U(2e-4, 8e-4) as IEEE binary16 bit patterns."""
    rng = _rng(cfg_id, T_Q8, kind, layer)
    qs = rng.integers(-127, 128, size=(E, N, K), dtype=np.int64).astype(np.int8)
    d = rng.uniform(2e-4, 8e-4, size=(E, N, K // 32)).astype(np.float16).view(np.uint16)
    return qs, d


def integer_exact_weight(seed, n, k, rows):
    """A Q4 matrix and activations whose products and sums are exact in fp32.

    scale = 2^-6, bias = m * 2^-6 with m in [-6, 6], x integers in [-8, 8]:
    every partial sum is a multiple of 2^-6 below 2^24 * 2^-6 in magnitude,
    so any summation order gives the same fp32 result."""
    rng = np.random.default_rng([SEED, 99, seed])
    g = k // 64
    codes = rng.integers(0, 1 << 32, size=(n, k // 8), dtype=np.uint64).astype(np.uint32)
    scales = np.full((n, g), 0x3C80, dtype=np.uint16)            # bf16 of 2^-6
    m = rng.integers(-6, 7, size=(n, g)).astype(np.float32)
    biases = bf16_bits_from_f32(m * np.float32(2.0 ** -6))
    x = bf16_bits_from_f32(rng.integers(-8, 9, size=(rows, k)).astype(np.float32))
    return codes, scales, biases, x


def verify_block(cfg_id, step, rows, vocab, accepted=None, margin=4.0, eos=-1):
    """Next-token logits [rows, vocab] fp32 ~ N(0,1) and the drafts [rows - 1]
    of one verify block, with ``accepted`` (default ~ U{0..rows-1}) drafts
    planted to be accepted under greedy sampling: for t < accepted, row t's
    logit of drafts[t] is set ``margin`` above the row's maximum; when
    accepted < rows - 1 (and vocab > 1), row ``accepted`` gets its raised
    token on a token other than drafts[accepted].  Drafts never equal ``eos`` unless planted
    by the caller.  Returns (logits, drafts, accepted)."""
    rng = _rng(cfg_id, T_VLOGITS, step)
    logits = rng.standard_normal((rows, vocab), dtype=np.float32)
    drng = _rng(cfg_id, T_DRAFTS, step)
    drafts = drng.integers(0, vocab, size=max(rows - 1, 0)).astype(np.int32)
    if eos >= 0:
        drafts[drafts == eos] = (eos + 1) % vocab
    if accepted is None:
        accepted = int(drng.integers(0, rows))
    for t in range(min(accepted, rows - 1)):
        logits[t, drafts[t]] = logits[t].max() + np.float32(margin)
    if accepted < rows - 1 and vocab > 1:
        other = (int(drafts[accepted]) + 1 + int(drng.integers(0, vocab - 1))) % vocab
        if other == drafts[accepted]:
            other = (other + 1) % vocab
        logits[accepted, other] = logits[accepted].max() + np.float32(margin)
    return logits, drafts, accepted


def gumbel_noise(cfg_id, step, rows, vocab):
    """Gumbel(0, 1) noise [rows, vocab] fp32: -log(-log(u)) with u uniform in (0, 1)."""
    u = _rng(cfg_id, T_GUMBEL, step).random((rows, vocab))
    u = np.clip(u, 2.0 ** -53, 1.0 - 2.0 ** -53)
    return (-np.log(-np.log(u))).astype(np.float32)


def gdn_raw_inputs(cfg_id, layer, rows, hv, hk, dk, dv, step=0):
    """Projections of one GDN layer before the preparation: qkv [rows, C]
    (C = 2 hk dk + hv dv, channels q | k | v), the conv history [3, C], the
    depthwise conv weights [C, 4], a, b [rows, hv], A_log, dt_bias [hv], the
    output gate z [rows, hv, dv] and the output norm weight [dv] (fp32)."""
    C = 2 * hk * dk + hv * dv
    f = np.float32
    out = {
        "qkv": _rng(cfg_id, T_QKV, layer, step).standard_normal((rows, C), dtype=f),
        "hist": _rng(cfg_id, T_HIST, layer).standard_normal((3, C), dtype=f),
        "conv_w": _rng(cfg_id, T_CONVW, layer).uniform(-0.5, 0.5, (C, 4)).astype(f),
        "a": _rng(cfg_id, T_A, layer, step).standard_normal((rows, hv), dtype=f),
        "b": _rng(cfg_id, T_B, layer, step).standard_normal((rows, hv), dtype=f),
        "A_log": _rng(cfg_id, T_ALOG, layer).uniform(-1.0, 1.0, hv).astype(f),
        "dt_bias": _rng(cfg_id, T_DTB, layer).uniform(-1.0, 1.0, hv).astype(f),
        "z": _rng(cfg_id, T_GATEZ, layer, step).standard_normal((rows, hv, dv), dtype=f),
        "norm_w": _rng(cfg_id, T_NORMW, layer).uniform(0.5, 1.5, dv).astype(f),
    }
    return out
