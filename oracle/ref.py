"""Plain fp64 definitions of every step of the k-row verification step.

TEST INFRASTRUCTURE ONLY (see the package docstring).  No blocking, fusion or
reordering beyond what each definition states; numpy's matmul and sort serve
as library steps.
"""

import numpy as np

GROUP = 64


# ---------------------------------------------------------------------------
# affine Q4 (mere.run transfer report, "Shared architecture and implemented
# paths": affine Q4, group size 64, compatible bf16 tensors)
# ---------------------------------------------------------------------------

def bf16_to_f64(bits):
    """bf16 bit patterns (uint16) to fp64: the fp32 whose high half is the
    pattern, widened exactly."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32).astype(np.float64)


def unpack_q4(codes):
    """Unsigned 4-bit codes from packed u32 words ``[..., K/8]``.

    Element ``8*w + i`` of a row sits in bits ``[4i, 4i+4)`` of word ``w``.
    The pages do not fix a nibble order; this layout is our definition
    (parity unpinned by the pages; pinned by tests against an independently
    written packer)."""
    codes = np.asarray(codes, dtype=np.uint32)
    shifts = (4 * np.arange(8, dtype=np.uint32))
    q = (codes[..., None] >> shifts) & np.uint32(15)
    return q.reshape(*codes.shape[:-1], codes.shape[-1] * 8).astype(np.uint8)


def dequant(codes, scales, biases):
    """Dense fp64 weights: ``W[n, c] = s[n, c // 64] * q[n, c] + b[n, c // 64]``.

    Affine Q4 with unsigned codes: value = scale * code + bias, one (scale,
    bias) pair per 64 consecutive input elements.  Exact in fp64 (a 8-bit
    scale times a 4-bit code plus an 8-bit bias needs far fewer than 53
    bits)."""
    q = unpack_q4(codes).astype(np.float64)
    s = np.repeat(bf16_to_f64(scales), GROUP, axis=-1)
    b = np.repeat(bf16_to_f64(biases), GROUP, axis=-1)
    return s * q + b


def qmv(codes, scales, biases, x):
    """Multi-row affine-Q4 matvec, each row computed on its own.

    ``x``: fp64 ``[k, K]``; returns fp64 ``[k, N]`` with ``y[r] = W @ x[r]``.
    A width-k verification row must equal the serial width-1 product (mere.run
    transfer report, "Exact verification kernels and benchmark admission";
    Red Lite dev45, "What it is": each row summed as the one-row product sums it), so the
    definition is the 1-row product applied per row."""
    w = dequant(codes, scales, biases)
    x = np.asarray(x, dtype=np.float64)
    y = np.empty((x.shape[0], w.shape[0]), dtype=np.float64)
    for r in range(x.shape[0]):
        y[r] = w @ x[r]
    return y


# ---------------------------------------------------------------------------
# routing and union (mere.run report: 256-expert top-8 gathered experts;
# Red Lite "What it is": one router dispatch for both rows, the (expert, row)
# pairs of the rows' union; Flash-Next plan "2.3 MoE": a bank of 512 experts,
# each row routed to 10 of them, plus one shared expert)
# ---------------------------------------------------------------------------

# ---------------------------------------------------------------------------
# affine Q3 (mere.run transfer report, "Shared architecture and implemented
# paths": the gathered expert kernel's Flash-Next Q3 specialization beside
# affine Q4/g64).  Same affine form and group as Q4, 3-bit codes.
# ---------------------------------------------------------------------------

def unpack_q3(codes):
    """Unsigned 3-bit codes from packed bytes ``[..., 3K/8]``: element c of a
    row is bits ``[3c, 3c+3)`` of the row's little-endian bit stream (eight
    codes in every three bytes).  The pages do not fix the packing; this is
    our definition (pinned against an independently written packer)."""
    b = np.asarray(codes, dtype=np.uint8)
    nbytes = b.shape[-1]
    n = nbytes * 8 // 3
    bits = np.unpackbits(b, axis=-1, bitorder="little")            # [..., 8 * nbytes], bit i of the stream
    trip = bits[..., :3 * n].reshape(*b.shape[:-1], n, 3).astype(np.uint8)
    return (trip[..., 0] | (trip[..., 1] << 1) | (trip[..., 2] << 2)).astype(np.uint8)


def dequant_q3(codes, scales, biases):
    """Dense fp64 weights: ``W[n, c] = s[n, c // 64] * q[n, c] + b[n, c // 64]``
    with 3-bit codes q (0..7).  Exact in fp64."""
    q = unpack_q3(codes).astype(np.float64)
    s = np.repeat(bf16_to_f64(scales), GROUP, axis=-1)
    b = np.repeat(bf16_to_f64(biases), GROUP, axis=-1)
    return s * q + b


def qmv_q3(codes, scales, biases, x):
    """Multi-row affine-Q3 matvec, each row on its own (as ``qmv``)."""
    w = dequant_q3(codes, scales, biases)
    x = np.asarray(x, dtype=np.float64)
    return np.stack([w @ x[r] for r in range(x.shape[0])])


# ---------------------------------------------------------------------------
# Q8_0 (Red Lite dev45, "What it is": the MTP block keeps its 512 experts in
# Q8_0, each code decoding to the same value as in the dense decode; mere.run transfer
# report, "Shared architecture and implemented paths": the checkpoint's Q8
# router and shared-gate weights).  The GGUF Q8_0 block: 32 signed 8-bit codes
# sharing one IEEE half scale.
# ---------------------------------------------------------------------------

Q8_BLOCK = 32


def fp16_to_f64(bits):
    """IEEE binary16 bit patterns (uint16) to fp64, from the fields: sign,
    5-bit exponent with bias 15, 10-bit fraction; exponent 0 is subnormal
    (f * 2^-24), exponent 31 is infinity (f = 0) or NaN."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.int64)
    sign = np.where((b >> 15) & 1, -1.0, 1.0)
    e = (b >> 10) & 31
    f = (b & 1023).astype(np.float64)
    normal = (1.0 + f / 1024.0) * np.exp2((e - 15).astype(np.float64))
    val = np.where(e == 0, f * 2.0 ** -24, normal)
    val = np.where(e == 31, np.where(f == 0, np.inf, np.nan), val)
    return sign * val


def dequant_q8_0(qs, d):
    """Dense fp64 weights: ``W[n, c] = d[n, c // 32] * q[n, c]`` with q the
    signed 8-bit code ``qs[n, c]`` and d the half scale of its 32-element
    block.  Exact in fp64."""
    q = np.asarray(qs, dtype=np.int8).astype(np.float64)
    s = np.repeat(fp16_to_f64(d), Q8_BLOCK, axis=-1)
    return s * q


def qmv_q8_0(qs, d, x):
    """Multi-row Q8_0 matvec, each row on its own: ``y[r] = W @ x[r]`` (the
    same per-row definition as ``qmv``)."""
    w = dequant_q8_0(qs, d)
    x = np.asarray(x, dtype=np.float64)
    return np.stack([w @ x[r] for r in range(x.shape[0])])


def route(logits, topk, mode, renorm):
    """Per-row top-k experts and their weights.

    Selection: experts sorted by (logit descending, index ascending), first
    ``topk`` kept; output slots are in that order.  The pages do not state a
    tie rule; ties to the lower index is our definition (parity unpinned by
    the pages).  Softmax and sigmoid are monotone, so selecting on the raw
    logit selects on the score.

    Weights (fp64): ``mode == "softmax"``: p_e = exp(l_e - m) / sum_all exp(l - m);
    ``mode == "sigmoid"``: p_e = 1 / (1 + exp(-l_e)).  ``w[r, s] = p[idx[r, s]]``,
    divided by ``sum_s p`` when ``renorm``.  The Ornith configuration is read
    literally as softmax over all experts without renormalisation; the
    Flash-Next configuration as sigmoid scores renormalised over the top-10
    (no score bias)."""
    l = np.asarray(logits, dtype=np.float64)
    k, e = l.shape
    idx = np.empty((k, topk), dtype=np.int32)
    w = np.empty((k, topk), dtype=np.float64)
    for r in range(k):
        order = np.lexsort((np.arange(e), -l[r]))
        idx[r] = order[:topk]
        if mode == "softmax":
            ex = np.exp(l[r] - l[r].max())
            p = ex / ex.sum()
        elif mode == "sigmoid":
            p = 1.0 / (1.0 + np.exp(-l[r]))
        else:
            raise ValueError(mode)
        w[r] = p[idx[r]]
        if renorm:
            w[r] = w[r] / w[r].sum()
    return idx, w


def union_pairs(idx):
    """The union of the rows' experts and the (expert, row, slot) pairs.

    ``union_ids``: distinct experts ascending.  Pairs ordered by (expert
    ascending, row ascending); ``pair_off[u] .. pair_off[u+1]`` are the pairs
    of union entry ``u``; ``pair_slot`` is the position of the expert in that
    row's top-k.  The orders are our definition (parity unpinned by the pages,
    which state only that the union of the rows' experts is loaded)."""
    idx = np.asarray(idx)
    k, topk = idx.shape
    union_ids = np.array(sorted(set(int(e) for e in idx.ravel())), dtype=np.int32)
    pair_off = [0]
    pair_row, pair_slot = [], []
    for e in union_ids:
        for r in range(k):
            hits = np.nonzero(idx[r] == e)[0]
            for s in hits:
                pair_row.append(r)
                pair_slot.append(int(s))
        pair_off.append(len(pair_row))
    return (union_ids, np.array(pair_off, dtype=np.int32), np.array(pair_row, dtype=np.int32),
            np.array(pair_slot, dtype=np.int32))


def silu(a):
    return a / (1.0 + np.exp(-a))


def swiglu(a):
    """SwiGLU over a fused gate/up output: rows ``[0, I)`` are the gate and
    rows ``[I, 2I)`` the up projection (gate and up concatenated, Flash-Next
    plan "2.3 MoE"); ``h = silu(gate) * up`` with ``silu(x) = x * sigmoid(x)``.
    Gate-first order is our reading (parity unpinned by the pages)."""
    a = np.asarray(a, dtype=np.float64)
    i = a.shape[-1] // 2
    return silu(a[..., :i]) * a[..., i:]


def _sigmoid(z):
    return 1.0 / (1.0 + np.exp(-np.asarray(z, dtype=np.float64)))


def combine(partial, w, shared=None, z=None):
    """MoE tail: ``y[r] = sum_s w[r, s] * partial[r, s]`` in slot order, then
    ``+ sigmoid(z[r]) * shared[r]`` (gate 1 when ``z`` is None) when a shared
    expert output is given.  Slot order, then the shared expert last, is our
    reading (parity unpinned by the pages)."""
    partial = np.asarray(partial, dtype=np.float64)
    w = np.asarray(w, dtype=np.float64)
    k, topk = w.shape
    y = np.zeros((k, partial.shape[-1]), dtype=np.float64)
    for r in range(k):
        for s in range(topk):
            y[r] = y[r] + w[r, s] * partial[r, s]
    if shared is not None:
        shared = np.asarray(shared, dtype=np.float64)
        gate = np.ones(k) if z is None else _sigmoid(z)
        for r in range(k):
            y[r] = y[r] + gate[r] * shared[r]
    return y


def moe_verify(x, logits, gate_up, down, topk, mode, renorm, z=None, shared_gate_up=None,
               shared_down=None):
    """One MoE layer for k rows (fp64).

    ``x``: fp64 ``[k, H]``.  ``gate_up(e)`` / ``down(e)`` return dense fp64
    matrices ``[2I, H]`` / ``[H, I]`` of expert ``e`` (so a caller can build
    only the experts it needs).  For each row r and slot s with e =
    idx[r, s]: ``h[r, s] = swiglu(W_gu[e] @ x[r])`` (kept in fp64),
    ``partial[r, s] = W_dn[e] @ h[r, s]``, ``y[r] = sum_s w[r, s] * partial[r, s]``
    in slot order, plus, when a shared expert is given,
    ``sigmoid(z[r]) * W_sdn @ swiglu(W_sgu @ x[r])`` added last.  The shared
    expert's scalar sigmoid gate follows the lineage's sigmoid-gated shared
    expert (Flash-Next plan, "3 Reference implementations"); with no ``z`` its
    weight is 1 (parity unpinned by the pages)."""
    x = np.asarray(x, dtype=np.float64)
    k = x.shape[0]
    idx, w = route(logits, topk, mode, renorm)
    union_ids, pair_off, pair_row, pair_slot = union_pairs(idx)
    cache = {}

    def mats(e):
        if e not in cache:
            cache[e] = (gate_up(e), down(e))
        return cache[e]

    h, partial = [], []
    for r in range(k):
        hr, pr = [], []
        for s in range(topk):
            wgu, wdn = mats(int(idx[r, s]))
            hs = swiglu(wgu @ x[r])
            hr.append(hs)
            pr.append(wdn @ hs)
        h.append(hr)
        partial.append(pr)
    h = np.array(h)
    partial = np.array(partial)
    shared = None
    if shared_gate_up is not None:
        shared = np.empty((k, partial.shape[-1]), dtype=np.float64)
        for r in range(k):
            shared[r] = shared_down @ swiglu(shared_gate_up @ x[r])
    y = combine(partial, w, shared, z)
    return {"idx": idx, "w": w, "union_ids": union_ids, "pair_off": pair_off,
            "pair_row": pair_row, "pair_slot": pair_slot, "h": h, "partial": partial,
            "shared": shared, "y": y, "n_union": len(union_ids)}


# ---------------------------------------------------------------------------
# Gated DeltaNet (Flash-Next plan, section 2.1 on the model's GDN layers;
# "3.1 Overlap": per-head scalar decay and beta, k heads shared by v heads;
# Red Lite dev45 "What it is": row t runs from row t-1's state, the state
# after each row is snapshotted; rejection selects the snapshot)
# ---------------------------------------------------------------------------

def gdn_verify(S_in, q, k, v, g, beta):
    """k-row delta-rule recurrence with a snapshot after every row.

    ``S_in`` fp ``[Hv, Dv, Dk]``; ``q, k`` ``[rows, Hk, Dk]``; ``v``
    ``[rows, Hv, Dv]``; ``g, beta`` ``[rows, Hv]``.  For t = 0..rows-1 and each
    v head h with qk head c = h // (Hv / Hk):

    1. ``S_h <- g[t, h] * S_h``            (decay)
    2. ``m = S_h @ k[t, c]``                (kv_mem: sum over the key axis)
    3. ``delta = beta[t, h] * (v[t, h] - m)``
    4. ``S_h[i, j] += delta[i] * k[t, c][j]``  (rank-1 update)
    5. ``y[t, h] = S_h @ q[t, c]``          (readout)
    6. ``snaps[t] = S``

    The plan writes step 4 as "S + k (outer) delta"; with S laid out
    [Dv, Dk] and step 2 summing over the key axis, the update that makes
    step 2 retrieve v after the write is delta along Dv times k along Dk,
    which is what is written here.  Contiguous head groups (c = h // ratio)
    and no 1/sqrt(Dk) scaling on q are our readings (parity unpinned by the
    pages).  Returns (y fp64 ``[rows, Hv, Dv]``, snaps fp64
    ``[rows, Hv, Dv, Dk]``); ``S_in`` is not modified."""
    S = np.array(S_in, dtype=np.float64, copy=True)
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    g = np.asarray(g, dtype=np.float64)
    beta = np.asarray(beta, dtype=np.float64)
    hv, dv, dk = S.shape
    hk = q.shape[1]
    if hv % hk != 0:
        raise ValueError("Hv must be a multiple of Hk")
    ratio = hv // hk
    rows = q.shape[0]
    y = np.empty((rows, hv, dv), dtype=np.float64)
    snaps = np.empty((rows, hv, dv, dk), dtype=np.float64)
    for t in range(rows):
        for h in range(hv):
            c = h // ratio
            kt, qt = k[t, c], q[t, c]
            S[h] = g[t, h] * S[h]
            m = S[h] @ kt
            delta = beta[t, h] * (v[t, h] - m)
            S[h] = S[h] + np.outer(delta, kt)
            y[t, h] = S[h] @ qt
        snaps[t] = S
    return y, snaps


def rollback(S_in, snaps, j):
    """State after the accepted prefix of length j: S_in for j = 0, the
    snapshot after row j-1 for 1 <= j <= rows; any other j is an error."""
    rows = len(snaps)
    if not (0 <= j <= rows):
        raise ValueError(f"accepted prefix {j} outside 0..{rows}")
    return np.array(S_in, copy=True) if j == 0 else np.array(snaps[j - 1], copy=True)


# ---------------------------------------------------------------------------
# acceptance (Red Lite dev45, "Acceptance": draft t stands when it equals the
# token sampled from row t-1's logits, so the output distribution stays that
# of plain decoding for any sampler; dev45b: a draft that matches the
# end-of-answer token is refused, so that token is kept out of the state)
# ---------------------------------------------------------------------------

def sample_tokens(logits, noise=None, inv_temp=1.0):
    """The token sampled from each row of ``logits`` [rows, V]: the index of
    the largest z, the lowest such index on ties, a NaN z never chosen (-1 for
    a row with no number).  Greedy: z = logits.  With Gumbel noise g (one
    value per logit, passed in): z = fl32(fl32(logits * inv_temp) + g), each
    operation rounded to fp32, so the decision is taken in the precision of
    the kernel; Gumbel-max of z samples the softmax at temperature 1 /
    inv_temp.  -0 and +0 compare equal.  (The sampler is our reading: the
    pages allow any sampler and measure greedy.)"""
    l = np.asarray(logits, dtype=np.float32)
    if noise is None:
        z = l
    else:
        z = (l * np.float32(inv_temp)).astype(np.float32) + np.asarray(noise, dtype=np.float32)
        z = z.astype(np.float32)
    out = np.full(z.shape[0], -1, dtype=np.int32)
    for r in range(z.shape[0]):
        valid = np.flatnonzero(~np.isnan(z[r]))
        if valid.size == 0:
            continue
        best = z[r][valid].max()
        out[r] = valid[z[r][valid] == best][0]
    return out


def accept(tokens, drafts, eos=-1):
    """Number of leading drafts accepted.  ``drafts[t]`` is the token of row
    t + 1; it is accepted when every earlier draft was, it equals the token
    sampled from row t, and it is not the end-of-answer token ``eos`` (-1:
    none).  With n accepted, rows 0..n stay in the state (rollback to the
    prefix of n + 1 rows) and tokens[0..n] are emitted, tokens[n] becoming the
    next pending token."""
    n = 0
    for t in range(len(drafts)):
        if drafts[t] == tokens[t] and (eos < 0 or drafts[t] != eos):
            n += 1
        else:
            break
    return n


def verify_cycle(logits, drafts, eos=-1, noise=None, inv_temp=1.0):
    """Acceptance of one verified block: the sampled tokens, the accepted
    draft count n, the accepted prefix length n + 1 (rows kept in the state)
    and the emitted tokens (the n accepted drafts, then the token sampled
    after them)."""
    tokens = sample_tokens(logits, noise, inv_temp)
    n = accept(tokens, drafts, eos)
    emitted = [int(d) for d in drafts[:n]] + [int(tokens[n])]
    return {"tokens": tokens, "accepted": n, "prefix": n + 1, "emitted": emitted}


# ---------------------------------------------------------------------------
# GDN preparation and tail (Flash-Next plan, "2.1 Gated DeltaNet": each q,
# k and v channel filtered along time by its own filter over the current and
# earlier inputs, the earlier inputs kept between calls; q and k scaled to
# unit L2 norm per head; g from A_log and dt_bias through softplus and exp,
# beta = sigmoid(b); the output is the RMS-normalised y times act(gate);
# "5.1 Gated DeltaNet": 4 taps, sigmoid gate for this model)
# ---------------------------------------------------------------------------

CONV_TAPS = 4


def softplus(x):
    """log(1 + e^x), written stably: max(x, 0) + log1p(e^-|x|)."""
    x = np.asarray(x, dtype=np.float64)
    return np.maximum(x, 0.0) + np.log1p(np.exp(-np.abs(x)))


def gdn_prepare(qkv, hist, conv_w, a, b, A_log, dt_bias, hk, hv, dk, dv, act="none", eps=1e-6):
    """The k rows' inputs of the recurrence from their projections.

    qkv [k, C] with C = 2 hk dk + hv dv, channels [q | k | v] (q, k head-major);
    hist [CONV_TAPS - 1, C], the inputs before row 0 (oldest first); conv_w
    [C, CONV_TAPS], tap i applied to the input CONV_TAPS - 1 - i steps before
    the current one (tap 3 to the current input): with X = [hist; qkv]
    (k + 3 columns), conv[t, c] = sum_i conv_w[c, i] * X[t + i, c].  act "silu" applies silu
    after the conv, "none" nothing (the page names no activation; reading).
    q and k are divided per (row, head) by sqrt(sum of squares + eps) (eps is
    our reading).  g[t, h] = exp(-exp(A_log[h]) * softplus(a[t, h] +
    dt_bias[h])), beta[t, h] = sigmoid(b[t, h]).  Returns q [k, hk, dk], k,
    v [k, hv, dv], g, beta [k, hv] and the window X [k + 3, C]; the conv
    history after an accepted prefix of j rows is X[j : j + 3]."""
    qkv = np.asarray(qkv, dtype=np.float64)
    rows, C = qkv.shape
    assert C == 2 * hk * dk + hv * dv
    X = np.concatenate([np.asarray(hist, dtype=np.float64), qkv], axis=0)
    w = np.asarray(conv_w, dtype=np.float64)
    conv = np.zeros((rows, C))
    for t in range(rows):
        for i in range(CONV_TAPS):
            conv[t] = conv[t] + w[:, i] * X[t + i]
    if act == "silu":
        conv = silu(conv)
    elif act != "none":
        raise ValueError(act)
    q = conv[:, :hk * dk].reshape(rows, hk, dk)
    k = conv[:, hk * dk:2 * hk * dk].reshape(rows, hk, dk)
    v = conv[:, 2 * hk * dk:].reshape(rows, hv, dv)
    q = q / np.sqrt((q * q).sum(axis=-1, keepdims=True) + eps)
    k = k / np.sqrt((k * k).sum(axis=-1, keepdims=True) + eps)
    g = np.exp(-np.exp(np.asarray(A_log, dtype=np.float64))[None, :] *
               softplus(np.asarray(a, dtype=np.float64) + np.asarray(dt_bias, dtype=np.float64)[None, :]))
    beta = 1.0 / (1.0 + np.exp(-np.asarray(b, dtype=np.float64)))
    return {"q": q, "k": k, "v": v, "g": g, "beta": beta, "window": X}


def gdn_gated_norm(y, z, w, act="sigmoid", eps=1e-6):
    """The GDN output: per (row, v head), rmsnorm over Dv times the weight w
    [Dv], times act(z): y / sqrt(mean(y^2) + eps) * w * act(z).  act
    "sigmoid" (the page's note for this model) or "silu"; eps is our
    reading."""
    y = np.asarray(y, dtype=np.float64)
    z = np.asarray(z, dtype=np.float64)
    n = y / np.sqrt((y * y).mean(axis=-1, keepdims=True) + eps)
    if act == "sigmoid":
        gate = 1.0 / (1.0 + np.exp(-z))
    elif act == "silu":
        gate = silu(z)
    else:
        raise ValueError(act)
    return n * np.asarray(w, dtype=np.float64) * gate
