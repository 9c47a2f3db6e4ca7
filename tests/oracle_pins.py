"""Pins for the CPU oracle: each check takes the oracle module and raises
AssertionError when the oracle disagrees with something fixed independently
of it (exact rational brute force, integer-exact arithmetic, closed forms,
invariants stated by the pages, reductions to textbook routines).

The checks are functions of the module so that tests/test_oracle_mutants.py
can run them against copies of the oracle with planted mistakes.
"""

from fractions import Fraction
import math
import struct

import numpy as np

import synth


# ---------------------------------------------------------------------------
# independent helpers (exact arithmetic, written without the oracle's code)
# ---------------------------------------------------------------------------

def bf16_exact(bits):
    """Exact rational value of a finite bf16 pattern from its fields."""
    bits = int(bits)
    sign = -1 if bits >> 15 else 1
    e = (bits >> 7) & 0xFF
    m = bits & 0x7F
    assert e != 0xFF
    if e == 0:
        return sign * Fraction(m, 128) * Fraction(2) ** (-126)
    return sign * (1 + Fraction(m, 128)) * Fraction(2) ** (e - 127)


def nibble(word, i):
    return (int(word) // 16 ** i) % 16


def pack_q4(q):
    """Pack codes [N, K] (0..15) into u32 words: element 8w+i at bits 4i."""
    n, k = q.shape
    out = np.zeros((n, k // 8), dtype=np.uint32)
    for r in range(n):
        for w in range(k // 8):
            acc = 0
            for i in range(8):
                acc += int(q[r, 8 * w + i]) * 16 ** i
            out[r, w] = acc
    return out


def exact_qmv(codes, scales, biases, xbits):
    n = codes.shape[0]
    k = codes.shape[1] * 8
    rows = xbits.shape[0]
    y = [[Fraction(0)] * n for _ in range(rows)]
    for r in range(rows):
        for o in range(n):
            acc = Fraction(0)
            for c in range(k):
                g = c // 64
                wv = bf16_exact(scales[o, g]) * nibble(codes[o, c // 8], c % 8) + bf16_exact(biases[o, g])
                acc += bf16_exact(xbits[r, c]) * wv
            y[r][o] = acc
    return y


def _f32(a):
    return np.asarray(a, dtype=np.float32)


# ---------------------------------------------------------------------------
# Q4 pins
# ---------------------------------------------------------------------------

def check_bf16_decode(ref):
    pats = np.arange(0, 1 << 16, 97, dtype=np.uint32).astype(np.uint16)
    pats = np.array([p for p in pats if ((int(p) >> 7) & 0xFF) != 0xFF], dtype=np.uint16)
    got = ref.bf16_to_f64(pats)
    for p, v in zip(pats, got):
        assert Fraction(float(v)) == bf16_exact(p), hex(int(p))
    assert ref.bf16_to_f64(np.array([0x3F80, 0xC000, 0x3C80], dtype=np.uint16)).tolist() == [1.0, -2.0, 2.0 ** -6]


def check_unpack_roundtrip(ref):
    rng = np.random.default_rng(7)
    q = rng.integers(0, 16, size=(3, 128)).astype(np.uint8)
    assert np.array_equal(ref.unpack_q4(pack_q4(q)), q)
    words = rng.integers(0, 1 << 32, size=(2, 4), dtype=np.uint64).astype(np.uint32)
    un = ref.unpack_q4(words)
    for r in range(2):
        for c in range(32):
            assert un[r, c] == nibble(words[r, c // 8], c % 8)


def check_qmv_bruteforce(ref):
    """P1: exact rational brute force on tiny random inputs."""
    keys = synth.bank_keys(0, 7, 0)
    for (n, k, rows) in [(3, 64, 1), (5, 128, 3), (8, 128, 2)]:
        codes, scales, biases = synth.q4_rows(keys, 1, n, k, expert=0)
        xb = synth.bf16_bits_from_f32(np.random.default_rng(n + k).standard_normal((rows, k), dtype=np.float32))
        y = ref.qmv(codes, scales, biases, ref.bf16_to_f64(xb))
        ex = exact_qmv(codes, scales, biases, xb)
        for r in range(rows):
            scale = max(abs(float(v)) for v in ex[r])
            for o in range(n):
                assert abs(float(Fraction(float(y[r, o])) - ex[r][o])) <= 1e-13 * scale, (n, k, r, o)


def check_qmv_integer_exact(ref):
    """P2: scales 2^-6, biases m*2^-6, integer x: the result is an exact
    multiple of 2^-6 computed here with Python integers."""
    codes, scales, biases, xb = synth.integer_exact_weight(1, 16, 256, 3)
    y = ref.qmv(codes, scales, biases, ref.bf16_to_f64(xb))
    xi = [[int(bf16_exact(v)) for v in row] for row in xb]
    for r in range(3):
        for o in range(16):
            acc = 0
            for c in range(256):
                g = c // 64
                m = int(bf16_exact(biases[o, g]) * 64)
                acc += xi[r][c] * (nibble(codes[o, c // 8], c % 8) + m)
            assert y[r, o] == acc / 64.0, (r, o)


def check_qmv_closed_forms(ref):
    """Constant codes give W[n, :] = s*c + b per group, so y = sum_g (s_g c + b_g) X_g."""
    n, k = 4, 192
    for c in (0, 7, 15):
        q = np.full((n, k), c, dtype=np.uint8)
        codes = pack_q4(q)
        rng = np.random.default_rng(c)
        sb = synth.bf16_bits_from_f32(rng.uniform(0.005, 0.02, size=(n, 3)).astype(np.float32))
        bb = synth.bf16_bits_from_f32(rng.uniform(-0.1, 0.1, size=(n, 3)).astype(np.float32))
        xb = synth.bf16_bits_from_f32(rng.standard_normal((2, k), dtype=np.float32))
        y = ref.qmv(codes, sb, bb, ref.bf16_to_f64(xb))
        for r in range(2):
            for o in range(n):
                exact = Fraction(0)
                for g in range(3):
                    xs = sum((bf16_exact(v) for v in xb[r, 64 * g:64 * g + 64]), Fraction(0))
                    exact += (bf16_exact(sb[o, g]) * c + bf16_exact(bb[o, g])) * xs
                assert abs(float(Fraction(float(y[r, o])) - exact)) <= 1e-13 * (1 + abs(float(exact)))


def check_qmv_rows_independent(ref):
    """P4: a k-row product equals k serial 1-row products exactly."""
    keys = synth.bank_keys(0, 8, 0)
    codes, scales, biases = synth.q4_rows(keys, 1, 32, 256, expert=0)
    xb = synth.bf16_bits_from_f32(np.random.default_rng(3).standard_normal((9, 256), dtype=np.float32))
    x = ref.bf16_to_f64(xb)
    y = ref.qmv(codes, scales, biases, x)
    for r in range(9):
        assert np.array_equal(y[r], ref.qmv(codes, scales, biases, x[r:r + 1])[0])


# ---------------------------------------------------------------------------
# routing pins
# ---------------------------------------------------------------------------

def check_route_selection(ref):
    """P5: selection against a brute-force full sort, with engineered ties."""
    rng = np.random.default_rng(11)
    for (k, e, topk) in [(3, 16, 4), (9, 256, 8), (9, 512, 10)]:
        l = rng.standard_normal((k, e)).astype(np.float32)
        l[0, :] = np.float32(0.25)                     # all tied
        l[1, 3] = l[1, 1] = l[1, 7] = np.float32(4.0)  # ties at the top
        l[2, 5] = l[2, 9] = np.float32(-0.0)
        l[2, 6] = np.float32(0.0)
        for mode in ("softmax", "sigmoid"):
            idx, _ = ref.route(l, topk, mode, False)
            for r in range(k):
                brute = sorted(range(e), key=lambda j: (-float(l[r, j]), j))[:topk]
                assert list(idx[r]) == brute, (k, e, r)


def check_route_weights(ref):
    """Closed forms: uniform logits give 1/E (softmax) and 1/topk (renorm);
    sigmoid(0) = 1/2; two-expert softmax equals the sigmoid of the gap;
    renormalised weights sum to one; weights follow their slot."""
    e = 64
    l = np.zeros((1, e), dtype=np.float32)
    _, w = ref.route(l, 4, "softmax", False)
    assert np.allclose(w, 1.0 / e, rtol=1e-15, atol=0)
    _, w = ref.route(l, 4, "softmax", True)
    assert np.allclose(w, 0.25, rtol=1e-15, atol=0)
    _, w = ref.route(l, 4, "sigmoid", False)
    assert np.allclose(w, 0.5, rtol=1e-15, atol=0)
    a = np.float32(1.75)
    idx, w = ref.route(np.array([[a, 0.0]], dtype=np.float32), 2, "softmax", False)
    assert list(idx[0]) == [0, 1]
    assert abs(w[0, 0] - 1.0 / (1.0 + math.exp(-float(a)))) < 1e-15
    assert abs(w[0, 1] - 1.0 / (1.0 + math.exp(float(a)))) < 1e-15
    # sigmoid scores 1/2 and 3/4 (logits 0 and ln 3), renormalised: 2/5 and 3/5
    idx, w = ref.route(np.array([[0.0, math.log(3.0)]]), 2, "sigmoid", True)
    assert list(idx[0]) == [1, 0]
    assert abs(w[0, 0] - 0.6) < 1e-15 and abs(w[0, 1] - 0.4) < 1e-15
    rng = np.random.default_rng(5)
    l = rng.standard_normal((9, 512)).astype(np.float32)
    _, w = ref.route(l, 10, "sigmoid", True)
    assert np.allclose(w.sum(axis=1), 1.0, rtol=0, atol=1e-15)
    assert np.all(np.diff(w, axis=1) <= 0)


def check_union_pairs(ref):
    rng = np.random.default_rng(2)
    for (k, e, topk) in [(1, 8, 3), (4, 16, 4), (9, 256, 8), (9, 512, 10)]:
        idx = np.stack([rng.permutation(e)[:topk] for _ in range(k)]).astype(np.int32)
        idx[-1, :2] = idx[0, :2] if k > 1 else idx[-1, :2]  # force sharing
        uid, off, prow, pslot = ref.union_pairs(idx)
        assert list(uid) == sorted(set(idx.ravel().tolist()))
        assert off[0] == 0 and off[-1] == k * topk and len(off) == len(uid) + 1
        seen = set()
        for u, ex in enumerate(uid):
            rows = list(prow[off[u]:off[u + 1]])
            assert rows == sorted(rows)
            expect = [r for r in range(k) if ex in set(idx[r].tolist())]
            assert rows == expect
            for p in range(off[u], off[u + 1]):
                assert idx[prow[p], pslot[p]] == ex
                seen.add((int(prow[p]), int(pslot[p])))
        assert len(seen) == k * topk


# ---------------------------------------------------------------------------
# MoE pins
# ---------------------------------------------------------------------------

def check_swiglu(ref):
    x = np.linspace(-6, 6, 25)
    assert ref.silu(np.array([0.0]))[0] == 0.0
    assert np.allclose(ref.silu(x) - ref.silu(-x), x, rtol=0, atol=1e-14)
    a = np.concatenate([x, np.full_like(x, 2.0)])
    assert np.allclose(ref.swiglu(a), 2.0 * ref.silu(x), rtol=1e-15, atol=0)
    a = np.concatenate([np.zeros(5), np.arange(5.0)])
    assert np.all(ref.swiglu(a) == 0.0)


def _tiny_bank(cfg, kind, e, n, k):
    keys = synth.bank_keys(cfg, kind, 0)
    mats = []
    for ex in range(e):
        c, s, b = synth.q4_rows(keys, e, n, k, expert=ex)
        mats.append((c, s, b))
    return mats


def check_moe_pairs_dense(ref):
    """P6: every (row, slot) output equals the dense product with the selected
    expert's matrices (gathered == dense)."""
    H, I, E, topk, k = 128, 64, 8, 3, 4
    gu = _tiny_bank(5, 1, E, 2 * I, H)
    dn = _tiny_bank(5, 2, E, H, I)
    inp = synth.moe_layer_inputs(5, 0, k, H, E)
    x = ref.bf16_to_f64(inp["x"])
    out = ref.moe_verify(x, inp["logits"], lambda e: ref.dequant(*gu[e]), lambda e: ref.dequant(*dn[e]),
                         topk, "softmax", False)
    for r in range(k):
        for s in range(topk):
            e = int(out["idx"][r, s])
            a = ref.qmv(*gu[e], x[r:r + 1])[0]
            assert np.array_equal(out["h"][r, s], ref.swiglu(a))
            assert np.array_equal(out["partial"][r, s], ref.qmv(*dn[e], out["h"][r, s][None, :].astype(np.float64))[0])


def check_moe_single_expert(ref):
    """E = 1, top-1: the routed weight is exactly 1 and the layer reduces to
    the dense down(swiglu(gate_up x))."""
    H, I, k = 128, 64, 3
    gu = _tiny_bank(6, 1, 1, 2 * I, H)[0]
    dn = _tiny_bank(6, 2, 1, H, I)[0]
    x = ref.bf16_to_f64(synth.moe_layer_inputs(6, 0, k, H, 1)["x"])
    l = np.random.default_rng(0).standard_normal((k, 1)).astype(np.float32)
    for mode, renorm in (("softmax", False), ("sigmoid", True)):
        out = ref.moe_verify(x, l, lambda e: ref.dequant(*gu), lambda e: ref.dequant(*dn), 1, mode, renorm)
        assert np.all(out["w"] == 1.0)
        for r in range(k):
            h = ref.swiglu(ref.qmv(*gu, x[r:r + 1])[0])
            assert np.array_equal(out["y"][r], ref.qmv(*dn, h[None, :])[0])


def check_moe_combine_closed_form(ref):
    """Sigmoid scores 1/2 and 3/4 renormalised to 2/5 and 3/5: y is that
    mix of the two experts' outputs; a zero routed bank with gate logit 0
    leaves half the shared expert."""
    H, I, k = 64, 64, 2
    gu = _tiny_bank(7, 1, 2, 2 * I, H)
    dn = _tiny_bank(7, 2, 2, H, I)
    x = ref.bf16_to_f64(synth.moe_layer_inputs(7, 0, k, H, 2)["x"])
    l = np.array([[0.0, math.log(3.0)], [math.log(3.0), 0.0]])
    out = ref.moe_verify(x, l, lambda e: ref.dequant(*gu[e]), lambda e: ref.dequant(*dn[e]), 2, "sigmoid", True)
    for r in range(k):
        p = [ref.qmv(*dn[e], ref.swiglu(ref.qmv(*gu[e], x[r:r + 1])[0])[None, :])[0] for e in range(2)]
        hi, lo = (1, 0) if r == 0 else (0, 1)
        assert np.allclose(out["y"][r], 0.6 * p[hi] + 0.4 * p[lo], rtol=1e-14, atol=1e-14)
    zero = (np.zeros((2 * I, H // 8), np.uint32), np.zeros((2 * I, 1), np.uint16), np.zeros((2 * I, 1), np.uint16))
    zdn = (np.zeros((H, I // 8), np.uint32), np.zeros((H, 1), np.uint16), np.zeros((H, 1), np.uint16))
    sgu, sdn = gu[0], dn[1]
    out = ref.moe_verify(x, l, lambda e: ref.dequant(*zero), lambda e: ref.dequant(*zdn), 2, "sigmoid", True,
                         z=np.zeros(k), shared_gate_up=ref.dequant(*sgu), shared_down=ref.dequant(*sdn))
    for r in range(k):
        sh = ref.qmv(*sdn, ref.swiglu(ref.qmv(*sgu, x[r:r + 1])[0])[None, :])[0]
        assert np.allclose(out["y"][r], 0.5 * sh, rtol=1e-14, atol=1e-15)


def check_shared_gate_closed_form(ref):
    """The shared expert's scalar gate at z = +-ln 3: sigma(ln 3) = 3 / (3 + 1)
    = 3/4 and sigma(-ln 3) = 1/4.  With no routed contribution the output is
    exactly that fraction of the shared expert's output, through the combine
    alone and through the whole layer; at z = +-40 the gate is 1 and 0 to
    below 1e-17."""
    H, I, k = 64, 64, 2
    ln3 = math.log(3.0)
    rng = np.random.default_rng(41)
    sh = rng.standard_normal((k, H))
    part = np.zeros((k, 3, H))
    w = rng.uniform(0.1, 1.0, (k, 3))
    y = ref.combine(part, w, shared=sh, z=np.array([ln3, -ln3]))
    assert np.allclose(y[0], 0.75 * sh[0], rtol=1e-15, atol=1e-16)
    assert np.allclose(y[1], 0.25 * sh[1], rtol=1e-15, atol=1e-16)
    y = ref.combine(part, w, shared=sh, z=np.array([40.0, -40.0]))
    assert np.allclose(y[0], sh[0], rtol=1e-15, atol=0.0)
    assert np.max(np.abs(y[1])) <= 1e-17 * np.max(np.abs(sh[1]))
    gu = _tiny_bank(7, 1, 2, 2 * I, H)
    dn = _tiny_bank(7, 2, 2, H, I)
    x = ref.bf16_to_f64(synth.moe_layer_inputs(7, 0, k, H, 2)["x"])
    l = np.array([[0.0, ln3], [ln3, 0.0]])
    zero = (np.zeros((2 * I, H // 8), np.uint32), np.zeros((2 * I, 1), np.uint16), np.zeros((2 * I, 1), np.uint16))
    zdn = (np.zeros((H, I // 8), np.uint32), np.zeros((H, 1), np.uint16), np.zeros((H, 1), np.uint16))
    sgu, sdn = gu[1], dn[0]
    out = ref.moe_verify(x, l, lambda e: ref.dequant(*zero), lambda e: ref.dequant(*zdn), 2, "sigmoid", True,
                         z=np.array([-ln3, ln3]), shared_gate_up=ref.dequant(*sgu), shared_down=ref.dequant(*sdn))
    for r, frac in ((0, 0.25), (1, 0.75)):
        s = ref.qmv(*sdn, ref.swiglu(ref.qmv(*sgu, x[r:r + 1])[0])[None, :])[0]
        assert np.allclose(out["y"][r], frac * s, rtol=1e-14, atol=1e-15)


def check_moe_identical_experts(ref):
    """Identical experts: the weights sum to one, so the layer output is the
    single expert's output (softmax over all experts with top-k = E, or any
    top-k with renormalisation)."""
    H, I, E, k = 64, 64, 4, 3
    gu = _tiny_bank(8, 1, 1, 2 * I, H)[0]
    dn = _tiny_bank(8, 2, 1, H, I)[0]
    x = ref.bf16_to_f64(synth.moe_layer_inputs(8, 0, k, H, E)["x"])
    l = np.random.default_rng(1).standard_normal((k, E)).astype(np.float32)
    for topk, mode, renorm in ((E, "softmax", False), (2, "sigmoid", True), (3, "softmax", True)):
        out = ref.moe_verify(x, l, lambda e: ref.dequant(*gu), lambda e: ref.dequant(*dn), topk, mode, renorm)
        for r in range(k):
            d = ref.qmv(*dn, ref.swiglu(ref.qmv(*gu, x[r:r + 1])[0])[None, :])[0]
            assert np.allclose(out["y"][r], d, rtol=1e-13, atol=1e-13)


# ---------------------------------------------------------------------------
# GDN pins
# ---------------------------------------------------------------------------

def _dyadic(rng, shape, denom=8, lo=-8, hi=8):
    return rng.integers(lo, hi + 1, size=shape) / float(denom)


def exact_gdn(S, q, k, v, g, beta, ratio):
    """Fractions brute force of the recurrence with explicit index loops."""
    hv, dv, dk = len(S), len(S[0]), len(S[0][0])
    S = [[[Fraction(S[h][i][j]) for j in range(dk)] for i in range(dv)] for h in range(hv)]
    ys, snaps = [], []
    for t in range(len(q)):
        yt = []
        for h in range(hv):
            c = h // ratio
            gg, bb = Fraction(g[t][h]), Fraction(beta[t][h])
            kk = [Fraction(k[t][c][j]) for j in range(dk)]
            qq = [Fraction(q[t][c][j]) for j in range(dk)]
            for i in range(dv):
                for j in range(dk):
                    S[h][i][j] = gg * S[h][i][j]
            for i in range(dv):
                m = sum((S[h][i][j] * kk[j] for j in range(dk)), Fraction(0))
                d = bb * (Fraction(v[t][h][i]) - m)
                for j in range(dk):
                    S[h][i][j] += d * kk[j]
            yt.append([sum((S[h][i][j] * qq[j] for j in range(dk)), Fraction(0)) for i in range(dv)])
        ys.append(yt)
        snaps.append([[list(row) for row in S[h]] for h in range(hv)])
    return ys, snaps


def check_gdn_bruteforce(ref):
    """P7: exact rationals on tiny dyadic cases (all fp64 steps exact there)."""
    rng = np.random.default_rng(17)
    for (hv, hk, dk, dv, rows) in [(2, 1, 3, 2, 3), (2, 2, 4, 4, 2), (4, 2, 2, 3, 3)]:
        S = _dyadic(rng, (hv, dv, dk))
        q = _dyadic(rng, (rows, hk, dk), 4, -4, 4)
        k = _dyadic(rng, (rows, hk, dk), 4, -4, 4)
        v = _dyadic(rng, (rows, hv, dv))
        g = rng.choice([0.5, 0.75, 1.0], size=(rows, hv))
        beta = rng.choice([0.25, 0.5, 1.0], size=(rows, hv))
        y, snaps = ref.gdn_verify(S, q, k, v, g, beta)
        ey, es = exact_gdn(S.tolist(), q.tolist(), k.tolist(), v.tolist(), g.tolist(), beta.tolist(), hv // hk)
        for t in range(rows):
            for h in range(hv):
                for i in range(dv):
                    assert Fraction(float(y[t, h, i])) == ey[t][h][i], (t, h, i)
                    for j in range(dk):
                        assert Fraction(float(snaps[t, h, i, j])) == es[t][h][i][j]


def check_gdn_no_write(ref):
    """P8: beta = 0 leaves only the decay: S_t = (g_0 ... g_t) S_in, y = S_t q."""
    rng = np.random.default_rng(4)
    hv, hk, d, rows = 4, 2, 8, 5
    S = rng.standard_normal((hv, d, d))
    inp = synth.gdn_layer_inputs(9, 0, rows, hv, hk, d, d)
    beta = np.zeros((rows, hv))
    y, snaps = ref.gdn_verify(S, inp["q"], inp["k"], inp["v"], inp["g"], beta)
    prod = np.ones(hv)
    for t in range(rows):
        prod = prod * inp["g"][t].astype(np.float64)
        for h in range(hv):
            assert np.allclose(snaps[t, h], prod[h] * S[h], rtol=1e-14, atol=1e-15)
            assert np.allclose(y[t, h], (prod[h] * S[h]) @ inp["q"][t, h // 2].astype(np.float64),
                               rtol=1e-13, atol=1e-14)


def check_gdn_scalar(ref):
    """Dk = Dv = 1: S' = g S (1 - beta k^2) + beta v k, y = S' q."""
    rng = np.random.default_rng(8)
    for _ in range(5):
        S0, q, k, v, g, b = rng.uniform(-1, 1, 6)
        g, b = abs(g), abs(b)
        y, snaps = ref.gdn_verify([[[S0]]], [[[q]]], [[[k]]], [[[v]]], [[g]], [[b]])
        s1 = g * S0 * (1 - b * k * k) + b * v * k
        assert abs(snaps[0, 0, 0, 0] - s1) < 1e-15
        assert abs(y[0, 0, 0] - s1 * q) < 1e-15


def check_gdn_basis(ref):
    """P9: g = beta = 1 and k = e_j: column j of every head becomes v exactly,
    every other column is unchanged."""
    rng = np.random.default_rng(9)
    hv, hk, d = 3, 1, 6
    S = _dyadic(rng, (hv, d, d))
    for j in range(d):
        kk = np.zeros((1, hk, d)); kk[0, 0, j] = 1.0
        q = _dyadic(rng, (1, hk, d))
        v = _dyadic(rng, (1, hv, d))
        y, snaps = ref.gdn_verify(S, q, kk, v, np.ones((1, hv)), np.ones((1, hv)))
        for h in range(hv):
            assert np.array_equal(snaps[0, h, :, j], v[0, h])
            other = [c for c in range(d) if c != j]
            assert np.array_equal(snaps[0, h][:, other], S[h][:, other])


def check_gdn_retrieval(ref):
    """P10: the delta rule writes v under key k: with g = beta = 1 and a unit
    key, reading the new state with k returns v."""
    rng = np.random.default_rng(10)
    hv, hk, d = 6, 2, 16
    S = rng.standard_normal((hv, d, d))
    inp = synth.gdn_layer_inputs(10, 0, 1, hv, hk, d, d)
    y, snaps = ref.gdn_verify(S, inp["q"], inp["k"], inp["v"], np.ones((1, hv)), np.ones((1, hv)))
    for h in range(hv):
        got = snaps[0, h] @ inp["k"][0, h // 3].astype(np.float64)
        n2 = float(np.dot(inp["k"][0, h // 3].astype(np.float64), inp["k"][0, h // 3].astype(np.float64)))
        # exact identity for any key: S' k = v n2 + (S k)(1 - n2)
        sk = S[h] @ inp["k"][0, h // 3].astype(np.float64)
        vh = inp["v"][0, h].astype(np.float64)
        assert np.allclose(got, vh * n2 + sk * (1 - n2), rtol=1e-12, atol=1e-12)
        assert np.allclose(got, inp["v"][0, h], rtol=0, atol=1e-5)


def check_gdn_head_groups(ref):
    """Hk < Hv equals the Hk = Hv run with each qk head repeated over its
    contiguous group of Hv/Hk value heads."""
    hv, hk, d, rows = 6, 2, 8, 3
    inp = synth.gdn_layer_inputs(11, 0, rows, hv, hk, d, d)
    S = synth.gdn_state(11, 0, hv, d, d)
    y1, s1 = ref.gdn_verify(S, inp["q"], inp["k"], inp["v"], inp["g"], inp["beta"])
    qe = np.repeat(inp["q"], hv // hk, axis=1)
    ke = np.repeat(inp["k"], hv // hk, axis=1)
    y2, s2 = ref.gdn_verify(S, qe, ke, inp["v"], inp["g"], inp["beta"])
    assert np.array_equal(y1, y2) and np.array_equal(s1, s2)


def check_gdn_rollback(ref):
    """P11 + P12: rollback to every prefix j equals a fresh j-row run; the
    input state is not modified."""
    hv, hk, d, rows = 4, 2, 8, 9
    inp = synth.gdn_layer_inputs(12, 0, rows, hv, hk, d, d)
    S = synth.gdn_state(12, 0, hv, d, d)
    S_copy = S.copy()
    y, snaps = ref.gdn_verify(S, inp["q"], inp["k"], inp["v"], inp["g"], inp["beta"])
    assert np.array_equal(S, S_copy)
    for j in range(rows + 1):
        st = ref.rollback(S, snaps, j)
        if j == 0:
            assert np.array_equal(st, S.astype(np.float64))
            continue
        yj, sj = ref.gdn_verify(S, *(inp[n][:j] for n in ("q", "k", "v", "g", "beta")))
        assert np.array_equal(st, sj[-1])
        assert np.array_equal(yj, y[:j])
    for bad in (-1, rows + 1):
        try:
            ref.rollback(S, snaps, bad)
        except ValueError:
            pass
        else:
            raise AssertionError("rollback accepted an out-of-range prefix")


# ---------------------------------------------------------------------------
# acceptance
# ---------------------------------------------------------------------------

def _scan_argmax(row):
    """Independent scan: first index of the largest non-NaN value (-1 if none)."""
    best, arg = None, -1
    for i, v in enumerate(row):
        v = float(v)
        if math.isnan(v):
            continue
        if best is None or v > best:
            best, arg = v, i
    return arg


def check_sample_greedy(ref):
    """P13: greedy tokens equal an element-by-element scan: ties (including
    -0 against +0 and equal infinities) go to the lower index, NaN is never
    chosen, an all-NaN row gives -1."""
    nan, inf = float("nan"), float("inf")
    rows = np.array([[0.5, 2.0, 2.0, -1.0, 1.0],
                     [nan, -3.0, nan, -3.0, -4.0],
                     [-0.0, 0.0, -1.0, -2.0, -0.0],
                     [nan, nan, nan, nan, nan],
                     [-inf, inf, 3.0, inf, nan],
                     [-inf, -inf, -inf, -inf, -inf]], dtype=np.float32)
    got = ref.sample_tokens(rows)
    assert [int(t) for t in got] == [_scan_argmax(r) for r in rows] == [1, 1, 0, -1, 1, 0]
    rng = np.random.default_rng(7)
    rnd = rng.integers(-3, 4, size=(40, 12)).astype(np.float32)  # many ties
    assert [int(t) for t in ref.sample_tokens(rnd)] == [_scan_argmax(r) for r in rnd]


def check_sample_noise_rounding(ref):
    """P13: with noise, z is fp32(fp32(l * inv_temp) + g) with each operation
    rounded; near-ties decided in fp32 match a scalar fp32 evaluation."""
    rng = np.random.default_rng(8)
    l = rng.standard_normal((30, 16)).astype(np.float32)
    g = rng.gumbel(size=(30, 16)).astype(np.float32)
    inv_t = np.float32(0.7)
    expect = []
    for r in range(30):
        z = [np.float32(np.float32(l[r, i] * inv_t) + g[r, i]) for i in range(16)]
        expect.append(_scan_argmax(z))
    assert [int(t) for t in ref.sample_tokens(l, g, float(inv_t))] == expect


def check_sample_gumbel_is_softmax(ref):
    """P14: Gumbel-max sampling: over many noise draws the token frequencies
    match softmax(l * inv_temp) (chi-square with 5 degrees of freedom below
    40, p ~ 1e-7 for a correct sampler)."""
    l = np.array([0.0, 1.0, 2.0, 3.0, -1.0, 0.5], dtype=np.float32)
    inv_t = 0.7
    n = 40000
    g = np.random.default_rng(9).gumbel(size=(n, l.size)).astype(np.float32)
    toks = ref.sample_tokens(np.broadcast_to(l, (n, l.size)), g, inv_t)
    counts = np.bincount(toks, minlength=l.size).astype(float)
    w = [math.exp(inv_t * float(x)) for x in l]
    p = [x / sum(w) for x in w]
    chi2 = sum((counts[i] - n * p[i]) ** 2 / (n * p[i]) for i in range(l.size))
    assert chi2 < 40.0, chi2


def check_accept_cases(ref):
    """P15: acceptance stops at the first draft that differs from the token
    sampled from the previous row, and at a draft equal to the end-of-answer
    token even when it matches; no drafts (one row) accepts none."""
    cases = [
        ([5, 6, 7, 8], [5, 6, 7], -1, 3),
        ([5, 6, 7, 8], [4, 6, 7], -1, 0),
        ([5, 6, 7, 8], [5, 9, 7], -1, 1),
        ([5, 6, 7, 8], [5, 6, 1], -1, 2),
        ([5, 6, 7, 8], [5, 6, 7], 6, 1),   # row 2's draft is the end-of-answer token
        ([5, 6, 7, 8], [5, 6, 7], 5, 0),
        ([5], [], 3, 0),
        ([-1, 4], [-1], -1, 1),            # an all-NaN row's token still compares by value
    ]
    for tokens, drafts, eos, n in cases:
        assert ref.accept(tokens, drafts, eos) == n, (tokens, drafts, eos)


def check_verify_cycle_rollback(ref):
    """P16: the emitted tokens are the accepted drafts and then the token
    sampled after them, and rolling the GDN state back to the accepted prefix
    equals a fresh run over those rows only."""
    hv, hk, d, rows = 4, 2, 8, 6
    inp = synth.gdn_layer_inputs(13, 0, rows, hv, hk, d, d)
    S = synth.gdn_state(13, 0, hv, d, d)
    y, snaps = ref.gdn_verify(S, inp["q"], inp["k"], inp["v"], inp["g"], inp["beta"])
    for planted in range(rows):
        logits, drafts, _ = synth.verify_block(13, planted, rows, 50, accepted=planted)
        out = ref.verify_cycle(logits, drafts)
        n = out["accepted"]
        assert n == planted
        toks = [_scan_argmax(r) for r in logits]
        assert out["emitted"] == [int(x) for x in drafts[:n]] + [toks[n]]
        assert out["prefix"] == n + 1
        st = ref.rollback(S, snaps, out["prefix"])
        _, sj = ref.gdn_verify(S, *(inp[m][:n + 1] for m in ("q", "k", "v", "g", "beta")))
        assert np.array_equal(st, sj[-1])


# ---------------------------------------------------------------------------
# GDN preparation and tail
# ---------------------------------------------------------------------------

def _prep(ref, raw, hk, hv, dk, dv, **kw):
    return ref.gdn_prepare(raw["qkv"], raw["hist"], raw["conv_w"], raw["a"], raw["b"], raw["A_log"],
                           raw["dt_bias"], hk, hv, dk, dv, **kw)


def check_conv_is_convolution(ref):
    """P17: the v channels (no norm) of the preparation are numpy's 'valid'
    convolution of [history; inputs] with the reversed taps."""
    hk, hv, dk, dv, rows = 1, 2, 4, 3, 5
    raw = synth.gdn_raw_inputs(14, 0, rows, hv, hk, dk, dv)
    out = _prep(ref, raw, hk, hv, dk, dv)
    X = np.concatenate([raw["hist"], raw["qkv"]]).astype(np.float64)
    v = out["v"].reshape(rows, hv * dv)
    for j in range(hv * dv):
        c = 2 * hk * dk + j
        expect = np.convolve(X[:, c], raw["conv_w"][c, ::-1].astype(np.float64), mode="valid")
        assert np.allclose(v[:, j], expect, rtol=1e-13, atol=1e-13)
    assert np.array_equal(out["window"], X)


def check_conv_alignment(ref):
    """P17: a tap on the current input passes the rows through; a tap three
    steps back passes the history, then the rows, through; with act silu the
    pass-through is x / (1 + e^-x)."""
    hk, hv, dk, dv, rows = 1, 1, 2, 2, 5
    raw = synth.gdn_raw_inputs(15, 0, rows, hv, hk, dk, dv)
    C = raw["qkv"].shape[1]
    for tap, shift in ((3, 0), (0, 3), (2, 1)):
        w = np.zeros((C, 4), dtype=np.float32)
        w[:, tap] = 1.0
        out = ref.gdn_prepare(raw["qkv"], raw["hist"], w, raw["a"], raw["b"], raw["A_log"], raw["dt_bias"],
                              hk, hv, dk, dv)
        X = np.concatenate([raw["hist"], raw["qkv"]]).astype(np.float64)
        assert np.array_equal(out["v"].reshape(rows, -1), X[3 - shift:3 - shift + rows, 2 * hk * dk:])
        act = ref.gdn_prepare(raw["qkv"], raw["hist"], w, raw["a"], raw["b"], raw["A_log"], raw["dt_bias"],
                              hk, hv, dk, dv, act="silu")
        xs = X[3 - shift:3 - shift + rows, 2 * hk * dk:]
        assert np.allclose(act["v"].reshape(rows, -1), xs / (1.0 + np.exp(-xs)), rtol=1e-14)


def check_conv_history_chain(ref):
    """P18: continuing from the history after an accepted prefix j
    (window[j:j+3]) gives the later rows exactly as one call over all rows."""
    hk, hv, dk, dv, rows = 1, 2, 4, 4, 7
    raw = synth.gdn_raw_inputs(16, 0, rows, hv, hk, dk, dv)
    full = _prep(ref, raw, hk, hv, dk, dv, act="silu")
    for j in range(rows + 1):
        part = dict(raw)
        part["qkv"] = raw["qkv"][j:]
        part["hist"] = full["window"][j:j + 3]
        part["a"], part["b"] = raw["a"][j:], raw["b"][j:]
        if j == rows:
            assert np.array_equal(full["window"][rows:rows + 3], np.concatenate([raw["hist"], raw["qkv"]])[-3:])
            continue
        out = _prep(ref, part, hk, hv, dk, dv, act="silu")
        for n in ("q", "k", "v", "g", "beta"):
            assert np.array_equal(out[n], full[n][j:]), (n, j)


def check_qk_l2_norm(ref):
    """P19: with eps = 0 every (row, head) of q and k has unit norm and the
    direction of the conv output; eps enters as sqrt(sum + eps)."""
    hk, hv, dk, dv, rows = 2, 2, 8, 2, 3
    raw = synth.gdn_raw_inputs(17, 0, rows, hv, hk, dk, dv)
    w = np.zeros((raw["qkv"].shape[1], 4), dtype=np.float32)
    w[:, 3] = 1.0
    raw["conv_w"] = w
    out = _prep(ref, raw, hk, hv, dk, dv, eps=0.0)
    for n, off in (("q", 0), ("k", hk * dk)):
        t = out[n]
        assert np.allclose((t * t).sum(-1), 1.0, rtol=1e-14)
        src = raw["qkv"][:, off:off + hk * dk].reshape(rows, hk, dk).astype(np.float64)
        assert np.allclose(t * np.linalg.norm(src, axis=-1, keepdims=True), src, rtol=1e-13)
    big = _prep(ref, raw, hk, hv, dk, dv, eps=3.0)
    src = raw["qkv"][:, :hk * dk].reshape(rows, hk, dk).astype(np.float64)
    assert np.allclose(big["q"], src / np.sqrt((src * src).sum(-1, keepdims=True) + 3.0), rtol=1e-14)


def check_gates(ref):
    """P20: beta = sigmoid(b); with A_log = 0 the decay is exp(-softplus(a +
    dt)) = 1 / (1 + e^(a + dt)); with A_log = log 2 it is the square of that;
    softplus(x) - softplus(-x) = x and softplus(0) = log 2."""
    hk, hv, dk, dv, rows = 1, 3, 2, 2, 4
    raw = synth.gdn_raw_inputs(18, 0, rows, hv, hk, dk, dv)
    for alog, power in ((0.0, 1), (math.log(2.0), 2)):
        raw["A_log"] = np.full(hv, alog, dtype=np.float64)
        out = _prep(ref, raw, hk, hv, dk, dv)
        x = raw["a"].astype(np.float64) + raw["dt_bias"].astype(np.float64)[None, :]
        assert np.allclose(out["g"], (1.0 / (1.0 + np.exp(x))) ** power, rtol=1e-13)
        b = raw["b"].astype(np.float64)
        assert np.allclose(out["beta"], np.exp(b) / (1.0 + np.exp(b)), rtol=1e-14)
    xs = np.linspace(-30, 30, 61)
    assert np.allclose(ref.softplus(xs) - ref.softplus(-xs), xs, atol=1e-12)
    assert abs(float(ref.softplus(0.0)) - math.log(2.0)) < 1e-15


def check_gated_norm(ref):
    """P21: a constant row c normalises to c / sqrt(c^2 + eps); with eps = 0
    the norm is scale-free and has unit rms; sigmoid(0) halves, silu(0)
    zeroes, and the weight multiplies elementwise."""
    rng = np.random.default_rng(19)
    y = rng.standard_normal((3, 2, 6))
    z = rng.standard_normal((3, 2, 6))
    w = rng.uniform(0.5, 1.5, 6)
    c = np.full((1, 1, 6), -2.5)
    out = ref.gdn_gated_norm(c, np.zeros_like(c), np.ones(6), eps=0.25)
    assert np.allclose(out, 0.5 * (-2.5) / math.sqrt(6.25 + 0.25), rtol=1e-14)
    big = np.full_like(z, 60.0)
    n1 = ref.gdn_gated_norm(y, big, np.ones(6), eps=0.0)
    assert np.allclose(np.sqrt((n1 * n1).mean(-1)), 1.0, rtol=1e-12)
    assert np.allclose(ref.gdn_gated_norm(7.0 * y, big, np.ones(6), eps=0.0), n1, rtol=1e-12)
    assert np.allclose(ref.gdn_gated_norm(y, big, w, eps=0.0), n1 * w, rtol=1e-12)
    assert np.array_equal(ref.gdn_gated_norm(y, np.zeros_like(z), w, act="silu"), np.zeros_like(y))
    half = ref.gdn_gated_norm(y, np.zeros_like(z), w, act="sigmoid")
    assert np.allclose(half, 0.5 * ref.gdn_gated_norm(y, big, w), rtol=1e-12)
    # Both gates at z = +-ln 3 on a constant row: sigmoid gives 3/4 and 1/4,
    # silu(z) = z * sigmoid(z) gives (3/4) ln 3 and -(1/4) ln 3.
    ln3 = math.log(3.0)
    n0 = -2.5 / math.sqrt(6.25 + 0.25)
    zz = np.array([ln3, -ln3]).reshape(2, 1, 1) * np.ones((2, 1, 6))
    cc = np.full((2, 1, 6), -2.5)
    sig = ref.gdn_gated_norm(cc, zz, np.ones(6), act="sigmoid", eps=0.25)
    assert np.allclose(sig[0], 0.75 * n0, rtol=1e-14) and np.allclose(sig[1], 0.25 * n0, rtol=1e-14)
    sl = ref.gdn_gated_norm(cc, zz, np.ones(6), act="silu", eps=0.25)
    assert np.allclose(sl[0], 0.75 * ln3 * n0, rtol=1e-14) and np.allclose(sl[1], -0.25 * ln3 * n0, rtol=1e-14)
    # silu's limits: silu(z) / z -> 1 for large z, -> 0 for large -z.
    zl = np.full((2, 1, 6), 40.0)
    zl[1] = -40.0
    sl = ref.gdn_gated_norm(cc, zl, np.ones(6), act="silu", eps=0.25)
    assert np.allclose(sl[0], 40.0 * n0, rtol=1e-15) and np.max(np.abs(sl[1])) < 1e-15


def half_exact(bits):
    """Exact value of an IEEE binary16 bit pattern, decoded by Python's struct
    module (format 'e')."""
    return Fraction(struct.unpack("<e", struct.pack("<H", int(bits)))[0])


def check_fp16_decode(ref):
    """Q8_0 scales: every 97th finite half pattern against struct's decoder,
    and the special values."""
    pats = [p for p in range(0, 65536, 97) if (p >> 10) & 31 != 31]
    got = ref.fp16_to_f64(np.array(pats, dtype=np.uint16))
    for p, g in zip(pats, got):
        assert Fraction(float(g)) == half_exact(p), hex(p)
    sp = ref.fp16_to_f64(np.array([0x7C00, 0xFC00, 0x7E00, 0x0001, 0x8000, 0x3C00, 0x03FF, 0x7BFF], dtype=np.uint16))
    assert sp[0] == np.inf and sp[1] == -np.inf and np.isnan(sp[2])
    assert sp[3] == 2.0 ** -24 and sp[4] == 0.0 and np.signbit(sp[4]) and sp[5] == 1.0
    assert sp[6] == 1023 * 2.0 ** -24 and sp[7] == 65504.0


def check_q8_0_bruteforce(ref):
    """Q8_0 product: exact rational brute force on tiny inputs (codes over the
    whole int8 range, one scale per 32 inputs)."""
    for (n, k, rows) in [(3, 64, 1), (4, 96, 2), (2, 32, 3)]:
        qs, d = synth.q8_0_weight(0, 9, n + k, 1, n, k)
        qs, d = qs[0], d[0]
        qs[0, :3] = np.array([-128, 127, 0], dtype=np.int8)
        xb = synth.bf16_bits_from_f32(np.random.default_rng(n * k).standard_normal((rows, k), dtype=np.float32))
        y = ref.qmv_q8_0(qs, d, ref.bf16_to_f64(xb))
        for r in range(rows):
            ex = [sum(half_exact(d[o, c // 32]) * int(qs[o, c]) * bf16_exact(xb[r, c]) for c in range(k))
                  for o in range(n)]
            scale = max(abs(float(v)) for v in ex)
            for o in range(n):
                assert abs(float(Fraction(float(y[r, o])) - ex[o])) <= 1e-13 * scale, (n, k, r, o)


def check_q8_0_blocks(ref):
    """Unit activations read single weights: with x = e_c, y[n] = d[n, c // 32]
    * q[n, c] exactly, so every block boundary and the sign of every code are
    checked."""
    n, k = 3, 128
    qs, d = synth.q8_0_weight(0, 10, 0, 1, n, k)
    qs, d = qs[0], d[0]
    for c in (0, 31, 32, 63, 64, 127):
        x = np.zeros((1, k))
        x[0, c] = 1.0
        y = ref.qmv_q8_0(qs, d, x)[0]
        for o in range(n):
            assert Fraction(float(y[o])) == half_exact(d[o, c // 32]) * int(qs[o, c]), (c, o)


def pack_q3_ints(q):
    """Independent packer: codes of one row summed into a Python integer at
    bit 3c, written out little-endian."""
    v = 0
    for c, code in enumerate(q):
        v |= int(code) << (3 * c)
    return np.frombuffer(v.to_bytes(3 * len(q) // 8, "little"), dtype=np.uint8)


def check_q3_unpack_roundtrip(ref):
    """Affine Q3: packed rows from the independent packer unpack to the codes,
    and every byte boundary (codes straddling bytes) is covered."""
    rng = np.random.default_rng(30)
    for k in (8, 64, 192):
        rows = rng.integers(0, 8, size=(3, k))
        packed = np.stack([pack_q3_ints(r) for r in rows])
        assert np.array_equal(ref.unpack_q3(packed), rows.astype(np.uint8)), k
    # all eight codes in one three-byte triplet, in order
    assert np.array_equal(ref.unpack_q3(pack_q3_ints(list(range(8)))[None])[0], np.arange(8))


def check_q3_bruteforce(ref):
    """Affine Q3 product: exact rational brute force (codes from the
    independent packer)."""
    rng = np.random.default_rng(31)
    for (n, k, rows) in [(3, 64, 1), (4, 128, 2)]:
        q = rng.integers(0, 8, size=(n, k))
        codes = np.stack([pack_q3_ints(r) for r in q])
        sc = synth.bf16_bits_from_f32(rng.uniform(0.01, 0.04, size=(n, k // 64)).astype(np.float32))
        bi = synth.bf16_bits_from_f32(rng.uniform(-0.1, 0.1, size=(n, k // 64)).astype(np.float32))
        xb = synth.bf16_bits_from_f32(rng.standard_normal((rows, k), dtype=np.float32))
        y = ref.qmv_q3(codes, sc, bi, ref.bf16_to_f64(xb))
        for r in range(rows):
            ex = [sum((bf16_exact(sc[o, c // 64]) * int(q[o, c]) + bf16_exact(bi[o, c // 64])) * bf16_exact(xb[r, c])
                      for c in range(k)) for o in range(n)]
            scale = max(abs(float(v)) for v in ex)
            for o in range(n):
                assert abs(float(Fraction(float(y[r, o])) - ex[o])) <= 1e-13 * scale, (n, k, r, o)


def check_q3_closed_form(ref):
    """Constant 3-bit codes c give y = sum_g (s_g c + b_g) X_g."""
    n, k = 3, 128
    rng = np.random.default_rng(32)
    for c in (0, 5, 7):
        codes = np.stack([pack_q3_ints([c] * k) for _ in range(n)])
        sc = synth.bf16_bits_from_f32(rng.uniform(0.01, 0.04, size=(n, 2)).astype(np.float32))
        bi = synth.bf16_bits_from_f32(rng.uniform(-0.1, 0.1, size=(n, 2)).astype(np.float32))
        xb = synth.bf16_bits_from_f32(rng.standard_normal((1, k), dtype=np.float32))
        y = ref.qmv_q3(codes, sc, bi, ref.bf16_to_f64(xb))[0]
        xs = [sum(bf16_exact(v) for v in xb[0, 64 * g:64 * (g + 1)]) for g in range(2)]
        for o in range(n):
            ex = sum((bf16_exact(sc[o, g]) * c + bf16_exact(bi[o, g])) * xs[g] for g in range(2))
            assert abs(float(Fraction(float(y[o])) - ex)) <= 1e-13 * max(1.0, abs(float(ex))), (c, o)


ALL_CHECKS = [
    check_bf16_decode, check_unpack_roundtrip, check_qmv_bruteforce, check_qmv_integer_exact,
    check_qmv_closed_forms, check_qmv_rows_independent, check_route_selection, check_route_weights,
    check_union_pairs, check_swiglu, check_moe_pairs_dense, check_moe_single_expert,
    check_moe_combine_closed_form, check_shared_gate_closed_form, check_moe_identical_experts, check_gdn_bruteforce,
    check_gdn_no_write, check_gdn_scalar, check_gdn_basis, check_gdn_retrieval,
    check_gdn_head_groups, check_gdn_rollback, check_sample_greedy, check_sample_noise_rounding,
    check_sample_gumbel_is_softmax, check_accept_cases, check_verify_cycle_rollback,
    check_conv_is_convolution, check_conv_alignment, check_conv_history_chain, check_qk_l2_norm, check_gates,
    check_gated_norm, check_fp16_decode, check_q8_0_bruteforce, check_q8_0_blocks, check_q3_unpack_roundtrip,
    check_q3_bruteforce, check_q3_closed_form,
]
