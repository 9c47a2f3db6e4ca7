"""Python binding of libsdv: argument marshalling over the C ABI.

Every function checks that the tensors it is handed are CUDA, contiguous, of
the expected dtype and large enough for the sizes it passes, then calls the
matching ``sdv_*`` entry point on the current stream.  All arithmetic runs in
the library's HIP kernels; nothing here computes results.
"""

import ctypes
from collections import namedtuple

import torch

from ._lib import (ACT_BF16, ACT_F32, CONV_NONE, CONV_SILU, FMT_AFFINE_Q3, FMT_AFFINE_Q4, FMT_Q8_0, GATE_SIGMOID,
                   GATE_SILU, MODE_GATEUP_SWIGLU, MODE_PLAIN, ROUTE_SIGMOID, ROUTE_SOFTMAX, SdvError, SdvGdnLayer,
                   SdvQ3, SdvQ4, SdvQ4T, SdvQ8_0, check, lib)

__all__ = ["Q4Weight", "Q8Weight", "Q3Weight", "TiledQ4", "FMT_AFFINE_Q4", "FMT_Q8_0", "FMT_AFFINE_Q3", "RouteResult", "qmv_k", "moe_route_k", "gather_qmv_k", "moe_experts_k", "moe_route_experts_k", "moe_combine_k",
           "gdn_verify_k", "gdn_rollback", "gdn_rollback_copy", "gdn_prepare_k", "gdn_verify_prep_k", "gdn_verify_prep_norm_k", "gdn_norm_counters", "gdn_gated_norm_k", "GdnLayersLaunch",
           "CONV_NONE", "CONV_SILU", "GATE_SIGMOID", "GATE_SILU", "SdvError", "MODE_PLAIN",
           "MODE_GATEUP_SWIGLU", "ACT_BF16", "ACT_F32", "ROUTE_SOFTMAX", "ROUTE_SIGMOID"]

RouteResult = namedtuple("RouteResult", "idx w union_ids n_union pair_off pair_row pair_slot")


def _stream(t):
    return ctypes.c_void_p(torch.cuda.current_stream(t.device).cuda_stream)


def _need(t, name, dtype, numel=None, device=None):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a CUDA (HIP) tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if numel is not None and t.numel() < numel:
        raise ValueError(f"{name} holds {t.numel()} elements, needs {numel}")
    if device is not None and t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    return ctypes.c_void_p(t.data_ptr())


class Q4Weight:
    """Affine-Q4/g64 weights on the device: codes int32 (bit patterns of the
    u32 words) [E, N, K/8], scales and biases int16 (bf16 bits) [E, N, K/64].
    A 2-D layout [N, K/8] is a dense matrix (E = 1)."""

    def __init__(self, codes, scales, biases):
        if codes.dim() == 2:
            codes, scales, biases = codes[None], scales[None], biases[None]
        if codes.dim() != 3 or scales.shape != biases.shape or scales.dim() != 3:
            raise ValueError("codes [E,N,K/8], scales/biases [E,N,K/64] expected")
        self.E, self.N, kw = codes.shape
        self.K = kw * 8
        if scales.shape != (self.E, self.N, self.K // 64):
            raise ValueError(f"scales shape {tuple(scales.shape)} does not match codes {tuple(codes.shape)}")
        self.codes, self.scales, self.biases = codes, scales, biases
        self.device = codes.device
        self._desc = SdvQ4(_need(codes, "codes", torch.int32).value,
                           _need(scales, "scales", torch.int16, device=self.device).value,
                           _need(biases, "biases", torch.int16, device=self.device).value,
                           self.E, self.N, self.K, 64)

    @property
    def desc(self):
        return ctypes.byref(self._desc)

    def nbytes(self):
        return self.E * self.N * (self.K // 2 + (self.K // 64) * 4)

    def tiled(self, fused_gateup=False):
        """The weight rewritten on the device into the tiled layout the
        products read (sdv_q4_repack)."""
        return TiledQ4.from_rowmajor(self, fused_gateup)


class Q3Weight:
    """Affine-Q3/g64 weights on the device: codes uint8 [E, N, 3K/8] (a
    little-endian 3-bit stream per row), scales and biases int16 (bf16 bits)
    [E, N, K/64].  A 2-D layout is a dense matrix (E = 1)."""

    def __init__(self, codes, scales, biases):
        if codes.dim() == 2:
            codes, scales, biases = codes[None], scales[None], biases[None]
        if codes.dim() != 3 or scales.shape != biases.shape or scales.dim() != 3:
            raise ValueError("codes [E,N,3K/8], scales/biases [E,N,K/64] expected")
        self.E, self.N, nb = codes.shape
        self.K = nb * 8 // 3
        if nb * 8 != self.K * 3 or scales.shape != (self.E, self.N, self.K // 64):
            raise ValueError(f"scales shape {tuple(scales.shape)} does not match codes {tuple(codes.shape)}")
        self.codes, self.scales, self.biases = codes, scales, biases
        self.device = codes.device
        self._desc = SdvQ3(_need(codes, "codes", torch.uint8).value,
                           _need(scales, "scales", torch.int16, device=self.device).value,
                           _need(biases, "biases", torch.int16, device=self.device).value, self.E, self.N, self.K)

    @property
    def desc(self):
        return ctypes.byref(self._desc)

    def nbytes(self):
        return self.E * self.N * (3 * self.K // 8 + (self.K // 64) * 4)

    def tiled(self, fused_gateup=False):
        """The weight rewritten on the device into the tiled Q3 layout (sdv_q3_repack)."""
        return TiledQ4.from_rowmajor(self, fused_gateup)


class Q8Weight:
    """Q8_0 weights on the device in the GGUF interchange form: codes int8
    [E, N, K], half scales int16 (binary16 bits) [E, N, K/32].  A 2-D layout
    [N, K] is a dense matrix (E = 1)."""

    def __init__(self, qs, d):
        if qs.dim() == 2:
            qs, d = qs[None], d[None]
        if qs.dim() != 3 or d.dim() != 3:
            raise ValueError("qs [E,N,K], d [E,N,K/32] expected")
        self.E, self.N, self.K = qs.shape
        if d.shape != (self.E, self.N, self.K // 32):
            raise ValueError(f"d shape {tuple(d.shape)} does not match qs {tuple(qs.shape)}")
        self.qs, self.d = qs, d
        self.device = qs.device
        self._desc = SdvQ8_0(_need(qs, "qs", torch.int8).value, _need(d, "d", torch.int16, device=self.device).value,
                             self.E, self.N, self.K)

    @property
    def desc(self):
        return ctypes.byref(self._desc)

    def nbytes(self):
        return self.E * self.N * (self.K + (self.K // 32) * 2)

    def tiled(self, fused_gateup=False):
        """The weight rewritten on the device into the tiled Q8_0 layout
        (sdv_q8_0_repack)."""
        return TiledQ4.from_rowmajor(self, fused_gateup)


_CODES_BYTES = {FMT_AFFINE_Q4: "sdv_q4t_codes_bytes", FMT_Q8_0: "sdv_q8_0t_codes_bytes",
                FMT_AFFINE_Q3: "sdv_q3t_codes_bytes"}


class TiledQ4:
    """A tiled weight of ``sdv_q4t`` (device tensors ``codes`` uint8 and ``sb``
    int32): affine Q4/g64 (``fmt`` FMT_AFFINE_Q4), Q8_0 (FMT_Q8_0) or affine
    Q3/g64 (FMT_AFFINE_Q3)."""

    def __init__(self, codes, sb, E, N, K, fused_gateup, fmt=FMT_AFFINE_Q4):
        self.E, self.N, self.K, self.fused, self.fmt = E, N, K, bool(fused_gateup), fmt
        L = lib()
        need_c = getattr(L, _CODES_BYTES[fmt])(E, N, K, int(self.fused))
        need_s = L.sdv_q4t_sb_bytes(E, N, K, int(self.fused))
        if codes.numel() * codes.element_size() < need_c or sb.numel() * 4 < need_s:
            raise ValueError("tiled buffers are smaller than the layout needs")
        self.codes, self.sb = codes, sb
        self.device = codes.device
        self._desc = SdvQ4T(_need(codes, "codes", codes.dtype).value,
                            _need(sb, "sb", torch.int32, device=self.device).value, E, N, K, 64, int(self.fused),
                            int(fmt))

    @staticmethod
    def empty(E, N, K, fused_gateup, device, fmt=FMT_AFFINE_Q4):
        L = lib()
        nc = getattr(L, _CODES_BYTES[fmt])(E, N, K, int(bool(fused_gateup)))
        ns = L.sdv_q4t_sb_bytes(E, N, K, int(bool(fused_gateup)))
        codes = torch.empty((nc,), dtype=torch.uint8, device=device)
        sb = torch.empty((ns // 4,), dtype=torch.int32, device=device)
        return codes, sb

    @classmethod
    def from_rowmajor(cls, W, fused_gateup=False, out=None):
        fmt = FMT_Q8_0 if isinstance(W, Q8Weight) else (FMT_AFFINE_Q3 if isinstance(W, Q3Weight) else FMT_AFFINE_Q4)
        codes, sb = out if out is not None else cls.empty(W.E, W.N, W.K, fused_gateup, W.device, fmt)
        repack = {FMT_Q8_0: lib().sdv_q8_0_repack, FMT_AFFINE_Q3: lib().sdv_q3_repack}.get(fmt, lib().sdv_q4_repack)
        check(repack(W.desc, int(bool(fused_gateup)), _need(codes, "codes_out", codes.dtype),
                     _need(sb, "sb_out", torch.int32), _stream(codes)))
        return cls(codes, sb, W.E, W.N, W.K, fused_gateup, fmt)

    @property
    def desc(self):
        return ctypes.byref(self._desc)

    def nbytes(self):
        return self.codes.numel() * self.codes.element_size() + self.sb.numel() * 4


def _act_kind(act):
    if act.dtype == torch.int16:
        return ACT_BF16
    if act.dtype == torch.float32:
        return ACT_F32
    raise TypeError("activations must be bf16 bits (torch.int16) or float32")


def qmv_k(W, act, mode=MODE_PLAIN, out=None):
    """Dense k-row product with a tiled weight: act [k, K] (bf16 bits as
    int16, or fp32) -> fp32 [k, N] (plain) or [k, N/2] (fused gate/up with
    SwiGLU; the weight must be tiled with fused_gateup=True)."""
    k = act.shape[0]
    kind = _act_kind(act)
    if act.dim() != 2 or act.shape[1] != W.K:
        raise ValueError(f"act must be [k, {W.K}]")
    n_out = W.N if mode == MODE_PLAIN else W.N // 2
    if out is None:
        out = torch.empty((k, n_out), dtype=torch.float32, device=W.device)
    pa = _need(act, "act", act.dtype, device=W.device)
    py = _need(out, "out", torch.float32, k * n_out, device=W.device)
    check(lib().sdv_qmv_k(W.desc, pa, kind, k, mode, py, _stream(out)))
    return out


def _qmv_multi_args(Ws, act, mode, outs):
    k = act.shape[0]
    W0 = Ws[0]
    n_out = W0.N if mode == MODE_PLAIN else W0.N // 2
    if act.dim() != 2 or act.shape[1] != W0.K:
        raise ValueError(f"act must be [k, {W0.K}]")
    if len(Ws) != len(outs):
        raise ValueError("one output per weight")
    descs = (SdvQ4T * len(Ws))(*[W._desc for W in Ws])
    ys = (ctypes.c_void_p * len(outs))(*[_need(o, "out", torch.float32, k * n_out, W0.device).value for o in outs])
    return [descs, len(Ws), _need(act, "act", act.dtype, device=W0.device), _act_kind(act), k, mode, ys,
            _stream(act)]


def qmv_k_multi(Ws, act, mode=MODE_PLAIN, outs=None):
    """``qmv_k`` for several weights of one shape that read the same
    activation rows, in one launch (sdv_qmv_k_multi); returns the outputs."""
    k = act.shape[0]
    n_out = Ws[0].N if mode == MODE_PLAIN else Ws[0].N // 2
    if outs is None:
        outs = [torch.empty((k, n_out), dtype=torch.float32, device=Ws[0].device) for _ in Ws]
    check(lib().sdv_qmv_k_multi(*_qmv_multi_args(Ws, act, mode, outs)))
    return outs


def bind_qmv_k_multi(Ws, act, mode, outs):
    return BoundCall("sdv_qmv_k_multi", _qmv_multi_args(Ws, act, mode, outs))


def route_buffers(k, topk, device):
    kt = k * topk
    return RouteResult(
        idx=torch.empty((k, topk), dtype=torch.int32, device=device),
        w=torch.empty((k, topk), dtype=torch.float32, device=device),
        union_ids=torch.empty((kt,), dtype=torch.int32, device=device),
        n_union=torch.empty((1,), dtype=torch.int32, device=device),
        pair_off=torch.empty((kt + 1,), dtype=torch.int32, device=device),
        pair_row=torch.empty((kt,), dtype=torch.int32, device=device),
        pair_slot=torch.empty((kt,), dtype=torch.int32, device=device))


def moe_route_k(logits, topk, score_mode, renorm, out=None):
    """Per-row top-k, weights, union and pairs for logits fp32 [k, E]."""
    k, E = logits.shape
    if out is None:
        out = route_buffers(k, topk, logits.device)
    kt = k * topk
    dev = logits.device
    args = [_need(logits, "logits", torch.float32)]
    check(lib().sdv_moe_route_k(args[0], k, E, topk, score_mode, int(bool(renorm)),
                                _need(out.idx, "idx", torch.int32, kt, dev),
                                _need(out.w, "w", torch.float32, kt, dev),
                                _need(out.union_ids, "union_ids", torch.int32, kt, dev),
                                _need(out.n_union, "n_union", torch.int32, 1, dev),
                                _need(out.pair_off, "pair_off", torch.int32, kt + 1, dev),
                                _need(out.pair_row, "pair_row", torch.int32, kt, dev),
                                _need(out.pair_slot, "pair_slot", torch.int32, kt, dev),
                                _stream(logits)))
    return out


def _gather_args(bank, mode, act, route, k, topk, out, shared, shared_act, shared_out):
    kind = _act_kind(act)
    kt = k * topk
    need_act = kt * bank.K if kind == ACT_F32 else k * bank.K
    n_out = bank.N if mode == MODE_PLAIN else bank.N // 2
    dev = bank.device
    if shared is not None:
        sh = (shared.desc, _need(shared_act, "shared_act", act.dtype, k * bank.K, dev),
              _need(shared_out, "shared_out", torch.float32, k * n_out, dev))
    else:
        sh = (None, None, None)
    return [bank.desc, mode, _need(act, "act", act.dtype, need_act, dev), kind,
            _need(route.union_ids, "union_ids", torch.int32, kt, dev),
            _need(route.n_union, "n_union", torch.int32, 1, dev),
            _need(route.pair_off, "pair_off", torch.int32, kt + 1, dev),
            _need(route.pair_row, "pair_row", torch.int32, kt, dev),
            _need(route.pair_slot, "pair_slot", torch.int32, kt, dev), k, topk,
            _need(out, "out", torch.float32, kt * n_out, dev), *sh, _stream(out)]


def gather_qmv_k(bank, mode, act, route, k, topk, out=None, shared=None, shared_act=None, shared_out=None):
    """Gathered-expert product over the union in ``route``.  act: bf16 bits
    [k, K] shared by a row's slots, or fp32 [k, topk, K] per pair.  Returns
    fp32 [k, topk, N or N/2]; entry (r, s) is expert idx[r, s]'s output.

    ``shared`` (a TiledQ4 with E = 1 and the bank's geometry) adds the
    always-on expert to the same launch: it reads ``shared_act`` [k, K] (same
    dtype as act) and writes ``shared_out`` [k, N or N/2] (allocated if None).
    Returns ``out`` or ``(out, shared_out)``."""
    n_out = bank.N if mode == MODE_PLAIN else bank.N // 2
    if out is None:
        out = torch.empty((k, topk, n_out), dtype=torch.float32, device=bank.device)
    if shared is not None and shared_out is None:
        shared_out = torch.empty((k, n_out), dtype=torch.float32, device=bank.device)
    check(lib().sdv_gather_qmv_k(*_gather_args(bank, mode, act, route, k, topk, out, shared, shared_act,
                                               shared_out)))
    return out if shared is None else (out, shared_out)


def expert_slices(I):
    """Intermediate slices of the fused expert product (128 columns each)."""
    return (I + 127) // 128


def _experts_args(gate_up, down, x, route, k, topk, shared_gate_up, shared_down, partial):
    kt = k * topk
    dev = gate_up.device
    H, I = gate_up.K, gate_up.N // 2
    need = lib().sdv_moe_experts_partial_bytes(k, topk, H, I) // 4
    return [gate_up.desc, down.desc, _need(x, "x", x.dtype, k * H, dev),
            _need(route.union_ids, "union_ids", torch.int32, kt, dev),
            _need(route.n_union, "n_union", torch.int32, 1, dev),
            _need(route.pair_off, "pair_off", torch.int32, kt + 1, dev),
            _need(route.pair_row, "pair_row", torch.int32, kt, dev),
            _need(route.pair_slot, "pair_slot", torch.int32, kt, dev), k, topk,
            shared_gate_up.desc if shared_gate_up is not None else None,
            shared_down.desc if shared_down is not None else None,
            _need(partial, "partial", torch.float32, need, dev), _stream(partial)]


def experts_partial(k, topk, H, I, device):
    return torch.empty((expert_slices(I), k, topk + 1, H), dtype=torch.float32, device=device)


def moe_experts_k(gate_up, down, x, route, k, topk, shared_gate_up=None, shared_down=None, partial=None):
    """Fused gate/up + SwiGLU + down over the union in ``route`` (and the
    shared expert, slot ``topk``).  Returns the per-slice partial outputs
    fp32 [S, k, topk + 1, H]; their sum over S is each slot's expert output."""
    H, I = gate_up.K, gate_up.N // 2
    if partial is None:
        partial = experts_partial(k, topk, H, I, gate_up.device)
    check(lib().sdv_moe_experts_k(*_experts_args(gate_up, down, x, route, k, topk, shared_gate_up, shared_down,
                                                 partial)))
    return partial


def _route_experts_args(logits, score_mode, renorm, gate_up, down, x, route, topk, shared_gate_up, shared_down,
                        partial):
    k, E = logits.shape
    if E != gate_up.E:
        raise ValueError(f"logits have {E} experts, the bank {gate_up.E}")
    kt = k * topk
    dev = gate_up.device
    H, I = gate_up.K, gate_up.N // 2
    need = lib().sdv_moe_experts_partial_bytes(k, topk, H, I) // 4
    return [_need(logits, "logits", torch.float32, k * E, dev), score_mode, int(bool(renorm)),
            gate_up.desc, down.desc, _need(x, "x", x.dtype, k * H, dev), k, topk,
            shared_gate_up.desc if shared_gate_up is not None else None,
            shared_down.desc if shared_down is not None else None,
            _need(route.idx, "idx", torch.int32, kt, dev), _need(route.w, "w", torch.float32, kt, dev),
            _need(route.union_ids, "union_ids", torch.int32, kt, dev),
            _need(route.n_union, "n_union", torch.int32, 1, dev),
            _need(route.pair_off, "pair_off", torch.int32, kt + 1, dev),
            _need(route.pair_row, "pair_row", torch.int32, kt, dev),
            _need(route.pair_slot, "pair_slot", torch.int32, kt, dev),
            _need(partial, "partial", torch.float32, need, dev), _stream(partial)]


def moe_route_experts_k(logits, score_mode, renorm, gate_up, down, x, topk, shared_gate_up=None, shared_down=None,
                        route=None, partial=None):
    """moe_route_k and moe_experts_k as one call (one launch when k <= 9 and
    E <= 512).  Returns (route, partial), equal bit for bit to the two calls'."""
    k = logits.shape[0]
    H, I = gate_up.K, gate_up.N // 2
    if route is None:
        route = route_buffers(k, topk, gate_up.device)
    if partial is None:
        partial = experts_partial(k, topk, H, I, gate_up.device)
    check(lib().sdv_moe_route_experts_k(*_route_experts_args(logits, score_mode, renorm, gate_up, down, x, route,
                                                             topk, shared_gate_up, shared_down, partial)))
    return route, partial


def _combine_sliced_args(partial, route, shared_logit, has_shared, I, out):
    S, k, tp1, H = partial.shape
    topk = tp1 - 1
    dev = partial.device
    pz = _need(shared_logit, "shared_logit", torch.float32, k, dev) if shared_logit is not None else None
    return [_need(partial, "partial", torch.float32, S * k * tp1 * H, dev),
            _need(route.idx, "idx", torch.int32, k * topk, dev), _need(route.w, "w", torch.float32, k * topk, dev),
            pz, k, topk, H, I, int(bool(has_shared)), _need(out, "out", torch.float32, k * H, dev), _stream(out)]


def moe_combine_sliced_k(partial, route, I, has_shared=False, shared_logit=None, out=None):
    """y[r] = sum_s w[r, s] (sum_j partial[j, r, s]) over slots with an expert,
    plus sigmoid(z_r) times the shared slot's sum when ``has_shared``."""
    S, k, tp1, H = partial.shape
    if out is None:
        out = torch.empty((k, H), dtype=torch.float32, device=partial.device)
    check(lib().sdv_moe_combine_sliced_k(*_combine_sliced_args(partial, route, shared_logit, has_shared, I, out)))
    return out


def moe_combine_k(partial, w, shared_out=None, shared_logit=None, out=None):
    """y[r] = sum_s w[r, s] partial[r, s] (slot order) + sigmoid(z_r) shared[r]."""
    k, topk, H = partial.shape
    dev = partial.device
    if out is None:
        out = torch.empty((k, H), dtype=torch.float32, device=dev)
    ps = _need(shared_out, "shared_out", torch.float32, k * H, dev) if shared_out is not None else None
    pz = _need(shared_logit, "shared_logit", torch.float32, k, dev) if shared_logit is not None else None
    check(lib().sdv_moe_combine_k(_need(partial, "partial", torch.float32, k * topk * H, dev),
                                  _need(w, "w", torch.float32, k * topk, dev), ps, pz, k, topk, H,
                                  _need(out, "out", torch.float32, k * H, dev), _stream(out)))
    return out


def gdn_verify_k(S_in, q, kk, v, g, beta, snaps, y=None):
    """k-row Gated DeltaNet step with a snapshot after every row.

    S_in fp32 [Hv, Dv, Dk]; q, kk [k, Hk, Dk]; v [k, Hv, Dv]; g, beta [k, Hv];
    snaps: k fp32 tensors of S_in's shape (written).  Returns y [k, Hv, Dv]."""
    Hv, Dv, Dk = S_in.shape
    k, Hk, dk2 = q.shape
    dev = S_in.device
    if dk2 != Dk or tuple(kk.shape) != (k, Hk, Dk) or tuple(v.shape) != (k, Hv, Dv):
        raise ValueError("q/kk/v shapes do not match S_in")
    if tuple(g.shape) != (k, Hv) or tuple(beta.shape) != (k, Hv):
        raise ValueError("g/beta must be [k, Hv]")
    if len(snaps) != k:
        raise ValueError(f"{len(snaps)} snapshot buffers for k={k} rows")
    if y is None:
        y = torch.empty((k, Hv, Dv), dtype=torch.float32, device=dev)
    st = Hv * Dv * Dk
    arr = (ctypes.c_void_p * k)(*[_need(s, f"snaps[{t}]", torch.float32, st, dev).value for t, s in enumerate(snaps)])
    check(lib().sdv_gdn_verify_k(_need(S_in, "S_in", torch.float32, st, dev), _need(q, "q", torch.float32, device=dev),
                                 _need(kk, "kk", torch.float32, device=dev), _need(v, "v", torch.float32, device=dev),
                                 _need(g, "g", torch.float32, device=dev), _need(beta, "beta", torch.float32, device=dev),
                                 k, Hv, Hk, Dk, Dv, _need(y, "y", torch.float32, k * Hv * Dv, dev), arr,
                                 _stream(y)))
    return y


def gdn_rollback(k, j):
    """Slot holding the state after an accepted prefix of j rows: 0 = the
    verify call's input state, t = snapshot t-1."""
    slot = ctypes.c_int(-1)
    check(lib().sdv_gdn_rollback(k, j, ctypes.byref(slot)))
    return slot.value


def gdn_rollback_copy(dst, S_in, snaps, j):
    """dst <- the selected state (device copy on the current stream)."""
    k = len(snaps)
    dev = dst.device
    n = S_in.numel()
    arr = (ctypes.c_void_p * k)(*[_need(s, f"snaps[{t}]", torch.float32, n, dev).value for t, s in enumerate(snaps)])
    check(lib().sdv_gdn_rollback_copy(_need(dst, "dst", torch.float32, n, dev), _need(S_in, "S_in", torch.float32, n, dev),
                                      arr, k, j, n, _stream(dst)))
    return dst


def _prepare_args(qkv, hist, conv_w, a, b, A_log, dt_bias, Hk, Dk, conv_act, eps, out):
    k, C = qkv.shape
    Hv = A_log.shape[0]
    Dv = Dk
    dev = qkv.device
    if C != 2 * Hk * Dk + Hv * Dv:
        raise ValueError(f"qkv has {C} channels, expected 2*{Hk}*{Dk} + {Hv}*{Dv}")
    f = torch.float32
    return [_need(qkv, "qkv", f, k * C, dev), _need(hist, "hist", f, 3 * C, dev),
            _need(conv_w, "conv_w", f, 4 * C, dev), _need(a, "a", f, k * Hv, dev), _need(b, "b", f, k * Hv, dev),
            _need(A_log, "A_log", f, Hv, dev), _need(dt_bias, "dt_bias", f, Hv, dev), k, Hv, Hk, Dk, Dv, conv_act,
            ctypes.c_float(eps), _need(out["q"], "q", f, k * Hk * Dk, dev), _need(out["k"], "k", f, k * Hk * Dk, dev),
            _need(out["v"], "v", f, k * Hv * Dv, dev), _need(out["g"], "g", f, k * Hv, dev),
            _need(out["beta"], "beta", f, k * Hv, dev), _need(out["window"], "window", f, (k + 3) * C, dev),
            _stream(qkv)]


def gdn_prepare_outputs(k, Hv, Hk, Dk, device):
    f = torch.float32
    C = 2 * Hk * Dk + Hv * Dk
    return {"q": torch.empty((k, Hk, Dk), dtype=f, device=device), "k": torch.empty((k, Hk, Dk), dtype=f, device=device),
            "v": torch.empty((k, Hv, Dk), dtype=f, device=device), "g": torch.empty((k, Hv), dtype=f, device=device),
            "beta": torch.empty((k, Hv), dtype=f, device=device),
            "window": torch.empty((k + 3, C), dtype=f, device=device)}


def gdn_prepare_k(qkv, hist, conv_w, a, b, A_log, dt_bias, Hk, Dk, conv_act=CONV_NONE, eps=1e-6, out=None):
    """The recurrence inputs from the GDN projections: qkv fp32 [k, C] (channels
    q | k | v), hist [3, C], conv_w [C, 4], a, b [k, Hv], A_log, dt_bias [Hv].
    Returns {q, k, v, g, beta, window}; window [k+3, C] rows j..j+3 are the
    conv history after an accepted prefix of j rows."""
    k = qkv.shape[0]
    Hv = A_log.shape[0]
    if out is None:
        out = gdn_prepare_outputs(k, Hv, Hk, Dk, qkv.device)
    check(lib().sdv_gdn_prepare_k(*_prepare_args(qkv, hist, conv_w, a, b, A_log, dt_bias, Hk, Dk, conv_act, eps,
                                                 out)))
    return out


def _norm_args(y, z, w, gate_act, eps, out):
    k, Hv, Dv = y.shape
    dev = y.device
    f = torch.float32
    n = k * Hv * Dv
    return [_need(y, "y", f, n, dev), _need(z, "z", f, n, dev), _need(w, "w", f, Dv, dev), k, Hv, Dv, gate_act,
            ctypes.c_float(eps), _need(out, "out", f, n, dev), _stream(y)]


def _verify_prep_args(S_in, qkv, hist, conv_w, a, b, A_log, dt_bias, Hk, snaps, window, y, conv_act, eps):
    Hv, Dv, Dk = S_in.shape
    k, C = qkv.shape
    dev = S_in.device
    if C != 2 * Hk * Dk + Hv * Dv:
        raise ValueError(f"qkv has {C} channels, expected 2*{Hk}*{Dk} + {Hv}*{Dv}")
    if len(snaps) != k:
        raise ValueError(f"{len(snaps)} snapshot buffers for k={k} rows")
    f = torch.float32
    st = Hv * Dv * Dk
    arr = (ctypes.c_void_p * k)(*[_need(s, f"snaps[{t}]", f, st, dev).value for t, s in enumerate(snaps)])
    return [_need(S_in, "S_in", f, st, dev), _need(qkv, "qkv", f, k * C, dev), _need(hist, "hist", f, 3 * C, dev),
            _need(conv_w, "conv_w", f, 4 * C, dev), _need(a, "a", f, k * Hv, dev), _need(b, "b", f, k * Hv, dev),
            _need(A_log, "A_log", f, Hv, dev), _need(dt_bias, "dt_bias", f, Hv, dev), k, Hv, Hk, Dk, Dv, conv_act,
            ctypes.c_float(eps), _need(window, "window", f, (k + 3) * C, dev), _need(y, "y", f, k * Hv * Dv, dev),
            arr, _stream(y)]


def gdn_verify_prep_k(S_in, qkv, hist, conv_w, a, b, A_log, dt_bias, Hk, snaps, window, y=None,
                      conv_act=CONV_NONE, eps=1e-6):
    """gdn_prepare_k followed by gdn_verify_k in one launch: from the
    projections (qkv [k, C], hist [3, C], conv_w [C, 4], a, b [k, Hv], A_log,
    dt_bias [Hv]) and S_in [Hv, Dv, Dk], writes the snapshots, the window
    [k + 3, C] and returns y [k, Hv, Dv]."""
    Hv, Dv, _ = S_in.shape
    if y is None:
        y = torch.empty((qkv.shape[0], Hv, Dv), dtype=torch.float32, device=S_in.device)
    check(lib().sdv_gdn_verify_prep_k(*_verify_prep_args(S_in, qkv, hist, conv_w, a, b, A_log, dt_bias, Hk, snaps,
                                                         window, y, conv_act, eps)))
    return y


def bind_gdn_verify_prep_k(S_in, qkv, hist, conv_w, a, b, A_log, dt_bias, Hk, snaps, window, y, conv_act=CONV_NONE,
                           eps=1e-6):
    return BoundCall("sdv_gdn_verify_prep_k", _verify_prep_args(S_in, qkv, hist, conv_w, a, b, A_log, dt_bias, Hk,
                                                                snaps, window, y, conv_act, eps))


def _verify_prep_norm_args(S_in, qkv, hist, conv_w, a, b, A_log, dt_bias, Hk, snaps, window, y, conv_act, eps, z,
                           norm_w, gate_act, norm_eps, out, counters):
    args = _verify_prep_args(S_in, qkv, hist, conv_w, a, b, A_log, dt_bias, Hk, snaps, window, y, conv_act, eps)
    Hv, Dv, _ = S_in.shape
    n = qkv.shape[0] * Hv * Dv
    dev = S_in.device
    f = torch.float32
    return args[:-1] + [_need(z, "z", f, n, dev), _need(norm_w, "norm_w", f, Dv, dev), gate_act,
                        ctypes.c_float(norm_eps), _need(out, "out", f, n, dev),
                        _need(counters, "counters", torch.int32, Hv, dev), args[-1]]


def gdn_norm_counters(Hv, device):
    """The per-head counters of gdn_verify_prep_norm_k (zero; every call leaves them zero)."""
    return torch.zeros((Hv,), dtype=torch.int32, device=device)


def gdn_verify_prep_norm_k(S_in, qkv, hist, conv_w, a, b, A_log, dt_bias, Hk, snaps, window, z, norm_w, counters,
                           y=None, out=None, conv_act=CONV_NONE, eps=1e-6, gate_act=GATE_SIGMOID, norm_eps=1e-6):
    """gdn_verify_prep_k and gdn_gated_norm_k in one launch: returns (y, out),
    both [k, Hv, Dv]; ``counters`` int32 [Hv] (gdn_norm_counters)."""
    Hv, Dv, _ = S_in.shape
    k = qkv.shape[0]
    if y is None:
        y = torch.empty((k, Hv, Dv), dtype=torch.float32, device=S_in.device)
    if out is None:
        out = torch.empty((k, Hv, Dv), dtype=torch.float32, device=S_in.device)
    check(lib().sdv_gdn_verify_prep_norm_k(*_verify_prep_norm_args(S_in, qkv, hist, conv_w, a, b, A_log, dt_bias, Hk,
                                                                   snaps, window, y, conv_act, eps, z, norm_w,
                                                                   gate_act, norm_eps, out, counters)))
    return y, out


def bind_gdn_verify_prep_norm_k(S_in, qkv, hist, conv_w, a, b, A_log, dt_bias, Hk, snaps, window, y, z, norm_w, out,
                                counters, conv_act=CONV_NONE, eps=1e-6, gate_act=GATE_SIGMOID, norm_eps=1e-6):
    return BoundCall("sdv_gdn_verify_prep_norm_k",
                     _verify_prep_norm_args(S_in, qkv, hist, conv_w, a, b, A_log, dt_bias, Hk, snaps, window, y,
                                            conv_act, eps, z, norm_w, gate_act, norm_eps, out, counters))


def gdn_gated_norm_k(y, z, w, gate_act=GATE_SIGMOID, eps=1e-6, out=None):
    """y / sqrt(mean(y^2) + eps) * w * act(z) per (row, v head); y, z fp32 [k, Hv, Dv], w [Dv]."""
    if out is None:
        out = torch.empty_like(y)
    check(lib().sdv_gdn_gated_norm_k(*_norm_args(y, z, w, gate_act, eps, out)))
    return out


def bind_gdn_prepare_k(qkv, hist, conv_w, a, b, A_log, dt_bias, Hk, Dk, out, conv_act=CONV_NONE, eps=1e-6):
    return BoundCall("sdv_gdn_prepare_k", _prepare_args(qkv, hist, conv_w, a, b, A_log, dt_bias, Hk, Dk, conv_act,
                                                        eps, out))


def bind_gdn_gated_norm_k(y, z, w, out, gate_act=GATE_SIGMOID, eps=1e-6):
    return BoundCall("sdv_gdn_gated_norm_k", _norm_args(y, z, w, gate_act, eps, out))


def verify_accept_workspace(k, V, device):
    """Workspace for verify_accept_k (uint8 device buffer)."""
    n = lib().sdv_verify_accept_workspace_bytes(k, V)
    if n == 0:
        raise ValueError(f"no acceptance workspace for k={k}, V={V}")
    return torch.empty(n, dtype=torch.uint8, device=device)


def _accept_args(logits, drafts, noise, inv_temp, eos, tokens, accepted, workspace):
    k, V = logits.shape
    dev = logits.device
    pn = _need(noise, "noise", torch.float32, k * V, dev) if noise is not None else None
    pd = _need(drafts, "drafts", torch.int32, k - 1, dev) if k > 1 else None
    return [_need(logits, "logits", torch.float32, k * V, dev), pn, ctypes.c_float(inv_temp), pd, k, V, eos,
            _need(tokens, "tokens", torch.int32, k, dev), _need(accepted, "accepted", torch.int32, 1, dev),
            _need(workspace, "workspace", torch.uint8, device=dev), workspace.numel(), _stream(tokens)]


def verify_accept_k(logits, drafts, noise=None, inv_temp=1.0, eos=-1, tokens=None, accepted=None, workspace=None):
    """Acceptance of a verified block: logits fp32 [k, V], drafts int32 [k-1]
    (the tokens of rows 1..k-1), optional Gumbel noise fp32 [k, V].  Returns
    (tokens int32 [k], accepted int32 [1]) on the device: the token sampled
    from each row and the number of leading drafts accepted."""
    k, V = logits.shape
    dev = logits.device
    if tokens is None:
        tokens = torch.empty(k, dtype=torch.int32, device=dev)
    if accepted is None:
        accepted = torch.empty(1, dtype=torch.int32, device=dev)
    if workspace is None:
        workspace = verify_accept_workspace(k, V, dev)
    check(lib().sdv_verify_accept_k(*_accept_args(logits, drafts, noise, inv_temp, eos, tokens, accepted,
                                                  workspace)))
    return tokens, accepted


def verify_accept_k_noalloc(logits, drafts, tokens, accepted, noise=None, inv_temp=1.0, eos=-1):
    """``verify_accept_k`` through sdv_verify_accept_k_noalloc: the library's
    built-in per-device scratch instead of a caller workspace (no allocation
    in the call).  tokens int32 [k] and accepted int32 [1] are caller
    buffers."""
    k, V = logits.shape
    dev = logits.device
    pn = _need(noise, "noise", torch.float32, k * V, dev) if noise is not None else None
    pd = _need(drafts, "drafts", torch.int32, k - 1, dev) if k > 1 else None
    check(lib().sdv_verify_accept_k_noalloc(
        _need(logits, "logits", torch.float32, k * V, dev), pn, ctypes.c_float(inv_temp), pd, k, V, eos,
        _need(tokens, "tokens", torch.int32, k, dev), _need(accepted, "accepted", torch.int32, 1, dev),
        _stream(tokens)))
    return tokens, accepted


def bind_verify_accept_k(logits, drafts, tokens, accepted, workspace, noise=None, inv_temp=1.0, eos=-1):
    return BoundCall("sdv_verify_accept_k",
                     _accept_args(logits, drafts, noise, inv_temp, eos, tokens, accepted, workspace))


class GdnLayersLaunch:
    """sdv_gdn_verify_prep_k_layers over the layers of bound
    sdv_gdn_verify_prep_k calls (``bind_gdn_verify_prep_k``,
    ``GdnLayer.prep_call``): independent layers of one shape in one launch, a
    measurement form.  The device table is checked and written once, from the
    calls' buffers; calling the object re-issues the launch."""

    # argument positions of sdv_gdn_verify_prep_k
    _PTRS = {"S_in": 0, "qkv": 1, "hist": 2, "conv_w": 3, "a": 4, "b": 5, "A_log": 6, "dt_bias": 7,
             "window": 15, "y": 16}
    _SHAPE = slice(8, 15)  # k, Hv, Hk, Dk, Dv, conv_act, eps
    _SNAPS, _STREAM = 17, 18

    def __init__(self, calls, device):
        if not calls or any(c.name != "sdv_gdn_verify_prep_k" for c in calls):
            raise ValueError("GdnLayersLaunch takes bound sdv_gdn_verify_prep_k calls")
        args = [c._args for c in calls]
        val = lambda v: v.value if isinstance(v, ctypes.c_float) else v
        shape = [val(v) for v in args[0][self._SHAPE]]
        if any([val(v) for v in a[self._SHAPE]] != shape for a in args):
            raise ValueError("the layers of one launch share k, Hv, Hk, Dk, Dv, conv_act and eps")
        k = shape[0]
        n = len(calls)
        entries = (SdvGdnLayer * n)()
        for e, a in zip(entries, args):
            for name, i in self._PTRS.items():
                setattr(e, name, a[i].value)
            for t in range(k):
                e.snaps[t] = a[self._SNAPS][t]
        nbytes = n * ctypes.sizeof(SdvGdnLayer)
        self.table = torch.empty((nbytes,), dtype=torch.uint8, device=device)
        check(lib().sdv_gdn_layers_table(ctypes.addressof(entries), n, *shape[:5],
                                         ctypes.c_void_p(self.table.data_ptr()), nbytes))
        self.layers = n
        self._args = (ctypes.c_void_p(self.table.data_ptr()), n, *shape[:6], ctypes.c_float(shape[6]),
                      args[0][self._STREAM])

    def __call__(self):
        check(lib().sdv_gdn_verify_prep_k_layers(*self._args))


class BoundCall:
    """A library call with its arguments marshalled once (fixed buffers).

    Calling it re-issues the same launch on the stream captured at bind time;
    used where the same buffers are reused every step, so the per-launch host
    cost is one ctypes call."""

    def __init__(self, fn_name, args):
        self._fn = getattr(lib(), fn_name)
        self._args = tuple(args)
        self.name = fn_name

    def __call__(self):
        check(self._fn(*self._args))

    def replaced(self, changes):
        """The same call with the arguments at the given positions replaced
        (already marshalled values, e.g. ctypes.c_void_p of a device pointer)."""
        args = list(self._args)
        for i, v in changes.items():
            args[i] = v
        out = BoundCall.__new__(BoundCall)
        out._fn, out._args, out.name = self._fn, tuple(args), self.name
        return out


def bind_qmv_k(W, act, mode, out):
    k = act.shape[0]
    n_out = W.N if mode == MODE_PLAIN else W.N // 2
    if act.dim() != 2 or act.shape[1] != W.K:
        raise ValueError(f"act must be [k, {W.K}]")
    return BoundCall("sdv_qmv_k", [W.desc, _need(act, "act", act.dtype, device=W.device), _act_kind(act), k, mode,
                                   _need(out, "out", torch.float32, k * n_out, W.device), _stream(out)])


def bind_moe_route_k(logits, topk, score_mode, renorm, out):
    k, E = logits.shape
    kt = k * topk
    dev = logits.device
    return BoundCall("sdv_moe_route_k", [
        _need(logits, "logits", torch.float32), k, E, topk, score_mode, int(bool(renorm)),
        _need(out.idx, "idx", torch.int32, kt, dev), _need(out.w, "w", torch.float32, kt, dev),
        _need(out.union_ids, "union_ids", torch.int32, kt, dev), _need(out.n_union, "n_union", torch.int32, 1, dev),
        _need(out.pair_off, "pair_off", torch.int32, kt + 1, dev),
        _need(out.pair_row, "pair_row", torch.int32, kt, dev),
        _need(out.pair_slot, "pair_slot", torch.int32, kt, dev), _stream(logits)])


def bind_gather_qmv_k(bank, mode, act, route, k, topk, out, shared=None, shared_act=None, shared_out=None):
    return BoundCall("sdv_gather_qmv_k",
                     _gather_args(bank, mode, act, route, k, topk, out, shared, shared_act, shared_out))


def bind_moe_experts_k(gate_up, down, x, route, k, topk, shared_gate_up, shared_down, partial):
    return BoundCall("sdv_moe_experts_k",
                     _experts_args(gate_up, down, x, route, k, topk, shared_gate_up, shared_down, partial))


def bind_moe_route_experts_k(logits, score_mode, renorm, gate_up, down, x, route, topk, shared_gate_up, shared_down,
                             partial):
    return BoundCall("sdv_moe_route_experts_k",
                     _route_experts_args(logits, score_mode, renorm, gate_up, down, x, route, topk, shared_gate_up,
                                         shared_down, partial))


def bind_moe_combine_sliced_k(partial, route, I, has_shared, shared_logit, out):
    return BoundCall("sdv_moe_combine_sliced_k", _combine_sliced_args(partial, route, shared_logit, has_shared, I, out))


def bind_moe_combine_k(partial, w, shared_out, shared_logit, out):
    k, topk, H = partial.shape
    dev = partial.device
    ps = _need(shared_out, "shared_out", torch.float32, k * H, dev) if shared_out is not None else None
    pz = _need(shared_logit, "shared_logit", torch.float32, k, dev) if shared_logit is not None else None
    return BoundCall("sdv_moe_combine_k", [
        _need(partial, "partial", torch.float32, k * topk * H, dev), _need(w, "w", torch.float32, k * topk, dev),
        ps, pz, k, topk, H, _need(out, "out", torch.float32, k * H, dev), _stream(out)])


def bind_gdn_verify_k(S_in, q, kk, v, g, beta, snaps, y):
    Hv, Dv, Dk = S_in.shape
    k, Hk, _ = q.shape
    dev = S_in.device
    if len(snaps) != k or tuple(kk.shape) != (k, Hk, Dk) or tuple(v.shape) != (k, Hv, Dv):
        raise ValueError("gdn shapes do not match")
    if tuple(g.shape) != (k, Hv) or tuple(beta.shape) != (k, Hv):
        raise ValueError("g/beta must be [k, Hv]")
    st = Hv * Dv * Dk
    arr = (ctypes.c_void_p * k)(*[_need(sn, f"snaps[{t}]", torch.float32, st, dev).value for t, sn in enumerate(snaps)])
    return BoundCall("sdv_gdn_verify_k", [
        _need(S_in, "S_in", torch.float32, st, dev), _need(q, "q", torch.float32, device=dev),
        _need(kk, "kk", torch.float32, device=dev), _need(v, "v", torch.float32, device=dev),
        _need(g, "g", torch.float32, device=dev), _need(beta, "beta", torch.float32, device=dev),
        k, Hv, Hk, Dk, Dv, _need(y, "y", torch.float32, k * Hv * Dv, dev), arr, _stream(y)])
