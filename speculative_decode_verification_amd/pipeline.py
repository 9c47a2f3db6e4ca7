"""One verification step composed from the library's entry points.

``MoeLayer`` runs the MoE half of a layer for k rows: router dispatch and
union, gathered fused gate/up with SwiGLU, gathered down projection, the
optional shared expert and the fixed-order combine, all on the device with no
host synchronisation.  When the shared expert has the routed experts'
geometry it rides in the two gathered launches as one more unit; otherwise
it runs as two dense products.  ``GdnLayer`` keeps a pool of
k+1 state buffers per layer: the live state and k snapshot slots.  A verify
call writes the snapshots; rollback to an accepted prefix j only swaps which
buffer is live (Red Lite dev45, "What it is": rejection by choosing the
live buffer), so no state is copied.
"""

import ctypes

import torch

from . import ops
from ._lib import MODE_GATEUP_SWIGLU, MODE_PLAIN, ROUTE_SIGMOID, ROUTE_SOFTMAX


class MoeLayer:
    def __init__(self, gate_up, down, k, topk, score_mode, renorm, shared_gate_up=None, shared_down=None,
                 fuse_shared=True, fused_experts=None, route_in_experts=False):
        """fused_experts: the one-launch expert kernel; None picks it when the
        four weights share one format (affine Q4, Q8_0 or affine Q3) and the
        two gathered launches otherwise.  route_in_experts: with the fused expert
        kernel, the router dispatch runs in one call with it
        (sdv_moe_route_experts_k) rather than in a launch of its own.  Off by
        default: every expert workgroup then waits for its own dispatch, which
        costs more than the separate launch at 512 experts and nine rows."""
        self.gate_up, self.down = gate_up, down
        weights = [w for w in (gate_up, down, shared_gate_up, shared_down) if w is not None]
        if fused_experts is None:
            fused_experts = len({w.fmt for w in weights}) == 1
        self.fused_experts = fused_experts
        if route_in_experts and gate_up.fmt != ops.FMT_AFFINE_Q4:
            raise ValueError("the router dispatch inside the expert kernel takes affine-Q4 weights")
        self.route_in_experts = bool(fused_experts and route_in_experts)
        self.shared_gate_up, self.shared_down = shared_gate_up, shared_down
        self.fused_shared = (fuse_shared and shared_gate_up is not None and
                             (shared_gate_up.N, shared_gate_up.K, shared_gate_up.fmt) ==
                             (gate_up.N, gate_up.K, gate_up.fmt) and
                             (shared_down.N, shared_down.K, shared_down.fmt) == (down.N, down.K, down.fmt))
        self.k, self.topk = k, topk
        self.score_mode, self.renorm = score_mode, renorm
        dev = gate_up.device
        self.H = gate_up.K
        self.I = gate_up.N // 2
        if down.K != self.I or down.N != self.H:
            raise ValueError("down bank must be [E, H, I]")
        self.route = ops.route_buffers(k, topk, dev)
        self.h = torch.empty((k, topk, self.I), dtype=torch.float32, device=dev)
        self.partial = torch.empty((k, topk, self.H), dtype=torch.float32, device=dev)
        self.y = torch.empty((k, self.H), dtype=torch.float32, device=dev)
        if shared_gate_up is not None:
            self.sh_h = torch.empty((k, shared_gate_up.N // 2), dtype=torch.float32, device=dev)
            self.sh_out = torch.empty((k, self.H), dtype=torch.float32, device=dev)
        else:
            self.sh_h = self.sh_out = None
        if fused_experts:
            if shared_gate_up is not None and not self.fused_shared:
                raise ValueError("the fused expert path needs the shared expert in the routed experts' geometry")
            self.xpartial = ops.experts_partial(k, topk, self.H, self.I, dev)

    def bind(self, x, logits, z=None):
        """Marshal the layer's launches once for fixed input buffers; returns a
        list of (name, call) pairs to run in order."""
        if self.fused_experts:
            has = self.shared_gate_up is not None
            if self.route_in_experts:
                calls = [("experts", ops.bind_moe_route_experts_k(logits, self.score_mode, self.renorm, self.gate_up,
                                                                  self.down, x, self.route, self.topk,
                                                                  self.shared_gate_up, self.shared_down,
                                                                  self.xpartial))]
            else:
                calls = [("route", ops.bind_moe_route_k(logits, self.topk, self.score_mode, self.renorm, self.route)),
                         ("experts", ops.bind_moe_experts_k(self.gate_up, self.down, x, self.route, self.k, self.topk,
                                                            self.shared_gate_up, self.shared_down, self.xpartial))]
            return calls + [("combine", ops.bind_moe_combine_sliced_k(self.xpartial, self.route, self.I, has,
                                                              z if has else None, self.y))]
        fs = self.fused_shared
        sg = dict(shared=self.shared_gate_up, shared_act=x, shared_out=self.sh_h) if fs else {}
        sd = dict(shared=self.shared_down, shared_act=self.sh_h, shared_out=self.sh_out) if fs else {}
        calls = [("route", ops.bind_moe_route_k(logits, self.topk, self.score_mode, self.renorm, self.route)),
                 ("gate_up", ops.bind_gather_qmv_k(self.gate_up, MODE_GATEUP_SWIGLU, x, self.route, self.k,
                                                   self.topk, self.h, **sg)),
                 ("down", ops.bind_gather_qmv_k(self.down, MODE_PLAIN, self.h, self.route, self.k, self.topk,
                                                self.partial, **sd))]
        if self.shared_gate_up is not None and not fs:
            calls.append(("shared_gate_up", ops.bind_qmv_k(self.shared_gate_up, x, MODE_GATEUP_SWIGLU, self.sh_h)))
            calls.append(("shared_down", ops.bind_qmv_k(self.shared_down, self.sh_h, MODE_PLAIN, self.sh_out)))
        calls.append(("combine", ops.bind_moe_combine_k(self.partial, self.route.w, self.sh_out,
                                                        z if self.sh_out is not None else None, self.y)))
        return calls

    def __call__(self, x, logits, z=None):
        """x: bf16 bits [k, H] (int16); logits fp32 [k, E]; z fp32 [k] or None."""
        if self.route_in_experts:
            has = self.shared_gate_up is not None
            ops.moe_route_experts_k(logits, self.score_mode, self.renorm, self.gate_up, self.down, x, self.topk,
                                    self.shared_gate_up, self.shared_down, route=self.route, partial=self.xpartial)
            return ops.moe_combine_sliced_k(self.xpartial, self.route, self.I, has, z if has else None, out=self.y)
        ops.moe_route_k(logits, self.topk, self.score_mode, self.renorm, out=self.route)
        if self.fused_experts:
            has = self.shared_gate_up is not None
            ops.moe_experts_k(self.gate_up, self.down, x, self.route, self.k, self.topk, self.shared_gate_up,
                              self.shared_down, partial=self.xpartial)
            return ops.moe_combine_sliced_k(self.xpartial, self.route, self.I, has, z if has else None, out=self.y)
        fs = self.fused_shared
        sg = dict(shared=self.shared_gate_up, shared_act=x, shared_out=self.sh_h) if fs else {}
        sd = dict(shared=self.shared_down, shared_act=self.sh_h, shared_out=self.sh_out) if fs else {}
        ops.gather_qmv_k(self.gate_up, MODE_GATEUP_SWIGLU, x, self.route, self.k, self.topk, out=self.h, **sg)
        ops.gather_qmv_k(self.down, MODE_PLAIN, self.h, self.route, self.k, self.topk, out=self.partial, **sd)
        if self.shared_gate_up is not None and not fs:
            ops.qmv_k(self.shared_gate_up, x, MODE_GATEUP_SWIGLU, out=self.sh_h)
            ops.qmv_k(self.shared_down, self.sh_h, MODE_PLAIN, out=self.sh_out)
        ops.moe_combine_k(self.partial, self.route.w, self.sh_out, z if self.sh_out is not None else None,
                          out=self.y)
        return self.y


class GdnLayer:
    """State pool of one GDN layer: slot ``live`` holds the current state, the
    other k slots receive the next verify call's snapshots."""

    def __init__(self, S0, k):
        self.k = k
        self.Hv, self.Dv, self.Dk = S0.shape
        self.slots = [S0.contiguous()] + [torch.empty_like(S0) for _ in range(k)]
        self.live = 0
        self.snap_ids = None
        self._pending = None
        self.y = torch.empty((k, self.Hv, self.Dv), dtype=torch.float32, device=S0.device)

    @property
    def state(self):
        self.apply_rollback()
        return self.slots[self.live]

    def verify(self, q, kk, v, g, beta):
        self.apply_rollback()
        rows = q.shape[0]
        self.snap_ids = [i for i in range(len(self.slots)) if i != self.live][:rows]
        y = self.y[:rows]
        ops.gdn_verify_k(self.state, q, kk, v, g, beta, [self.slots[i] for i in self.snap_ids], y=y)
        return y

    def bind(self, q, kk, v, g, beta):
        """Marshal the verify launch once per possible live slot for fixed
        input buffers; ``run_bound`` then issues the one matching the live slot."""
        self.apply_rollback()
        rows = q.shape[0]
        self._bound = []
        for live in range(len(self.slots)):
            ids = [i for i in range(len(self.slots)) if i != live][:rows]
            call = ops.bind_gdn_verify_k(self.slots[live], q, kk, v, g, beta, [self.slots[i] for i in ids],
                                         self.y[:rows])
            self._bound.append((ids, call))
        return self

    def run_bound(self):
        self.apply_rollback()
        ids, call = self._bound[self.live]
        self.snap_ids = ids
        call()
        return self.y

    def attach_prep(self, hist, conv_w, A_log, dt_bias, Hk, conv_act=ops.CONV_NONE, eps=1e-6):
        """Run the layer from its projections: the conv history hist [3, C]
        (copied), depthwise taps conv_w [C, 4], A_log and dt_bias [Hv], Hk
        q/k heads.  Two windows [k + 3, C] alternate: rollback makes rows j..j+2
        of the last window the history (no copy), and the next preparation
        writes the other window."""
        C = hist.shape[1]
        dev = hist.device
        self.prep_params = (conv_w.contiguous(), A_log.contiguous(), dt_bias.contiguous(), Hk, conv_act, eps)
        self.hist = hist.contiguous().clone()
        self.windows = [torch.empty((self.k + 3, C), dtype=torch.float32, device=dev) for _ in range(2)]
        self.win = 0
        self.prepped = False
        self.prep_out = {n: t for n, t in ops.gdn_prepare_outputs(self.k, self.Hv, Hk, self.Dk, dev).items()
                         if n != "window"}
        self._bound_prep = {}
        return self

    def _prep_out(self, rows):
        out = {n: t[:rows] for n, t in self.prep_out.items()}
        out["window"] = self.windows[self.win][:rows + 3]
        return out

    def prepare(self, qkv, a, b):
        """The recurrence inputs of rows qkv [rows, C], a, b [rows, Hv];
        returns {q, k, v, g, beta, window}."""
        self.apply_rollback()
        conv_w, A_log, dt_bias, Hk, act, eps = self.prep_params
        out = ops.gdn_prepare_k(qkv, self.hist, conv_w, a, b, A_log, dt_bias, Hk, self.Dk, act, eps,
                                self._prep_out(qkv.shape[0]))
        self.prepped = True
        return out

    def bind_tail(self, z, norm_w, out, gate_act=ops.GATE_SIGMOID, eps=1e-6):
        """The output norm of all k rows for fixed z [k, Hv, Dv] and out."""
        self._bound_tail = ops.bind_gdn_gated_norm_k(self.y, z, norm_w, out, gate_act, eps)
        return self

    def run_tail_bound(self):
        self._bound_tail()

    def _prep_call(self, qkv, a, b, win, hist):
        key = (win, hist.data_ptr(), qkv.data_ptr(), a.data_ptr(), b.data_ptr())
        call = self._bound_prep.get(key)
        if call is None:
            conv_w, A_log, dt_bias, Hk, act, eps = self.prep_params
            rows = qkv.shape[0]
            out = {n: t[:rows] for n, t in self.prep_out.items()}
            out["window"] = self.windows[win][:rows + 3]
            call = ops.bind_gdn_prepare_k(qkv, hist, conv_w, a, b, A_log, dt_bias, Hk, self.Dk, out, act, eps)
            self._bound_prep[key] = call
        return call

    def prebind_prepare(self, qkv, a, b):
        """Marshal ``run_prepare_bound`` for every (window, history source)
        pair it can meet, so later steps only look the call up."""
        self.apply_rollback()
        for win in (0, 1):
            self._prep_call(qkv, a, b, win, self.hist)
            for j in range(self.k + 1):
                self._prep_call(qkv, a, b, win, self.windows[win ^ 1][j:j + 3])
        return self

    def run_prepare_bound(self, qkv, a, b):
        """``prepare`` for fixed qkv, a, b buffers, marshalled once per
        (window, history source) pair."""
        self.apply_rollback()
        self._prep_call(qkv, a, b, self.win, self.hist)()
        self.prepped = True
        return self._prep_out(qkv.shape[0])

    def verify_from_proj(self, qkv, a, b):
        """Preparation and recurrence in one launch from the projections qkv
        [rows, C], a, b [rows, Hv]; returns y [rows, Hv, Dv]."""
        self.apply_rollback()
        conv_w, A_log, dt_bias, Hk, act, eps = self.prep_params
        rows = qkv.shape[0]
        self.snap_ids = [i for i in range(len(self.slots)) if i != self.live][:rows]
        y = self.y[:rows]
        ops.gdn_verify_prep_k(self.state, qkv, self.hist, conv_w, a, b, A_log, dt_bias, Hk,
                              [self.slots[i] for i in self.snap_ids], self.windows[self.win][:rows + 3], y, act, eps)
        self.prepped = True
        return y

    # argument positions of sdv_gdn_verify_prep_k that change between steps
    _FP_S_IN, _FP_HIST, _FP_WINDOW, _FP_SNAPS = 0, 2, 15, 17

    def bind_from_proj(self, qkv, a, b):
        """Marshal ``verify_from_proj`` for fixed qkv, a, b buffers; the state,
        history, window and snapshot pointers are patched per step from
        prebuilt values (no argument checks on the host path after this)."""
        self.apply_rollback()
        conv_w, A_log, dt_bias, Hk, act, eps = self.prep_params
        rows = qkv.shape[0]
        self._fp_rows = rows
        self._fp_snaps = {}
        for live in range(len(self.slots)):
            ids = [i for i in range(len(self.slots)) if i != live][:rows]
            arr = (ctypes.c_void_p * rows)(*[self.slots[i].data_ptr() for i in ids])
            self._fp_snaps[live] = (ids, arr)
        ids0 = self._fp_snaps[self.live][0]
        self._fp_template = ops.bind_gdn_verify_prep_k(self.state, qkv, self.hist, conv_w, a, b, A_log, dt_bias, Hk,
                                                       [self.slots[i] for i in ids0],
                                                       self.windows[self.win][:rows + 3], self.y[:rows], act, eps)
        self._fp_cache = {}
        return self

    def verify_from_proj_norm(self, qkv, a, b, z, norm_w, out, gate_act=ops.GATE_SIGMOID, norm_eps=1e-6):
        """``verify_from_proj`` with the gated output norm in the same launch:
        out [rows, Hv, Dv] = rmsnorm(y) * norm_w * act(z); returns (y, out)."""
        self.apply_rollback()
        conv_w, A_log, dt_bias, Hk, act, eps = self.prep_params
        rows = qkv.shape[0]
        self.snap_ids = [i for i in range(len(self.slots)) if i != self.live][:rows]
        y = self.y[:rows]
        ops.gdn_verify_prep_norm_k(self.state, qkv, self.hist, conv_w, a, b, A_log, dt_bias, Hk,
                                   [self.slots[i] for i in self.snap_ids], self.windows[self.win][:rows + 3], z,
                                   norm_w, self._counters(), y, out, act, eps, gate_act, norm_eps)
        self.prepped = True
        return y, out

    def _counters(self):
        if getattr(self, "norm_counters", None) is None:
            self.norm_counters = ops.gdn_norm_counters(self.Hv, self.state.device)
        return self.norm_counters

    def bind_from_proj_norm(self, qkv, a, b, z, norm_w, out, gate_act=ops.GATE_SIGMOID, norm_eps=1e-6):
        """``bind_from_proj`` with the gated output norm in the same launch
        (``run_from_proj_bound`` then also writes out)."""
        self.bind_from_proj(qkv, a, b)
        conv_w, A_log, dt_bias, Hk, act, eps = self.prep_params
        rows = qkv.shape[0]
        ids0 = self._fp_snaps[self.live][0]
        self._fp_template = ops.bind_gdn_verify_prep_norm_k(
            self.state, qkv, self.hist, conv_w, a, b, A_log, dt_bias, Hk, [self.slots[i] for i in ids0],
            self.windows[self.win][:rows + 3], self.y[:rows], z, norm_w, out, self._counters(), act, eps, gate_act,
            norm_eps)
        return self

    def prep_call(self):
        """The bound call ``run_from_proj_bound`` issues next (the live state,
        history, window and snapshot slots), without issuing it."""
        self.apply_rollback()
        key = (self.live, self.win, self.hist.data_ptr())
        call = self._fp_cache.get(key)
        if call is None:
            ids, arr = self._fp_snaps[self.live]
            call = self._fp_template.replaced({
                self._FP_S_IN: ctypes.c_void_p(self.state.data_ptr()),
                self._FP_HIST: ctypes.c_void_p(self.hist.data_ptr()),
                self._FP_WINDOW: ctypes.c_void_p(self.windows[self.win].data_ptr()),
                self._FP_SNAPS: arr})
            self._fp_cache[key] = call
        return call

    def run_from_proj_bound(self):
        call = self.prep_call()
        self.snap_ids = self._fp_snaps[self.live][0]
        call()
        self.prepped = True
        return self.y[:self._fp_rows]

    def rollback_later(self, j):
        """``rollback(j)``, applied when the layer next runs or its state is
        read (or by ``apply_rollback``).  A decoding loop that reads the
        accepted count back then launches the next step's first layer after
        that layer's rollback alone, instead of after every layer's."""
        if self._pending is not None:
            raise RuntimeError("a rollback is already pending")
        ops.gdn_rollback(len(self.snap_ids), j)  # checks j before it is stored
        self._pending = j

    def apply_rollback(self):
        j, self._pending = self._pending, None
        if j is not None:
            self.rollback(j)

    def rollback(self, j):
        """Make the state after the accepted prefix of j rows live (no copy);
        with a preparation stage, rows j..j+2 of its window become the conv
        history."""
        if self._pending is not None:
            raise RuntimeError("a rollback is already pending")
        slot = ops.gdn_rollback(len(self.snap_ids), j)
        if slot > 0:
            self.live = self.snap_ids[slot - 1]
        self.snap_ids = None
        if getattr(self, "prepped", False):
            self.hist = self.windows[self.win][j:j + 3]
            self.win ^= 1
            self.prepped = False
        return self.slots[self.live]


__all__ = ["MoeLayer", "GdnLayer", "MODE_PLAIN", "MODE_GATEUP_SWIGLU", "ROUTE_SOFTMAX", "ROUTE_SIGMOID"]


class VerifyCycle:
    """Closes a verify step: the acceptance of the block on the device, then
    every GDN layer rolled back to the accepted prefix by selecting its
    snapshot (Red Lite dev45, "Acceptance" and "What it is": rejection
    picks which state buffer is live, nothing is copied).

    The accepted count is read back to the host, which holds the slot choice
    of each layer's state pool."""

    def __init__(self, gdn_layers, k, vocab, device, eos=-1):
        self.layers = list(gdn_layers)
        self.k, self.vocab, self.eos = k, vocab, eos
        self.tokens = torch.empty(k, dtype=torch.int32, device=device)
        self.accepted = torch.empty(1, dtype=torch.int32, device=device)
        self.workspace = ops.verify_accept_workspace(k, vocab, device)

    def accept(self, logits, drafts, noise=None, inv_temp=1.0):
        """Device acceptance only: (tokens, accepted) device tensors."""
        return ops.verify_accept_k(logits, drafts, noise, inv_temp, self.eos, self.tokens, self.accepted,
                                   self.workspace)

    def bind(self, logits, drafts, noise=None, inv_temp=1.0):
        return ops.bind_verify_accept_k(logits, drafts, self.tokens, self.accepted, self.workspace, noise, inv_temp,
                                        self.eos)

    def __call__(self, logits, drafts, noise=None, inv_temp=1.0, defer=False):
        """Accept, roll every layer back to the accepted prefix, and return
        (n accepted drafts, emitted tokens: the accepted drafts, then the
        token sampled after them).  With ``defer`` each layer's rollback is
        applied when the layer next runs (``GdnLayer.rollback_later``)."""
        self.accept(logits, drafts, noise, inv_temp)
        n = int(self.accepted.item())
        for layer in self.layers:
            if defer:
                layer.rollback_later(n + 1)
            else:
                layer.rollback(n + 1)
        toks = self.tokens.cpu().tolist()
        accepted_drafts = drafts[:n].cpu().tolist() if n > 0 else []
        return n, accepted_drafts + [toks[n]]
