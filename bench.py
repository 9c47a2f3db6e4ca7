#!/usr/bin/env python3
"""Benchmark of one exact k-row verification step on one MI355X.

Workload (default ``flashnext_k9``): the Flash-Next-shaped hybrid at k = 9
draft rows (``flashnext_k16`` and ``flashnext_k32``: the same step at the
verifier's wide widths).  One step runs, for each of the 48 layers, the Gated
DeltaNet verify from the layer's projections on the 36 layers with l % 4 != 3
(one launch: causal conv over q/k/v with the carried conv history, q/k L2
norm, decay and beta gates, the recurrence with per-row snapshots; then the
gated output norm) and the MoE verify (router dispatch and union over 512
experts, top-10 sigmoid scores renormalised; the fused expert kernel:
gate/up + SwiGLU + down over the union's affine-Q4/g64 experts
[512, 1280, 2560] / [512, 2560, 640] and the sigmoid-gated shared expert;
the fixed-order combine); then the acceptance of the block over a
248,320-token vocabulary, and every GDN layer rolls back (state and conv
history) to the accepted prefix by selection.  All inputs are synthetic
(synth/), generated before timing and resident in HBM: 67.9 GB of expert
weights, 48 shared experts and 36 fp32 GDN state pools.

Prints one JSON line: verified rows/s (k rows per step), the roofline of the
dominant kernel (the fused expert kernel, timed with HIP events on its
stream inside the timed region), a per-kernel breakdown from a separate
instrumented pass, and the CPU oracle timed on a bounded sample.
"""

import argparse
import hashlib
import json
import os
import platform
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "verified rows/s and achieved HBM GB/s (% of peak) for k-row Q4 verify + GDN"
PEAK_HBM_GBS = 8000.0  # MI355X HBM3E
PEAK_BF16_TFLOPS = 2500.0  # MI355X dense bf16 matrix-core peak
DOMINANT = "experts"
# the dominant kernel is bracketed by timing events in every SAMPLE_EVERY-th
# layer of each timed step: each event pair adds a few microseconds of idle
# time to the stream, so sampling keeps the step time close to untimed runs
SAMPLE_EVERY = 4
ACCEPT_BLOCKS = 8  # distinct verify blocks (logits, drafts) cycled through the steps
PROFILE_DIR = os.path.join(ROOT, "profiles")


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def parse_args():
    p = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=100)
    p.add_argument("--warmup", type=int, default=10)
    p.add_argument("--workload", default="flashnext_k9",
                   choices=["flashnext_k9", "flashnext_k16", "flashnext_k32"])
    p.add_argument("--no-cpu-baseline", action="store_true", help="skip the CPU oracle timing")
    p.add_argument("--no-breakdown", action="store_true", help="skip the per-kernel instrumented pass")
    p.add_argument("--fused-norm", action="store_true",
                   help="the GDN gated output norm inside the GDN launch (default: its own launch, faster here)")
    p.add_argument("--no-extra-configs", action="store_true",
                   help="skip the 256-expert MoE, 36-layer GDN and weight-format MoE lines")
    p.add_argument("--copy-probe", action="store_true",
                   help="only run a plain device copy of known size (PMC counter calibration)")
    return p.parse_args()


def q4_bytes(n, k):
    return n * k // 2 + n * (k // 64) * 4


def kernel_source_hash():
    """Hash of the dominant kernel's sources: a counter summary taken on other
    sources no longer describes it."""
    h = hashlib.sha256()
    for f in ("moe_experts.hip", "q4_core.h", "common.h", "route_core.h"):
        with open(os.path.join(ROOT, "speculative_decode_verification_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def _hip_runtime():
    """The HIP runtime already mapped into this process (the one torch and
    libsdv use), so events and streams are the same objects."""
    import ctypes
    paths = []
    with open("/proc/self/maps") as f:
        for line in f:
            part = line.split()
            if len(part) >= 6 and "libamdhip64" in part[-1] and part[-1] not in paths:
                paths.append(part[-1])
    if len(paths) != 1:
        raise RuntimeError(f"expected one HIP runtime in the process, found {paths}")
    return ctypes.CDLL(paths[0]), paths[0]


class HipTimer:
    """Timing events recorded on the launch stream without the system-scope
    fence default events carry (hipEventDisableSystemFence): recording them
    between kernels then costs no cache write-back and invalidation, so the
    timed sequence runs as it would untimed.  Events are created up front."""

    DISABLE_SYSTEM_FENCE = 0x20000000

    def __init__(self, pairs):
        import ctypes
        import torch
        self.ct = ctypes
        self.rt, self.path = _hip_runtime()
        self.rt.hipEventCreateWithFlags.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_uint]
        self.rt.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
        self.rt.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
        self.rt.hipEventDestroy.argtypes = [ctypes.c_void_p]
        self.stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
        self.pool = []
        for _ in range(2 * pairs):
            ev = ctypes.c_void_p()
            rc = self.rt.hipEventCreateWithFlags(ctypes.byref(ev), self.DISABLE_SYSTEM_FENCE)
            if rc != 0:
                raise RuntimeError(f"hipEventCreateWithFlags failed ({rc})")
            self.pool.append(ev)
        self.next = 0

    def start(self):
        ev = self.pool[self.next]
        self.next += 1
        self.rt.hipEventRecord(ev, self.stream)
        return ev

    stop = start

    def elapsed_us(self, a, b):
        ms = self.ct.c_float()
        rc = self.rt.hipEventElapsedTime(self.ct.byref(ms), a, b)
        if rc != 0:
            raise RuntimeError(f"hipEventElapsedTime failed ({rc})")
        return ms.value * 1e3

    def close(self):
        for ev in self.pool:
            self.rt.hipEventDestroy(ev)
        self.pool = []


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return platform.processor() or "unknown"


class Workload:
    """Device-resident inputs and bound launches of the flashnext step at k rows."""

    def __init__(self, dev, k=9, fused_norm=False):
        import torch
        import synth
        from synth import configs
        from synth import device as sdev
        from synth.inputs import DOWN, GATEUP, SHARED_DOWN, SHARED_GATEUP
        from speculative_decode_verification_amd import ops, pipeline

        cfg = configs.C4
        m, gs = cfg.moe, cfg.gdn
        self.k, self.cfg = k, cfg
        self.E, self.H, self.I, self.topk = m.experts, m.hidden, m.inter, m.topk
        self.layers = cfg.layers
        self.gdn_ids = list(cfg.gdn_layers)
        self.gs = gs
        self.moe, self.calls, self.gdn = [], [], {}
        t0 = time.time()
        def bank(kind, l, E, N, K, fused):
            # generated row-major in a scratch bank, then rewritten in the tiled layout
            rm = ops.Q4Weight(*sdev.q4_bank(synth.bank_keys(cfg.cid, kind, l), E, N, K, dev))
            return rm.tiled(fused_gateup=fused)

        for l in range(self.layers):
            gu = bank(GATEUP, l, self.E, 2 * self.I, self.H, True)
            dn = bank(DOWN, l, self.E, self.H, self.I, False)
            sgu = bank(SHARED_GATEUP, l, 1, 2 * self.I, self.H, True)
            sdn = bank(SHARED_DOWN, l, 1, self.H, self.I, False)
            inp = synth.moe_layer_inputs(cfg.cid, l, k, self.H, self.E)
            x, lg, z = (sdev.upload_bf16(inp["x"], dev), sdev.upload_f32(inp["logits"], dev),
                        sdev.upload_f32(inp["z"], dev))
            layer = pipeline.MoeLayer(gu, dn, k, self.topk, ops.ROUTE_SIGMOID, m.renorm, sgu, sdn)
            self.moe.append((layer, x, lg, z))
            self.calls.append(layer.bind(x, lg, z))
        for l in self.gdn_ids:
            # from the layer's projections: preparation (conv, q/k norm, gates),
            # the recurrence with snapshots, the gated output norm
            S0 = sdev.upload_f32(synth.gdn_state(cfg.cid, l, gs.hv, gs.dv, gs.dk), dev)
            raw = synth.gdn_raw_inputs(cfg.cid, l, k, gs.hv, gs.hk, gs.dk, gs.dv)
            d = {n: sdev.upload_f32(v, dev) for n, v in raw.items()}
            gl = pipeline.GdnLayer(S0, k).attach_prep(d["hist"], d["conv_w"], d["A_log"], d["dt_bias"], gs.hk)
            d["out"] = torch.empty((k, gs.hv, gs.dv), dtype=torch.float32, device=dev)
            if fused_norm:
                # the gated output norm in the same launch (the last workgroup
                # of each head applies it)
                gl.bind_from_proj_norm(d["qkv"], d["a"], d["b"], d["z"], d["norm_w"], d["out"])
            else:
                gl.bind_from_proj(d["qkv"], d["a"], d["b"])
                gl.bind_tail(d["z"], d["norm_w"], d["out"])
            self.gdn[l] = (gl, d)
        # acceptance of the block: next-token logits over the vocabulary with a
        # planted accepted-draft count per step (greedy), and the accepted
        # prefix n + 1 the GDN layers roll back to
        self.vocab = cfg.extra["vocab"]
        self.cycle = pipeline.VerifyCycle([gl for gl, _ in self.gdn.values()], k, self.vocab, dev)
        self.blocks = []
        for s in range(ACCEPT_BLOCKS):
            lg, dr, n = synth.verify_block(cfg.cid, s, k, self.vocab)
            lg_d = sdev.upload_f32(lg, dev)
            dr_d = torch.from_numpy(dr).to(dev)
            self.blocks.append((self.cycle.bind(lg_d, dr_d), n, lg_d, dr_d))
        torch.cuda.synchronize()
        self.fused_norm = fused_norm
        self.setup_s = time.time() - t0
        self.bank_bytes = self.layers * (self.E + 1) * (q4_bytes(2 * self.I, self.H) + q4_bytes(self.H, self.I))

    def step(self, s, timer=None, events=None, per_kernel=None):
        """One verify step over all layers, the acceptance of the block, then
        rollback of every GDN layer to the accepted prefix the device
        returned (its count is read back, one host synchronisation per step,
        as a decoding loop must).  With ``events``, the dominant kernel of
        every layer is bracketed by timer events; with ``per_kernel``, every
        launch is."""
        def run(name, l, call):
            if per_kernel is not None or (events is not None and name == DOMINANT and l % SAMPLE_EVERY == 0):
                a = timer.start()
                call()
                b = timer.stop()
                (per_kernel if per_kernel is not None else events).append((name, l, a, b))
            else:
                call()

        for l in range(self.layers):
            g = self.gdn.get(l)
            if g is not None:
                run("gdn", l, g[0].run_from_proj_bound)
                if not self.fused_norm:
                    run("gdn_norm", l, g[0].run_tail_bound)
            for name, call in self.calls[l]:
                run(name, l, call)
        accept, _, _, _ = self.blocks[s % len(self.blocks)]
        run("accept", self.layers, accept)
        n = int(self.cycle.accepted.item())
        # each GDN layer applies its rollback just before it runs again, so
        # between reading the count and the next step's first launch the host
        # handles one layer only
        for gl, _ in self.gdn.values():
            gl.rollback_later(n + 1)
        return n

    def check_acceptance(self):
        """Every block's device acceptance equals its planted count (outside timing)."""
        for call, n, _, _ in self.blocks:
            call()
            got = int(self.cycle.accepted.item())
            if got != n:
                raise RuntimeError(f"acceptance returned {got} drafts, planted {n}")

    def unions(self):
        return [int(layer.route.n_union.item()) for layer, *_ in self.moe]

    def kernel_bytes(self, name, l, unions):
        k, H, I, topk, E = self.k, self.H, self.I, self.topk, self.E
        if name == "accept":  # logits once, drafts, tokens and the count
            return k * self.vocab * 4 + (k - 1) * 4 + k * 4 + 4
        U = unions[l]
        if name == "route":
            return k * E * 4 + k * topk * 4 * 5 + 8
        # with the shared expert in the gathered launches, each reads one more
        # weight (its activations: the same x for gate/up, its own h for down)
        sh = 1 if self.moe[l][0].fused_shared else 0
        if name == "gate_up":
            return (U + sh) * q4_bytes(2 * I, H) + k * H * 2 + (k * topk + sh * k) * I * 4
        if name == "down":
            return (U + sh) * q4_bytes(H, I) + (k * topk + sh * k) * (I + H) * 4
        if name == "shared_gate_up":
            return q4_bytes(2 * I, H) + k * H * 2 + k * I * 4
        if name == "shared_down":
            return q4_bytes(H, I) + k * I * 4 + k * H * 4
        if name == "experts":
            # algorithmic: the union experts (and the shared expert) read
            # once, x read once, one output per used (row, slot) written once
            # (the method's per-slot expert outputs); the kernel's per-slice
            # partial sums beyond that are design traffic (design_bytes)
            used = k * topk + sh * k
            b = (U + sh) * (q4_bytes(2 * I, H) + q4_bytes(H, I)) + k * H * 2 + used * H * 4
            if self.moe[l][0].route_in_experts:
                # the router dispatch in the same launch: logits in, its
                # outputs out (as the "route" launch)
                b += k * E * 4 + k * topk * 4 * 5 + 8
            return b
        if name == "combine" and self.moe[l][0].fused_experts:
            # algorithmic: the per-slot outputs in, slot weights and indices,
            # the shared gate logits, y out
            used = k * topk + sh * k
            return used * H * 4 + k * topk * 8 + k * 4 + k * H * 4
        if name == "combine":
            return k * topk * H * 4 + k * topk * 4 + k * H * 4 + k * 4 + k * H * 4
        if name == "gdn":
            # preparation and recurrence in one launch: the state in, k
            # snapshots and y out; qkv rows, history, taps, a, b, A_log and
            # dt_bias in, the window [history; rows] out
            g = self.gs
            C = 2 * g.hk * g.dk + g.hv * g.dv
            b = ((k + 1) * g.hv * g.dv * g.dk * 4 + k * g.hv * g.dv * 4
                 + (k * C + 3 * C + 4 * C + 2 * k * g.hv + 2 * g.hv + (k + 3) * C) * 4)
            if self.fused_norm:
                # the gated norm in the same launch: z and the weight in, out written
                b += (2 * k * g.hv * g.dv + g.dv) * 4
            return b
        if name == "gdn_norm":
            g = self.gs
            return (3 * k * g.hv * g.dv + g.dv) * 4
        raise KeyError(name)

    def design_bytes(self, name, l):
        """HBM bytes a launch moves beyond its algorithmic bytes because of
        this design: the fused expert kernel writes one partial sum per
        128-wide intermediate slice of each used slot (S of them instead of
        one), and the combine reads them all back."""
        if name not in ("experts", "combine") or not self.moe[l][0].fused_experts:
            return 0
        S = (self.I + 127) // 128
        sh = 1 if self.moe[l][0].fused_shared else 0
        used = self.k * self.topk + sh * self.k
        return (S - 1) * used * self.H * 4

    def step_bytes(self, unions):
        total = 0
        for l in range(self.layers):
            for name, _ in self.calls[l]:
                total += self.kernel_bytes(name, l, unions)
            if l in self.gdn:
                for name in (("gdn",) if self.fused_norm else ("gdn", "gdn_norm")):
                    total += self.kernel_bytes(name, l, unions)
        return total + self.kernel_bytes("accept", self.layers, unions)


TRAFFIC_SUMMARY = "traffic_moe_experts_flashnext_k9.md"


def traffic_for(kernel_hash):
    """Counter-measured HBM bytes per launch of the dominant kernel, read from
    the committed counter summary (lines ``kernel_source_hash: H`` and
    ``hbm_bytes_per_launch: N``), or None if that summary was taken on other
    kernel sources."""
    path = os.path.join(PROFILE_DIR, TRAFFIC_SUMMARY)
    rec = {}
    try:
        with open(path) as f:
            for line in f:
                m = re.match(r"^\s*[-*]?\s*`?(kernel_source_hash|hbm_bytes_per_launch)`?:\s*`?([0-9a-f]+)`?", line)
                if m:
                    rec[m.group(1)] = m.group(2)
    except OSError:
        return None
    if rec.get("kernel_source_hash") != kernel_hash or "hbm_bytes_per_launch" not in rec:
        return None
    return int(rec["hbm_bytes_per_launch"])


def cpu_baseline(k=9, min_seconds=10.0, max_layers=16, threads_limit=None):
    """The CPU oracle on a bounded sample of the same workload: whole layers
    (MoE: route, union, gate/up, down, shared expert, combine, with the layer's
    union experts regenerated on the host before timing; GDN: preparation,
    the k-row recurrence with snapshots, the gated output norm), layer by
    layer until at least ``min_seconds`` of oracle time or ``max_layers``
    layers, then scaled to the 48 MoE + 36 GDN layers of a step."""
    import oracle
    import synth
    from synth import configs
    from synth.inputs import DOWN, GATEUP, SHARED_DOWN, SHARED_GATEUP

    cfg = configs.C4
    m, gs = cfg.moe, cfg.gdn
    E, H, I, topk = m.experts, m.hidden, m.inter, m.topk
    if threads_limit is not None:
        from threadpoolctl import threadpool_limits
        with threadpool_limits(limits=threads_limit):
            return cpu_baseline(k, min_seconds, max_layers)
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        threads = os.cpu_count() or 1
    t_moe, t_gdn, n_moe, n_gdn, unions = 0.0, 0.0, 0, 0, []
    for l in range(min(max_layers, cfg.layers)):
        inp = synth.moe_layer_inputs(cfg.cid, l, k, H, E)
        idx, _ = oracle.route(inp["logits"], topk, m.mode, m.renorm)
        used = sorted(set(idx.ravel().tolist()))
        gk, dk = synth.bank_keys(cfg.cid, GATEUP, l), synth.bank_keys(cfg.cid, DOWN, l)
        packed_g = {e: synth.q4_rows(gk, E, 2 * I, H, expert=e) for e in used}
        packed_d = {e: synth.q4_rows(dk, E, H, I, expert=e) for e in used}
        sgu = synth.dense_weight(cfg.cid, SHARED_GATEUP, l, 2 * I, H)
        sdn = synth.dense_weight(cfg.cid, SHARED_DOWN, l, H, I)
        t0 = time.perf_counter()
        oracle.moe_verify(oracle.bf16_to_f64(inp["x"]), inp["logits"], lambda e: oracle.dequant(*packed_g[e]),
                          lambda e: oracle.dequant(*packed_d[e]), topk, m.mode, m.renorm, z=inp["z"],
                          shared_gate_up=oracle.dequant(*sgu), shared_down=oracle.dequant(*sdn))
        t_moe += time.perf_counter() - t0
        n_moe += 1
        unions.append(len(used))
        if l in cfg.gdn_layers:
            S = synth.gdn_state(cfg.cid, l, gs.hv, gs.dv, gs.dk)
            raw = synth.gdn_raw_inputs(cfg.cid, l, k, gs.hv, gs.hk, gs.dk, gs.dv)
            t0 = time.perf_counter()
            p = oracle.gdn_prepare(raw["qkv"], raw["hist"], raw["conv_w"], raw["a"], raw["b"], raw["A_log"],
                                   raw["dt_bias"], gs.hk, gs.hv, gs.dk, gs.dv)
            y, _ = oracle.gdn_verify(S, p["q"], p["k"], p["v"], p["g"], p["beta"])
            oracle.gdn_gated_norm(y, raw["z"], raw["norm_w"])
            t_gdn += time.perf_counter() - t0
            n_gdn += 1
        if t_moe + t_gdn >= min_seconds:
            break
    lg, dr, _ = synth.verify_block(cfg.cid, 0, k, cfg.extra["vocab"])
    t0 = time.perf_counter()
    oracle.verify_cycle(lg, dr)
    t_acc = time.perf_counter() - t0
    step = cfg.layers * t_moe / n_moe + len(cfg.gdn_layers) * t_gdn / n_gdn + t_acc
    return {"value": k / step, "unit": "rows/s", "cores": threads, "kind": "oracle",
            "sample": (f"flashnext_k{k} layers 0..{n_moe - 1}: {n_moe} MoE layers (union experts {unions}, "
                       f"{t_moe:.1f} s) and {n_gdn} GDN layers ({t_gdn:.2f} s) of the oracle (numpy fp64, "
                       f"{t_moe + t_gdn:.1f} s in all), scaled to 48 MoE + 36 GDN layers per step, plus one "
                       f"acceptance of the block ({t_acc:.2f} s) ({step:.1f} s per {k}-row step)"),
            "host_cpu": cpu_model(), "host_logical_cpus": os.cpu_count()}


def cpu_configs(threads_limit=None):
    """The CPU oracle (untuned numpy fp64) on one unit of each other
    configuration, per width: the dense 5120 x 5120 projection (rows/s of one
    projection, widths 1/4/8/9), one 256-expert MoE layer (rows/s of a
    40-layer step, widths 2..9: route, union experts dequantised from the
    layer's bank, gate/up, down, combine) and one 36-layer GDN step's layer
    (rows/s of a 36-layer step, widths 1..9: the k-row recurrence with its
    snapshots).  Each unit runs once per width; generation is outside the
    timed region; each configuration's first run is an untimed warm-up."""
    import oracle
    import synth
    from synth import configs
    from synth.inputs import DENSE_W, DOWN, GATEUP

    if threads_limit is not None:
        from threadpoolctl import threadpool_limits
        with threadpool_limits(limits=threads_limit):
            r = cpu_configs()
        r["cores"] = threads_limit
        return r
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        threads = os.cpu_count() or 1
    out = {"cores": threads, "kind": "oracle", "unit": "rows/s"}
    c1 = configs.C1
    N, K = c1.dense
    codes, sc, bi = synth.dense_weight(c1.cid, DENSE_W, 0, N, K)
    dense = {}
    oracle.qmv(codes, sc, bi, oracle.bf16_to_f64(synth.activations(c1.cid, 0, 1, K)))  # warm-up, untimed
    for k in c1.widths:
        x = oracle.bf16_to_f64(synth.activations(c1.cid, 0, k, K))
        t0 = time.perf_counter()
        oracle.qmv(codes, sc, bi, x)
        dense[f"k{k}"] = round(k / (time.perf_counter() - t0), 2)
    out["dense5120"] = {"what": "rows/s of one 5120 x 5120 projection", "widths": dense}
    c2 = configs.C2
    m = c2.moe
    E, H, I, topk = m.experts, m.hidden, m.inter, m.topk
    gk, dk = synth.bank_keys(c2.cid, GATEUP, 0), synth.bank_keys(c2.cid, DOWN, 0)
    moe, cache_g, cache_d = {}, {}, {}
    for k in (c2.widths[0],) + tuple(c2.widths):  # the first width twice: its first run is a warm-up
        inp = synth.moe_layer_inputs(c2.cid, 0, k, H, E)
        idx, _ = oracle.route(inp["logits"], topk, m.mode, m.renorm)
        for e in sorted(set(idx.ravel().tolist())):
            if e not in cache_g:
                cache_g[e] = synth.q4_rows(gk, E, 2 * I, H, expert=e)
                cache_d[e] = synth.q4_rows(dk, E, H, I, expert=e)
        t0 = time.perf_counter()
        oracle.moe_verify(oracle.bf16_to_f64(inp["x"]), inp["logits"], lambda e: oracle.dequant(*cache_g[e]),
                          lambda e: oracle.dequant(*cache_d[e]), topk, m.mode, m.renorm)
        moe[f"k{k}"] = round(k / ((time.perf_counter() - t0) * c2.layers), 3)
    out["ornith_moe"] = {"what": f"rows/s of a {c2.layers}-layer step, one layer timed", "widths": moe}
    c3 = configs.C3
    g = c3.gdn
    S = synth.gdn_state(c3.cid, 0, g.hv, g.dv, g.dk)
    gdn = {}
    for k in (c3.widths[0],) + tuple(c3.widths):  # the first width twice: its first run is a warm-up
        inp = synth.gdn_layer_inputs(c3.cid, 0, k, g.hv, g.hk, g.dk, g.dv)
        t0 = time.perf_counter()
        oracle.gdn_verify(S, inp["q"], inp["k"], inp["v"], inp["g"], inp["beta"])
        gdn[f"k{k}"] = round(k / ((time.perf_counter() - t0) * c3.layers), 2)
    out["gdn36"] = {"what": f"rows/s of a {c3.layers}-layer step, one layer timed", "widths": gdn}
    return out


def dense_projection(dev, timer, n_weights=64, reps=4):
    """sdv_qmv_k on the dense 5120 x 5120 shape: 64 distinct weights (944 MB
    of affine Q4, more than the last-level cache) launched back to back at
    each width, timed with HIP events around each width's launches; then the
    same for the Q8_0 (1.7 GB) and affine-Q3 (0.66 GB) formats; 16 and 32
    rows take the one-pass wide form (affine Q4 and Q3).  Reported per
    projection: time and algorithmic GB/s (weights, activations and outputs
    once)."""
    import torch
    import synth
    from synth import device as sdev
    from synth.inputs import DENSE_W
    from speculative_decode_verification_amd import ops
    N = K = 5120
    x = sdev.upload_bf16(synth.activations(1, 0, 32, K), dev)

    def time_widths(Ws, wbytes, widths):
        res = {}
        for k in widths:
            xs = x[:k].contiguous()
            ys = torch.empty((k, N), dtype=torch.float32, device=dev)
            calls = [ops.bind_qmv_k(W, xs, ops.MODE_PLAIN, ys) for W in Ws]
            for c in calls:
                c()
            torch.cuda.synchronize()
            a = timer.start()
            for _ in range(reps):
                for c in calls:
                    c()
            b = timer.stop()
            torch.cuda.synchronize()
            us = timer.elapsed_us(a, b) / (reps * len(Ws))
            nbytes = wbytes + k * (2 * K + 4 * N)
            # algorithmic flops 2 k N K against the dense bf16 matrix-core
            # peak (the products run on bf16 MFMA)
            tflops = 2.0 * k * N * K / us / 1e6
            res[f"k{k}"] = {"us": round(us, 2), "gbs": round(nbytes / us / 1e3, 1),
                            "frac_hbm": round(nbytes / us / 1e3 / PEAK_HBM_GBS, 3),
                            "tflops": round(tflops, 2), "frac_mfma_bf16": round(tflops / PEAK_BF16_TFLOPS, 4)}
        return res

    def time_multi(Ws, wbytes, widths, per_call=16):
        """sdv_qmv_k_multi: the weights in launches of 16 that share the
        activation rows (one launch ramp per 16 projections)."""
        res = {}
        for k in widths:
            xs = x[:k].contiguous()
            groups = [Ws[i:i + per_call] for i in range(0, len(Ws), per_call)]
            outs = [[torch.empty((k, N), dtype=torch.float32, device=dev) for _ in g] for g in groups]
            calls = [ops.bind_qmv_k_multi(g, xs, ops.MODE_PLAIN, o) for g, o in zip(groups, outs)]
            for c in calls:
                c()
            torch.cuda.synchronize()
            a = timer.start()
            for _ in range(reps):
                for c in calls:
                    c()
            b = timer.stop()
            torch.cuda.synchronize()
            us = timer.elapsed_us(a, b) / (reps * len(Ws))
            nbytes = wbytes + k * 2 * K + k * 4 * N
            res[f"k{k}"] = {"us_per_projection": round(us, 2), "gbs": round(nbytes / us / 1e3, 1),
                            "frac_hbm": round(nbytes / us / 1e3 / PEAK_HBM_GBS, 3)}
        return {"weights_per_launch": per_call, "widths": res}

    Ws = [ops.Q4Weight(*sdev.q4_bank(synth.bank_keys(1, DENSE_W, l), 1, N, K, dev)).tiled()
          for l in range(n_weights)]
    out = time_widths(Ws, q4_bytes(N, K), (1, 4, 8, 9, 16, 32))
    multi = time_multi(Ws, q4_bytes(N, K), (1, 9, 32))
    del Ws
    # Q8_0 and affine Q3 weights filled on the device (any codes are valid;
    # parity of these formats is covered by the tests)
    g = torch.Generator(device=dev)
    g.manual_seed(5120)
    Ws = []
    for _ in range(n_weights):
        qs = torch.randint(-127, 128, (N, K), dtype=torch.int8, device=dev, generator=g)
        d = (torch.rand((N, K // 32), device=dev, generator=g) * 6e-4 + 2e-4).to(torch.float16).view(torch.int16)
        Ws.append(ops.Q8Weight(qs, d).tiled())
        del qs, d
    q8 = time_widths(Ws, N * K + N * (K // 64) * 4, (1, 9))
    del Ws
    Ws = []
    for _ in range(n_weights):
        codes = torch.randint(0, 256, (N, 3 * K // 8), dtype=torch.uint8, device=dev, generator=g)
        sc = (torch.rand((N, K // 64), device=dev, generator=g) * 0.03 + 0.01).to(torch.bfloat16).view(torch.int16)
        bi = (torch.rand((N, K // 64), device=dev, generator=g) * 0.2 - 0.1).to(torch.bfloat16).view(torch.int16)
        Ws.append(ops.Q3Weight(codes, sc, bi).tiled())
        del codes, sc, bi
    q3 = time_widths(Ws, N * 3 * K // 8 + N * (K // 64) * 4, (1, 9, 32))
    del Ws
    torch.cuda.empty_cache()
    return {"shape": [N, K], "weights": n_weights, "widths": out, "multi_weight_launch": multi, "q8_0": q8,
            "q3": q3}


def ornith_moe(dev, widths=tuple(range(2, 10)), reps=3):
    """The 256-expert MoE verify (hidden 2048, intermediate 512, softmax
    top-8, no shared expert) over 40 distinct layer banks (18.1 GB of affine
    Q4, rotated so no layer's experts are cache-resident): router dispatch,
    the fused expert kernel and the combine of every layer, back to back, at
    each width.  Reported per width: the layer time, verified rows/s of a
    40-layer step, the mean union, algorithmic bytes per layer (the union
    experts once, x, logits and y) as GB/s, and the expert kernel alone
    (events around its launches in a separate pass)."""
    import torch
    import synth
    from synth import configs
    from synth import device as sdev
    from synth.inputs import DOWN, GATEUP
    from speculative_decode_verification_amd import ops, pipeline
    cfg = configs.C2
    m = cfg.moe
    E, H, I, topk = m.experts, m.hidden, m.inter, m.topk
    banks = []
    for l in range(cfg.layers):
        gu = ops.Q4Weight(*sdev.q4_bank(synth.bank_keys(cfg.cid, GATEUP, l), E, 2 * I, H, dev)).tiled(True)
        dn = ops.Q4Weight(*sdev.q4_bank(synth.bank_keys(cfg.cid, DOWN, l), E, H, I, dev)).tiled()
        banks.append((gu, dn))
    ex_bytes = q4_bytes(2 * I, H) + q4_bytes(H, I)
    out = {}
    for k in widths:
        layers, calls = [], []
        for l, (gu, dn) in enumerate(banks):
            inp = synth.moe_layer_inputs(cfg.cid, l, k, H, E)
            x, lg = sdev.upload_bf16(inp["x"], dev), sdev.upload_f32(inp["logits"], dev)
            layer = pipeline.MoeLayer(gu, dn, k, topk, ops.ROUTE_SOFTMAX, m.renorm)
            layers.append((layer, x, lg))
            calls.append(layer.bind(x, lg))
        for cl in calls:
            for _, c in cl:
                c()
        torch.cuda.synchronize()
        timer = HipTimer(1 + cfg.layers)
        a = timer.start()
        for _ in range(reps):
            for cl in calls:
                for _, c in cl:
                    c()
        b = timer.stop()
        torch.cuda.synchronize()
        us_layer = timer.elapsed_us(a, b) / (reps * cfg.layers)
        ev = []
        for cl in calls:
            for name, c in cl:
                if name == "experts":
                    e0 = timer.start()
                    c()
                    ev.append((e0, timer.stop()))
                else:
                    c()
        torch.cuda.synchronize()
        ex_us = sum(timer.elapsed_us(e0, e1) for e0, e1 in ev) / len(ev)
        timer.close()
        unions = [int(layer.route.n_union.item()) for layer, _, _ in layers]
        mu = sum(unions) / len(unions)
        lb = mu * ex_bytes + k * H * 2 + k * E * 4 + k * H * 4
        eb = mu * ex_bytes + k * H * 2 + k * topk * H * 4
        out[f"k{k}"] = {"us_per_layer": round(us_layer, 2),
                        "rows_per_s_40_layers": round(k / (us_layer * cfg.layers * 1e-6), 1),
                        "mean_union": round(mu, 2), "bytes_per_layer": round(lb),
                        "gbs": round(lb / us_layer / 1e3, 1), "frac_hbm": round(lb / us_layer / 1e3 / PEAK_HBM_GBS, 3),
                        "experts_us": round(ex_us, 2), "experts_frac_hbm": round(eb / ex_us / 1e3 / PEAK_HBM_GBS, 3)}
        del layers, calls
    del banks
    torch.cuda.empty_cache()
    return {"workload": "ornith_moe: 40 layers x [256 experts: gate/up 1024x2048 + down 2048x512, affine Q4/g64], "
                        "softmax top-8", "widths": out}


def format_bytes(fmt, n, k):
    """Bytes of one [n, k] matrix in a weight format: affine Q4/g64 (nibbles,
    bf16 scale and bias per 64), Q8_0 (bytes, a half scale per 32) or affine
    Q3/g64 (three bits, bf16 scale and bias per 64)."""
    if fmt == "q4":
        return q4_bytes(n, k)
    if fmt == "q8_0":
        return n * k + n * (k // 32) * 2
    if fmt == "q3":
        return n * k * 3 // 8 + n * (k // 64) * 4
    raise KeyError(fmt)


def _format_bank(fmt, E, N, K, fused, dev, gen):
    """A whole [E, N, K] bank of uniformly random codes in device memory
    (seeded torch generator; any byte pattern is a valid code), scales and
    biases in the synthetic inputs' ranges, repacked to the tiled layout."""
    import torch
    from speculative_decode_verification_amd import ops
    bf16 = lambda shape, lo, hi: (torch.empty(shape, dtype=torch.float32, device=dev).uniform_(lo, hi, generator=gen)
                                  .to(torch.bfloat16).view(torch.int16))
    if fmt == "q8_0":
        qs = torch.randint(-127, 128, (E, N, K), dtype=torch.int8, device=dev, generator=gen)
        d = (torch.empty((E, N, K // 32), dtype=torch.float32, device=dev).uniform_(2e-4, 8e-4, generator=gen)
             .to(torch.float16).view(torch.int16))
        W = ops.Q8Weight(qs, d)
    elif fmt == "q3":
        codes = torch.randint(0, 256, (E, N, 3 * K // 8), dtype=torch.uint8, device=dev, generator=gen)
        W = ops.Q3Weight(codes, bf16((E, N, K // 64), 0.01, 0.04), bf16((E, N, K // 64), -0.1, 0.1))
    else:
        codes = torch.randint(-2 ** 31, 2 ** 31 - 1, (E, N, K // 8), dtype=torch.int32, device=dev, generator=gen)
        W = ops.Q4Weight(codes, bf16((E, N, K // 64), 0.01, 0.04), bf16((E, N, K // 64), -0.1, 0.1))
    T = W.tiled(fused_gateup=fused)
    del W
    return T


def format_moe(dev, widths=(2, 9), formats=("q4", "q8_0", "q3"), layers=6, reps=3):
    """The Flash-Next MoE layer geometry (512 experts, hidden 2560,
    intermediate 640, sigmoid top-10 with renormalisation, the gated shared
    expert) with the routed and shared experts in affine Q4, Q8_0 or affine
    Q3, over `layers` distinct banks rotated so no layer's experts are
    cache-resident.  Per format and width: the fused path (router, expert
    kernel, sliced combine) and the gathered path (router, gate/up and down
    gathered launches carrying the shared expert, combine), the layer time
    each, and the expert kernel alone against its algorithmic bytes (union
    and shared experts once, x, one output per used slot)."""
    import torch
    import synth
    from synth import configs
    from synth import device as sdev
    from speculative_decode_verification_amd import ops, pipeline
    m = configs.C4.moe
    E, H, I, topk = m.experts, m.hidden, m.inter, m.topk
    out = {}
    for fmt in formats:
        gen = torch.Generator(device=dev)
        gen.manual_seed(4242)
        banks = []
        for _ in range(layers):
            banks.append(tuple(_format_bank(fmt, e, n, kk, f, dev, gen) for e, n, kk, f in
                               ((E, 2 * I, H, True), (E, H, I, False), (1, 2 * I, H, True), (1, H, I, False))))
        ex_bytes = format_bytes(fmt, 2 * I, H) + format_bytes(fmt, H, I)
        res = {}
        for k in widths:
            row = {}
            for path, fused in (("fused", True), ("gathered", False)):
                layer_objs, calls = [], []
                for l, (gu, dn, sgu, sdn) in enumerate(banks):
                    inp = synth.moe_layer_inputs(configs.C4.cid, l, k, H, E)
                    args = (sdev.upload_bf16(inp["x"], dev), sdev.upload_f32(inp["logits"], dev),
                            sdev.upload_f32(inp["z"], dev))
                    layer = pipeline.MoeLayer(gu, dn, k, topk, ops.ROUTE_SIGMOID, m.renorm, sgu, sdn,
                                              fused_experts=fused)
                    layer_objs.append((layer, args))
                    calls.append(layer.bind(*args))
                for cl in calls:
                    for _, c in cl:
                        c()
                torch.cuda.synchronize()
                timer = HipTimer(1 + layers)
                a = timer.start()
                for _ in range(reps):
                    for cl in calls:
                        for _, c in cl:
                            c()
                b = timer.stop()
                torch.cuda.synchronize()
                us_layer = timer.elapsed_us(a, b) / (reps * layers)
                ev = []
                for cl in calls:
                    for name, c in cl:
                        if name == "experts":
                            e0 = timer.start()
                            c()
                            ev.append((e0, timer.stop()))
                        else:
                            c()
                torch.cuda.synchronize()
                r = {"us_per_layer": round(us_layer, 2)}
                if ev:
                    ex_us = sum(timer.elapsed_us(e0, e1) for e0, e1 in ev) / len(ev)
                    unions = [int(lo.route.n_union.item()) for lo, _ in layer_objs]
                    mu = sum(unions) / len(unions)
                    eb = (mu + 1) * ex_bytes + k * H * 2 + (k * topk + k) * H * 4
                    r.update({"mean_union": round(mu, 2), "experts_us": round(ex_us, 2),
                              "experts_bytes": round(eb),
                              "experts_frac_hbm": round(eb / ex_us / 1e3 / PEAK_HBM_GBS, 3)})
                timer.close()
                row[path] = r
                del layer_objs, calls
            res[f"k{k}"] = row
        out[fmt] = {"bank_bytes_per_layer": E * ex_bytes + ex_bytes, "widths": res}
        del banks
        torch.cuda.empty_cache()
    return {"workload": f"format_moe: {layers} layers x [512 experts + shared: gate/up 1280x2560 + down 2560x640], "
                        "sigmoid top-10, affine Q4 / Q8_0 / affine Q3", "formats": out}


def gdn36_chains(dev, widths=tuple(range(1, 10)), steps=16):
    """The GDN verify of 36 layers (48 v heads, 16 qk heads, Dk = Dv = 128,
    3 MB of fp32 state per layer, 113 MB in all) at each width: 16-step
    chains, each step the k-row recurrence with snapshots on every layer,
    then rollback of every layer to an accepted prefix j ~ U{0..k} by slot
    selection.  Reported per width: verified rows/s (k rows per 36-layer
    step), the per-layer time, and algorithmic bytes per layer (the state in,
    k snapshots out, q, k, v, g, beta in and y out per row) as GB/s."""
    import torch
    import synth
    from synth import configs
    from synth import device as sdev
    from speculative_decode_verification_amd import pipeline
    cfg = configs.C3
    g = cfg.gdn
    S0 = [sdev.upload_f32(synth.gdn_state(cfg.cid, l, g.hv, g.dv, g.dk), dev) for l in range(cfg.layers)]
    out = {}
    for k in widths:
        layers = []
        for l in range(cfg.layers):
            d = {n: sdev.upload_f32(v, dev)
                 for n, v in synth.gdn_layer_inputs(cfg.cid, l, k, g.hv, g.hk, g.dk, g.dv).items()}
            gl = pipeline.GdnLayer(S0[l], k).bind(d["q"], d["k"], d["v"], d["g"], d["beta"])
            layers.append((gl, d))
        js = [synth.accepted_prefix(cfg.cid, s, k) for s in range(steps)]
        for gl, _ in layers:  # warm-up step
            gl.run_bound()
        for gl, _ in layers:
            gl.rollback(js[0])
        torch.cuda.synchronize()
        timer = HipTimer(1)
        a = timer.start()
        for s in range(steps):
            for gl, _ in layers:
                gl.run_bound()
            for gl, _ in layers:
                gl.rollback(js[s])
        b = timer.stop()
        torch.cuda.synchronize()
        us = timer.elapsed_us(a, b)
        timer.close()
        per_layer = us / (steps * cfg.layers)
        lb = (k + 1) * g.hv * g.dv * g.dk * 4 + k * (2 * g.hk * g.dk + 2 * g.hv * g.dv + 2 * g.hv) * 4
        out[f"k{k}"] = {"rows_per_s": round(k * steps / (us * 1e-6), 1), "us_per_layer": round(per_layer, 2),
                        "bytes_per_layer": lb, "gbs": round(lb / per_layer / 1e3, 1),
                        "frac_hbm": round(lb / per_layer / 1e3 / PEAK_HBM_GBS, 3),
                        "accepted_prefixes": js}
        del layers
    del S0
    torch.cuda.empty_cache()
    return {"workload": "gdn36: 36 layers x state [48,128,128] fp32, 16-step chains with rollback", "widths": out}


def gdn_layers_one_launch(wl, dev, unions, reps=20):
    """The step's GDN layers (preparation + recurrence with snapshots) as
    independent layers in one launch (sdv_gdn_verify_prep_k_layers), a
    measurement form labelled as such: it shows the kernel's bandwidth
    without the ramp of each launch.  The step itself runs one launch per
    layer, since each layer's input depends on the layer before."""
    import torch
    from speculative_decode_verification_amd import ops
    layers = sorted(wl.gdn)
    launch = ops.GdnLayersLaunch([wl.gdn[l][0].prep_call() for l in layers], dev)
    for _ in range(3):
        launch()
    torch.cuda.synchronize()
    timer = HipTimer(1)
    a = timer.start()
    for _ in range(reps):
        launch()
    b = timer.stop()
    torch.cuda.synchronize()
    us = timer.elapsed_us(a, b) / reps
    timer.close()
    lb = sum(wl.kernel_bytes("gdn", l, unions) for l in layers)
    return {"what": f"{len(layers)} independent GDN layers (preparation + recurrence, k = {wl.k}) in one launch; "
                    "a measurement form, not the step's launch sequence",
            "layers": len(layers), "us_per_launch": round(us, 2), "us_per_layer": round(us / len(layers), 2),
            "bytes_per_layer": round(lb / len(layers)), "gbs": round(lb / us / 1e3, 1),
            "frac_hbm": round(lb / us / 1e3 / PEAK_HBM_GBS, 3)}


def copy_probe():
    """A plain device copy of known size, for scaling HBM counters."""
    import torch
    n = 1 << 28  # 1 GiB of fp32
    a = torch.ones(n, dtype=torch.float32, device="cuda:0")
    b = torch.empty_like(a)
    for _ in range(3):
        b.copy_(a)
    torch.cuda.synchronize()
    log(f"copy probe: 3 copies of {a.numel() * 4} bytes")


def main():
    args = parse_args()
    if args.gpus != 1:
        log(f"bench.py runs on one GPU: this build has no multi-GPU path (asked for --gpus {args.gpus}); "
            "the per-GPU shard of the verify step is the single-GPU workload.")
        sys.exit(2)
    import torch
    if not torch.cuda.is_available():
        log("bench.py needs a GPU")
        sys.exit(1)
    if args.copy_probe:
        copy_probe()
        return
    from speculative_decode_verification_amd import _lib
    _lib.lib()  # fail loudly if the HIP library is missing
    dev = torch.device("cuda:0")
    k = int(args.workload.rsplit("_k", 1)[1])
    log(f"building workload {args.workload} (device-filled banks) ...")
    wl = Workload(dev, k, fused_norm=args.fused_norm)
    log(f"workload ready in {wl.setup_s:.1f} s: {wl.bank_bytes / 1e9:.1f} GB of Q4 banks, "
        f"{len(wl.gdn)} GDN layers")
    wl.check_acceptance()
    for s in range(args.warmup):
        wl.step(s)
    torch.cuda.synchronize()
    unions = wl.unions()

    per_step = len(wl.calls[0]) * wl.layers + (1 if wl.fused_norm else 2) * len(wl.gdn) + 1
    # the dominant kernel's events, one mark per step boundary, the breakdown
    # pass and the dense widths
    timer = HipTimer((wl.layers // SAMPLE_EVERY + 1) * args.steps + args.steps + 1 + per_step + 1 + 9)
    log(f"timing events on the launch stream (HIP runtime {timer.path})")
    events = []
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    t_start = timer.start()
    marks = [t_start]
    for s in range(args.steps):
        wl.step(args.warmup + s, timer=timer, events=events)
        marks.append(timer.stop())
    t_end = marks[-1]
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    ms_total = timer.elapsed_us(t_start, t_end) / 1e3
    step_us = sorted(timer.elapsed_us(a, b) for a, b in zip(marks[:-1], marks[1:]))
    pct = lambda q: step_us[min(len(step_us) - 1, int(q * len(step_us)))]
    # rows/s of single steps: the median, and p10 / p90 (p10 of rows/s is the
    # p90 of step time)
    step_rows = {"median": round(k / (pct(0.5) * 1e-6), 1), "p10": round(k / (pct(0.9) * 1e-6), 1),
                 "p90": round(k / (pct(0.1) * 1e-6), 1)}
    ms_step = ms_total / args.steps
    rows_per_s = k * args.steps / (ms_total / 1e3)
    step_bytes = wl.step_bytes(unions)

    dom_us = [timer.elapsed_us(a, b) for (_, _, a, b) in events]
    dom_bytes = [wl.kernel_bytes(DOMINANT, l, unions) for (_, l, _, _) in events]
    dom_design = [wl.design_bytes(DOMINANT, l) for (_, l, _, _) in events]
    dom_avg_us = sum(dom_us) / len(dom_us)
    dom_gbs = sum(dom_bytes) / (sum(dom_us) * 1e-6) / 1e9
    khash = kernel_source_hash()
    traffic = traffic_for(khash) if args.workload == "flashnext_k9" else None

    breakdown = None
    if not args.no_breakdown:
        per = []
        wl.step(args.warmup + args.steps, timer=timer, per_kernel=per)
        torch.cuda.synchronize()
        agg = {}
        for name, l, a, b in per:
            us = timer.elapsed_us(a, b)
            d = agg.setdefault(name, {"launches": 0, "us": 0.0, "bytes": 0})
            d["launches"] += 1
            d["us"] += us
            d["bytes"] += wl.kernel_bytes(name, l, unions)
        breakdown = {n: {"launches": d["launches"], "avg_us": round(d["us"] / d["launches"], 2),
                         "share_of_step": round(d["us"] / 1e3 / ms_step, 3),
                         "gbs": round(d["bytes"] / (d["us"] * 1e-6) / 1e9, 1),
                         "frac_hbm": round(d["bytes"] / (d["us"] * 1e-6) / 1e9 / PEAK_HBM_GBS, 3)}
                     for n, d in agg.items()}

    gdn_batched = None
    if not args.no_breakdown and not wl.fused_norm:
        log("timing the GDN layers in one launch (measurement form) ...")
        gdn_batched = gdn_layers_one_launch(wl, dev, unions)

    dense = None
    if not args.no_breakdown:
        log("timing the dense 5120 x 5120 projection ...")
        dense = dense_projection(dev, timer)

    extra = {}
    if not args.no_extra_configs:
        log("timing the 256-expert MoE layers (k = 2..9) ...")
        extra["ornith_moe"] = ornith_moe(dev)
        log("timing the 36-layer GDN chains (k = 1..9) ...")
        extra["gdn36"] = gdn36_chains(dev)
        log("timing the Flash-Next MoE layer in affine Q4, Q8_0 and affine Q3 (fused and gathered) ...")
        extra["format_moe"] = format_moe(dev)

    cpu = cpu1 = cpu_cfg = None
    if not args.no_cpu_baseline:
        log("timing the CPU oracle on a bounded sample (all host cores, then one) ...")
        cpu = cpu_baseline(k)
        cpu1 = cpu_baseline(k, min_seconds=10.0, max_layers=2, threads_limit=1)
        if not args.no_extra_configs:
            log("timing the CPU oracle on the other configurations' units (all host cores, then one) ...")
            cpu_cfg = {"all_cores": cpu_configs(), "one_core": cpu_configs(threads_limit=1)}

    out = {
        "metric": METRIC,
        "value": round(rows_per_s, 1),
        "unit": "rows/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": args.workload, "rows": k, "layers": wl.layers, "gdn_layers": len(wl.gdn),
                   "experts": wl.E, "topk": wl.topk, "hidden": wl.H, "inter": wl.I, "shared_expert": True,
                   "gdn_heads": [wl.gs.hv, wl.gs.hk, wl.gs.dk], "vocab": wl.vocab,
                   "mean_union": round(sum(unions) / len(unions), 2),
                   "bytes_per_step": step_bytes},
        "step_rows_per_s": step_rows,
        "hbm_gbs_step": round(step_bytes / (ms_step * 1e-3) / 1e9, 1),
        "hbm_frac_step": round(step_bytes / (ms_step * 1e-3) / 1e9 / PEAK_HBM_GBS, 3),
        "roofline": {"bound": "hbm", "achieved": round(dom_gbs, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                     "frac": round(dom_gbs / PEAK_HBM_GBS, 3), "traffic": traffic,
                     "kernel": "moe_experts_kernel (sdv_moe_experts_k: fused gate/up + SwiGLU + down)",
                     "avg_launch_us": round(dom_avg_us, 2),
                     "bytes_per_launch": round(sum(dom_bytes) / len(dom_bytes)),
                     "design_traffic": {"bytes_per_launch": round(sum(dom_design) / len(dom_design)),
                                        "what": "per-slice partial sums written beyond one output per used slot "
                                                "(read back by the combine); not in achieved"},
                     "kernel_source_hash": khash},
        "kernels": breakdown,
        "gdn_layers_one_launch": gdn_batched,
        "dense_qmv_k": dense,
        "cpu_baseline": cpu,
        "cpu_baseline_1core": cpu1,
        "cpu_other_configs": cpu_cfg,
        "accepted_count": ("read back from the device every timed step (one host synchronisation per step); "
                           "each GDN layer's rollback to it is applied before the layer's next launch"),
        **extra,
        "wall_s_timed": round(wall, 3),
        "env": {"gpu": torch.cuda.get_device_name(0), "torch": torch.__version__, "host_cpu": cpu_model()},
    }
    timer.close()
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
