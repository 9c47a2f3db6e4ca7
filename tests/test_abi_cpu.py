"""The C ABI on the CPU: the library loads, exports every declared symbol,
and rejects bad arguments before any launch (no GPU is touched: every call
here fails host validation, which runs before any HIP call)."""

import ctypes
import os
import re
import subprocess

import pytest

from speculative_decode_verification_amd import _lib as L

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "sdv.h")

P = 0x10000  # fake, 16-byte aligned "device" addresses; validation fails before any use


def declared():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"SDV_API\s+[\w\s\*]+?\b(sdv_\w+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(L.LIB_PATH):
        pytest.fail("libsdv.so is not built (run `python __graft_entry__.py build`)")
    return L.lib()


def test_exports_match_header(lib):
    names = declared()
    assert len(names) == 32
    assert tuple(sorted(L.EXPORTS)) == tuple(names)
    for n in names:
        assert hasattr(lib, n), n
    nm = subprocess.run(["nm", "-D", "--defined-only", L.LIB_PATH], capture_output=True, text=True).stdout
    exported = sorted(set(re.findall(r"\bT (sdv_\w+)", nm)))
    assert exported == names


def test_status_strings(lib):
    for code, text in [(0, "ok"), (-1, "invalid argument"), (-2, "unsupported row width"),
                       (-3, "unsupported layout"), (-4, "value out of range"), (-5, "output aliases"),
                       (-6, "HIP runtime error")]:
        assert lib.sdv_status_string(code).decode().startswith(text)
    assert b"gfx950" in lib.sdv_build_info()


def q4(E=1, N=64, K=128, group=64, codes=P, scales=P + 0x100000, biases=P + 0x200000):
    return L.SdvQ4(codes, scales, biases, E, N, K, group)


def q4t(E=1, N=64, K=128, group=64, codes=P, sb=P + 0x100000, fused=0, fmt=0):
    return L.SdvQ4T(codes, sb, E, N, K, group, fused, fmt)


def qmv(lib, W, act=P + 0x400000, dtype=L.ACT_BF16, k=2, mode=L.MODE_PLAIN, y=P + 0x800000):
    return lib.sdv_qmv_k(ctypes.byref(W), act, dtype, k, mode, y, None)


def test_tiled_sizes(lib):
    # T tiles x G groups x (1 KB of codes, 128 B of scale/bias words)
    assert lib.sdv_q4t_codes_bytes(512, 1280, 2560, 1) == 512 * 40 * 40 * 1024
    assert lib.sdv_q4t_sb_bytes(512, 1280, 2560, 1) == 512 * 40 * 40 * 128
    assert lib.sdv_q4t_codes_bytes(1, 1000, 576, 0) == 32 * 9 * 1024
    assert lib.sdv_q4t_codes_bytes(1, 34, 64, 1) == 2 * 1 * 1024
    assert lib.sdv_q4t_codes_bytes(1, 64, 100, 0) == 0


def test_repack_validation(lib):
    f = lib.sdv_q4_repack
    out_c, out_s = P + 0x4000000, P + 0x8000000
    assert f(ctypes.byref(q4(group=32)), 0, out_c, out_s, None) == L.SDV_ELAYOUT
    assert f(ctypes.byref(q4(N=63)), 1, out_c, out_s, None) == L.SDV_ELAYOUT
    assert f(ctypes.byref(q4()), 2, out_c, out_s, None) == L.SDV_ELAYOUT
    assert f(ctypes.byref(q4()), 0, 0, out_s, None) == L.SDV_EINVAL
    assert f(ctypes.byref(q4()), 0, P + 16, out_s, None) == L.SDV_EALIAS      # over the source codes
    assert f(ctypes.byref(q4()), 0, out_c, out_c + 64, None) == L.SDV_EALIAS  # outputs overlap


def test_q8_0_sizes_and_repack_validation(lib):
    # T tiles x G groups x (2 KB of codes, 128 B of half-scale words)
    assert lib.sdv_q8_0t_codes_bytes(512, 1280, 2560, 1) == 512 * 40 * 40 * 2048
    assert lib.sdv_q8_0t_codes_bytes(1, 1000, 576, 0) == 32 * 9 * 2048
    assert lib.sdv_q8_0t_codes_bytes(1, 64, 96, 0) == 0                         # K not a multiple of 64
    f = lib.sdv_q8_0_repack
    src = lambda **kw: ctypes.byref(L.SdvQ8_0(kw.get("qs", P), kw.get("d", P + 0x100000), kw.get("E", 1),
                                               kw.get("N", 64), kw.get("K", 128)))
    out_c, out_s = P + 0x4000000, P + 0x8000000
    assert f(None, 0, out_c, out_s, None) == L.SDV_EINVAL
    assert f(src(K=96), 0, out_c, out_s, None) == L.SDV_ELAYOUT
    assert f(src(N=63), 1, out_c, out_s, None) == L.SDV_ELAYOUT
    assert f(src(E=0), 0, out_c, out_s, None) == L.SDV_EINVAL
    assert f(src(qs=0), 0, out_c, out_s, None) == L.SDV_EINVAL
    assert f(src(), 0, P + 64, out_s, None) == L.SDV_EALIAS                     # over the source codes
    assert f(src(), 0, out_c, P + 0x100000 + 16, None) == L.SDV_EALIAS          # sb over the scales
    assert f(src(), 0, out_c, out_c + 64, None) == L.SDV_EALIAS


def test_q3_sizes_and_repack_validation(lib):
    # T tiles x G groups x (768 B of codes: three words per lane)
    assert lib.sdv_q3t_codes_bytes(512, 1280, 2560, 1) == 512 * 40 * 40 * 768
    assert lib.sdv_q3t_codes_bytes(1, 64, 96, 0) == 0
    f = lib.sdv_q3_repack
    src = lambda **kw: ctypes.byref(L.SdvQ3(kw.get("codes", P), kw.get("scales", P + 0x100000),
                                             kw.get("biases", P + 0x200000), kw.get("E", 1), kw.get("N", 64),
                                             kw.get("K", 128)))
    out_c, out_s = P + 0x4000000, P + 0x8000000
    assert f(None, 0, out_c, out_s, None) == L.SDV_EINVAL
    assert f(src(K=100), 0, out_c, out_s, None) == L.SDV_ELAYOUT
    assert f(src(N=63), 1, out_c, out_s, None) == L.SDV_ELAYOUT
    assert f(src(biases=0), 0, out_c, out_s, None) == L.SDV_EINVAL
    assert f(src(), 0, P + 16, out_s, None) == L.SDV_EALIAS                     # over the source codes
    assert f(src(), 0, out_c, P + 0x200000 + 16, None) == L.SDV_EALIAS          # sb over the biases


def test_format_validation(lib):
    assert qmv(lib, q4t(fmt=3)) == L.SDV_ELAYOUT
    assert "format" in lib.sdv_last_error().decode()
    # a Q8_0 weight's codes are twice a Q4 weight's: an output right after
    # the Q4-sized codes still overlaps them
    assert qmv(lib, q4t(fmt=1), y=P + 64 * 128 // 2 + 64) == L.SDV_EALIAS


def test_qmv_validation(lib):
    assert qmv(lib, q4t(), k=0) == L.SDV_EWIDTH
    assert qmv(lib, q4t(), k=33) == L.SDV_EWIDTH
    assert qmv(lib, q4t(group=32)) == L.SDV_ELAYOUT
    assert qmv(lib, q4t(K=100)) == L.SDV_ELAYOUT
    assert qmv(lib, q4t(K=0)) == L.SDV_ELAYOUT
    assert qmv(lib, q4t(E=2)) == L.SDV_EINVAL
    assert qmv(lib, q4t(N=0)) == L.SDV_EINVAL
    assert qmv(lib, q4t(codes=0)) == L.SDV_EINVAL
    assert qmv(lib, q4t(sb=P + 4)) == L.SDV_EINVAL
    assert qmv(lib, q4t(), act=0) == L.SDV_EINVAL
    assert qmv(lib, q4t(), y=P + 0x800008) == L.SDV_EINVAL
    assert qmv(lib, q4t(N=63, fused=1), mode=L.MODE_GATEUP_SWIGLU) == L.SDV_ELAYOUT
    assert qmv(lib, q4t(fused=3)) == L.SDV_ELAYOUT
    assert qmv(lib, q4t(), mode=7) == L.SDV_EINVAL
    assert qmv(lib, q4t(), dtype=5) == L.SDV_EINVAL
    # the product mode must match the tile layout
    assert qmv(lib, q4t(fused=0), mode=L.MODE_GATEUP_SWIGLU) == L.SDV_ELAYOUT
    assert qmv(lib, q4t(fused=1), mode=L.MODE_PLAIN) == L.SDV_ELAYOUT
    # output inside the codes array
    assert qmv(lib, q4t(), y=P + 64) == L.SDV_EALIAS
    # output overlapping the activations
    assert qmv(lib, q4t(), y=P + 0x400000 + 16) == L.SDV_EALIAS
    # fp32 activation rows that cannot be staged in LDS
    assert qmv(lib, q4t(K=8192), dtype=L.ACT_F32, k=9) == L.SDV_ELAYOUT
    assert "LDS" in lib.sdv_last_error().decode()


def qmv_multi(lib, Ws, act=P + 0x400000, dtype=L.ACT_BF16, k=2, mode=L.MODE_PLAIN, ys=None, nw=None):
    arr = (L.SdvQ4T * len(Ws))(*Ws)
    ys = ys if ys is not None else [P + 0x800000 + 0x10000 * m for m in range(len(Ws))]
    yarr = (ctypes.c_void_p * len(ys))(*ys)
    return lib.sdv_qmv_k_multi(arr, len(Ws) if nw is None else nw, act, dtype, k, mode, yarr, None)


def test_qmv_multi_validation(lib):
    """The multi-weight dense call: the single call's checks for every
    weight, one shape, format and layout for all, 1..16 weights, no output
    over any weight, the activations or another output."""
    base = [q4t(codes=P + 0x20000 * m, sb=P + 0x100000 + 0x2000 * m) for m in range(3)]
    assert qmv_multi(lib, base, nw=0) == L.SDV_ERANGE
    assert qmv_multi(lib, base, nw=17) == L.SDV_ERANGE
    assert qmv_multi(lib, base, k=0) == L.SDV_EWIDTH
    assert qmv_multi(lib, base, act=0) == L.SDV_EINVAL
    assert qmv_multi(lib, base[:1] + [q4t(N=128, codes=P + 0x20000, sb=P + 0x102000)]) == L.SDV_ELAYOUT
    assert qmv_multi(lib, base[:1] + [q4t(fmt=1, codes=P + 0x20000, sb=P + 0x102000)]) == L.SDV_ELAYOUT
    assert qmv_multi(lib, base[:1] + [q4t(E=2, codes=P + 0x20000, sb=P + 0x102000)]) == L.SDV_EINVAL
    assert qmv_multi(lib, base[:1] + [q4t(codes=0)]) == L.SDV_EINVAL
    assert qmv_multi(lib, base, ys=[P + 0x800000, 0, P + 0x820000]) == L.SDV_EINVAL
    assert qmv_multi(lib, base, ys=[P + 0x800000, P + 0x20000 + 64, P + 0x820000]) == L.SDV_EALIAS  # over codes
    assert qmv_multi(lib, base, ys=[P + 0x800000, P + 0x800000 + 16, P + 0x820000]) == L.SDV_EALIAS  # outputs
    assert qmv_multi(lib, base, ys=[P + 0x400000 + 16, P + 0x810000, P + 0x820000]) == L.SDV_EALIAS  # over act
    assert qmv_multi(lib, base, mode=L.MODE_GATEUP_SWIGLU) == L.SDV_ELAYOUT


def route(lib, k=2, E=64, topk=4, mode=L.ROUTE_SOFTMAX, logits=P, outs=None):
    outs = outs or [P + 0x100000 * (i + 1) for i in range(7)]
    return lib.sdv_moe_route_k(logits, k, E, topk, mode, 0, *outs, None)


def test_route_validation(lib):
    assert route(lib, k=0) == L.SDV_EWIDTH
    assert route(lib, topk=0) == L.SDV_ERANGE
    assert route(lib, topk=17, E=64) == L.SDV_ERANGE
    assert route(lib, topk=8, E=4) == L.SDV_ERANGE
    assert route(lib, E=1025) == L.SDV_ERANGE
    assert route(lib, mode=3) == L.SDV_EINVAL
    assert route(lib, logits=0) == L.SDV_EINVAL
    outs = [P + 0x100000 * (i + 1) for i in range(7)]
    outs[1] = P  # weights written over the logits
    assert route(lib, outs=outs) == L.SDV_EALIAS
    outs = [P + 0x100000 * (i + 1) for i in range(7)]
    outs[6] = outs[5] + 16  # pair_slot overlapping pair_row
    assert route(lib, outs=outs) == L.SDV_EALIAS


def gather(lib, bank, k=2, topk=4, mode=L.MODE_GATEUP_SWIGLU, dtype=L.ACT_BF16, out=P + 0x2000000,
           shared=None, shared_act=None, shared_out=None):
    ptrs = [P + 0x800000 + 0x10000 * i for i in range(6)]
    return lib.sdv_gather_qmv_k(ctypes.byref(bank), mode, ptrs[0], dtype, ptrs[1], ptrs[2], ptrs[3], ptrs[4],
                                ptrs[5], k, topk, out, ctypes.byref(shared) if shared is not None else None,
                                shared_act, shared_out, None)


def test_gather_validation(lib):
    bank = q4t(E=8, N=128, K=128, fused=1)
    assert gather(lib, bank, k=33) == L.SDV_EWIDTH
    assert gather(lib, bank, topk=9) == L.SDV_ERANGE
    assert gather(lib, q4t(E=8, N=127, K=128, fused=1)) == L.SDV_ELAYOUT
    assert gather(lib, q4t(E=8, N=128, K=96, fused=1)) == L.SDV_ELAYOUT
    assert gather(lib, q4t(E=8, N=128, K=128, fused=0)) == L.SDV_ELAYOUT
    assert gather(lib, bank, out=0) == L.SDV_EINVAL
    assert gather(lib, bank, out=P + 0x800000) == L.SDV_EALIAS


def test_gather_shared_validation(lib):
    bank = q4t(E=8, N=128, K=128, fused=1)
    sh = q4t(E=1, N=128, K=128, fused=1)
    sh.codes, sh.sb = P + 0x4000000, P + 0x5000000
    ok = dict(shared=sh, shared_act=P + 0x6000000, shared_out=P + 0x7000000)
    assert gather(lib, bank, shared_act=P + 0x6000000) == L.SDV_EINVAL      # no shared weight
    assert gather(lib, bank, shared_out=P + 0x7000000) == L.SDV_EINVAL
    assert gather(lib, bank, **{**ok, "shared_out": None}) == L.SDV_EINVAL
    assert gather(lib, bank, **{**ok, "shared_act": None}) == L.SDV_EINVAL
    bad = q4t(E=2, N=128, K=128, fused=1)
    assert gather(lib, bank, **{**ok, "shared": bad}) == L.SDV_EINVAL       # E must be 1
    for geo in (dict(N=256, K=128, fused=1), dict(N=128, K=192, fused=1), dict(N=128, K=128, fused=0)):
        other = q4t(E=1, **geo)
        other.codes, other.sb = sh.codes, sh.sb
        assert gather(lib, bank, **{**ok, "shared": other}) == L.SDV_ELAYOUT
    assert gather(lib, bank, **{**ok, "shared_out": P + 0x2000000 + 64}) == L.SDV_EALIAS  # over out
    assert gather(lib, bank, **{**ok, "shared_out": sh.codes}) == L.SDV_EALIAS
    assert "shared" in lib.sdv_last_error().decode()


def experts(lib, gu, dn, k=2, topk=4, x=P + 0x3000000, partial=P + 0x4000000, sgu=None, sdn=None):
    ptrs = [P + 0x800000 + 0x10000 * i for i in range(5)]
    return lib.sdv_moe_experts_k(ctypes.byref(gu), ctypes.byref(dn), x, *ptrs, k, topk,
                                 ctypes.byref(sgu) if sgu is not None else None,
                                 ctypes.byref(sdn) if sdn is not None else None, partial, None)


def test_experts_partial_bytes(lib):
    # S = ceil(I / 128) slices of [k][topk + 1][H] fp32
    assert lib.sdv_moe_experts_partial_bytes(9, 10, 2560, 640) == 5 * 9 * 11 * 2560 * 4
    assert lib.sdv_moe_experts_partial_bytes(2, 4, 256, 192) == 2 * 2 * 5 * 256 * 4
    assert lib.sdv_moe_experts_partial_bytes(32, 10, 2560, 640) == 5 * 32 * 11 * 2560 * 4
    assert lib.sdv_moe_experts_partial_bytes(33, 4, 256, 128) == 0
    assert lib.sdv_moe_experts_partial_bytes(2, 4, 250, 128) == 0
    assert lib.sdv_moe_experts_partial_bytes(2, 4, 256, 96) == 0


def test_experts_validation(lib):
    E, H, I = 8, 256, 128
    gu = q4t(E=E, N=2 * I, K=H, fused=1, codes=P, sb=P + 0x100000)
    dn = q4t(E=E, N=H, K=I, fused=0, codes=P + 0x200000, sb=P + 0x300000)
    assert experts(lib, gu, dn, k=33) == L.SDV_EWIDTH
    assert experts(lib, gu, dn, topk=9) == L.SDV_ERANGE
    assert experts(lib, q4t(E=E, N=2 * I, K=H, fused=0), dn) == L.SDV_ELAYOUT            # gate/up not fused
    assert experts(lib, gu, q4t(E=E, N=H, K=I, fused=1, codes=P + 0x200000)) == L.SDV_ELAYOUT
    assert experts(lib, gu, q4t(E=E, N=H + 32, K=I, codes=P + 0x200000, sb=P + 0x300000)) == L.SDV_ELAYOUT
    assert experts(lib, gu, q4t(E=E - 1, N=H, K=I, codes=P + 0x200000, sb=P + 0x300000)) == L.SDV_ELAYOUT
    gu96 = q4t(E=E, N=2 * 96, K=H, fused=1)
    dn96 = q4t(E=E, N=H, K=96, codes=P + 0x200000, sb=P + 0x300000)
    assert experts(lib, gu96, dn96) == L.SDV_ELAYOUT                                     # K=96 not a group multiple
    assert experts(lib, gu, dn, x=0) == L.SDV_EINVAL
    assert experts(lib, gu, dn, partial=P + 0x80) == L.SDV_EALIAS                        # over the gate/up codes
    assert experts(lib, gu, dn, partial=P + 0x800000) == L.SDV_EALIAS                    # over union_ids
    sgu = q4t(E=1, N=2 * I, K=H, fused=1, codes=P + 0x5000000, sb=P + 0x5100000)
    sdn = q4t(E=1, N=H, K=I, codes=P + 0x5200000, sb=P + 0x5300000)
    assert experts(lib, gu, dn, sgu=sgu) == L.SDV_EINVAL                                 # one of the pair
    assert experts(lib, gu, dn, sgu=q4t(E=2, N=2 * I, K=H, fused=1), sdn=sdn) == L.SDV_EINVAL
    assert experts(lib, gu, dn, sgu=q4t(E=1, N=2 * I, K=H, fused=0), sdn=sdn) == L.SDV_ELAYOUT
    assert experts(lib, gu, dn, sgu=sgu, sdn=sdn, partial=P + 0x5000000 + 64) == L.SDV_EALIAS
    # too much LDS: k = 9 rows of a very wide hidden size
    wide = q4t(E=E, N=2 * I, K=16384, fused=1)
    assert experts(lib, wide, q4t(E=E, N=16384, K=I, codes=P + 0x200000, sb=P + 0x300000), k=9) == L.SDV_ELAYOUT
    assert "LDS" in lib.sdv_last_error().decode()
    # the four weights of the fused expert kernel share one format
    assert experts(lib, q4t(E=E, N=2 * I, K=H, fused=1, fmt=L.FMT_Q8_0), dn) == L.SDV_ELAYOUT
    assert "one weight format" in lib.sdv_last_error().decode()
    q3dn = q4t(E=E, N=H, K=I, codes=P + 0x200000, sb=P + 0x300000, fmt=L.FMT_AFFINE_Q3)
    assert experts(lib, q4t(E=E, N=2 * I, K=H, fused=1, fmt=L.FMT_AFFINE_Q3), q3dn, sgu=sgu, sdn=sdn) == L.SDV_ELAYOUT
    assert "one weight format" in lib.sdv_last_error().decode()
    gu9 = q4t(E=E, N=2 * 1088, K=H, fused=1)
    assert experts(lib, gu9, q4t(E=E, N=H, K=1088, codes=P + 0x2000000, sb=P + 0x3000000)) == L.SDV_ERANGE


def route_experts(lib, gu, dn, k=2, topk=4, mode=L.ROUTE_SIGMOID, logits=P + 0x6000000, x=P + 0x3000000,
                  partial=P + 0x4000000, outs=None, sgu=None, sdn=None):
    outs = outs if outs is not None else [P + 0x800000 + 0x10000 * i for i in range(7)]
    return lib.sdv_moe_route_experts_k(logits, mode, 1, ctypes.byref(gu), ctypes.byref(dn), x, k, topk,
                                       ctypes.byref(sgu) if sgu is not None else None,
                                       ctypes.byref(sdn) if sdn is not None else None, *outs, partial, None)


def test_route_experts_validation(lib):
    """The one-call router dispatch + expert MLP: the router's checks, the
    expert kernel's checks, and aliasing across both sets of buffers, all
    before any launch."""
    E, H, I = 8, 256, 128
    gu = q4t(E=E, N=2 * I, K=H, fused=1, codes=P, sb=P + 0x100000)
    dn = q4t(E=E, N=H, K=I, fused=0, codes=P + 0x200000, sb=P + 0x300000)
    assert route_experts(lib, gu, dn, mode=7) == L.SDV_EINVAL
    assert route_experts(lib, gu, dn, k=33) == L.SDV_EWIDTH
    assert route_experts(lib, gu, dn, topk=9) == L.SDV_ERANGE                            # topk > E
    big = q4t(E=1025, N=2 * I, K=H, fused=1, codes=P, sb=P + 0x100000)
    assert route_experts(lib, big, dn) == L.SDV_ERANGE                                    # E above 1024
    assert route_experts(lib, q4t(E=E, N=2 * I, K=H, fused=0), dn) == L.SDV_ELAYOUT       # gate/up not fused
    assert route_experts(lib, gu, dn, logits=0) == L.SDV_EINVAL
    assert route_experts(lib, gu, dn, x=0) == L.SDV_EINVAL
    outs = [P + 0x800000 + 0x10000 * i for i in range(7)]
    assert route_experts(lib, gu, dn, outs=outs[:3] + [0] + outs[4:]) == L.SDV_EINVAL    # n_union NULL
    assert route_experts(lib, gu, dn, logits=outs[1]) == L.SDV_EALIAS                     # w over the logits
    assert route_experts(lib, gu, dn, partial=P + 0x80) == L.SDV_EALIAS                   # over the gate/up codes
    assert route_experts(lib, gu, dn, partial=outs[2]) == L.SDV_EALIAS                    # over union_ids
    assert route_experts(lib, gu, dn, outs=[outs[0]] * 7) == L.SDV_EALIAS                 # outputs overlap
    q8 = q4t(E=E, N=2 * I, K=H, fused=1, codes=P, sb=P + 0x100000, fmt=L.FMT_Q8_0)
    q8dn = q4t(E=E, N=H, K=I, codes=dn.codes, sb=dn.sb, fmt=L.FMT_Q8_0)
    assert route_experts(lib, q8, q8dn) == L.SDV_ELAYOUT                                  # affine Q4 only
    assert "affine Q4" in lib.sdv_last_error().decode()


def test_combine_sliced_validation(lib):
    f = lib.sdv_moe_combine_sliced_k
    part, idx, w, y = P, P + 0x1000000, P + 0x1100000, P + 0x1200000
    assert f(part, idx, w, None, 0, 4, 256, 128, 0, y, None) == L.SDV_EWIDTH
    assert f(part, idx, w, None, 2, 17, 256, 128, 0, y, None) == L.SDV_ERANGE
    assert f(part, idx, w, None, 2, 4, 250, 128, 0, y, None) == L.SDV_EINVAL
    assert f(part, idx, w, None, 2, 4, 256, 100, 0, y, None) == L.SDV_EINVAL
    assert f(part, idx, w, None, 2, 4, 256, 128, 2, y, None) == L.SDV_EINVAL
    assert f(part, idx, w, None, 2, 4, 256, 1088, 0, y, None) == L.SDV_ERANGE              # 9 slices
    assert f(part, idx, w, P + 0x1300000, 2, 4, 256, 128, 0, y, None) == L.SDV_EINVAL    # logit without shared slot
    assert f(part, idx, w, None, 2, 4, 256, 128, 0, P + 0x100, None) == L.SDV_EALIAS
    assert f(part, idx, w, None, 2, 4, 256, 128, 0, idx + 16, None) == L.SDV_EALIAS


def test_combine_validation(lib):
    f = lib.sdv_moe_combine_k
    assert f(P, P + 0x10000, None, None, 0, 4, 64, P + 0x20000, None) == L.SDV_EWIDTH
    assert f(P, P + 0x10000, None, None, 2, 0, 64, P + 0x20000, None) == L.SDV_ERANGE
    assert f(P, P + 0x10000, None, None, 2, 4, 62, P + 0x20000, None) == L.SDV_EINVAL
    assert f(P, P + 0x10000, None, P + 0x30000, 2, 4, 64, P + 0x20000, None) == L.SDV_EINVAL
    assert f(P, P + 0x10000, None, None, 2, 4, 64, P + 0x100, None) == L.SDV_EALIAS


def gdn(lib, k=2, Hv=4, Hk=4, Dk=64, Dv=64, snaps=None, S_in=P, y=P + 0x700000):
    base = [P + 0x100000 * (i + 1) for i in range(5)]
    snaps = snaps if snaps is not None else [P + 0x1000000 * (t + 1) for t in range(k)]
    arr = (ctypes.c_void_p * max(1, len(snaps)))(*snaps)
    return lib.sdv_gdn_verify_k(S_in, base[0], base[1], base[2], base[3], base[4], k, Hv, Hk, Dk, Dv, y, arr, None)


def test_gdn_validation(lib):
    assert gdn(lib, k=0) == L.SDV_EWIDTH
    assert gdn(lib, k=33) == L.SDV_EWIDTH
    assert gdn(lib, Dk=96) == L.SDV_ELAYOUT
    assert gdn(lib, Dk=256) == L.SDV_ELAYOUT
    assert gdn(lib, Hv=6, Hk=4) == L.SDV_ELAYOUT
    assert gdn(lib, Hv=0) == L.SDV_EINVAL
    assert gdn(lib, S_in=0) == L.SDV_EINVAL
    s = P + 0x1000000
    assert gdn(lib, snaps=[s, s]) == L.SDV_EALIAS                   # two rows, one snapshot buffer
    assert "snaps" in lib.sdv_last_error().decode()
    assert gdn(lib, snaps=[s, P + 8 * 1024]) == L.SDV_EALIAS        # snapshot over S_in
    assert gdn(lib, snaps=[s, 0]) == L.SDV_EINVAL
    assert gdn(lib, y=P + 0x100000) == L.SDV_EALIAS                 # y over q
    assert lib.sdv_last_error().decode() == "output y overlaps input q"


def test_rollback_selection(lib):
    slot = ctypes.c_int(-7)
    for k in range(1, 33):
        for j in range(0, k + 1):
            assert lib.sdv_gdn_rollback(k, j, ctypes.byref(slot)) == 0
            assert slot.value == j
        assert lib.sdv_gdn_rollback(k, k + 1, ctypes.byref(slot)) == L.SDV_ERANGE
        assert lib.sdv_gdn_rollback(k, -1, ctypes.byref(slot)) == L.SDV_ERANGE
    assert lib.sdv_gdn_rollback(33, 1, ctypes.byref(slot)) == L.SDV_EWIDTH
    assert lib.sdv_gdn_rollback(2, 1, None) == L.SDV_EINVAL


def test_rollback_copy_validation(lib):
    snaps = (ctypes.c_void_p * 2)(P + 0x100000, P + 0x200000)
    f = lib.sdv_gdn_rollback_copy
    # selecting the state the destination already is: nothing to copy, no HIP call
    assert f(P, P, snaps, 2, 0, 1024, None) == 0
    assert f(P + 0x200000, P, snaps, 2, 2, 1024, None) == 0
    assert f(P + 16, P, snaps, 2, 0, 1024, None) == L.SDV_EALIAS
    assert f(P + 0x900000, P, snaps, 2, 3, 1024, None) == L.SDV_ERANGE
    assert f(P + 0x900000, P, snaps, 2, 1, 0, None) == L.SDV_EINVAL
    assert f(0, P, snaps, 2, 1, 1024, None) == L.SDV_EINVAL


def test_accept_workspace_bytes(lib):
    assert lib.sdv_verify_accept_workspace_bytes(9, 248320) == 9 * 61 * 8
    assert lib.sdv_verify_accept_workspace_bytes(1, 1) == 8
    assert lib.sdv_verify_accept_workspace_bytes(2, 4097) == 2 * 2 * 8
    assert lib.sdv_verify_accept_workspace_bytes(32, 248320) == 32 * 61 * 8
    for k, V in [(0, 10), (33, 10), (2, 0), (2, -5)]:
        assert lib.sdv_verify_accept_workspace_bytes(k, V) == 0


def test_accept_validation(lib):
    f = lib.sdv_verify_accept_k
    logits, noise, drafts = P, P + 0x1000000, P + 0x2000000
    tok, acc, ws = P + 0x2100000, P + 0x2200000, P + 0x2300000
    ok = dict(logits=logits, noise=None, inv=1.0, drafts=drafts, k=3, V=1000, eos=-1, tok=tok, acc=acc,
              ws=ws, wsb=1 << 20)

    def call(**kw):
        a = dict(ok, **kw)
        return f(a["logits"], a["noise"], a["inv"], a["drafts"], a["k"], a["V"], a["eos"], a["tok"], a["acc"],
                 a["ws"], a["wsb"], None)

    assert call(k=0) == L.SDV_EWIDTH
    assert call(k=33) == L.SDV_EWIDTH
    assert call(V=0) == L.SDV_ERANGE
    assert call(V=(1 << 30) + 1) == L.SDV_ERANGE
    assert call(logits=None) == L.SDV_EINVAL
    assert call(logits=P + 4) == L.SDV_EINVAL                       # misaligned
    assert call(noise=noise, inv=0.0) == L.SDV_ERANGE
    assert call(noise=noise, inv=float("inf")) == L.SDV_ERANGE
    assert call(noise=noise, inv=float("nan")) == L.SDV_ERANGE
    assert call(drafts=None) == L.SDV_EINVAL
    assert call(tok=None) == L.SDV_EINVAL
    assert call(acc=None) == L.SDV_EINVAL
    assert call(ws=None) == L.SDV_EINVAL
    assert call(wsb=3 * 8 - 1) == L.SDV_EINVAL
    assert "workspace" in lib.sdv_last_error().decode()
    assert call(tok=logits + 64) == L.SDV_EALIAS                    # tokens over logits
    assert call(ws=tok) == L.SDV_EALIAS                             # workspace over tokens
    assert call(acc=noise + 16, noise=noise) == L.SDV_EALIAS         # accepted over noise


def test_accept_noalloc_validation(lib):
    """The allocation-free acceptance: the same argument checks as the
    workspace form, and sizes whose workspace exceeds the built-in 1 MiB
    scratch are rejected before any launch."""
    f = lib.sdv_verify_accept_k_noalloc
    assert lib.sdv_verify_accept_scratch_bytes() == 1 << 20
    logits, noise, drafts = P, P + 0x1000000, P + 0x2000000
    tok, acc = P + 0x2100000, P + 0x2200000
    ok = dict(logits=logits, noise=None, inv=1.0, drafts=drafts, k=3, V=1000, eos=-1, tok=tok, acc=acc)

    def call(**kw):
        a = dict(ok, **kw)
        return f(a["logits"], a["noise"], a["inv"], a["drafts"], a["k"], a["V"], a["eos"], a["tok"], a["acc"], None)

    assert call(k=0) == L.SDV_EWIDTH
    assert call(k=33) == L.SDV_EWIDTH
    assert call(V=0) == L.SDV_ERANGE
    # 32 rows x ceil(V / 4096) chunks x 8 bytes: 4096 chunks fit (1 MiB), 4097 do not
    assert lib.sdv_verify_accept_workspace_bytes(32, 4096 * 4096) == 1 << 20
    assert call(k=32, V=4096 * 4096 + 1, logits=None) == L.SDV_ERANGE
    assert "scratch" in lib.sdv_last_error().decode()
    assert call(k=32, V=1 << 30, logits=None) == L.SDV_ERANGE
    assert call(k=32, V=4096 * 4096, logits=None) == L.SDV_EINVAL  # fits: the next check fails
    assert call(logits=None) == L.SDV_EINVAL
    assert call(logits=P + 4) == L.SDV_EINVAL
    assert call(noise=noise, inv=0.0) == L.SDV_ERANGE
    assert call(drafts=None) == L.SDV_EINVAL
    assert call(tok=None) == L.SDV_EINVAL
    assert call(acc=None) == L.SDV_EINVAL
    assert call(tok=logits + 64) == L.SDV_EALIAS
    assert call(acc=tok) == L.SDV_EALIAS


def prep(lib, k=2, Hv=4, Hk=2, Dk=64, Dv=64, act=0, eps=1e-6, **over):
    C = 2 * Hk * Dk + Hv * Dv
    ptr = dict(qkv=P, hist=P + 0x100000, conv_w=P + 0x200000, a=P + 0x300000, b=P + 0x310000,
               A_log=P + 0x320000, dt_bias=P + 0x330000, q=P + 0x400000, kk=P + 0x500000, v=P + 0x600000,
               g=P + 0x700000, beta=P + 0x710000, window=P + 0x800000)
    ptr.update(over)
    assert C * 4 * 12 < 0x100000
    return lib.sdv_gdn_prepare_k(ptr["qkv"], ptr["hist"], ptr["conv_w"], ptr["a"], ptr["b"], ptr["A_log"],
                                 ptr["dt_bias"], k, Hv, Hk, Dk, Dv, act, eps, ptr["q"], ptr["kk"], ptr["v"],
                                 ptr["g"], ptr["beta"], ptr["window"], None)


def test_prepare_validation(lib):
    assert prep(lib, k=0) == L.SDV_EWIDTH
    assert prep(lib, k=33) == L.SDV_EWIDTH
    assert prep(lib, Hv=0) == L.SDV_EINVAL
    assert prep(lib, Hv=5, Hk=2) == L.SDV_ELAYOUT
    assert prep(lib, Dk=128, Dv=64) == L.SDV_ELAYOUT
    assert prep(lib, Dk=96, Dv=96) == L.SDV_ELAYOUT
    assert prep(lib, act=2) == L.SDV_EINVAL
    assert prep(lib, eps=-1.0) == L.SDV_ERANGE
    assert prep(lib, eps=float("nan")) == L.SDV_ERANGE
    assert prep(lib, eps=float("inf")) == L.SDV_ERANGE
    assert prep(lib, hist=0) == L.SDV_EINVAL
    assert lib.sdv_last_error().decode() == "hist is NULL"
    assert prep(lib, conv_w=P + 0x200004) == L.SDV_EINVAL            # taps are read as float4
    # the window (k + 3 rows) over the conv history: the next step reads it
    assert prep(lib, window=P + 0x100000 + 64) == L.SDV_EALIAS
    assert lib.sdv_last_error().decode() == "output window overlaps input hist"
    assert prep(lib, q=P + 0x500000) == L.SDV_EALIAS                 # q over kk
    assert prep(lib, beta=P + 0x700000 + 16) == L.SDV_EALIAS         # beta over g
    assert prep(lib, g=P + 0x300000) == L.SDV_EALIAS                 # g over a


def norm(lib, k=2, Hv=4, Dv=64, act=0, eps=1e-6, y=P, z=P + 0x100000, w=P + 0x200000, out=P + 0x300000):
    return lib.sdv_gdn_gated_norm_k(y, z, w, k, Hv, Dv, act, eps, out, None)


def test_gated_norm_validation(lib):
    assert norm(lib, k=0) == L.SDV_EWIDTH
    assert norm(lib, Hv=0) == L.SDV_EINVAL
    assert norm(lib, Dv=32) == L.SDV_ELAYOUT
    assert norm(lib, act=5) == L.SDV_EINVAL
    assert norm(lib, eps=-0.5) == L.SDV_ERANGE
    assert norm(lib, w=0) == L.SDV_EINVAL
    assert norm(lib, out=P + 16) == L.SDV_EALIAS                     # in place over y
    assert lib.sdv_last_error().decode() == "output out overlaps input y"
    assert norm(lib, out=P + 0x200000) == L.SDV_EALIAS


def verify_prep(lib, k=2, Hv=4, Hk=2, D=64, Dv=None, act=0, eps=1e-6, snaps=None, **over):
    ptr = dict(S_in=P + 0x4000000, qkv=P, hist=P + 0x100000, conv_w=P + 0x200000, a=P + 0x300000, b=P + 0x310000,
               A_log=P + 0x320000, dt_bias=P + 0x330000, window=P + 0x800000, y=P + 0x900000)
    ptr.update(over)
    snaps = snaps if snaps is not None else [P + 0x5000000 + 0x1000000 * t for t in range(k)]
    arr = (ctypes.c_void_p * max(1, len(snaps)))(*snaps)
    return lib.sdv_gdn_verify_prep_k(ptr["S_in"], ptr["qkv"], ptr["hist"], ptr["conv_w"], ptr["a"], ptr["b"],
                                     ptr["A_log"], ptr["dt_bias"], k, Hv, Hk, D, D if Dv is None else Dv, act, eps,
                                     ptr["window"], ptr["y"], arr, None)


def test_verify_prep_validation(lib):
    assert verify_prep(lib, k=0) == L.SDV_EWIDTH
    assert verify_prep(lib, k=33) == L.SDV_EWIDTH
    assert verify_prep(lib, Hv=5) == L.SDV_ELAYOUT
    assert verify_prep(lib, D=128, Dv=64) == L.SDV_ELAYOUT
    assert verify_prep(lib, D=32) == L.SDV_ELAYOUT
    assert verify_prep(lib, act=7) == L.SDV_EINVAL
    assert verify_prep(lib, eps=float("nan")) == L.SDV_ERANGE
    assert verify_prep(lib, S_in=0) == L.SDV_EINVAL
    assert verify_prep(lib, snaps=[P + 0x5000000, 0]) == L.SDV_EINVAL
    s = P + 0x5000000
    assert verify_prep(lib, snaps=[s, s]) == L.SDV_EALIAS
    assert verify_prep(lib, snaps=[s, P + 0x4000000 + 64]) == L.SDV_EALIAS      # snapshot over S_in
    assert verify_prep(lib, window=P + 0x100000) == L.SDV_EALIAS                # window over hist
    assert lib.sdv_last_error().decode() == "output window overlaps input hist"
    assert verify_prep(lib, y=P + 0x800000 + 4096) == L.SDV_EALIAS              # y over window
    assert verify_prep(lib, y=P + 0x5000000 + 64) == L.SDV_EALIAS               # y over a snapshot


def verify_prep_norm(lib, k=2, Hv=4, Hk=2, D=64, gate=0, neps=1e-6, **over):
    ptr = dict(S_in=P + 0x4000000, qkv=P, hist=P + 0x100000, conv_w=P + 0x200000, a=P + 0x300000, b=P + 0x310000,
               A_log=P + 0x320000, dt_bias=P + 0x330000, window=P + 0x800000, y=P + 0x900000, z=P + 0xA00000,
               norm_w=P + 0xB00000, out=P + 0xC00000, counters=P + 0xD00000)
    ptr.update(over)
    snaps = [P + 0x5000000 + 0x1000000 * t for t in range(k)]
    arr = (ctypes.c_void_p * k)(*snaps)
    return lib.sdv_gdn_verify_prep_norm_k(ptr["S_in"], ptr["qkv"], ptr["hist"], ptr["conv_w"], ptr["a"], ptr["b"],
                                          ptr["A_log"], ptr["dt_bias"], k, Hv, Hk, D, D, 0, 1e-6, ptr["window"],
                                          ptr["y"], arr, ptr["z"], ptr["norm_w"], gate, neps, ptr["out"],
                                          ptr["counters"], None)


def test_verify_prep_norm_validation(lib):
    """The preparation + recurrence checks, the norm's checks, and aliasing
    of out and the counters, before any launch."""
    assert verify_prep_norm(lib, k=33) == L.SDV_EWIDTH
    assert verify_prep_norm(lib, Hv=5) == L.SDV_ELAYOUT
    assert verify_prep_norm(lib, gate=5) == L.SDV_EINVAL
    assert verify_prep_norm(lib, neps=float("inf")) == L.SDV_ERANGE
    assert verify_prep_norm(lib, z=0) == L.SDV_EINVAL
    assert verify_prep_norm(lib, counters=0) == L.SDV_EINVAL
    assert verify_prep_norm(lib, counters=P + 0xD00002) == L.SDV_EINVAL                  # misaligned
    assert verify_prep_norm(lib, out=P + 0xA00000 + 64) == L.SDV_EALIAS                 # out over z
    assert verify_prep_norm(lib, out=P + 0x900000) == L.SDV_EALIAS                       # out over y
    assert verify_prep_norm(lib, counters=P + 0xB00000) == L.SDV_EALIAS                  # counters over norm_w
    assert verify_prep_norm(lib, counters=P + 0xC00000 + 4) == L.SDV_EALIAS              # counters over out


def gdn_layer(base, k):
    """A sdv_gdn_layer of fake addresses in its own 256 MB window."""
    e = L.SdvGdnLayer()
    for name, off in (("S_in", 0x4000000), ("qkv", 0), ("hist", 0x100000), ("conv_w", 0x200000), ("a", 0x300000),
                      ("b", 0x310000), ("A_log", 0x320000), ("dt_bias", 0x330000), ("window", 0x800000),
                      ("y", 0x900000)):
        setattr(e, name, base + off)
    for t in range(k):
        e.snaps[t] = base + 0x5000000 + 0x1000000 * t
    return e


def test_gdn_layers_validation(lib):
    """The layer table is checked layer by layer as sdv_gdn_verify_prep_k
    checks its arguments, and for overlaps across layers and with the table;
    the layered launch checks its shape, all before any HIP call."""
    k, n = 2, 3
    arr = (L.SdvGdnLayer * n)(*[gdn_layer(P + 0x10000000 * (l + 1), k) for l in range(n)])
    size = n * ctypes.sizeof(L.SdvGdnLayer)
    assert ctypes.sizeof(L.SdvGdnLayer) == 42 * 8
    table = P + 0x80000000
    tab = lambda a=arr, nl=n, kk=k, Hv=4, Hk=2, D=64, t=table, nb=size: lib.sdv_gdn_layers_table(
        ctypes.addressof(a), nl, kk, Hv, Hk, D, D, t, nb)
    assert lib.sdv_gdn_layers_table(None, n, k, 4, 2, 64, 64, table, size) == L.SDV_EINVAL
    assert tab(nl=0) == L.SDV_EINVAL
    assert tab(nl=65536) == L.SDV_EINVAL
    assert tab(t=0) == L.SDV_EINVAL
    assert tab(t=table + 8) == L.SDV_EINVAL                              # misaligned
    assert tab(nb=size - 1) == L.SDV_EINVAL
    assert tab(kk=33) == L.SDV_EWIDTH
    assert tab(Hv=5) == L.SDV_ELAYOUT
    arr[1].conv_w = 0
    assert tab() == L.SDV_EINVAL
    assert lib.sdv_last_error().decode() == "conv_w is NULL (layer 1)"
    arr[1].conv_w = P + 0x20000000 + 0x200000
    arr[2].y = arr[0].window                                             # y of one layer over another's window
    assert tab() == L.SDV_EALIAS
    arr[2].y = arr[1].S_in                                               # an output over another layer's input
    assert tab() == L.SDV_EALIAS
    arr[2].y = P + 0x30000000 + 0x900000
    assert tab(t=arr[0].qkv) == L.SDV_EALIAS                             # the table over an input
    assert lib.sdv_last_error().decode() == "output table overlaps input qkv"
    launch = lambda nl=n, kk=k, Hv=4, Hk=2, D=64, Dv=None, act=0, eps=1e-6, t=table: \
        lib.sdv_gdn_verify_prep_k_layers(t, nl, kk, Hv, Hk, D, D if Dv is None else Dv, act, eps, None)
    assert launch(t=0) == L.SDV_EINVAL
    assert launch(nl=0) == L.SDV_EINVAL
    assert launch(kk=0) == L.SDV_EWIDTH
    assert launch(Hv=6, Hk=4) == L.SDV_ELAYOUT
    assert launch(D=128, Dv=64) == L.SDV_ELAYOUT
    assert launch(act=9) == L.SDV_EINVAL
    assert launch(eps=-1.0) == L.SDV_ERANGE
