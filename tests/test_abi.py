"""The C-ABI library loads, exports every symbol include/quads.h declares, and
rejects bad arguments on the host before any launch (CPU only: no compute)."""

import ctypes
import os
import re

import pytest

import nvfp4_w4a4_quantized_act_amd as Q

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared():
    with open(os.path.join(ROOT, "include", "quads.h")) as f:
        src = f.read()
    return sorted(set(re.findall(r"\b(quads_[a-z0-9_]+)\s*\(", src)))


def test_library_exports_every_declared_symbol():
    lib = Q.lib()
    names = _declared()
    assert "quads_moe_w4a4_gemm" in names and len(names) == 29
    missing = [n for n in names if not hasattr(lib, n)]
    assert not missing, missing
    assert lib.quads_version().startswith(b"quads-mi355x")


def test_status_strings():
    lib = Q.lib()
    for st in (0, -1, -2, -3, -4):
        assert lib.quads_status_string(st)


FAKE = ctypes.c_void_p(0x10000)          # aligned, never dereferenced (checks fail first)
MIS = ctypes.c_void_p(0x10004)           # misaligned
MIS2 = ctypes.c_void_p(0x10002)          # misaligned for a 32-bit word


def test_quantize_validation():
    lib = Q.lib()
    ws = lib.quads_nvfp4_quantize_ws(4, 32)
    assert ws > 0
    f = lib.quads_nvfp4_quantize
    assert f(FAKE, 4, 30, None, FAKE, FAKE, FAKE, FAKE, ws, None) == -2      # K % 16
    assert f(FAKE, -1, 32, None, FAKE, FAKE, FAKE, FAKE, ws, None) == -2     # M < 0
    assert f(None, 4, 32, None, FAKE, FAKE, FAKE, FAKE, ws, None) == -1      # null x
    assert f(MIS, 4, 32, None, FAKE, FAKE, FAKE, FAKE, ws, None) == -1       # misaligned
    assert f(FAKE, 4, 32, None, FAKE, FAKE, FAKE, FAKE, ws - 1, None) == -3  # workspace
    assert f(FAKE, 4, 32, None, FAKE, FAKE, FAKE, None, ws, None) == -3


def test_quantize_rows_validation():
    f = Q.lib().quads_nvfp4_quantize_rows
    assert f(FAKE, 4, 24, FAKE, FAKE, FAKE, None) == -2        # K % 16
    assert f(FAKE, -1, 32, FAKE, FAKE, FAKE, None) == -2       # M < 0
    assert f(FAKE, 4, 32, FAKE, FAKE, None, None) == -1        # ts missing
    assert f(FAKE, 4, 32, MIS, FAKE, FAKE, None) == -1         # misaligned
    assert f(None, 0, 32, None, None, None, None) == 0         # empty: no-op


def test_rac_validation():
    lib = Q.lib()
    f = lib.quads_rac_quantize
    ws = lib.quads_rac_quantize_ws(64, 256, 32)
    args = lambda m, k_dim, k, wsz: f(FAKE, m, k_dim, k, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE,
                                      FAKE, None, FAKE, wsz, None)
    assert args(64, 256, 8, ws) == -2          # k % 16
    assert args(64, 256, 272, ws) == -2        # k > K
    assert args(64, 250, 16, ws) == -2         # K % 16
    assert args(64, 256, 32, ws - 1) == -3
    assert f(FAKE, 64, 256, 32, FAKE, FAKE, FAKE, None, FAKE, FAKE, FAKE, None, FAKE, ws,
             None) == -1                        # sel missing with k > 0


def test_rac_noalloc_validation():
    """The no-allocation RAC: the argument checks of quads_rac_quantize, then
    QUADS_ESCRATCH for sizes whose workspace exceeds the static scratch; all
    before any device call."""
    lib = Q.lib()
    f = lib.quads_rac_quantize_noalloc
    cap = Q.RAC_NOALLOC_SCRATCH_BYTES
    call = lambda m, k_dim, k: f(FAKE, m, k_dim, k, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE,
                                 None, None)
    assert call(64, 256, 8) == -2              # k % 16
    assert call(64, 250, 16) == -2             # K % 16
    assert f(FAKE, 64, 256, 32, FAKE, FAKE, FAKE, None, FAKE, FAKE, FAKE, None,
             None) == -1                        # sel missing with k > 0
    # the largest M (multiple of 64) that fits at K = 4096, and the next
    k_dim = 4096
    m = 64
    while lib.quads_rac_quantize_ws(2 * m, k_dim, 64) <= cap:
        m *= 2
    while lib.quads_rac_quantize_ws(m + 64, k_dim, 64) <= cap:
        m += 64
    assert lib.quads_rac_quantize_ws(m, k_dim, 64) <= cap
    assert call(m + 64, k_dim, 64) == -5
    assert call(4 * m, k_dim, 64) == -5
    assert "scratch" in lib.quads_status_string(-5).decode()
    # the scratch covers every RAC site of the five workloads
    for mm, kk, k in ((32, 256, 16), (4096, 4096, 128), (4096, 2048, 64), (32768, 768, 64),
                      (16384, 4096, 256), (131072, 1536, 64)):
        assert lib.quads_rac_quantize_ws(mm, kk, k) <= cap, (mm, kk)


def test_mx_rac_validation():
    lib = Q.lib()
    f = lib.quads_mx_rac_quantize
    ws = lib.quads_mx_rac_quantize_ws(64, 256, 32)
    call = lambda m, kd, k, wsz: f(FAKE, m, kd, k, FAKE, FAKE, FAKE, FAKE, FAKE, None, FAKE, wsz,
                                   None)
    assert call(64, 256, 16, ws) == -2           # k % 32
    assert call(64, 240, 32, ws) == -2           # K % 32
    assert call(64, 256, 288, ws) == -2          # k > K
    assert call(64, 256, 32, ws - 1) == -3
    assert f(FAKE, 64, 256, 32, FAKE, FAKE, None, FAKE, FAKE, None, FAKE, ws, None) == -1
    g = lib.quads_moe_mx_rac_gemm
    gws = lib.quads_moe_mx_rac_gemm_ws(2, 64, 32)
    assert gws == 2 * 64 * 32 * 2
    args = lambda k, kd, wsz: g(FAKE, FAKE, None, 32, kd, FAKE, FAKE, FAKE, k, FAKE, FAKE, FAKE,
                                2, 64, 0, 0, FAKE, FAKE, wsz, None)
    assert args(48, 256, gws) == -2              # k % 32
    assert args(32, 192, gws) == -2              # K % 128
    assert args(32, 256, gws - 1) == -3
    assert g(FAKE, FAKE, None, 32, 256, None, FAKE, FAKE, 32, FAKE, FAKE, FAKE, 2, 64, 0, 0, FAKE,
             FAKE, gws, None) == -1              # r_codes missing with k > 0


def test_weight_qdq_validation():
    lib = Q.lib()
    f = lib.quads_nvfp4_weight_qdq
    ws = lib.quads_nvfp4_weight_qdq_ws(2, 8, 32)
    assert f(FAKE, 0, 8, 32, FAKE, FAKE, FAKE, None, FAKE, ws, None) == -2
    assert f(FAKE, 2, 8, 40, FAKE, FAKE, FAKE, None, FAKE, ws, None) == -2
    assert f(FAKE, 2, 8, 32, FAKE, FAKE, FAKE, MIS, FAKE, ws, None) == -1
    assert f(FAKE, 2, 8, 32, FAKE, FAKE, FAKE, None, FAKE, ws - 4, None) == -3


def test_pack_validation():
    lib = Q.lib()
    f = lib.quads_moe_pack
    ws = lib.quads_moe_pack_ws(16, 2, 4)
    assert f(FAKE, 16, 0, 4, FAKE, FAKE, FAKE, FAKE, ws, None) == -2
    assert f(FAKE, 16, 2, 0, FAKE, FAKE, FAKE, FAKE, ws, None) == -2
    assert f(FAKE, 16, 2, 4, None, FAKE, FAKE, FAKE, ws, None) == -1


def test_gemm_validation():
    lib = Q.lib()
    f = lib.quads_moe_w4a4_gemm
    ws = lib.quads_moe_w4a4_gemm_ws(64, 256, 16, 4, 64)

    def call(rows=64, k_dim=256, k=16, e=4, n=64, epi=0, odt=0, offsets=FAKE, sel=FAKE,
             wsz=ws, out=FAKE):
        return f(FAKE, FAKE, FAKE, None, rows, k_dim, FAKE, FAKE, FAKE, sel, k, FAKE, FAKE, FAKE,
                 offsets, e, n, epi, odt, out, FAKE, wsz, None)
    assert call(k_dim=250) == -2
    assert call(k=8) == -2
    assert call(k=512) == -2
    assert call(e=0) == -2
    assert call(n=63, epi=1, odt=1) == -2      # SwiGLU needs even N
    assert call(epi=1, odt=0) == -1            # SwiGLU needs bf16 output
    assert call(epi=7) == -1
    assert call(offsets=None) == -1            # offsets required for E > 1
    assert call(sel=None) == -1                # sel required for k > 0
    assert call(out=MIS) == -1


def test_empty_gemm_calls_are_no_ops():
    """rows = 0 returns QUADS_OK before any row-sized pointer is looked at, as the
    header promises for size-0 inputs (a size-0 torch tensor has a null data
    pointer), on every grouped-GEMM entry point and the combine."""
    lib = Q.lib()
    n0 = None
    assert lib.quads_moe_w4a4_gemm(n0, n0, n0, n0, 0, 256, n0, n0, n0, n0, 16, n0, n0, n0, n0,
                                   1, 64, 0, 0, n0, n0, 0, n0) == 0
    assert lib.quads_moe_w4a4_gemm_amax(n0, n0, n0, n0, 0, 256, n0, n0, n0, n0, 16, n0, n0, n0,
                                        n0, 1, 64, n0, n0, 0, n0, 0, n0) == 0
    assert lib.quads_moe_w4a4_gemm_rowscale(n0, n0, n0, n0, 0, 256, n0, n0, n0, n0, 1, 64, 0, 0,
                                            n0, n0, 0, n0) == 0
    assert lib.quads_moe_w4a4_gemm_sel_experts(n0, n0, n0, 0, 256, n0, n0, FAKE, n0, 16, n0, n0,
                                               n0, FAKE, 4, 64, 0, 0, n0, n0, 0, n0) == 0
    assert lib.quads_moe_mx_gemm(n0, n0, n0, 0, 256, n0, n0, n0, 1, 64, 0, 0, 0, n0, n0) == 0
    assert lib.quads_moe_mx_rac_gemm(n0, n0, n0, 0, 256, n0, n0, n0, 32, n0, n0, n0, 1, 64, 0, 0,
                                     n0, n0, 0, n0) == 0
    assert lib.quads_moe_combine(n0, 0, n0, n0, 0, 8, 16, n0, n0) == 0
    # the shape and enum checks still come first
    assert lib.quads_moe_w4a4_gemm(n0, n0, n0, n0, 0, 250, n0, n0, n0, n0, 16, n0, n0, n0, n0,
                                   1, 64, 0, 0, n0, n0, 0, n0) == -2
    assert lib.quads_moe_w4a4_gemm(n0, n0, n0, n0, 0, 256, n0, n0, n0, n0, 16, n0, n0, n0, n0,
                                   1, 64, 7, 0, n0, n0, 0, n0) == -1


def test_gemm_amax_slots():
    """Slot count of the SwiGLU GEMM with partial maxima: the work-groups of its launches,
    worked out here from the launch rules (host logic only)."""
    lib = Q.lib()
    f = lib.quads_moe_w4a4_gemm_amax_groups
    # 128-expert layer gate/up (32768 packed rows, K = 2048 + 64): the decode kernel for the
    # experts' tails, 12 slabs x 8 x ceil(128 / 8), then the tiled kernel, 12 N-tiles x
    # (128 + 128) M-tiles rounded up to whole spans of 2 x 12 x 8 work-groups
    assert f(32768, 2048, 64, 128, 1536) == 12 * 8 * 16 + 3072
    # the decode step (512 packed rows): the decode kernel alone, 128 + 512 / 128 units
    assert f(512, 2048, 64, 128, 1536) == 12 * 8 * 17
    # a single chain (K + k <= 1152), 256 x 256 tiles: 3 N-tiles x (5 + 4) M-tiles, rounded
    # up to a whole span of 2 x 3 x 8 work-groups
    assert f(4 * 256 + 64, 768, 64, 4, 384 * 2) == 48
    assert f(0, 2048, 64, 128, 1536) == 0                 # rejected sizes
    assert f(512, 2048, 64, 128, 1535) == 0               # SwiGLU needs even N
    g = lib.quads_moe_w4a4_gemm_amax
    ws = lib.quads_moe_w4a4_gemm_ws(512, 2048, 64, 128, 1536)

    def call(groups=1632, amax=FAKE, k=64):
        return g(FAKE, FAKE, FAKE, None, 512, 2048, FAKE, FAKE, FAKE, FAKE, k, FAKE, FAKE, FAKE,
                 FAKE, 128, 1536, FAKE, amax, groups, FAKE, ws, None)
    assert call(amax=None) == -1
    assert call(amax=MIS2) == -1
    assert call(groups=0) == -1
    assert call(groups=1631) == -3                        # fewer slots than work-groups
    assert call(k=8) == -2


def test_partials_validation():
    lib = Q.lib()
    f = lib.quads_nvfp4_quantize_partials
    assert f(FAKE, 4, 32, FAKE, 0, FAKE, FAKE, FAKE, None) == -2           # groups >= 1
    assert f(FAKE, 4, 30, FAKE, 8, FAKE, FAKE, FAKE, None) == -2           # K % 16
    assert f(FAKE, 4, 32, MIS2, 8, FAKE, FAKE, FAKE, None) == -1
    assert f(FAKE, 4, 32, None, 8, FAKE, FAKE, FAKE, None) == -1
    g = lib.quads_rac_quantize_partials
    ws = lib.quads_rac_quantize_ws(64, 256, 16)

    def call(groups=8, amax=FAKE, wsz=ws, k=16):
        return g(FAKE, 64, 256, k, amax, groups, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None,
                 FAKE, wsz, None)
    assert call(groups=0) == -2
    assert call(amax=None) == -1
    assert call(k=8) == -2
    assert call(wsz=ws - 1) == -3


def test_gemm_rowscale_validation():
    f = Q.lib().quads_moe_w4a4_gemm_rowscale
    ws = Q.lib().quads_moe_w4a4_gemm_ws(64, 256, 0, 4, 64)

    def call(k_dim=256, e=4, ts=FAKE, offsets=FAKE, epi=0, odt=0, out=FAKE):
        return f(FAKE, FAKE, ts, None, 64, k_dim, FAKE, FAKE, FAKE, offsets, e, 64, epi, odt,
                 out, FAKE, ws, None)
    assert call(ts=None) == -1                 # per-row scales required
    assert call(ts=MIS) == -1
    assert call(k_dim=250) == -2
    assert call(offsets=None) == -1
    assert call(epi=1, odt=0) == -1
    assert call(out=MIS) == -1


def test_experts_validation():
    lib = Q.lib()
    f = lib.quads_rac_quantize_experts
    ws = lib.quads_rac_quantize_experts_ws(64, 256, 16, 4)
    assert ws > 0

    def call(m=64, kd=256, k=16, e=4, off=FAKE, wsz=ws):
        return f(FAKE, m, kd, k, off, e, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None, FAKE, wsz,
                 None)
    assert call(off=None) == -1                 # offsets required
    assert call(k=8) == -2
    assert call(m=64 ** 3 + 1) == -2            # rows per expert bound
    assert call(e=0) == -2
    assert call(wsz=ws - 1) == -3
    g = lib.quads_moe_w4a4_gemm_sel_experts
    gws = lib.quads_moe_w4a4_gemm_ws(64, 256, 16, 4, 64)
    assert g(FAKE, FAKE, FAKE, 64, 256, FAKE, FAKE, FAKE, FAKE, 16, FAKE, FAKE, FAKE, None, 4, 64,
             0, 0, FAKE, FAKE, gws, None) == -1      # offsets required
    assert g(FAKE, FAKE, FAKE, 64, 256, FAKE, FAKE, None, FAKE, 16, FAKE, FAKE, FAKE, FAKE, 4, 64,
             0, 0, FAKE, FAKE, gws, None) == -1      # residual scales required


def test_combine_validation():
    lib = Q.lib()
    f = lib.quads_moe_combine
    assert f(FAKE, 0, FAKE, FAKE, 4, 2, 12, FAKE, None) == -2     # N % 8
    assert f(FAKE, 5, FAKE, FAKE, 4, 2, 16, FAKE, None) == -1     # dtype
    assert f(None, 0, FAKE, FAKE, 4, 2, 16, FAKE, None) == -1


def test_mx_validation():
    lib = Q.lib()
    q = lib.quads_mx_quantize
    assert q(FAKE, 4, 48, 0, FAKE, FAKE, None) == -2              # K % 32
    assert q(FAKE, 4, 64, 1, FAKE, FAKE, None) == -1              # format
    assert q(FAKE, 4, 64, 4, MIS, FAKE, None) == -1
    assert q(None, 0, 64, 0, None, None, None) == 0               # empty: no-op
    g = lib.quads_moe_mx_gemm

    def call(rows=64, k_dim=256, e=4, n=64, fmt=0, epi=0, odt=0, offsets=FAKE, out=FAKE):
        return g(FAKE, FAKE, None, rows, k_dim, FAKE, FAKE, offsets, e, n, fmt, epi, odt, out,
                 None)
    assert call(k_dim=192) == -2                                  # K % 128
    assert call(fmt=2) == -1
    assert call(epi=1, odt=0) == -1
    assert call(n=63, epi=1, odt=1) == -2
    assert call(offsets=None) == -1
    assert call(out=MIS) == -1
    assert call(rows=0) == 0
