"""C-ABI checks that need no GPU: the library loads, exports every function
include/libfp4q.h declares, and rejects bad arguments on the host (status
codes) before anything reaches the device."""
import ctypes as ct
import os
import re

import pytest

import mxfp4_block_scaled_fp4q_amd as fq

HEADER = os.path.join(os.path.dirname(os.path.dirname(__file__)), "include", "libfp4q.h")


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(fq.LIB_PATH):
        pytest.fail("libfp4q.so not built (run __graft_entry__.build())")
    return fq.lib()


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(fp4q_[a-z_0-9]+)\s*\(", src)))


def test_exports_every_declared_function(L):
    names = declared_functions()
    assert set(names) == set(fq.EXPORTS)
    for n in names:
        assert hasattr(L, n), n


def test_version_and_strings(L):
    assert L.fp4q_abi_version() == 1
    for s in range(6):
        assert L.fp4q_status_string(s).decode()
    assert L.fp4q_status_string(99).decode() == "unknown status"


FAKE = ct.c_void_p(0x10000)       # 16-byte aligned, never dereferenced
FAKE_MIS = ct.c_void_p(0x10008)   # misaligned
NUL = ct.c_void_p(0)


def q(L, x=FAKE, dt=1, rows=64, cols=64, ld=64, block=32, axis=0, rnd=0, codes=FAKE,
      scales=FAKE):
    return L.fp4q_quantize(x, dt, rows, cols, ld, block, axis, rnd, 0, 0, codes, scales, NUL)


@pytest.mark.parametrize("kw,status", [
    (dict(x=NUL), 1), (dict(codes=NUL), 1), (dict(scales=NUL), 1),
    (dict(dt=7), 1), (dict(rows=0), 1), (dict(cols=-1), 1), (dict(ld=32), 1),
    (dict(block=8), 1), (dict(block=48), 1), (dict(block=256), 1),
    (dict(axis=2), 1), (dict(rnd=3), 1),
    (dict(cols=48, ld=48), 1),               # ROW needs cols % block == 0
    (dict(rows=48, axis=1), 1),              # COL needs rows % block == 0
    (dict(x=FAKE_MIS), 3), (dict(codes=FAKE_MIS), 3), (dict(scales=FAKE_MIS), 3),
    (dict(ld=68), 3),                        # bf16 row stride 136 bytes
    (dict(rows=1 << 40), 1),                 # too large
])
def test_quantize_validation(L, kw, status):
    assert q(L, **kw) == status
    assert L.fp4q_last_error().decode()


def test_dequantize_validation(L):
    d = L.fp4q_dequantize
    assert d(NUL, FAKE, 4, 64, 32, FAKE, 1, NUL) == 1
    assert d(FAKE, FAKE, 4, 64, 24, FAKE, 1, NUL) == 1
    assert d(FAKE, FAKE, 4, 48, 32, FAKE, 1, NUL) == 1
    assert d(FAKE, FAKE, 4, 64, 32, FAKE, 5, NUL) == 1
    assert d(FAKE, FAKE, 4, 64, 32, FAKE_MIS, 1, NUL) == 3


def test_grad_validation(L):
    g = L.fp4q_grad_estimate
    # DGE needs x
    assert g(1, NUL, 1, FAKE, 1, 64, 64, 32, 0, 5.0, 3.0, FAKE, 1, NUL) == 1
    assert g(2, FAKE, 1, FAKE, 1, 64, 64, 32, 0, 5.0, 3.0, FAKE, 1, NUL) == 1
    assert g(1, FAKE, 1, FAKE, 1, 64, 64, 32, 0, 0.5, 3.0, FAKE, 1, NUL) == 1  # k < 1
    assert g(1, FAKE, 1, FAKE, 1, 64, 64, 32, 0, 5.0, 0.0, FAKE, 1, NUL) == 1  # clamp <= 0
    assert g(1, FAKE, 1, FAKE, 1, 64, 48, 32, 0, 5.0, 3.0, FAKE, 1, NUL) == 1  # ROW cols%b
    assert g(1, FAKE, 1, FAKE, 1, 48, 64, 32, 1, 5.0, 3.0, FAKE, 1, NUL) == 1  # COL rows%b
    assert g(1, FAKE, 1, FAKE_MIS, 1, 64, 64, 32, 0, 5.0, 3.0, FAKE, 1, NUL) == 3
    assert g(0, NUL, 1, FAKE, 1, 0, 64, 32, 0, 5.0, 3.0, FAKE, 1, NUL) == 1


def test_gemm_validation(L):
    g = L.fp4q_gemm
    ok = dict(M=64, N=64, K=256, a=FAKE, sa=FAKE, b=FAKE, sb=FAKE, blk=32, c=FAKE, cdt=0,
              ldc=64, acc=0)

    def call(**kw):
        a = dict(ok, **kw)
        return g(a["M"], a["N"], a["K"], a["a"], a["sa"], a["b"], a["sb"], a["blk"], a["c"],
                 a["cdt"], a["ldc"], a["acc"], NUL)
    assert call(a=NUL) == 1
    assert call(M=0) == 1
    assert call(blk=16) == 2            # valid block, not the MX hardware block
    assert call(blk=12) == 1
    assert call(K=160) == 1             # K % 64
    assert call(K=96) == 1
    assert call(K=1 << 24) == 2         # 256 rows of codes exceed 32-bit offsets
    assert call(ldc=32) == 1
    assert call(acc=1, cdt=1) == 2      # accumulate into bf16
    assert call(acc=2) == 1
    assert call(c=ct.c_void_p(0x10002)) == 3   # fp32 C not 4-byte aligned
    assert call(a=FAKE_MIS) == 3
    assert call(sb=FAKE_MIS) == 3


def test_hcp_validation(L):
    h = L.fp4q_hcp_residual_add
    ws = L.fp4q_hcp_workspace_bytes(128, 64, 10)
    assert ws >= (128 + 64) * (2 * 10) * 2   # gathered bf16 operands, 2 n_hot columns
    assert L.fp4q_hcp_workspace_bytes(128, 64, 0) == 0
    args = [128, 64, 256, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 10, FAKE, FAKE, ws, NUL]
    bad = list(args)
    bad[13] = ws - 1
    assert h(*bad) == 4
    bad = list(args)
    bad[10] = 300        # n_hot > K
    assert h(*bad) == 1
    bad = list(args)
    bad[2] = 1 << 22
    bad[10] = (1 << 20) + 1    # more hot channels than the residual GEMM addresses
    assert h(*bad) == 2
    bad = list(args)
    bad[2] = 100         # K % 32
    assert h(*bad) == 1
    bad = list(args)
    bad[3] = NUL
    assert h(*bad) == 1
    bad = list(args)
    bad[11] = FAKE_MIS
    assert h(*bad) == 3
    bad = list(args)
    bad[10] = 0          # no hot channels: a no-op that touches nothing
    bad[3] = NUL
    assert h(*bad) == 0


def test_fastdiv_formula():
    """The 32-bit division-by-invariant multiplier the streaming kernels use
    (Granlund & Montgomery round-up variant), checked against // on the host."""
    import random
    random.seed(3)
    for d in [1, 2, 3, 7, 64, 176, 256, 640, 704, 2047, 2048, 2049, (1 << 31) - 1] + \
            [random.randrange(1, 1 << 31) for _ in range(200)]:
        l = 0
        while (1 << l) < d:
            l += 1
        mul = ((1 << 32) * ((1 << l) - d)) // d + 1
        assert mul < (1 << 32)
        for n in [0, 1, d - 1, d, d + 1, (1 << 31) - 1] + \
                [random.randrange(0, 1 << 31) for _ in range(500)]:
            assert ((((n * mul) >> 32) + n) >> l) == n // d


def test_quantize_dual_validation(L):
    d = L.fp4q_quantize_dual

    def call(x=FAKE, dt=1, rows=64, cols=64, ld=64, block=32, rr=0, rc=1, a=FAKE, b=FAKE,
             c=FAKE, e=FAKE):
        return d(x, dt, rows, cols, ld, block, rr, 1, rc, 2, 0, a, b, c, e, NUL)
    assert call(x=NUL) == 1
    assert call(e=NUL) == 1
    assert call(rows=48) == 1          # rows % block
    assert call(cols=48, ld=48) == 1   # cols % block
    assert call(rr=2) == 1
    assert call(rc=5) == 1
    assert call(block=24) == 1
    assert call(ld=32) == 1
    assert call(c=FAKE_MIS) == 3
    assert call(ld=68) == 3            # bf16 row stride 136 bytes
    assert L.fp4q_last_error().decode()


def test_gemm_hcp_validation(L):
    h = L.fp4q_gemm_hcp
    ws = L.fp4q_hcp_workspace_bytes(128, 64, 10)
    args = [128, 64, 256, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 10, FAKE, 64, FAKE, ws, NUL]
    bad = list(args)
    bad[14] = ws - 1
    assert h(*bad) == 4
    bad = list(args)
    bad[10] = 300        # n_hot > K
    assert h(*bad) == 1
    bad = list(args)
    bad[2] = 1 << 22
    bad[10] = (1 << 20) + 1
    assert h(*bad) == 2
    bad = list(args)
    bad[2] = 160         # K % 64 (the FP4 GEMM's half step)
    assert h(*bad) == 1
    bad = list(args)
    bad[2] = 1 << 24     # K beyond the GEMM's 32-bit row offsets
    assert h(*bad) == 2
    bad = list(args)
    bad[12] = 63         # ld_y < N
    assert h(*bad) == 1
    bad = list(args)
    bad[3] = NUL         # x needed when there are hot channels
    assert h(*bad) == 1
    bad = list(args)
    bad[4] = NUL         # quantised X always needed
    assert h(*bad) == 1
    bad = list(args)
    bad[11] = ct.c_void_p(0x10002)   # y not 4-byte aligned
    assert h(*bad) == 3
    bad = list(args)
    bad[6] = FAKE_MIS    # W codes not 16-byte aligned
    assert h(*bad) == 3


def test_gemm_dge_validation(L):
    h = L.fp4q_gemm_dge
    F = ct.c_float
    args = [256, 64, 256, FAKE, FAKE, FAKE, FAKE, FAKE, 1, F(5.0), F(3.0), FAKE, 64, NUL]
    bad = list(args)
    bad[0] = 250         # M % 32 (column blocks of x)
    assert h(*bad) == 1
    bad = list(args)
    bad[2] = 160         # K % 64
    assert h(*bad) == 1
    bad = list(args)
    bad[8] = 0           # fp32 x
    assert h(*bad) == 2
    bad = list(args)
    bad[8] = 7           # not a dtype
    assert h(*bad) == 1
    bad = list(args)
    bad[9] = F(0.5)      # k < 1
    assert h(*bad) == 1
    bad = list(args)
    bad[10] = F(0.0)     # clamp
    assert h(*bad) == 1
    bad = list(args)
    bad[12] = 63         # ld_out < N
    assert h(*bad) == 1
    bad = list(args)
    bad[7] = NUL         # x
    assert h(*bad) == 1
    bad = list(args)
    bad[7] = FAKE_MIS    # x alignment
    assert h(*bad) == 3
    bad = list(args)
    bad[2] = 1 << 24
    assert h(*bad) == 2


def test_gemm_quant_validation(L):
    h = L.fp4q_gemm_quant
    args = [256, 64, 256, FAKE, FAKE, FAKE, FAKE, FAKE, 64, FAKE, FAKE, NUL]
    bad = list(args)
    bad[1] = 48          # N % 32 (ROW blocks of C)
    assert h(*bad) == 1
    bad = list(args)
    bad[2] = 160         # K % 64
    assert h(*bad) == 1
    bad = list(args)
    bad[8] = 63          # ld_c < N
    assert h(*bad) == 1
    bad = list(args)
    bad[9] = NUL         # codes
    assert h(*bad) == 1
    bad = list(args)
    bad[9] = FAKE_MIS    # codes alignment
    assert h(*bad) == 3
    bad = list(args)
    bad[7] = ct.c_void_p(0x10001)   # C not element-aligned
    assert h(*bad) == 3
    bad = list(args)
    bad[2] = 1 << 24
    assert h(*bad) == 2


def test_split_entry_points_validation(L):
    assert L.fp4q_channel_mask(FAKE, 3, 0, FAKE, NUL) == 1          # length
    assert L.fp4q_channel_mask(FAKE, -1, 10, FAKE, NUL) == 1        # n
    assert L.fp4q_channel_mask(FAKE, 3, 10, NUL, NUL) == 1          # mask
    assert L.fp4q_channel_mask(ct.c_void_p(0x10002), 3, 10, FAKE, NUL) == 3
    q = L.fp4q_quantize_masked
    args = [FAKE, 1, 64, 64, 64, 32, 0, 0, ct.c_uint64(0), ct.c_uint64(0), FAKE, FAKE, FAKE, NUL]
    bad = list(args)
    bad[10] = NUL        # zero mask
    assert q(*bad) == 1
    bad = list(args)
    bad[10] = ct.c_void_p(0x10002)
    assert q(*bad) == 3
    bad = list(args)
    bad[3] = 48          # cols % block for ROW
    bad[4] = 48
    assert q(*bad) == 1
    h = L.fp4q_gemm_hcp_split
    ws = L.fp4q_hcp_workspace_bytes(128, 64, 10)
    args = [128, 64, 256, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 10, FAKE, 64, FAKE, ws, NUL]
    bad = list(args)
    bad[14] = ws - 1
    assert h(*bad) == 4
    bad = list(args)
    bad[2] = 160
    assert h(*bad) == 1
    bad = list(args)
    bad[10] = 300
    assert h(*bad) == 1


def test_hot_channels_validation(L):
    ws = L.fp4q_hot_channels_workspace_bytes(128, 64)
    assert ws >= (2 + 1) * 64 * 4        # partial rows + the error row
    assert L.fp4q_hot_channels_workspace_bytes(0, 64) == 0
    h = L.fp4q_hot_channels
    args = [FAKE, 128, 64, 64, 6, FAKE, NUL, FAKE, ws, NUL]
    for i, v, st in [(2, 48, 1),          # cols % 32
                     (3, 60, 1),          # ld_x < cols
                     (3, 68, 1),          # ld_x % 8
                     (4, 65, 1),          # n_hot > cols
                     (4, -1, 1),          # n_hot < 0
                     (1, 0, 1),           # rows
                     (5, NUL, 1),         # hot_idx with n_hot > 0
                     (7, NUL, 1),         # workspace
                     (8, ws - 1, 4),      # workspace size
                     (0, ct.c_void_p(0x10008), 3),   # x alignment
                     (6, ct.c_void_p(0x10002), 3)]:  # err alignment
        bad = list(args)
        bad[i] = v
        assert h(*bad) == st, (i, v)
    bad = list(args)
    bad[2] = bad[3] = 16384 + 32         # above the in-LDS selection limit
    bad[8] = L.fp4q_hot_channels_workspace_bytes(128, 16384 + 32)
    assert h(*bad) == 2


def test_quantize_2d_validation(L):
    q = L.fp4q_quantize_2d
    args = [FAKE, 64, 96, 96, 0, ct.c_uint64(0), ct.c_uint64(0), FAKE, FAKE, FAKE, FAKE, NUL]
    for i, v, st in [(1, 48, 1),          # rows % 32
                     (2, 80, 1),          # cols % 32
                     (3, 64, 1),          # ld_x < cols
                     (3, 100, 3),         # ld_x % 8
                     (4, 2, 1),           # round
                     (0, NUL, 1),
                     (9, NUL, 1),
                     (0, FAKE_MIS, 3),
                     (10, ct.c_void_p(0x10001), 3)]:
        bad = list(args)
        bad[i] = v
        assert q(*bad) == st, (i, v)


def test_quantize_rht_validation(L):
    q = L.fp4q_quantize_rht
    args = [FAKE, 64, 96, 96, 0, FAKE, 0, ct.c_uint64(0), ct.c_uint64(0), FAKE, FAKE, NUL]
    for i, v, st in [(2, 80, 1),          # ROW: cols % 32
                     (4, 2, 1),           # axis
                     (6, 3, 1),           # round
                     (5, NUL, 1),         # signs
                     (3, 90, 1),          # ld_x < cols
                     (3, 100, 3),         # ld_x % 8
                     (5, ct.c_void_p(0x10002), 3),
                     (9, FAKE_MIS, 3)]:
        bad = list(args)
        bad[i] = v
        assert q(*bad) == st, (i, v)
    bad = list(args)
    bad[4] = 1                            # COL: rows % 32
    bad[1] = 48
    assert q(*bad) == 1


def test_occ_validation(L):
    assert L.fp4q_occ_max_nnz(100, 64, ct.c_double(0.99)) == 6400 - 6336
    assert L.fp4q_occ_max_nnz(100, 64, ct.c_double(1.0)) == 0
    assert L.fp4q_occ_max_nnz(100, 64, ct.c_double(0.0)) == -1
    ws = L.fp4q_occ_workspace_bytes(100, 64)
    q = L.fp4q_occ_quantize
    args = [FAKE, 100, 64, 64, ct.c_double(0.99), 0, ct.c_uint64(0), ct.c_uint64(0), FAKE, FAKE,
            FAKE, FAKE, FAKE, 64, NUL, FAKE, ws, NUL]
    for i, v, st in [(2, 48, 1),                  # cols % 32
                     (4, ct.c_double(1.5), 1),    # quantile
                     (4, ct.c_double(0.0), 1),
                     (5, 2, 1),                   # round
                     (13, 63, 1),                 # nnz_cap below the bound
                     (11, NUL, 1),                # col_idx
                     (16, ws - 1, 4),             # workspace
                     (3, 60, 1),                  # ld_x
                     (10, ct.c_void_p(0x10004), 3)]:
        bad = list(args)
        bad[i] = v
        assert q(*bad) == st, (i, v)
    s = L.fp4q_occ_spmm
    args = [16, 64, 128, FAKE, FAKE, FAKE, FAKE, 64, FAKE, 64, NUL]
    for i, v, st in [(1, 60, 1), (7, 32, 1), (9, 32, 1), (3, NUL, 1), (8, FAKE_MIS, 3),
                     (9, 66, 3)]:
        bad = list(args)
        bad[i] = v
        assert s(*bad) == st, (i, v)


def test_hcp_noalloc_validation(L):
    """The workspace-free hot-channel call refuses, on the host, sizes whose
    gathered operands exceed its static scratch (nothing is launched)."""
    h = L.fp4q_hcp_residual_add_noalloc
    args = (FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE)
    assert h(64, 64, 1024, *args, 0, FAKE, NUL) == 0                      # no hot channels: no-op
    assert h(64, 64, 1000, *args, 8, FAKE, NUL) == 1                      # K % 32
    assert h(64, 64, 1024, *args, 2000, FAKE, NUL) == 1                   # n_hot > K
    assert h(64, 64, 1024, NUL, *args[1:], 8, FAKE, NUL) == 1             # null x
    assert h(64, 64, 1024, FAKE_MIS, *args[1:], 8, FAKE, NUL) == 3        # misaligned x
    assert h(1 << 20, 1 << 16, 1024, *args, 64, FAKE, NUL) == 4           # > 64 MiB of scratch
    assert b"static maximum" in L.fp4q_last_error()
    assert fq.hcp_workspace_bytes(1 << 20, 1 << 16, 64) > fq.HCP_NOALLOC_MAX_BYTES


def test_set_next_launch_flags(L):
    """Unknown flag bits are rejected and set nothing; the known ones and the
    clearing call succeed (host-side state only, no device work)."""
    assert L.fp4q_set_next_launch(None, None, 2) == 1
    assert "flags" in L.fp4q_last_error().decode()
    assert L.fp4q_set_next_launch(None, None, 0xFFFFFFFE) == 1
    assert L.fp4q_set_next_launch(None, None, fq.ANY_ORDER) == 0
    assert L.fp4q_set_next_launch(None, None, 0) == 0
