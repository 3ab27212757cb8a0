"""Shared helpers of the GPU parity tests: host <-> device moves and the
comparison rules (bit-exact codes/scales/dequant/STE; DGE within 2^-20 of the
oracle's derivative; GEMM/HCP within 1e-5 * sum|a_i b_i|)."""
import numpy as np
import torch

DGE_REL = 2.0 ** -20
GEMM_REL = 1e-5


def dev_bf16(bits: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).cuda()


def dev(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def host_bits(t: torch.Tensor) -> np.ndarray:
    """bf16 tensor -> uint16 bits; fp32 -> float32; uint8 -> uint8."""
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).cpu().numpy().view(np.uint16)
    return t.cpu().numpy()


def to_dev_input(x: np.ndarray) -> torch.Tensor:
    return dev_bf16(x) if x.dtype == np.uint16 else dev(x)


def f64_of(t: torch.Tensor, orc) -> np.ndarray:
    h = host_bits(t)
    if h.dtype == np.uint16:
        return orc.bf16_to_f64(h)
    return h.astype(np.float64)


def assert_same_bits(got: np.ndarray, want: np.ndarray, what=""):
    if not np.array_equal(got, want):
        bad = np.argwhere(got != want)
        i = tuple(bad[0])
        raise AssertionError(f"{what}: {len(bad)} mismatches; first at {i}: got {got[i]!r} "
                             f"want {want[i]!r}")


def assert_float_bits_equal(got: np.ndarray, want: np.ndarray, what=""):
    """Bit equality, except that any NaN matches any NaN."""
    if got.dtype == np.uint16:
        gn = (got & 0x7FFF) > 0x7F80
        wn = (want & 0x7FFF) > 0x7F80
    else:
        gn = np.isnan(got)
        wn = np.isnan(want)
        got = got.view(np.uint32)
        want = want.view(np.uint32)
    assert np.array_equal(gn, wn), f"{what}: NaN positions differ"
    assert_same_bits(np.where(gn, 0, got), np.where(wn, 0, want), what)


def check_gemm_f32(c: np.ndarray, C: np.ndarray, S: np.ndarray, what=""):
    err = np.abs(c.astype(np.float64) - C)
    tol = GEMM_REL * S
    ok = err <= tol
    if not ok.all():
        i = np.argwhere(~ok)[0]
        i = tuple(i)
        raise AssertionError(f"{what}: {int((~ok).sum())} entries out of tolerance; first {i}: "
                             f"got {c[i]!r} want {C[i]!r} S {S[i]!r}")


def check_gemm_bf16(c_bits: np.ndarray, C: np.ndarray, S: np.ndarray, orc, what=""):
    lo = orc.bf16_to_f64(orc.round_bf16(C - GEMM_REL * S))
    hi = orc.bf16_to_f64(orc.round_bf16(C + GEMM_REL * S))
    v = orc.bf16_to_f64(c_bits)
    ok = (v >= lo) & (v <= hi)
    if not ok.all():
        i = tuple(np.argwhere(~ok)[0])
        raise AssertionError(f"{what}: {int((~ok).sum())} bf16 entries out of bracket; first {i}:"
                             f" got {v[i]!r} bracket [{lo[i]!r}, {hi[i]!r}]")


def check_dge(out: torch.Tensor, d_ref: np.ndarray, g_f64: np.ndarray, orc, clamp_max, what=""):
    """Each output within the rounded bracket g*d_ref*(1 -+ 2^-20); bit-exact
    where d_ref is exactly clamp_max or 1 (the product is then formed exactly)."""
    rnd = orc.round_bf16 if out.dtype == torch.bfloat16 else orc.round_f32
    tof = orc.bf16_to_f64 if out.dtype == torch.bfloat16 else (lambda a: a.astype(np.float64))
    o = f64_of(out, orc)
    nan_ref = np.isnan(d_ref)
    assert np.array_equal(np.isnan(o) & nan_ref, nan_ref), f"{what}: NaN blocks"
    fin = ~nan_ref
    a = g_f64 * d_ref * (1 - DGE_REL)
    b = g_f64 * d_ref * (1 + DGE_REL)
    lo = tof(rnd(np.minimum(a, b)))
    hi = tof(rnd(np.maximum(a, b)))
    ok = (o >= lo) & (o <= hi) | ~fin
    if not ok.all():
        i = tuple(np.argwhere(~ok)[0])
        raise AssertionError(f"{what}: {int((~ok).sum())} out of bracket; first {i}: got {o[i]!r}"
                             f" bracket [{lo[i]!r}, {hi[i]!r}] d_ref {d_ref[i]!r} g {g_f64[i]!r}")
    exact = fin & ((d_ref == clamp_max) | (d_ref == 1.0))
    want = tof(rnd(g_f64 * d_ref))
    bad = exact & ~((o == want) | (np.isnan(o) & np.isnan(want)))
    assert not bad.any(), f"{what}: {int(bad.sum())} clamped/unit entries not bit-exact"


def edge_lines(n, k, seed):
    """k distinct indices of [0, n), always including 0 and n - 1 (all of
    them when n <= k), ascending."""
    if n <= k:
        return np.arange(n)
    rng = np.random.default_rng(seed)
    pick = rng.choice(np.arange(1, n - 1), k - 2, replace=False)
    return np.sort(np.concatenate([[0, n - 1], pick])).astype(np.int64)


def sample_positions(M, N, seed, per_tile=4, tile=128, full_rows=2, full_cols=2):
    """>= per_tile random entries in every tile x tile output tile, plus
    full_rows whole rows and full_cols whole columns that always include the
    first and the last (edge_lines)."""
    rng = np.random.default_rng(seed)
    ii, jj = [], []
    for t0 in range(0, M, tile):
        for u0 in range(0, N, tile):
            h = min(tile, M - t0)
            w = min(tile, N - u0)
            ii.append(t0 + rng.integers(0, h, per_tile))
            jj.append(u0 + rng.integers(0, w, per_tile))
    for r in edge_lines(M, max(full_rows, 2), seed + 1):
        ii.append(np.full(N, r))
        jj.append(np.arange(N))
    for c in edge_lines(N, max(full_cols, 2), seed + 2):
        ii.append(np.arange(M))
        jj.append(np.full(M, c))
    return np.concatenate(ii).astype(np.int64), np.concatenate(jj).astype(np.int64)


def check_lines_f32(orc, got, rows, cols, ref, what=""):
    """Whole rows `rows` and whole columns `cols` of an fp32 output `got`
    [M, N] against ref(rows=..., cols=...) -> (C, S) of those lines."""
    C, S = ref(rows=rows, cols=None)
    check_gemm_f32(got[rows], C, S, f"{what} rows")
    C, S = ref(rows=None, cols=cols)
    check_gemm_f32(got[:, cols], C, S, f"{what} cols")
