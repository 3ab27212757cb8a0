"""Python binding of libfp4q, the block-scaled MXFP4 linear-layer hot path for
AMD MI355X (gfx950).

Argument marshalling only: every step runs in the HIP kernels behind the C ABI
declared in ``include/libfp4q.h``; torch supplies device memory and the
current stream.  There is no fallback: if ``libfp4q.so`` has not been built,
loading the library raises.
"""
import ctypes as _ct
import os as _os

_HERE = _os.path.dirname(_os.path.abspath(__file__))
LIB_PATH = _os.path.join(_HERE, "libfp4q.so")

F32, BF16 = 0, 1
ROW, COL = 0, 1
RNE, SR = 0, 1
STE, DGE = 0, 1

STATUS = {0: "FP4Q_OK", 1: "FP4Q_ERR_INVALID", 2: "FP4Q_ERR_UNSUPPORTED",
          3: "FP4Q_ERR_ALIGNMENT", 4: "FP4Q_ERR_WORKSPACE", 5: "FP4Q_ERR_HIP"}

EXPORTS = ["fp4q_channel_mask", "fp4q_quantize_masked", "fp4q_gemm_hcp_split",
           "fp4q_quantize", "fp4q_quantize_dual", "fp4q_dequantize", "fp4q_grad_estimate",
           "fp4q_gemm",
           "fp4q_gemm_dge", "fp4q_gemm_quant", "fp4q_hcp_workspace_bytes",
           "fp4q_hcp_residual_add", "fp4q_hcp_residual_add_noalloc",
           "fp4q_gemm_hcp", "fp4q_hot_channels_workspace_bytes", "fp4q_hot_channels",
           "fp4q_quantize_2d", "fp4q_quantize_2d_tile", "fp4q_quantize_rht", "fp4q_occ_max_nnz",
           "fp4q_occ_workspace_bytes", "fp4q_occ_quantize", "fp4q_occ_spmm",
           "fp4q_set_next_launch", "fp4q_status_string",
           "fp4q_last_error", "fp4q_abi_version"]


class Fp4qError(RuntimeError):
    def __init__(self, status, detail):
        super().__init__(f"{STATUS.get(status, status)}: {detail}")
        self.status = status


_lib = None


def lib():
    """Load libfp4q.so (raises if it is not built)."""
    global _lib
    if _lib is None:
        if not _os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is not built; run "
                              "mxfp4_block_scaled_fp4q_amd/build.py (or __graft_entry__.build())")
        L = _ct.CDLL(LIB_PATH)
        P, I64, I32, U64, F, SZ = (_ct.c_void_p, _ct.c_int64, _ct.c_int32, _ct.c_uint64,
                                   _ct.c_float, _ct.c_size_t)
        sig = {
            "fp4q_quantize": (I32, [P, I32, I64, I64, I64, I32, I32, I32, U64, U64, P, P, P]),
            "fp4q_quantize_dual": (I32, [P, I32, I64, I64, I64, I32, I32, U64, I32, U64, U64, P, P,
                                         P, P, P]),
            "fp4q_dequantize": (I32, [P, P, I64, I64, I32, P, I32, P]),
            "fp4q_grad_estimate": (I32, [I32, P, I32, P, I32, I64, I64, I32, I32, F, F, P, I32,
                                         P]),
            "fp4q_gemm": (I32, [I64, I64, I64, P, P, P, P, I32, P, I32, I64, I32, P]),
            "fp4q_hcp_workspace_bytes": (SZ, [I64, I64, I32]),
            "fp4q_hcp_residual_add": (I32, [I64, I64, I64, P, P, P, P, P, P, P, I32, P, P, SZ,
                                            P]),
            "fp4q_hcp_residual_add_noalloc": (I32, [I64, I64, I64, P, P, P, P, P, P, P, I32, P,
                                                    P]),
            "fp4q_gemm_dge": (I32, [I64, I64, I64, P, P, P, P, P, I32, F, F, P, I64, P]),
            "fp4q_gemm_quant": (I32, [I64, I64, I64, P, P, P, P, P, I64, P, P, P]),
            "fp4q_channel_mask": (I32, [P, I32, I64, P, P]),
            "fp4q_quantize_masked": (I32, [P, I32, I64, I64, I64, I32, I32, I32, U64, U64, P, P,
                                           P, P]),
            "fp4q_gemm_hcp_split": (I32, [I64, I64, I64, P, P, P, P, P, P, P, I32, P, I64, P, SZ,
                                          P]),
            "fp4q_gemm_hcp": (I32, [I64, I64, I64, P, P, P, P, P, P, P, I32, P, I64, P, SZ, P]),
            "fp4q_hot_channels_workspace_bytes": (SZ, [I64, I64]),
            "fp4q_quantize_2d": (I32, [P, I64, I64, I64, I32, U64, U64, P, P, P, P, P]),
            "fp4q_quantize_2d_tile": (I32, [P, I64, I64, I64, I32, I32, U64, U64, P, P, P, P, P]),
            "fp4q_quantize_rht": (I32, [P, I64, I64, I64, I32, P, I32, U64, U64, P, P, P]),
            "fp4q_occ_max_nnz": (I64, [I64, I64, _ct.c_double]),
            "fp4q_occ_workspace_bytes": (SZ, [I64, I64]),
            "fp4q_occ_quantize": (I32, [P, I64, I64, I64, _ct.c_double, I32, U64, U64, P, P, P, P,
                                        P, I64, P, P, SZ, P]),
            "fp4q_occ_spmm": (I32, [I64, I64, I64, P, P, P, P, I64, P, I64, P]),
            "fp4q_hot_channels": (I32, [P, I64, I64, I64, I32, P, P, P, SZ, P]),
            "fp4q_set_next_launch": (I32, [P, P, _ct.c_uint32]),
            "fp4q_status_string": (_ct.c_char_p, [I32]),
            "fp4q_last_error": (_ct.c_char_p, []),
            "fp4q_abi_version": (I32, []),
        }
        for name, (res, args) in sig.items():
            f = getattr(L, name)
            f.restype = res
            f.argtypes = args
        _lib = L
    return _lib


def _check(status):
    if status != 0:
        raise Fp4qError(status, lib().fp4q_last_error().decode())


def _torch():
    import torch
    return torch


def _ptr(t):
    return _ct.c_void_p(t.data_ptr()) if t is not None else None


def _dt(t):
    torch = _torch()
    if t.dtype == torch.bfloat16:
        return BF16
    if t.dtype == torch.float32:
        return F32
    raise TypeError(f"libfp4q takes bf16 or fp32 tensors, got {t.dtype}")


def _stream(stream):
    torch = _torch()
    s = stream if stream is not None else torch.cuda.current_stream()
    return _ct.c_void_p(s.cuda_stream)


def _need_cuda(*ts):
    for t in ts:
        if t is not None and not t.is_cuda:
            raise ValueError("libfp4q takes device (cuda) tensors")


def _need(t, name, dtype, shape=None, dense=True):
    """Raise unless t has the dtype (and shape) the C call reads it as and,
    with dense, is contiguous (the C call takes no strides for it)."""
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    if dense and not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _scratch(nbytes, device, stream):
    """Caller-less workspace for one call: allocated from torch's pool and,
    when the kernels run on a stream other than the current one, recorded on
    that stream so the pool does not hand the block to other work before
    those kernels finish."""
    torch = _torch()
    ws = torch.empty(max(int(nbytes), 16), dtype=torch.uint8, device=device)
    if stream is not None:
        ws.record_stream(stream)
    return ws


def _hcp_operands(x, xq_codes, xq_scales, w, wq_codes, wq_scales, hot_idx):
    """Shapes and dtypes of the hot-channel calls' operands; returns M, N, K."""
    torch = _torch()
    _need_cuda(x, xq_codes, xq_scales, w, wq_codes, wq_scales, hot_idx)
    if x.dim() != 2 or w.dim() != 2:
        raise ValueError("x and w must be 2-D")
    M, K = x.shape
    N = w.shape[1]
    _need(x, "x", torch.bfloat16)
    _need(w, "w", torch.bfloat16, (K, N))
    _need(xq_codes, "xq_codes", torch.uint8, (M, K // 2))
    _need(xq_scales, "xq_scales", torch.uint8, (M, K // 32))
    _need(wq_codes, "wq_codes", torch.uint8, (N, K // 2))
    _need(wq_scales, "wq_scales", torch.uint8, (N, K // 32))
    _need(hot_idx, "hot_idx", torch.int32)
    if hot_idx.dim() != 1:
        raise ValueError("hot_idx must be 1-D")
    return M, N, K


def quantize(x, block=32, axis=ROW, rounding=RNE, seed=0, rng_offset=0, codes=None, scales=None,
             stream=None):
    """Fused MXFP4 quantisation of a 2-D bf16/fp32 tensor (row stride from x).
    Returns (codes uint8, scales uint8): ROW -> [R, C/2], [R, C/block];
    COL -> [C, R/2], [C, R/block] (the K-major quantisation of x^T)."""
    torch = _torch()
    _need_cuda(x)
    if x.dim() != 2 or x.stride(1) != 1:
        raise ValueError("x must be 2-D with unit column stride")
    rows, cols = x.shape
    if axis == ROW:
        cshape, sshape = (rows, cols // 2), (rows, cols // block)
    else:
        cshape, sshape = (cols, rows // 2), (cols, rows // block)
    if codes is None:
        codes = torch.empty(cshape, dtype=torch.uint8, device=x.device)
    if scales is None:
        scales = torch.empty(sshape, dtype=torch.uint8, device=x.device)
    _check(lib().fp4q_quantize(_ptr(x), _dt(x), rows, cols, x.stride(0), block, axis, rounding,
                               seed, rng_offset, _ptr(codes), _ptr(scales), _stream(stream)))
    return codes, scales


def quantize_dual(x, block=32, round_row=RNE, seed_row=0, round_col=RNE, seed_col=0,
                  rng_offset=0, out=None, stream=None):
    """Both orientations in one pass: returns ((row codes, row scales),
    (col codes, col scales)), identical to quantize(x, block, ROW, round_row,
    seed_row, rng_offset) and quantize(x, block, COL, round_col, seed_col,
    rng_offset).  `out` may give the four output tensors."""
    torch = _torch()
    _need_cuda(x)
    if x.dim() != 2 or x.stride(1) != 1:
        raise ValueError("x must be 2-D with unit column stride")
    rows, cols = x.shape
    if out is None:
        u8 = dict(dtype=torch.uint8, device=x.device)
        out = (torch.empty((rows, cols // 2), **u8), torch.empty((rows, cols // block), **u8),
               torch.empty((cols, rows // 2), **u8), torch.empty((cols, rows // block), **u8))
    rc, rs, cc, cs = out
    _check(lib().fp4q_quantize_dual(_ptr(x), _dt(x), rows, cols, x.stride(0), block, round_row,
                                    seed_row, round_col, seed_col, rng_offset, _ptr(rc), _ptr(rs),
                                    _ptr(cc), _ptr(cs), _stream(stream)))
    return (rc, rs), (cc, cs)


def dequantize(codes, scales, block=32, out_dtype=None, out=None, stream=None):
    """codes [R, K/2] + scales [R, K/block] -> dense [R, K] bf16 (default) or fp32."""
    torch = _torch()
    _need_cuda(codes, scales)
    rows, k = codes.shape[0], codes.shape[1] * 2
    if out is None:
        out = torch.empty((rows, k), dtype=out_dtype or torch.bfloat16, device=codes.device)
    _check(lib().fp4q_dequantize(_ptr(codes), _ptr(scales), rows, k, block, _ptr(out), _dt(out),
                                 _stream(stream)))
    return out


def grad_estimate(mode, x, grad, block=32, axis=ROW, k=5.0, clamp_max=3.0, out_dtype=None,
                  out=None, stream=None):
    """STE (mode 0) or DGE (mode 1) backward of the quantiser: out = grad * d."""
    torch = _torch()
    _need_cuda(x, grad)
    rows, cols = grad.shape
    if out is None:
        out = torch.empty((rows, cols), dtype=out_dtype or grad.dtype, device=grad.device)
    xdt = _dt(x) if x is not None else F32
    _check(lib().fp4q_grad_estimate(mode, _ptr(x), xdt, _ptr(grad), _dt(grad), rows, cols, block,
                                    axis, float(k), float(clamp_max), _ptr(out), _dt(out),
                                    _stream(stream)))
    return out


def gemm(a_codes, a_scales, b_codes, b_scales, out_dtype=None, c=None, accumulate=False,
         block=32, stream=None):
    """C[M,N] (+)= deq(A) deq(B)^T with A [M, K/2]+[M, K/32], B [N, K/2]+[N, K/32]."""
    torch = _torch()
    _need_cuda(a_codes, a_scales, b_codes, b_scales)
    M, N, K = a_codes.shape[0], b_codes.shape[0], a_codes.shape[1] * 2
    if b_codes.shape[1] * 2 != K:
        raise ValueError("A and B K dimensions differ")
    if c is None:
        c = torch.empty((M, N), dtype=out_dtype or torch.bfloat16, device=a_codes.device)
    _check(lib().fp4q_gemm(M, N, K, _ptr(a_codes), _ptr(a_scales), _ptr(b_codes),
                           _ptr(b_scales), block, _ptr(c), _dt(c), c.stride(0),
                           1 if accumulate else 0, _stream(stream)))
    return c


ANY_ORDER = 1


def set_next_launch(start_event=None, stop_event=None, any_order=False):
    """Options for the next kernel this thread launches through the library:
    hipEvent_t handles (ints or ctypes pointers, or None) that its dispatch
    records at its start and end, and whether it may start before earlier
    work on its stream has finished (the caller vouches that it does not
    depend on that work)."""
    _check(lib().fp4q_set_next_launch(start_event, stop_event, ANY_ORDER if any_order else 0))


def hcp_workspace_bytes(M, N, n_hot):
    return int(lib().fp4q_hcp_workspace_bytes(M, N, n_hot))


def hcp_residual_add(x, xq_codes, xq_scales, w, wq_codes, wq_scales, hot_idx, y, workspace=None,
                     stream=None):
    """y[M,N] (fp32, in place) += sum_{c in hot} X[:,c] W[c,:] - Xq[:,c] Wq[c,:]."""
    torch = _torch()
    M, N, K = _hcp_operands(x, xq_codes, xq_scales, w, wq_codes, wq_scales, hot_idx)
    _need_cuda(y)
    _need(y, "y", torch.float32, (M, N))
    n_hot = hot_idx.numel()
    if workspace is None:
        workspace = _scratch(hcp_workspace_bytes(M, N, n_hot), x.device, stream)
    _check(lib().fp4q_hcp_residual_add(M, N, K, _ptr(x), _ptr(xq_codes), _ptr(xq_scales), _ptr(w),
                                       _ptr(wq_codes), _ptr(wq_scales), _ptr(hot_idx), n_hot,
                                       _ptr(y), _ptr(workspace), workspace.numel(),
                                       _stream(stream)))
    return y


HCP_NOALLOC_MAX_BYTES = 64 << 20


def hcp_residual_add_noalloc(x, xq_codes, xq_scales, w, wq_codes, wq_scales, hot_idx, y,
                             stream=None):
    """hcp_residual_add without a workspace (fp4q_hcp_residual_add_noalloc):
    the library's own 64 MiB device scratch holds the gathered operands;
    nothing is allocated.  Calls overlapping on one GPU race."""
    torch = _torch()
    M, N, K = _hcp_operands(x, xq_codes, xq_scales, w, wq_codes, wq_scales, hot_idx)
    _need_cuda(y)
    _need(y, "y", torch.float32, (M, N))
    _check(lib().fp4q_hcp_residual_add_noalloc(M, N, K, _ptr(x), _ptr(xq_codes), _ptr(xq_scales),
                                               _ptr(w), _ptr(wq_codes), _ptr(wq_scales),
                                               _ptr(hot_idx), hot_idx.numel(), _ptr(y),
                                               _stream(stream)))
    return y


def gemm_hcp(x, xq_codes, xq_scales, w, wq_codes, wq_scales, hot_idx, y=None, workspace=None,
             stream=None):
    """Y[M,N] (fp32) = Xq Wq + sum_{c in hot} X[:,c] W[c,:] - Xq[:,c] Wq[c,:], in one GEMM
    kernel (fp4q_gemm_hcp); returns y."""
    torch = _torch()
    M, N, K = _hcp_operands(x, xq_codes, xq_scales, w, wq_codes, wq_scales, hot_idx)
    n_hot = hot_idx.numel()
    if y is None:
        y = torch.empty((M, N), dtype=torch.float32, device=x.device)
    _need_cuda(y)
    _need(y, "y", torch.float32, (M, N), dense=False)
    if y.stride(1) != 1:
        raise ValueError("y must have unit column stride")
    if workspace is None:
        workspace = _scratch(hcp_workspace_bytes(M, N, n_hot), x.device, stream)
    _check(lib().fp4q_gemm_hcp(M, N, K, _ptr(x), _ptr(xq_codes), _ptr(xq_scales), _ptr(w),
                               _ptr(wq_codes), _ptr(wq_scales), _ptr(hot_idx), n_hot, _ptr(y),
                               y.stride(0), _ptr(workspace), workspace.numel(), _stream(stream)))
    return y


def gemm_dge(a_codes, a_scales, b_codes, b_scales, x, k=5.0, clamp_max=3.0, out=None,
             stream=None):
    """out[M,N] (fp32) = deq(A) deq(B)^T times the DGE derivative of x (bf16 [M,N],
    column blocks of 32), in one kernel (fp4q_gemm_dge); returns out."""
    torch = _torch()
    _need_cuda(a_codes, a_scales, b_codes, b_scales, x)
    M, N, K = a_codes.shape[0], b_codes.shape[0], a_codes.shape[1] * 2
    if b_codes.shape[1] * 2 != K:
        raise ValueError("A and B K dimensions differ")
    if tuple(x.shape) != (M, N):
        raise ValueError("x must be [M, N]")
    if out is None:
        out = torch.empty((M, N), dtype=torch.float32, device=a_codes.device)
    _check(lib().fp4q_gemm_dge(M, N, K, _ptr(a_codes), _ptr(a_scales), _ptr(b_codes),
                               _ptr(b_scales), _ptr(x), _dt(x), k, clamp_max, _ptr(out),
                               out.stride(0), _stream(stream)))
    return out


def gemm_quant(a_codes, a_scales, b_codes, b_scales, c=None, write_c=True, out=None,
               stream=None):
    """C = deq(A) deq(B)^T in bf16 (written unless write_c is False) and C's ROW
    block-32 nearest-even quantisation, in one kernel (fp4q_gemm_quant).
    Returns (c or None, (codes, scales))."""
    torch = _torch()
    _need_cuda(a_codes, a_scales, b_codes, b_scales)
    M, N, K = a_codes.shape[0], b_codes.shape[0], a_codes.shape[1] * 2
    if b_codes.shape[1] * 2 != K:
        raise ValueError("A and B K dimensions differ")
    if write_c and c is None:
        c = torch.empty((M, N), dtype=torch.bfloat16, device=a_codes.device)
    if not write_c:
        c = None
    if out is None:
        u8 = dict(dtype=torch.uint8, device=a_codes.device)
        out = (torch.empty((M, N // 2), **u8), torch.empty((M, N // 32), **u8))
    _check(lib().fp4q_gemm_quant(M, N, K, _ptr(a_codes), _ptr(a_scales), _ptr(b_codes),
                                 _ptr(b_scales), _ptr(c), c.stride(0) if c is not None else N,
                                 _ptr(out[0]), _ptr(out[1]), _stream(stream)))
    return c, out


def channel_mask(idx, length, out=None, stream=None):
    """uint32 bit mask over `length` positions with the bits of idx set
    (fp4q_channel_mask); returns the mask tensor."""
    torch = _torch()
    _need_cuda(idx)
    if out is None:
        out = torch.empty(((length + 31) // 32,), dtype=torch.int32, device=idx.device)
    _check(lib().fp4q_channel_mask(_ptr(idx), idx.numel(), length, _ptr(out), _stream(stream)))
    return out


def quantize_masked(x, zero_mask, block=32, axis=ROW, rounding=RNE, seed=0, rng_offset=0,
                    codes=None, scales=None, stream=None):
    """fp4q_quantize of x with the zero_mask positions along the block axis
    taken as zeros (fp4q_quantize_masked); returns (codes, scales)."""
    torch = _torch()
    _need_cuda(x, zero_mask)
    R, C = x.shape
    if codes is None:
        shape_c = (R, C // 2) if axis == ROW else (C, R // 2)
        shape_s = (R, C // block) if axis == ROW else (C, R // block)
        codes = torch.empty(shape_c, dtype=torch.uint8, device=x.device)
        scales = torch.empty(shape_s, dtype=torch.uint8, device=x.device)
    _check(lib().fp4q_quantize_masked(_ptr(x), _dt(x), R, C, x.stride(0), block, axis, rounding,
                                      seed, rng_offset, _ptr(zero_mask), _ptr(codes),
                                      _ptr(scales), _stream(stream)))
    return codes, scales


def gemm_hcp_split(x, xq_codes, xq_scales, w, wq_codes, wq_scales, hot_idx, y=None,
                   workspace=None, stream=None):
    """Y[M,N] (fp32) = Xq' Wq' + X[:, hot] W[hot, :] in one kernel
    (fp4q_gemm_hcp_split; xq, wq quantised with the hot channels zeroed)."""
    torch = _torch()
    M, N, K = _hcp_operands(x, xq_codes, xq_scales, w, wq_codes, wq_scales, hot_idx)
    n_hot = hot_idx.numel()
    if y is None:
        y = torch.empty((M, N), dtype=torch.float32, device=x.device)
    _need_cuda(y)
    _need(y, "y", torch.float32, (M, N), dense=False)
    if y.stride(1) != 1:
        raise ValueError("y must have unit column stride")
    if workspace is None:
        workspace = _scratch(hcp_workspace_bytes(M, N, n_hot), x.device, stream)
    _check(lib().fp4q_gemm_hcp_split(M, N, K, _ptr(x), _ptr(xq_codes), _ptr(xq_scales), _ptr(w),
                                     _ptr(wq_codes), _ptr(wq_scales), _ptr(hot_idx), n_hot,
                                     _ptr(y), y.stride(0), _ptr(workspace), workspace.numel(),
                                     _stream(stream)))
    return y


def hot_channels_workspace_bytes(rows, cols):
    return int(lib().fp4q_hot_channels_workspace_bytes(rows, cols))


def hot_channels(x, n_hot, hot_idx=None, err=None, want_err=False, workspace=None, stream=None):
    """The n_hot channels (columns) of the bf16 x with the largest ROW block-32
    quantisation error, ascending (fp4q_hot_channels).  Returns hot_idx, or
    (hot_idx, err) when want_err (err: fp32 per-channel errors)."""
    torch = _torch()
    _need_cuda(x)
    _need(x, "x", torch.bfloat16, dense=False)
    if x.dim() != 2 or x.stride(1) != 1:
        raise ValueError("x must be 2-D with unit column stride")
    R, C = x.shape
    if hot_idx is None:
        hot_idx = torch.empty((max(n_hot, 0),), dtype=torch.int32, device=x.device)
    _need_cuda(hot_idx)
    _need(hot_idx, "hot_idx", torch.int32)
    if err is None and want_err:
        err = torch.empty((C,), dtype=torch.float32, device=x.device)
    if err is not None:
        _need_cuda(err)
        _need(err, "err", torch.float32, (C,))
    if workspace is None:
        workspace = _scratch(hot_channels_workspace_bytes(R, C), x.device, stream)
    _check(lib().fp4q_hot_channels(_ptr(x), R, C, x.stride(0), n_hot,
                                   _ptr(hot_idx) if n_hot > 0 else None,
                                   _ptr(err) if err is not None else None, _ptr(workspace),
                                   workspace.numel(), _stream(stream)))
    return (hot_idx, err) if want_err else hot_idx


def quantize_2d(x, rounding=RNE, seed=0, rng_offset=0, out=None, stream=None, tile=32):
    """One E8M0 scale per tile x tile square of the bf16 x (fp4q_quantize_2d,
    or fp4q_quantize_2d_tile for tile 16).  Returns (row_codes, row_scales,
    col_codes, col_scales): the same codes in the ROW layout [R, C/2],
    [R, C/tile] and the COL layout [C, R/2], [C, R/tile]."""
    torch = _torch()
    _need_cuda(x)
    R, C = x.shape
    if out is None:
        dev = x.device
        out = (torch.empty((R, C // 2), dtype=torch.uint8, device=dev),
               torch.empty((R, C // tile), dtype=torch.uint8, device=dev),
               torch.empty((C, R // 2), dtype=torch.uint8, device=dev),
               torch.empty((C, R // tile), dtype=torch.uint8, device=dev))
    if tile == 32:
        _check(lib().fp4q_quantize_2d(_ptr(x), R, C, x.stride(0), rounding, seed, rng_offset,
                                      *(_ptr(t) for t in out), _stream(stream)))
    else:
        _check(lib().fp4q_quantize_2d_tile(_ptr(x), R, C, x.stride(0), tile, rounding, seed,
                                           rng_offset, *(_ptr(t) for t in out), _stream(stream)))
    return out


def quantize_rht(x, signs, axis=ROW, rounding=RNE, seed=0, rng_offset=0, codes=None, scales=None,
                 stream=None):
    """Block-32 quantisation of c * H32 * D * x along the block axis
    (fp4q_quantize_rht); signs: int32/uint32 device bit mask over that axis.
    Returns (codes, scales) in the layout of quantize(x, 32, axis)."""
    torch = _torch()
    _need_cuda(x, signs)
    R, C = x.shape
    if codes is None:
        shape_c = (R, C // 2) if axis == ROW else (C, R // 2)
        shape_s = (R, C // 32) if axis == ROW else (C, R // 32)
        codes = torch.empty(shape_c, dtype=torch.uint8, device=x.device)
        scales = torch.empty(shape_s, dtype=torch.uint8, device=x.device)
    _check(lib().fp4q_quantize_rht(_ptr(x), R, C, x.stride(0), axis, _ptr(signs), rounding, seed,
                                   rng_offset, _ptr(codes), _ptr(scales), _stream(stream)))
    return codes, scales


def occ_max_nnz(rows, cols, quantile=0.99):
    return int(lib().fp4q_occ_max_nnz(rows, cols, quantile))


def occ_quantize(x, quantile=0.99, rounding=RNE, seed=0, rng_offset=0, workspace=None,
                 stream=None):
    """Outlier clamping and compensation (fp4q_occ_quantize).  Returns
    (codes, scales, row_ptr, col_idx, vals, threshold): the ROW block-32
    quantisation of the clamped x, the residual in CSR (arrays sized by the
    bound fp4q_occ_max_nnz; row_ptr[-1] entries are used) and T's bf16 bits."""
    torch = _torch()
    _need_cuda(x)
    _need(x, "x", torch.bfloat16, dense=False)
    if x.dim() != 2 or x.stride(1) != 1:
        raise ValueError("x must be 2-D with unit column stride")
    R, C = x.shape
    dev = x.device
    cap = occ_max_nnz(R, C, quantile)
    codes = torch.empty((R, C // 2), dtype=torch.uint8, device=dev)
    scales = torch.empty((R, C // 32), dtype=torch.uint8, device=dev)
    row_ptr = torch.empty((R + 1,), dtype=torch.int64, device=dev)
    col_idx = torch.empty((max(cap, 1),), dtype=torch.int32, device=dev)
    vals = torch.empty((max(cap, 1),), dtype=torch.float32, device=dev)
    thr = torch.empty((8,), dtype=torch.int16, device=dev)
    if workspace is None:
        workspace = _scratch(lib().fp4q_occ_workspace_bytes(R, C), dev, stream)
    _check(lib().fp4q_occ_quantize(_ptr(x), R, C, x.stride(0), quantile, rounding, seed,
                                   rng_offset, _ptr(codes), _ptr(scales), _ptr(row_ptr),
                                   _ptr(col_idx), _ptr(vals), cap, _ptr(thr), _ptr(workspace),
                                   workspace.numel(), _stream(stream)))
    return codes, scales, row_ptr, col_idx, vals, thr[:1]


def occ_spmm(row_ptr, col_idx, vals, w, y, stream=None):
    """y[M, N] (fp32, in place) += R W for the CSR residual R (fp4q_occ_spmm)."""
    torch = _torch()
    _need_cuda(row_ptr, col_idx, vals, w, y)
    _need(row_ptr, "row_ptr", torch.int64)
    _need(col_idx, "col_idx", torch.int32)
    _need(vals, "vals", torch.float32)
    _need(w, "w", torch.bfloat16, dense=False)
    _need(y, "y", torch.float32, dense=False)
    if w.stride(1) != 1 or y.stride(1) != 1:
        raise ValueError("w and y must have unit column stride")
    M, N = y.shape
    K = w.shape[0]
    _check(lib().fp4q_occ_spmm(M, N, K, _ptr(row_ptr), _ptr(col_idx), _ptr(vals), _ptr(w),
                               w.stride(0), _ptr(y), y.stride(0), _stream(stream)))
    return y
