"""Thin ctypes binding of ``libdg_mi355x.so`` (the C ABI in include/dg.h).

Argument marshalling only: every function takes torch tensors that already
live on the current HIP device, checks dtype/shape/contiguity, derives the
sizes and passes raw pointers plus the current torch stream to the library.
All arithmetic runs in the library's HIP kernels.  torch is used only for
device memory and streams.  If the shared library is missing or cannot be
loaded, every call raises: there is no fallback.
"""

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libdg_mi355x.so")

DG_OK = 0
DG_ERR_INVALID_ARG = 1
DG_ERR_SHAPE = 2
DG_ERR_ALIGN = 3
DG_ERR_WORKSPACE = 4
DG_ERR_DEVICE = 5
DG_ERR_LAUNCH = 6

DG_OP_GEMM_NT = 0
DG_OP_CONTIGUOUS = 1
DG_OP_MASKED = 2
DG_OP_BF16_GEMM_NT = 3
DG_OP_GEMM_NT_UE8M0 = 4
DG_OP_K_GROUPED = 5

EXPORTED = (
    "dg_fp8_gemm_nt",
    "dg_fp8_gemm_nt_noalloc",
    "dg_fp8_gemm_nt_acc",
    "dg_bf16_gemm_nt",
    "dg_m_grouped_fp8_gemm_nt_contiguous",
    "dg_m_grouped_fp8_gemm_nt_masked",
    "dg_k_grouped_fp8_gemm_nt_contiguous",
    "dg_quant_1x128",
    "dg_quant_128x128",
    "dg_quant_1x128_ue8m0",
    "dg_quant_128x128_ue8m0",
    "dg_fp8_gemm_nt_ue8m0",
    "dg_m_grouped_fp8_gemm_nt_contiguous_ue8m0",
    "dg_m_grouped_fp8_gemm_nt_masked_ue8m0",
    "dg_get_workspace_size",
    "dg_describe_plan",
    "dg_get_m_alignment_for_contiguous_layout",
    "dg_set_num_cus",
    "dg_get_num_cus",
    "dg_get_last_error",
    "dg_version",
)


class DGError(RuntimeError):
    def __init__(self, code, msg):
        super().__init__(f"dg error {code}: {msg}")
        self.code = code


_lib = None


def load_library():
    """Load (once) and return the ctypes handle of the in-tree library; raises
    if it is missing."""
    global _lib
    if _lib is not None:
        return _lib
    p = LIB_PATH
    if not os.path.exists(p):
        raise RuntimeError(
            f"{p} not found: build it first (python -m moe_grouped_matmul_amd.build); "
            "there is no fallback path")
    lib = ctypes.CDLL(p)
    P, I64, SZ, I = ctypes.c_void_p, ctypes.c_int64, ctypes.c_size_t, ctypes.c_int
    lib.dg_fp8_gemm_nt.argtypes = [P, P, P, P, P, I64, I64, I64, P, SZ, P]
    lib.dg_fp8_gemm_nt_noalloc.argtypes = [P, P, P, P, P, I64, I64, I64, P]
    lib.dg_bf16_gemm_nt.argtypes = [P, P, P, I64, I64, I64, P, SZ, P]
    lib.dg_fp8_gemm_nt_acc.argtypes = [P, P, P, P, P, P, I64, I64, I64, P, SZ, P]
    lib.dg_m_grouped_fp8_gemm_nt_contiguous.argtypes = [P, P, P, P, P, P, I64, I64, I64, I64, P, SZ, P]
    lib.dg_m_grouped_fp8_gemm_nt_masked.argtypes = [P, P, P, P, P, P, I64, I64, I64, I64, I64, P, SZ, P]
    lib.dg_m_grouped_fp8_gemm_nt_contiguous_ue8m0.argtypes = [P, P, P, P, P, P, I64, I64, I64, I64, P, SZ, P]
    lib.dg_m_grouped_fp8_gemm_nt_masked_ue8m0.argtypes = [P, P, P, P, P, P, I64, I64, I64, I64, I64, P, SZ, P]
    lib.dg_k_grouped_fp8_gemm_nt_contiguous.argtypes = [P, P, P, P, P, P, P, I64, I64, I64, I64, P, SZ, P]
    lib.dg_quant_1x128.argtypes = [P, P, P, I64, I64, I64, P]
    lib.dg_quant_128x128.argtypes = [P, P, P, I64, I64, I64, P]
    lib.dg_quant_1x128_ue8m0.argtypes = [P, P, P, I64, I64, I64, P]
    lib.dg_quant_128x128_ue8m0.argtypes = [P, P, P, I64, I64, I64, P]
    lib.dg_fp8_gemm_nt_ue8m0.argtypes = [P, P, P, P, P, I64, I64, I64, P, SZ, P]
    lib.dg_get_workspace_size.argtypes = [I, I64, I64, I64, I64]
    lib.dg_get_workspace_size.restype = SZ
    lib.dg_describe_plan.argtypes = [I, I64, I64, I64, I64]
    lib.dg_describe_plan.restype = ctypes.c_char_p
    lib.dg_get_m_alignment_for_contiguous_layout.argtypes = []
    lib.dg_set_num_cus.argtypes = [I]
    lib.dg_get_num_cus.argtypes = []
    lib.dg_get_last_error.restype = ctypes.c_char_p
    lib.dg_version.restype = ctypes.c_char_p
    for name in ("dg_fp8_gemm_nt", "dg_fp8_gemm_nt_noalloc", "dg_fp8_gemm_nt_acc", "dg_bf16_gemm_nt", "dg_m_grouped_fp8_gemm_nt_contiguous", "dg_m_grouped_fp8_gemm_nt_masked",
                 "dg_k_grouped_fp8_gemm_nt_contiguous", "dg_quant_1x128", "dg_quant_1x128_ue8m0",
                 "dg_quant_128x128_ue8m0", "dg_fp8_gemm_nt_ue8m0", "dg_m_grouped_fp8_gemm_nt_contiguous_ue8m0",
                 "dg_m_grouped_fp8_gemm_nt_masked_ue8m0", "dg_quant_128x128", "dg_set_num_cus", "dg_get_num_cus",
                 "dg_get_m_alignment_for_contiguous_layout"):
        getattr(lib, name).restype = I
    _lib = lib
    return lib


def _check(rc):
    if rc != DG_OK:
        msg = load_library().dg_get_last_error().decode()
        raise DGError(rc, msg)


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else ctypes.c_void_p(0)


def _stream(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _bytes_view(t, name):
    if t.dtype == torch.float8_e4m3fn:
        t = t.view(torch.uint8)
    if t.dtype != torch.uint8:
        raise TypeError(f"{name} must be uint8 or float8_e4m3fn (got {t.dtype})")
    return t


def _need(t, name, dtype, ndim):
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if t.device.index is not None and t.device.index != torch.cuda.current_device():
        raise ValueError(f"{name} is on {t.device}, but the library runs on the current device "
                         f"cuda:{torch.cuda.current_device()}")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype} (got {t.dtype})")
    if t.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dims (got shape {tuple(t.shape)})")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _bf16_out(d, name="D"):
    if d.dtype == torch.bfloat16:
        d = d.view(torch.int16)
    if d.dtype not in (torch.int16, torch.uint16):
        raise TypeError(f"{name} must be bfloat16 (got {d.dtype})")
    return d


def dg_get_workspace_size(op, rows, N, K, G=1):
    return int(load_library().dg_get_workspace_size(op, rows, N, K, G))


def dg_describe_plan(op, rows, N, K, G=1):
    """Text description of the launch plan for op at this shape (DG_OP_GEMM_NT only)."""
    return load_library().dg_describe_plan(op, rows, N, K, G).decode()


def dg_get_m_alignment_for_contiguous_layout():
    return int(load_library().dg_get_m_alignment_for_contiguous_layout())


def dg_set_num_cus(n):
    _check(load_library().dg_set_num_cus(int(n)))


def dg_get_num_cus():
    return int(load_library().dg_get_num_cus())


def dg_version():
    return load_library().dg_version().decode()


def dg_fp8_gemm_nt(A, sfa, B, sfb, D, workspace=None, stream=None):
    """D[M,N] (bf16, written) = A[M,K] . B[N,K]^T with sfa [K/128, M], sfb [ceil(N/128), K/128]."""
    A = _bytes_view(A, "A")
    B = _bytes_view(B, "B")
    D = _bf16_out(D)
    _need(A, "A", torch.uint8, 2)
    _need(B, "B", torch.uint8, 2)
    _need(sfa, "sfa", torch.float32, 2)
    _need(sfb, "sfb", torch.float32, 2)
    _need(D, "D", D.dtype, 2)
    M, K = A.shape
    N = B.shape[0]
    if B.shape[1] != K or tuple(sfa.shape) != (K // 128, M) or tuple(sfb.shape) != ((N + 127) // 128, K // 128) \
            or tuple(D.shape) != (M, N):
        raise ValueError("shape mismatch between A, sfa, B, sfb, D")
    ws_bytes = 0
    if workspace is not None:
        _need(workspace, "workspace", workspace.dtype, workspace.dim())
        ws_bytes = workspace.numel() * workspace.element_size()
    _check(load_library().dg_fp8_gemm_nt(_ptr(A), _ptr(sfa), _ptr(B), _ptr(sfb), _ptr(D), M, N, K,
                                         _ptr(workspace), ws_bytes, _stream(stream)))


def dg_fp8_gemm_nt_noalloc(A, sfa, B, sfb, D, stream=None):
    """dg_fp8_gemm_nt without a workspace argument: the split-K scratch is the
    library's static per-device array (calls that overlap on one GPU race)."""
    A = _bytes_view(A, "A")
    B = _bytes_view(B, "B")
    D = _bf16_out(D)
    _need(A, "A", torch.uint8, 2)
    _need(B, "B", torch.uint8, 2)
    _need(sfa, "sfa", torch.float32, 2)
    _need(sfb, "sfb", torch.float32, 2)
    _need(D, "D", D.dtype, 2)
    M, K = A.shape
    N = B.shape[0]
    if B.shape[1] != K or tuple(sfa.shape) != (K // 128, M) or tuple(sfb.shape) != ((N + 127) // 128, K // 128) \
            or tuple(D.shape) != (M, N):
        raise ValueError("shape mismatch between A, sfa, B, sfb, D")
    _check(load_library().dg_fp8_gemm_nt_noalloc(_ptr(A), _ptr(sfa), _ptr(B), _ptr(sfb), _ptr(D), M, N, K,
                                                 _stream(stream)))


def dg_fp8_gemm_nt_acc(A, sfa, B, sfb, C, D, workspace=None, stream=None):
    """D[M,N] (fp32, written) = C[M,N] (fp32, or None for zeros; may be D) + A[M,K] . B[N,K]^T."""
    A = _bytes_view(A, "A")
    B = _bytes_view(B, "B")
    _need(A, "A", torch.uint8, 2)
    _need(B, "B", torch.uint8, 2)
    _need(sfa, "sfa", torch.float32, 2)
    _need(sfb, "sfb", torch.float32, 2)
    _need(D, "D", torch.float32, 2)
    if C is not None:
        _need(C, "C", torch.float32, 2)
    M, K = A.shape
    N = B.shape[0]
    if B.shape[1] != K or tuple(sfa.shape) != (K // 128, M) or tuple(sfb.shape) != ((N + 127) // 128, K // 128) \
            or tuple(D.shape) != (M, N) or (C is not None and tuple(C.shape) != (M, N)):
        raise ValueError("shape mismatch between A, sfa, B, sfb, C, D")
    ws_bytes = 0
    if workspace is not None:
        _need(workspace, "workspace", workspace.dtype, workspace.dim())
        ws_bytes = workspace.numel() * workspace.element_size()
    _check(load_library().dg_fp8_gemm_nt_acc(_ptr(A), _ptr(sfa), _ptr(B), _ptr(sfb), _ptr(C), _ptr(D), M, N, K,
                                             _ptr(workspace), ws_bytes, _stream(stream)))


def dg_bf16_gemm_nt(A, B, D, workspace=None, stream=None):
    """D[M,N] (bf16, written) = A[M,K] . B[N,K]^T, all bf16 (int16/uint16 bit views accepted)."""
    A = _bf16_out(A, "A")
    B = _bf16_out(B, "B")
    D = _bf16_out(D)
    for t, n in ((A, "A"), (B, "B"), (D, "D")):
        _need(t, n, t.dtype, 2)
    M, K = A.shape
    N = B.shape[0]
    if B.shape[1] != K or tuple(D.shape) != (M, N):
        raise ValueError("shape mismatch between A, B, D")
    ws_bytes = 0
    if workspace is not None:
        _need(workspace, "workspace", workspace.dtype, workspace.dim())
        ws_bytes = workspace.numel() * workspace.element_size()
    _check(load_library().dg_bf16_gemm_nt(_ptr(A), _ptr(B), _ptr(D), M, N, K, _ptr(workspace), ws_bytes,
                                          _stream(stream)))


def dg_m_grouped_fp8_gemm_nt_contiguous(A, sfa, B, sfb, D, m_indices, stream=None):
    """M-grouped contiguous: A [M_total,K], sfa [K/128,M_total], B [G,N,K], sfb [G,ceil(N/128),K/128],
    D [M_total,N] bf16, m_indices [M_total] int32 (-1 = padding row, not written)."""
    A = _bytes_view(A, "A")
    B = _bytes_view(B, "B")
    D = _bf16_out(D)
    _need(A, "A", torch.uint8, 2)
    _need(B, "B", torch.uint8, 3)
    _need(sfa, "sfa", torch.float32, 2)
    _need(sfb, "sfb", torch.float32, 3)
    _need(D, "D", D.dtype, 2)
    _need(m_indices, "m_indices", torch.int32, 1)
    M_total, K = A.shape
    G, N, _ = B.shape
    if B.shape[2] != K or tuple(sfa.shape) != (K // 128, M_total) \
            or tuple(sfb.shape) != (G, (N + 127) // 128, K // 128) or tuple(D.shape) != (M_total, N) \
            or m_indices.shape[0] != M_total:
        raise ValueError("shape mismatch between A, sfa, B, sfb, D, m_indices")
    _check(load_library().dg_m_grouped_fp8_gemm_nt_contiguous(
        _ptr(A), _ptr(sfa), _ptr(B), _ptr(sfb), _ptr(D), _ptr(m_indices), M_total, N, K, G,
        ctypes.c_void_p(0), 0, _stream(stream)))


def dg_m_grouped_fp8_gemm_nt_masked(A, sfa, B, sfb, D, masked_m, expected_m=0, stream=None):
    """M-grouped masked: A [G,max_m,K], sfa [G,K/128,max_m], B [G,N,K], sfb [G,ceil(N/128),K/128],
    D [G,max_m,N] bf16, masked_m [G] int32 on device (rows past it are not written)."""
    A = _bytes_view(A, "A")
    B = _bytes_view(B, "B")
    D = _bf16_out(D)
    _need(A, "A", torch.uint8, 3)
    _need(B, "B", torch.uint8, 3)
    _need(sfa, "sfa", torch.float32, 3)
    _need(sfb, "sfb", torch.float32, 3)
    _need(D, "D", D.dtype, 3)
    _need(masked_m, "masked_m", torch.int32, 1)
    G, max_m, K = A.shape
    N = B.shape[1]
    if B.shape[0] != G or B.shape[2] != K or tuple(sfa.shape) != (G, K // 128, max_m) \
            or tuple(sfb.shape) != (G, (N + 127) // 128, K // 128) or tuple(D.shape) != (G, max_m, N) \
            or masked_m.shape[0] != G:
        raise ValueError("shape mismatch between A, sfa, B, sfb, D, masked_m")
    _check(load_library().dg_m_grouped_fp8_gemm_nt_masked(
        _ptr(A), _ptr(sfa), _ptr(B), _ptr(sfb), _ptr(D), _ptr(masked_m), G, max_m, N, K, int(expected_m),
        ctypes.c_void_p(0), 0, _stream(stream)))


def dg_k_grouped_fp8_gemm_nt_contiguous(A, sfa, B, sfb, C, D, ks, stream=None):
    """K-grouped contiguous: A [M,K], sfa [K/128,M], B [N,K], sfb [K/128,N] (per-row scales on both),
    ks [G] int32 on device (K length of each group, multiples of 128), C [G,M,N] fp32 or None (zeros;
    may be D), D [G,M,N] fp32 written: D[g] = C[g] + A[:, seg g] . B[:, seg g]^T."""
    A = _bytes_view(A, "A")
    B = _bytes_view(B, "B")
    _need(A, "A", torch.uint8, 2)
    _need(B, "B", torch.uint8, 2)
    _need(sfa, "sfa", torch.float32, 2)
    _need(sfb, "sfb", torch.float32, 2)
    _need(D, "D", torch.float32, 3)
    _need(ks, "ks", torch.int32, 1)
    if C is not None:
        _need(C, "C", torch.float32, 3)
    M, K = A.shape
    N = B.shape[0]
    G = ks.shape[0]
    if B.shape[1] != K or tuple(sfa.shape) != (K // 128, M) or tuple(sfb.shape) != (K // 128, N) \
            or tuple(D.shape) != (G, M, N) or (C is not None and tuple(C.shape) != (G, M, N)):
        raise ValueError("shape mismatch between A, sfa, B, sfb, C, D, ks")
    _check(load_library().dg_k_grouped_fp8_gemm_nt_contiguous(
        _ptr(A), _ptr(sfa), _ptr(B), _ptr(sfb), _ptr(C), _ptr(D), _ptr(ks), G, M, N, K,
        ctypes.c_void_p(0), 0, _stream(stream)))


def dg_quant_1x128(x, q, sfa, stream=None):
    """x [M,K] or [G,M,K] fp32 -> q (uint8, same shape), sfa [(G,) K/128, M] fp32."""
    q = _bytes_view(q, "q")
    _need(x, "x", torch.float32, x.dim())
    _need(q, "q", torch.uint8, x.dim())
    _need(sfa, "sfa", torch.float32, x.dim())
    if x.dim() == 2:
        G, (M, K) = 1, x.shape
    elif x.dim() == 3:
        G, M, K = x.shape
    else:
        raise ValueError("x must be [M,K] or [G,M,K]")
    exp_s = (K // 128, M) if x.dim() == 2 else (G, K // 128, M)
    if tuple(q.shape) != tuple(x.shape) or tuple(sfa.shape) != exp_s:
        raise ValueError("shape mismatch between x, q, sfa")
    _check(load_library().dg_quant_1x128(_ptr(x), _ptr(q), _ptr(sfa), G, M, K, _stream(stream)))


def dg_quant_128x128(x, q, sfb, stream=None):
    """x [N,K] or [G,N,K] fp32 -> q (uint8, same shape), sfb [(G,) ceil(N/128), K/128] fp32."""
    q = _bytes_view(q, "q")
    _need(x, "x", torch.float32, x.dim())
    _need(q, "q", torch.uint8, x.dim())
    _need(sfb, "sfb", torch.float32, x.dim())
    if x.dim() == 2:
        G, (N, K) = 1, x.shape
    elif x.dim() == 3:
        G, N, K = x.shape
    else:
        raise ValueError("x must be [N,K] or [G,N,K]")
    exp_s = ((N + 127) // 128, K // 128) if x.dim() == 2 else (G, (N + 127) // 128, K // 128)
    if tuple(q.shape) != tuple(x.shape) or tuple(sfb.shape) != exp_s:
        raise ValueError("shape mismatch between x, q, sfb")
    _check(load_library().dg_quant_128x128(_ptr(x), _ptr(q), _ptr(sfb), G, N, K, _stream(stream)))


def _kw(K):
    return (K // 128 + 3) // 4


def dg_quant_1x128_ue8m0(x, q, sfa, stream=None):
    """x [M,K] or [G,M,K] fp32 -> q (uint8, same shape), sfa [(G,) ceil(K/512), M] int32 (UE8M0
    codes of four K blocks per word, block 4w+j in byte j)."""
    q = _bytes_view(q, "q")
    _need(x, "x", torch.float32, x.dim())
    _need(q, "q", torch.uint8, x.dim())
    _need(sfa, "sfa", torch.int32, x.dim())
    if x.dim() == 2:
        G, (M, K) = 1, x.shape
    elif x.dim() == 3:
        G, M, K = x.shape
    else:
        raise ValueError("x must be [M,K] or [G,M,K]")
    exp_s = (_kw(K), M) if x.dim() == 2 else (G, _kw(K), M)
    if tuple(q.shape) != tuple(x.shape) or tuple(sfa.shape) != exp_s:
        raise ValueError("shape mismatch between x, q, sfa")
    _check(load_library().dg_quant_1x128_ue8m0(_ptr(x), _ptr(q), _ptr(sfa), G, M, K, _stream(stream)))


def dg_quant_128x128_ue8m0(x, q, sfb, stream=None):
    """x [N,K] or [G,N,K] fp32 -> q (uint8, same shape), sfb [(G,) ceil(N/128), ceil(K/512)] int32
    (UE8M0 codes, four K blocks per word)."""
    q = _bytes_view(q, "q")
    _need(x, "x", torch.float32, x.dim())
    _need(q, "q", torch.uint8, x.dim())
    _need(sfb, "sfb", torch.int32, x.dim())
    if x.dim() == 2:
        G, (N, K) = 1, x.shape
    elif x.dim() == 3:
        G, N, K = x.shape
    else:
        raise ValueError("x must be [N,K] or [G,N,K]")
    exp_s = ((N + 127) // 128, _kw(K)) if x.dim() == 2 else (G, (N + 127) // 128, _kw(K))
    if tuple(q.shape) != tuple(x.shape) or tuple(sfb.shape) != exp_s:
        raise ValueError("shape mismatch between x, q, sfb")
    _check(load_library().dg_quant_128x128_ue8m0(_ptr(x), _ptr(q), _ptr(sfb), G, N, K, _stream(stream)))


def dg_fp8_gemm_nt_ue8m0(A, sfa, B, sfb, D, workspace=None, stream=None):
    """D[M,N] (bf16, written) = A[M,K] . B[N,K]^T with packed UE8M0 scales: sfa [ceil(K/512), M] int32,
    sfb [ceil(N/128), ceil(K/512)] int32."""
    A = _bytes_view(A, "A")
    B = _bytes_view(B, "B")
    D = _bf16_out(D)
    _need(A, "A", torch.uint8, 2)
    _need(B, "B", torch.uint8, 2)
    _need(sfa, "sfa", torch.int32, 2)
    _need(sfb, "sfb", torch.int32, 2)
    _need(D, "D", D.dtype, 2)
    M, K = A.shape
    N = B.shape[0]
    if B.shape[1] != K or tuple(sfa.shape) != (_kw(K), M) or tuple(sfb.shape) != ((N + 127) // 128, _kw(K)) \
            or tuple(D.shape) != (M, N):
        raise ValueError("shape mismatch between A, sfa, B, sfb, D")
    ws_bytes = 0
    if workspace is not None:
        _need(workspace, "workspace", workspace.dtype, workspace.dim())
        ws_bytes = workspace.numel() * workspace.element_size()
    _check(load_library().dg_fp8_gemm_nt_ue8m0(_ptr(A), _ptr(sfa), _ptr(B), _ptr(sfb), _ptr(D), M, N, K,
                                               _ptr(workspace), ws_bytes, _stream(stream)))


def dg_m_grouped_fp8_gemm_nt_contiguous_ue8m0(A, sfa, B, sfb, D, m_indices, stream=None):
    """M-grouped contiguous with packed UE8M0 scales: A [M_total,K], sfa [ceil(K/512),M_total] int32,
    B [G,N,K], sfb [G,ceil(N/128),ceil(K/512)] int32, D [M_total,N] bf16, m_indices [M_total] int32."""
    A = _bytes_view(A, "A")
    B = _bytes_view(B, "B")
    D = _bf16_out(D)
    _need(A, "A", torch.uint8, 2)
    _need(B, "B", torch.uint8, 3)
    _need(sfa, "sfa", torch.int32, 2)
    _need(sfb, "sfb", torch.int32, 3)
    _need(D, "D", D.dtype, 2)
    _need(m_indices, "m_indices", torch.int32, 1)
    M_total, K = A.shape
    G, N, _ = B.shape
    if B.shape[2] != K or tuple(sfa.shape) != (_kw(K), M_total) or tuple(sfb.shape) != (G, (N + 127) // 128, _kw(K)) \
            or tuple(D.shape) != (M_total, N) or m_indices.shape[0] != M_total:
        raise ValueError("shape mismatch between A, sfa, B, sfb, D, m_indices")
    _check(load_library().dg_m_grouped_fp8_gemm_nt_contiguous_ue8m0(
        _ptr(A), _ptr(sfa), _ptr(B), _ptr(sfb), _ptr(D), _ptr(m_indices), M_total, N, K, G,
        ctypes.c_void_p(0), 0, _stream(stream)))


def dg_m_grouped_fp8_gemm_nt_masked_ue8m0(A, sfa, B, sfb, D, masked_m, expected_m=0, stream=None):
    """M-grouped masked with packed UE8M0 scales: A [G,max_m,K], sfa [G,ceil(K/512),max_m] int32,
    B [G,N,K], sfb [G,ceil(N/128),ceil(K/512)] int32, D [G,max_m,N] bf16, masked_m [G] int32."""
    A = _bytes_view(A, "A")
    B = _bytes_view(B, "B")
    D = _bf16_out(D)
    _need(A, "A", torch.uint8, 3)
    _need(B, "B", torch.uint8, 3)
    _need(sfa, "sfa", torch.int32, 3)
    _need(sfb, "sfb", torch.int32, 3)
    _need(D, "D", D.dtype, 3)
    _need(masked_m, "masked_m", torch.int32, 1)
    G, max_m, K = A.shape
    N = B.shape[1]
    if B.shape[0] != G or B.shape[2] != K or tuple(sfa.shape) != (G, _kw(K), max_m) \
            or tuple(sfb.shape) != (G, (N + 127) // 128, _kw(K)) or tuple(D.shape) != (G, max_m, N) \
            or masked_m.shape[0] != G:
        raise ValueError("shape mismatch between A, sfa, B, sfb, D, masked_m")
    _check(load_library().dg_m_grouped_fp8_gemm_nt_masked_ue8m0(
        _ptr(A), _ptr(sfa), _ptr(B), _ptr(sfb), _ptr(D), _ptr(masked_m), G, max_m, N, K, int(expected_m),
        ctypes.c_void_p(0), 0, _stream(stream)))
