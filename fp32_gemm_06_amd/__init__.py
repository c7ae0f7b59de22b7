"""Python binding of libfp32gemm.so (fp32 SGEMM / small-M SGEMV for MI355X).

Argument marshalling only: every step of the computation runs in the HIP
kernels of the shared library.  The functions with the C names (``sgemm``,
``sgemv``, ``fp32gemm_*``) take the same arguments as the C entry points,
with device pointers given as ints or torch tensors, and return the C return
code.  ``gemm`` is a torch-tensor convenience wrapper that raises on error.

PyTorch serves only for device memory and streams.  The library must be built
(``python -m fp32_gemm_06_amd.build``); there is no fallback of any kind when
it is missing.
"""
from __future__ import annotations

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libfp32gemm.so")
_lib = None

KIND_SGEMM = 0
KIND_SGEMV = 1
ERR_CONFIG = -100
ERR_SCRATCH = -101

_GEMM_ARGTYPES = [ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_float,
                  ctypes.c_void_p, ctypes.c_int, ctypes.c_void_p, ctypes.c_int,
                  ctypes.c_float, ctypes.c_void_p, ctypes.c_int, ctypes.c_void_p]

OP_N = 0
OP_T = 1

_EX_ARGTYPES = [ctypes.c_int, ctypes.c_int] + _GEMM_ARGTYPES
_BATCHED_ARGTYPES = [ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                     ctypes.c_float, ctypes.c_void_p, ctypes.c_int, ctypes.c_longlong,
                     ctypes.c_void_p, ctypes.c_int, ctypes.c_longlong, ctypes.c_float,
                     ctypes.c_void_p, ctypes.c_int, ctypes.c_longlong, ctypes.c_int,
                     ctypes.c_void_p]

_FUSED_ARGTYPES = _EX_ARGTYPES[:-1] + [ctypes.c_void_p, ctypes.c_int, ctypes.c_void_p]
ACT_NONE = 0
ACT_RELU = 1
_SPLITK_ARGTYPES = _EX_ARGTYPES[:-1] + [ctypes.c_int, ctypes.c_void_p, ctypes.c_size_t,
                                        ctypes.c_void_p]
_SPLITK_NOALLOC_ARGTYPES = _EX_ARGTYPES[:-1] + [ctypes.c_int, ctypes.c_void_p]
_STREAMK_ARGTYPES = _EX_ARGTYPES[:-1] + [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p]

# Every symbol include/fp32gemm.h declares.
EXPORTS = ("sgemm", "sgemv", "sgemm_ex", "sgemm_strided_batched", "sgemm_fused", "sgemm_splitk",
           "sgemm_splitk_noalloc", "sgemm_splitk_workspace_size", "fp32gemm_splitk_splits",
           "sgemm_streamk", "sgemm_streamk_workspace_size", "fp32gemm_streamk_tile_name",
           "fp32gemm_streamk_plan", "fp32gemm_streamk_with_config", "fp32gemm_strerror",
           "fp32gemm_num_configs", "fp32gemm_config_name", "fp32gemm_select_config",
           "fp32gemm_config_max_rows", "fp32gemm_round_split", "fp32gemm_sgemm_with_config",
           "fp32gemm_sgemv_with_config")


class Fp32GemmError(RuntimeError):
    def __init__(self, code: int):
        super().__init__(f"fp32gemm error {code}: {strerror(code)}")
        self.code = code


def lib():
    """Load the built library (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is not built; run `python -m fp32_gemm_06_amd.build`")
        # torch brings its own HIP runtime.  Loaded first, it is the one the
        # library binds to (same soname); loaded after the library, it would
        # be a second runtime in the process, and whichever of the two opens
        # the GPU second finds no device.  So torch goes first.
        import torch  # noqa: F401
        L = ctypes.CDLL(LIB_PATH)
        L.sgemm.argtypes = _GEMM_ARGTYPES
        L.sgemm.restype = ctypes.c_int
        L.sgemv.argtypes = _GEMM_ARGTYPES
        L.sgemv.restype = ctypes.c_int
        L.sgemm_ex.argtypes = _EX_ARGTYPES
        L.sgemm_ex.restype = ctypes.c_int
        L.sgemm_strided_batched.argtypes = _BATCHED_ARGTYPES
        L.sgemm_strided_batched.restype = ctypes.c_int
        L.sgemm_fused.argtypes = _FUSED_ARGTYPES
        L.sgemm_fused.restype = ctypes.c_int
        L.sgemm_splitk.argtypes = _SPLITK_ARGTYPES
        L.sgemm_splitk.restype = ctypes.c_int
        L.sgemm_splitk_noalloc.argtypes = _SPLITK_NOALLOC_ARGTYPES
        L.sgemm_splitk_noalloc.restype = ctypes.c_int
        L.sgemm_streamk.argtypes = _STREAMK_ARGTYPES
        L.sgemm_streamk.restype = ctypes.c_int
        L.sgemm_streamk_workspace_size.argtypes = [ctypes.c_int] * 3
        L.sgemm_streamk_workspace_size.restype = ctypes.c_size_t
        L.fp32gemm_streamk_tile_name.argtypes = [ctypes.c_int]
        L.fp32gemm_streamk_tile_name.restype = ctypes.c_char_p
        L.fp32gemm_streamk_plan.argtypes = [ctypes.c_int] * 5 + [ctypes.POINTER(ctypes.c_int)] * 3
        L.fp32gemm_streamk_plan.restype = ctypes.c_size_t
        L.fp32gemm_streamk_with_config.argtypes = [ctypes.c_int, ctypes.c_int] + _STREAMK_ARGTYPES
        L.fp32gemm_streamk_with_config.restype = ctypes.c_int
        L.sgemm_splitk_workspace_size.argtypes = [ctypes.c_int] * 4
        L.sgemm_splitk_workspace_size.restype = ctypes.c_size_t
        L.fp32gemm_splitk_splits.argtypes = [ctypes.c_int] * 3
        L.fp32gemm_splitk_splits.restype = ctypes.c_int
        L.fp32gemm_strerror.argtypes = [ctypes.c_int]
        L.fp32gemm_strerror.restype = ctypes.c_char_p
        L.fp32gemm_num_configs.argtypes = [ctypes.c_int]
        L.fp32gemm_num_configs.restype = ctypes.c_int
        L.fp32gemm_config_name.argtypes = [ctypes.c_int, ctypes.c_int]
        L.fp32gemm_config_name.restype = ctypes.c_char_p
        L.fp32gemm_select_config.argtypes = [ctypes.c_int] * 4
        L.fp32gemm_select_config.restype = ctypes.c_int
        L.fp32gemm_config_max_rows.argtypes = [ctypes.c_int, ctypes.c_int]
        L.fp32gemm_config_max_rows.restype = ctypes.c_int
        L.fp32gemm_round_split.argtypes = [ctypes.c_int] * 4 + [ctypes.POINTER(ctypes.c_int)]
        L.fp32gemm_round_split.restype = ctypes.c_int
        L.fp32gemm_sgemm_with_config.argtypes = [ctypes.c_int] + _GEMM_ARGTYPES
        L.fp32gemm_sgemm_with_config.restype = ctypes.c_int
        L.fp32gemm_sgemv_with_config.argtypes = [ctypes.c_int] + _GEMM_ARGTYPES
        L.fp32gemm_sgemv_with_config.restype = ctypes.c_int
        _lib = L
    return _lib


def _addr(x):
    """Device address of a tensor / int / None."""
    if x is None:
        return None
    if isinstance(x, int):
        return x
    return x.data_ptr()


def _stream(stream):
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def sgemm(M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, stream=None) -> int:
    """C <- alpha A B + beta C (row-major fp32); returns the C return code."""
    return lib().sgemm(M, N, K, alpha, _addr(A), lda, _addr(B), ldb, beta, _addr(C), ldc,
                       _stream(stream))


def sgemv(M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, stream=None) -> int:
    """Same operation for 1 <= M <= 128 (decode shapes: GEMV kernels up to
    M = 8, the skinny MFMA kernel above); returns the C return code."""
    return lib().sgemv(M, N, K, alpha, _addr(A), lda, _addr(B), ldb, beta, _addr(C), ldc,
                       _stream(stream))


def sgemm_ex(transA, transB, M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, stream=None) -> int:
    """C <- alpha op(A) op(B) + beta C with op = identity (0) or transpose (1)."""
    return lib().sgemm_ex(transA, transB, M, N, K, alpha, _addr(A), lda, _addr(B), ldb, beta,
                          _addr(C), ldc, _stream(stream))


def sgemm_strided_batched(transA, transB, M, N, K, alpha, A, lda, strideA, B, ldb, strideB,
                          beta, C, ldc, strideC, batch_count, stream=None) -> int:
    """batch_count products with element strides between the entries."""
    return lib().sgemm_strided_batched(transA, transB, M, N, K, alpha, _addr(A), lda, strideA,
                                       _addr(B), ldb, strideB, beta, _addr(C), ldc, strideC,
                                       batch_count, _stream(stream))


def sgemm_fused(transA, transB, M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, bias, act,
                stream=None) -> int:
    """C <- act(alpha op(A) op(B) + beta C + bias[None, :]); bias may be None,
    act is ACT_NONE or ACT_RELU."""
    return lib().sgemm_fused(transA, transB, M, N, K, alpha, _addr(A), lda, _addr(B), ldb, beta,
                             _addr(C), ldc, _addr(bias), act, _stream(stream))


def sgemm_splitk(transA, transB, M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, splits,
                 workspace, workspace_bytes, stream=None) -> int:
    """sgemm_ex computed as K chunks plus a fixed-order reduction; the caller
    provides the workspace (sgemm_splitk_workspace_size bytes)."""
    return lib().sgemm_splitk(transA, transB, M, N, K, alpha, _addr(A), lda, _addr(B), ldb, beta,
                              _addr(C), ldc, splits, _addr(workspace), workspace_bytes,
                              _stream(stream))


def sgemm_splitk_noalloc(transA, transB, M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, splits,
                         stream=None) -> int:
    """sgemm_splitk with the partial products in the library's static
    device scratch (no allocation; at most 4 Mi floats of partials)."""
    return lib().sgemm_splitk_noalloc(transA, transB, M, N, K, alpha, _addr(A), lda, _addr(B),
                                      ldb, beta, _addr(C), ldc, splits, _stream(stream))


def sgemm_streamk(transA, transB, M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, workspace,
                  workspace_bytes, stream=None) -> int:
    """sgemm_ex as one stream-K grid; the caller provides the workspace
    (sgemm_streamk_workspace_size bytes)."""
    return lib().sgemm_streamk(transA, transB, M, N, K, alpha, _addr(A), lda, _addr(B), ldb, beta,
                               _addr(C), ldc, _addr(workspace), workspace_bytes, _stream(stream))


def sgemm_streamk_workspace_size(M, N, K) -> int:
    return lib().sgemm_streamk_workspace_size(M, N, K)


def fp32gemm_streamk_tile_name(tile: int):
    s = lib().fp32gemm_streamk_tile_name(tile)
    return None if s is None else s.decode()


def fp32gemm_streamk_plan(M, N, K, tile=-1, groups=0):
    """(workspace bytes, tile, workgroups, K slices per workgroup) of the
    stream-K plan for this shape (tile -1 / groups 0: the library's choice)."""
    t, g, i = ctypes.c_int(-1), ctypes.c_int(0), ctypes.c_int(0)
    b = lib().fp32gemm_streamk_plan(M, N, K, tile, groups, ctypes.byref(t), ctypes.byref(g),
                                    ctypes.byref(i))
    return b, t.value, g.value, i.value


def fp32gemm_streamk_with_config(tile, groups, transA, transB, M, N, K, alpha, A, lda, B, ldb,
                                 beta, C, ldc, workspace, workspace_bytes, stream=None) -> int:
    return lib().fp32gemm_streamk_with_config(tile, groups, transA, transB, M, N, K, alpha,
                                              _addr(A), lda, _addr(B), ldb, beta, _addr(C), ldc,
                                              _addr(workspace), workspace_bytes, _stream(stream))


def sgemm_splitk_workspace_size(M, N, K, splits=0) -> int:
    """Workspace bytes sgemm_splitk needs (0 when it runs as one chunk)."""
    return lib().sgemm_splitk_workspace_size(M, N, K, splits)


def fp32gemm_splitk_splits(M, N, K) -> int:
    """The number of K chunks sgemm_splitk uses when splits = 0."""
    return lib().fp32gemm_splitk_splits(M, N, K)


def fp32gemm_sgemm_with_config(cfg, M, N, K, alpha, A, lda, B, ldb, beta, C, ldc,
                               stream=None) -> int:
    return lib().fp32gemm_sgemm_with_config(cfg, M, N, K, alpha, _addr(A), lda, _addr(B), ldb,
                                            beta, _addr(C), ldc, _stream(stream))


def fp32gemm_sgemv_with_config(cfg, M, N, K, alpha, A, lda, B, ldb, beta, C, ldc,
                               stream=None) -> int:
    return lib().fp32gemm_sgemv_with_config(cfg, M, N, K, alpha, _addr(A), lda, _addr(B), ldb,
                                            beta, _addr(C), ldc, _stream(stream))


def fp32gemm_strerror(code: int) -> str:
    return lib().fp32gemm_strerror(code).decode()


strerror = fp32gemm_strerror


def fp32gemm_num_configs(kind: int) -> int:
    return lib().fp32gemm_num_configs(kind)


def fp32gemm_config_name(kind: int, cfg: int):
    s = lib().fp32gemm_config_name(kind, cfg)
    return None if s is None else s.decode()


def fp32gemm_select_config(kind: int, M: int, N: int, K: int) -> int:
    return lib().fp32gemm_select_config(kind, M, N, K)


def fp32gemm_config_max_rows(kind: int, cfg: int) -> int:
    """The largest M a configuration runs (-1 for an unknown id)."""
    return lib().fp32gemm_config_max_rows(kind, cfg)


def fp32gemm_round_split(M: int, N: int, K: int, batch: int = 1):
    """(dim, first): how the tiled kernel splits this product into two launches
    (0 = one launch, 1 = columns [0, first) then the rest, 2 = the same over rows)."""
    first = ctypes.c_int(0)
    dim = lib().fp32gemm_round_split(M, N, K, batch, ctypes.byref(first))
    return dim, first.value


def config_names(kind: int):
    return [fp32gemm_config_name(kind, i) for i in range(fp32gemm_num_configs(kind))]


def _layout(t, name, allow_transposed=True):
    """(transposed, leading dimension) of a 2-D float32 GPU tensor that is
    row-major (unit column stride) or, when allowed, a transposed view of a
    row-major matrix (unit row stride)."""
    import torch
    if t.dtype != torch.float32:
        raise TypeError(f"{name} must be float32")
    if t.dim() != 2:
        raise ValueError(f"{name} must be 2-D")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be a GPU tensor")
    r, c = t.shape
    if c <= 1 or t.stride(1) == 1:
        return 0, (t.stride(0) if r > 1 else max(1, c))
    if allow_transposed and (r <= 1 or t.stride(0) == 1):
        return 1, (t.stride(1) if c > 1 else max(1, r))
    raise ValueError(f"{name} must be row-major or a transposed view of a row-major matrix")


def gemm(A, B, C=None, alpha: float = 1.0, beta: float = 0.0, config: int | None = None,
         stream=None, bias=None, act: int | str | None = None):
    """Torch wrapper: returns C = act(alpha A @ B + beta C + bias) (C allocated
    when None).

    A and B may be row-major or transposed views of row-major matrices
    (``W.t()`` of a stored N x K weight); C must be row-major.  ``bias`` (N
    floats) and ``act`` ("relu" or ACT_RELU) select the fused epilogue.
    ``config`` forces a configuration of the SGEMM family (``sgemv`` family
    when ``A`` has at most 8 rows and ``config`` is given as ("gemv", id));
    it needs row-major A and B and no epilogue.
    """
    import torch
    M, K = A.shape
    K2, N = B.shape
    if K2 != K:
        raise ValueError(f"inner dimensions differ: {A.shape} @ {B.shape}")
    if C is None:
        C = torch.empty((M, N), dtype=torch.float32, device=A.device)
        if beta != 0.0:
            raise ValueError("beta != 0 needs C")
    if tuple(C.shape) != (M, N):
        raise ValueError(f"C has shape {tuple(C.shape)}, expected {(M, N)}")
    ta, lda = _layout(A, "A")
    tb, ldb = _layout(B, "B")
    _, ldc = _layout(C, "C", allow_transposed=False)
    if act in (None, "none"):
        act = ACT_NONE
    elif act == "relu":
        act = ACT_RELU
    if bias is not None:
        if tuple(bias.shape) != (N,) or bias.dtype != torch.float32 or not bias.is_contiguous():
            raise ValueError(f"bias must be a contiguous float32 vector of {N} values")
    fused = bias is not None or act != ACT_NONE
    if config is not None:
        if ta or tb or fused:
            raise ValueError("a forced configuration needs row-major A and B and no epilogue")
        args = (M, N, K, float(alpha), A, lda, B, ldb, float(beta), C, ldc, stream)
        if isinstance(config, tuple) and config[0] == "gemv":
            rc = fp32gemm_sgemv_with_config(config[1], *args)
        else:
            rc = fp32gemm_sgemm_with_config(int(config), *args)
    elif fused:
        rc = sgemm_fused(ta, tb, M, N, K, float(alpha), A, lda, B, ldb, float(beta), C, ldc,
                         bias, int(act), stream)
    elif ta or tb:
        rc = sgemm_ex(ta, tb, M, N, K, float(alpha), A, lda, B, ldb, float(beta), C, ldc, stream)
    else:
        rc = sgemm(M, N, K, float(alpha), A, lda, B, ldb, float(beta), C, ldc, stream)
    if rc != 0:
        raise Fp32GemmError(rc)
    return C
