"""ctypes binding of libsla.so (argument marshalling only).

Every step of the SageSLA forward and backward runs in the HIP kernels behind the C ABI
declared in include/sla.h; this module only checks tensors, allocates outputs
and workspaces through torch, and passes raw device pointers and the current
HIP stream.  If the library is missing the calls raise: there is no fallback.
"""
from __future__ import annotations

import ctypes
import os

import torch

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libsla.so")

(SLA_OK, SLA_ERR_INVALID_ARG, SLA_ERR_UNSUPPORTED, SLA_ERR_WORKSPACE, SLA_ERR_DEVICE,
 SLA_ERR_SCRATCH) = range(6)
NOALLOC_SCRATCH_BYTES = 64 << 20
PHI = {"none": 0, "elu1": 1, "relu": 2}
OP_QUANTIZE, OP_SELECT, OP_ATTENTION, OP_ATTENTION_BWD = 0, 1, 2, 3
OPT_PHI_K_FP8 = 1
BLOCK = 64
HEAD_DIM = 128

_lib = None


class SLAError(RuntimeError):
    def __init__(self, status: int, what: str):
        self.status = status
        super().__init__(f"{what}: {load().sla_status_string(status).decode()}")


def load() -> ctypes.CDLL:
    """Load libsla.so once; raise if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is not built; run "
                           "`python -m sparse_linear_attention_sagesla_amd.build`")
    lib = ctypes.CDLL(LIB_PATH)
    c_int, c_double, c_size_t, c_void_p = ctypes.c_int, ctypes.c_double, ctypes.c_size_t, ctypes.c_void_p
    lib.sla_topk_count.argtypes = [ctypes.c_int32, c_double]
    lib.sla_topk_count.restype = ctypes.c_int32
    lib.sla_workspace_size.argtypes = [c_int] * 6 + [c_double, c_int, ctypes.POINTER(c_size_t)]
    lib.sla_workspace_size.restype = c_int
    lib.sla_workspace_bytes.argtypes = [c_int] * 5 + [c_double, c_int]
    lib.sla_workspace_bytes.restype = c_size_t
    lib.sla_quantize_qk.argtypes = [c_void_p, c_void_p] + [c_int] * 5 + [c_void_p] * 5 + [c_void_p, c_size_t, c_void_p]
    lib.sla_quantize_qk.restype = c_int
    lib.sla_block_select.argtypes = [c_void_p, c_void_p] + [c_int] * 5 + [c_double, c_void_p, c_void_p, c_void_p, c_size_t, c_void_p]
    lib.sla_block_select.restype = c_int
    lib.sla_attention_fwd.argtypes = [c_void_p] * 3 + [c_int] * 5 + [c_double, c_int, c_void_p, c_int, c_void_p, c_size_t, c_void_p]
    lib.sla_attention_fwd.restype = c_int
    lib.sla_attention_fwd_ex.argtypes = [c_void_p] * 3 + [c_int] * 5 + [c_double, c_int, c_void_p, c_int, c_void_p, c_void_p, c_size_t, c_void_p, c_void_p, c_int]
    lib.sla_attention_fwd_ex.restype = c_int
    lib.sla_attention_fwd_fork.argtypes = [c_void_p] * 3 + [c_int] * 5 + [c_double, c_int, c_void_p, c_int, c_void_p, c_size_t, c_void_p, c_void_p]
    lib.sla_attention_fwd_fork.restype = c_int
    lib.sla_attention_fwd_lowbit.argtypes = lib.sla_attention_fwd.argtypes
    lib.sla_attention_fwd_lowbit.restype = c_int
    lib.sla_attention_fwd_noalloc.argtypes = [c_void_p] * 3 + [c_int] * 5 + [c_double, c_int, c_void_p, c_int, c_void_p]
    lib.sla_attention_fwd_noalloc.restype = c_int
    lib.sla_attention_bwd.argtypes = [c_void_p] * 4 + [c_int] * 5 + [c_double, c_int] + [c_void_p] * 3 + [c_int, c_void_p, c_size_t, c_void_p]
    lib.sla_attention_bwd.restype = c_int
    lib.sla_attention_bwd_timed.argtypes = lib.sla_attention_bwd.argtypes + [c_void_p]
    lib.sla_attention_bwd_timed.restype = c_int
    lib.sla_train_residual_bytes.argtypes = [c_int] * 5 + [c_double, c_int]
    lib.sla_train_residual_bytes.restype = c_size_t
    lib.sla_attention_fwd_train.argtypes = [c_void_p] * 3 + [c_int] * 5 + [c_double, c_int, c_void_p, c_int,
                                                                          c_void_p, c_size_t, c_void_p,
                                                                          c_size_t, c_void_p]
    lib.sla_attention_fwd_train.restype = c_int
    lib.sla_attention_bwd_saved.argtypes = [c_void_p] * 5 + [c_size_t] + [c_int] * 5 + [c_double, c_int] + \
        [c_void_p] * 3 + [c_int, c_void_p, c_size_t, c_void_p, c_void_p]
    lib.sla_attention_bwd_saved.restype = c_int
    lib.sla_rowquant_i8.argtypes = [c_void_p, c_int, c_int, c_void_p, c_void_p, c_void_p]
    lib.sla_rowquant_i8.restype = c_int
    lib.sla_fused_norm_i8.argtypes = [c_void_p, c_int, c_int, c_void_p, c_void_p, ctypes.c_float,
                                      c_void_p, c_void_p, c_void_p, c_void_p, c_void_p]
    lib.sla_fused_norm_i8.restype = c_int
    lib.sla_w8a8_linear.argtypes = [c_void_p] * 5 + [c_int] * 3 + [c_void_p, c_int, c_void_p]
    lib.sla_w8a8_linear.restype = c_int
    lib.sla_debug_qk_i32.argtypes = [c_void_p, c_void_p] + [c_int] * 5 + [c_void_p, c_int, c_void_p, c_void_p]
    lib.sla_debug_qk_i32.restype = c_int
    lib.sla_status_string.argtypes = [c_int]
    lib.sla_status_string.restype = ctypes.c_char_p
    lib.sla_version.argtypes = []
    lib.sla_version.restype = c_int
    _lib = lib
    return lib


def _check(status: int, what: str):
    if status != SLA_OK:
        raise SLAError(status, what)


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else ctypes.c_void_p(0)


def _stream(device) -> ctypes.c_void_p:
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _bhnd(x: torch.Tensor, name: str):
    if not isinstance(x, torch.Tensor) or x.dim() != 4:
        raise ValueError(f"{name} must be a [B, H, N, 128] tensor")
    if not x.is_cuda:
        raise ValueError(f"{name} must live on a GPU")
    if x.dtype != torch.bfloat16:
        raise ValueError(f"{name} must be bfloat16")
    if x.shape[-1] != HEAD_DIM:
        raise ValueError(f"{name}: head dim must be {HEAD_DIM}")
    return x.contiguous()


def topk_count(n_blocks: int, keep: float) -> int:
    return int(load().sla_topk_count(int(n_blocks), float(keep)))


def n_blocks(N: int) -> int:
    return (N + BLOCK - 1) // BLOCK


def workspace_size(op: int, B: int, H: int, N: int, keep: float = 0.0, phi="none") -> int:
    out = ctypes.c_size_t(0)
    _check(load().sla_workspace_size(op, B, H, N, HEAD_DIM, BLOCK, float(keep),
                                     PHI[phi] if isinstance(phi, str) else int(phi),
                                     ctypes.byref(out)), "sla_workspace_size")
    return out.value


def workspace_bytes(B: int, H: int, N: int, keep: float, phi="elu1") -> int:
    """Bytes of the forward workspace (0 for arguments no forward call accepts)."""
    return int(load().sla_workspace_bytes(B, H, N, HEAD_DIM, BLOCK, float(keep),
                                          PHI[phi] if isinstance(phi, str) else int(phi)))


def _workspace(nbytes: int, device, ws):
    if ws is not None and ws.numel() >= nbytes:
        return ws
    return torch.empty(max(nbytes, 1), dtype=torch.uint8, device=device)


def quantize_qk(q: torch.Tensor, k: torch.Tensor, workspace=None):
    """INT8 codes/scales of Q and mean-smoothed K: (q8, k8, q_scale, k_scale, k_mean)."""
    q, k = _bhnd(q, "q"), _bhnd(k, "k")
    B, H, N, d = q.shape
    nb = n_blocks(N)
    dev = q.device
    q8 = torch.empty(B, H, nb * BLOCK, d, dtype=torch.int8, device=dev)
    k8 = torch.empty_like(q8)
    sq = torch.empty(B, H, nb, dtype=torch.float32, device=dev)
    sk = torch.empty_like(sq)
    mu = torch.empty(B, H, d, dtype=torch.float32, device=dev)
    nbytes = workspace_size(OP_QUANTIZE, B, H, N)
    ws = _workspace(nbytes, dev, workspace)
    _check(load().sla_quantize_qk(_ptr(q), _ptr(k), B, H, N, d, BLOCK, _ptr(q8), _ptr(k8),
                                  _ptr(sq), _ptr(sk), _ptr(mu), _ptr(ws), ws.numel(),
                                  _stream(dev)), "sla_quantize_qk")
    return q8, k8, sq, sk, mu


def block_select(q: torch.Tensor, k: torch.Tensor, keep: float, with_mask: bool = False,
                 workspace=None):
    """Kept key blocks per query block: idx int32 [B,H,Nb,k] ascending (and the bitmask)."""
    q, k = _bhnd(q, "q"), _bhnd(k, "k")
    B, H, N, d = q.shape
    nb = n_blocks(N)
    kk = topk_count(nb, keep)
    dev = q.device
    idx = torch.empty(B, H, nb, max(kk, 1), dtype=torch.int32, device=dev)
    mask = torch.empty(B, H, nb, (nb + 31) // 32, dtype=torch.int32, device=dev) if with_mask else None
    nbytes = workspace_size(OP_SELECT, B, H, N)
    ws = _workspace(nbytes, dev, workspace)
    _check(load().sla_block_select(_ptr(q), _ptr(k), B, H, N, d, BLOCK, float(keep), _ptr(idx),
                                   _ptr(mask), _ptr(ws), ws.numel(), _stream(dev)),
           "sla_block_select")
    return (idx, mask) if with_mask else idx


def attention(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, keep: float = 0.1,
              phi: str = "elu1", out_dtype=torch.bfloat16, return_linear: bool = False,
              out=None, workspace=None, lowbit: bool = False, side_stream=None):
    """SageSLA forward: softmax attention on the kept key blocks + linear attention on the rest.

    ``lowbit``: the opt-in variant with the linear branch's phi(K) in FP8
    (sla_attention_fwd_lowbit).  ``side_stream`` (a torch.cuda.Stream of q's
    device): the selection runs on it, concurrently with the linear staging
    (sla_attention_fwd_fork); not with ``return_linear`` or ``lowbit``."""
    q, k, v = _bhnd(q, "q"), _bhnd(k, "k"), _bhnd(v, "v")
    if k.shape != q.shape or v.shape != q.shape:
        raise ValueError("q, k, v must have the same shape")
    B, H, N, d = q.shape
    dev = q.device
    if out_dtype not in (torch.bfloat16, torch.float32):
        raise ValueError("out_dtype must be bfloat16 or float32")
    if out is None:
        out = torch.empty(B, H, N, d, dtype=out_dtype, device=dev)
    elif out.shape != q.shape or out.dtype != out_dtype or not out.is_contiguous():
        raise ValueError("out must be a contiguous tensor of q's shape and out_dtype")
    lin = torch.empty(B, H, N, d, dtype=torch.float32, device=dev) if return_linear else None
    ph = PHI[phi] if isinstance(phi, str) else int(phi)
    nbytes = workspace_size(OP_ATTENTION, B, H, N, keep, ph)
    ws = _workspace(nbytes, dev, workspace)
    f32 = 1 if out_dtype == torch.float32 else 0
    if side_stream is not None:
        if lin is not None or lowbit:
            raise ValueError("side_stream is not combined with return_linear or lowbit")
        _check(load().sla_attention_fwd_fork(_ptr(q), _ptr(k), _ptr(v), B, H, N, d, BLOCK, float(keep), ph,
                                             _ptr(out), f32, _ptr(ws), ws.numel(), _stream(dev),
                                             side_stream.cuda_stream), "sla_attention_fwd_fork")
        return out
    if lin is None:
        fn = load().sla_attention_fwd_lowbit if lowbit else load().sla_attention_fwd
        _check(fn(_ptr(q), _ptr(k), _ptr(v), B, H, N, d, BLOCK, float(keep), ph, _ptr(out), f32,
                  _ptr(ws), ws.numel(), _stream(dev)),
               "sla_attention_fwd_lowbit" if lowbit else "sla_attention_fwd")
    else:
        _check(load().sla_attention_fwd_ex(_ptr(q), _ptr(k), _ptr(v), B, H, N, d, BLOCK,
                                           float(keep), ph, _ptr(out), f32, _ptr(lin), _ptr(ws),
                                           ws.numel(), _stream(dev), None,
                                           OPT_PHI_K_FP8 if lowbit else 0), "sla_attention_fwd_ex")
    return (out, lin) if return_linear else out


def attention_noalloc(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, out: torch.Tensor,
                      keep: float = 0.1, phi: str = "elu1"):
    """SageSLA forward into a preallocated ``out`` (bf16 or fp32), with the
    library's static device scratch as workspace: nothing is allocated."""
    q, k, v = _bhnd(q, "q"), _bhnd(k, "k"), _bhnd(v, "v")
    if k.shape != q.shape or v.shape != q.shape:
        raise ValueError("q, k, v must have the same shape")
    if out.shape != q.shape or out.dtype not in (torch.bfloat16, torch.float32) or not out.is_contiguous():
        raise ValueError("out must be a contiguous bf16 or fp32 tensor of q's shape")
    B, H, N, d = q.shape
    ph = PHI[phi] if isinstance(phi, str) else int(phi)
    _check(load().sla_attention_fwd_noalloc(_ptr(q), _ptr(k), _ptr(v), B, H, N, d, BLOCK, float(keep),
                                            ph, _ptr(out), 1 if out.dtype == torch.float32 else 0,
                                            _stream(q.device)), "sla_attention_fwd_noalloc")
    return out


def train_residual_bytes(B: int, H: int, N: int, keep: float, phi="elu1") -> int:
    """Bytes of a training forward's residual buffer (sla_train_residual_bytes)."""
    ph = PHI[phi] if isinstance(phi, str) else int(phi)
    n = load().sla_train_residual_bytes(B, H, N, HEAD_DIM, BLOCK, float(keep), ph)
    if n == 0:
        raise SLAError(1, "sla_train_residual_bytes: invalid arguments")
    return int(n)


def attention_train(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, keep: float = 0.1,
                    phi: str = "elu1", out_dtype=torch.bfloat16, workspace=None):
    """SageSLA forward that also keeps what the backward needs
    (sla_attention_fwd_train): returns (out, residuals), residuals a uint8
    tensor to pass to attention_bwd(..., residuals=...)."""
    q, k, v = _bhnd(q, "q"), _bhnd(k, "k"), _bhnd(v, "v")
    if k.shape != q.shape or v.shape != q.shape:
        raise ValueError("q, k, v must have the same shape")
    if out_dtype not in (torch.bfloat16, torch.float32):
        raise ValueError("out_dtype must be bfloat16 or float32")
    B, H, N, d = q.shape
    dev = q.device
    out = torch.empty(B, H, N, d, dtype=out_dtype, device=dev)
    ph = PHI[phi] if isinstance(phi, str) else int(phi)
    res = torch.empty(train_residual_bytes(B, H, N, keep, ph), dtype=torch.uint8, device=dev)
    ws = _workspace(workspace_size(OP_ATTENTION, B, H, N, keep, ph), dev, workspace)
    _check(load().sla_attention_fwd_train(_ptr(q), _ptr(k), _ptr(v), B, H, N, d, BLOCK, float(keep), ph,
                                          _ptr(out), 1 if out_dtype == torch.float32 else 0,
                                          _ptr(res), res.numel(), _ptr(ws), ws.numel(), _stream(dev)),
           "sla_attention_fwd_train")
    return out, res


def attention_bwd(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, dout: torch.Tensor,
                  keep: float = 0.1, phi: str = "elu1", grad_dtype=torch.bfloat16, workspace=None,
                  residuals=None):
    """Gradients (dq, dk, dv) of the SageSLA forward for the output gradient dout.

    ``residuals``: the buffer of an attention_train call on the same q, k, v,
    keep and phi (sla_attention_bwd_saved); None recomputes the forward's part
    (sla_attention_bwd)."""
    q, k, v, dout = _bhnd(q, "q"), _bhnd(k, "k"), _bhnd(v, "v"), _bhnd(dout, "dout")
    if k.shape != q.shape or v.shape != q.shape or dout.shape != q.shape:
        raise ValueError("q, k, v, dout must have the same shape")
    if grad_dtype not in (torch.bfloat16, torch.float32):
        raise ValueError("grad_dtype must be bfloat16 or float32")
    B, H, N, d = q.shape
    dev = q.device
    dq, dk, dv = (torch.empty(B, H, N, d, dtype=grad_dtype, device=dev) for _ in range(3))
    ph = PHI[phi] if isinstance(phi, str) else int(phi)
    nbytes = workspace_size(OP_ATTENTION_BWD, B, H, N, keep, ph)
    ws = _workspace(nbytes, dev, workspace)
    f32 = 1 if grad_dtype == torch.float32 else 0
    if residuals is None:
        _check(load().sla_attention_bwd(_ptr(q), _ptr(k), _ptr(v), _ptr(dout), B, H, N, d, BLOCK,
                                        float(keep), ph, _ptr(dq), _ptr(dk), _ptr(dv), f32, _ptr(ws),
                                        ws.numel(), _stream(dev)), "sla_attention_bwd")
    else:
        if residuals.device != dev or residuals.dtype != torch.uint8 or not residuals.is_contiguous():
            raise ValueError("residuals must be the contiguous uint8 buffer of attention_train")
        _check(load().sla_attention_bwd_saved(_ptr(q), _ptr(k), _ptr(v), _ptr(dout), _ptr(residuals),
                                              residuals.numel(), B, H, N, d, BLOCK, float(keep), ph,
                                              _ptr(dq), _ptr(dk), _ptr(dv), f32, _ptr(ws), ws.numel(),
                                              _stream(dev), None), "sla_attention_bwd_saved")
    return dq, dk, dv


def _rows2d(x: torch.Tensor, name: str, dtype=torch.bfloat16):
    if not isinstance(x, torch.Tensor) or x.dim() != 2 or not x.is_cuda or x.dtype != dtype:
        raise ValueError(f"{name} must be a 2-D {dtype} GPU tensor")
    return x.contiguous()


def _vec(x, n: int, name: str):
    if x is None:
        return None
    if not isinstance(x, torch.Tensor) or x.dtype != torch.float32 or x.numel() != n or not x.is_cuda:
        raise ValueError(f"{name} must be a float32 GPU tensor of {n} elements")
    return x.contiguous()


def rowquant_i8(x: torch.Tensor):
    """Per-row INT8 codes and scales of a bf16 [rows, K] matrix: (codes, scale)."""
    x = _rows2d(x, "x")
    rows, K = x.shape
    codes = torch.empty(rows, K, dtype=torch.int8, device=x.device)
    scale = torch.empty(rows, dtype=torch.float32, device=x.device)
    _check(load().sla_rowquant_i8(_ptr(x), rows, K, _ptr(codes), _ptr(scale), _stream(x.device)),
           "sla_rowquant_i8")
    return codes, scale


def fused_norm_i8(x: torch.Tensor, gamma=None, beta=None, eps: float = 1e-6):
    """FusedNorm: LayerNorm (+ per-channel affine) then per-row INT8:
    (codes, scale, mean, rstd)."""
    x = _rows2d(x, "x")
    rows, K = x.shape
    gamma, beta = _vec(gamma, K, "gamma"), _vec(beta, K, "beta")
    dev = x.device
    codes = torch.empty(rows, K, dtype=torch.int8, device=dev)
    scale, mean, rstd = (torch.empty(rows, dtype=torch.float32, device=dev) for _ in range(3))
    _check(load().sla_fused_norm_i8(_ptr(x), rows, K, _ptr(gamma), _ptr(beta), float(eps),
                                    _ptr(codes), _ptr(scale), _ptr(mean), _ptr(rstd),
                                    _stream(dev)), "sla_fused_norm_i8")
    return codes, scale, mean, rstd


def w8a8_linear(x8: torch.Tensor, x_scale: torch.Tensor, w8: torch.Tensor, w_scale: torch.Tensor,
                bias=None, out_dtype=torch.bfloat16, out=None):
    """y = (x8 w8^T) * x_scale[:, None] * w_scale[None, :] + bias, [M, N]."""
    x8, w8 = _rows2d(x8, "x8", torch.int8), _rows2d(w8, "w8", torch.int8)
    M, K = x8.shape
    N, K2 = w8.shape
    if K2 != K:
        raise ValueError("x8 and w8 must have the same K")
    x_scale, w_scale, bias = _vec(x_scale, M, "x_scale"), _vec(w_scale, N, "w_scale"), _vec(bias, N, "bias")
    if out_dtype not in (torch.bfloat16, torch.float32):
        raise ValueError("out_dtype must be bfloat16 or float32")
    if out is None:
        out = torch.empty(M, N, dtype=out_dtype, device=x8.device)
    elif out.shape != (M, N) or out.dtype != out_dtype or not out.is_contiguous():
        raise ValueError("out must be a contiguous [M, N] tensor of out_dtype")
    _check(load().sla_w8a8_linear(_ptr(x8), _ptr(x_scale), _ptr(w8), _ptr(w_scale), _ptr(bias), M, N,
                                  K, _ptr(out), 1 if out_dtype == torch.float32 else 0,
                                  _stream(x8.device)), "sla_w8a8_linear")
    return out


def debug_qk_i32(q8: torch.Tensor, k8: torch.Tensor, N: int, pairs: torch.Tensor):
    """Integer Q.K^T tiles [P, 64, 64] for (b, h, i, j) rows of `pairs`."""
    B, H, Np, d = q8.shape
    pairs = pairs.to(device=q8.device, dtype=torch.int32).contiguous()
    acc = torch.zeros(pairs.shape[0], BLOCK, BLOCK, dtype=torch.int32, device=q8.device)
    _check(load().sla_debug_qk_i32(_ptr(q8.contiguous()), _ptr(k8.contiguous()), B, H, N, d,
                                   BLOCK, _ptr(pairs), pairs.shape[0], _ptr(acc),
                                   _stream(q8.device)), "sla_debug_qk_i32")
    return acc


class SLAAttention:
    """Repeated SageSLA forwards of one shape with a preallocated workspace and output."""

    def __init__(self, B, H, N, keep=0.1, phi="elu1", out_dtype=torch.bfloat16, device="cuda"):
        self.shape = (B, H, N, HEAD_DIM)
        self.keep, self.phi, self.out_dtype = keep, phi, out_dtype
        nbytes = workspace_size(OP_ATTENTION, B, H, N, keep, PHI[phi])
        self.workspace = torch.empty(nbytes, dtype=torch.uint8, device=device)
        self.out = torch.empty(*self.shape, dtype=out_dtype, device=device)

    def __call__(self, q, k, v):
        return attention(q, k, v, self.keep, self.phi, self.out_dtype, out=self.out,
                         workspace=self.workspace)
