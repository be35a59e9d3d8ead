"""Thin PyTorch binding of the SharQ C ABI (pack_weight, prepare, linear,
prepare_linear, and the plain baseline rmsnorm, quantize_mx, linear_dense).

PyTorch provides device memory and the stream; each function allocates its
outputs as torch tensors, fills the C structs with their device pointers and
calls the library.  No arithmetic of the method happens here.
"""
from __future__ import annotations

from dataclasses import dataclass
from typing import Optional

import torch

from . import _lib as L


def _stream_ptr(stream: Optional[torch.cuda.Stream]) -> int:
    s = stream if stream is not None else torch.cuda.current_stream()
    return s.cuda_stream


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.float32:
        return L.SHARQ_F32
    if t.dtype == torch.bfloat16:
        return L.SHARQ_BF16
    raise TypeError(f"unsupported dtype {t.dtype} (float32 or bfloat16)")


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _dev_check(*ts):
    for t in ts:
        if t is not None and not t.is_cuda:
            raise ValueError("tensors must live on the GPU")


@dataclass
class PackedWeight:
    """One shared FP4 payload + sparse and dense scale views (per group)."""
    fmt: str
    K: int
    D: int
    n_groups: int
    payload: torch.Tensor          # uint8 (n_groups, D, K/2)
    scale_sp: torch.Tensor         # uint8 (n_groups, D, K/32)
    scale_dn: torch.Tensor         # uint8 (n_groups, D, K/32 | K/16)
    tensor_scale: Optional[torch.Tensor]

    def struct(self) -> L.SharqWeight:
        return L.SharqWeight(L.FORMATS[self.fmt], self.K, self.D, self.n_groups, _ptr(self.payload),
                             _ptr(self.scale_sp), _ptr(self.scale_dn), _ptr(self.tensor_scale))


@dataclass
class PreparedAct:
    """Output of the fused preparation: compacted backbone + dense residual."""
    fmt: str
    T: int
    K: int
    bb_codes: torch.Tensor         # uint8 (T, K/4)
    bb_meta: torch.Tensor          # uint8 (T, K/16 | K/8 for the 2:4 backbone)
    bb_scale: torch.Tensor         # uint8 (T, K/32)
    res_codes: torch.Tensor        # uint8 (T, K/2)
    res_scale: torch.Tensor        # uint8 (T, K/32 | K/16)
    tensor_scales: Optional[torch.Tensor]
    workspace: Optional[torch.Tensor]

    def struct(self) -> L.SharqAct:
        return L.SharqAct(L.FORMATS[self.fmt], self.T, self.K, _ptr(self.bb_codes), _ptr(self.bb_meta),
                          _ptr(self.bb_scale), _ptr(self.res_codes), _ptr(self.res_scale),
                          _ptr(self.tensor_scales))

    def as_numpy(self) -> dict:
        """Host copies of the layouts (for tests and inspection)."""
        d = {k: getattr(self, k).cpu().numpy() for k in ("bb_codes", "bb_meta", "bb_scale", "res_codes", "res_scale")}
        d["tensor_scales"] = None if self.tensor_scales is None else self.tensor_scales.cpu().numpy()
        d["fmt"] = self.fmt
        return d


def empty_weight(fmt: str, K: int, D: int, n_groups: int = 1, device="cuda") -> PackedWeight:
    sz = L.weight_sizes(L.FORMATS[fmt], K, D, n_groups)
    u8 = dict(dtype=torch.uint8, device=device)
    payload = torch.empty((n_groups, D, K // 2), **u8)
    scale_sp = torch.empty((n_groups, D, K // 32), **u8)
    if fmt == "mxfp4":
        scale_dn, ts = scale_sp, None
    else:
        scale_dn = torch.empty((n_groups, D, K // 16), **u8)
        ts = torch.empty(n_groups, dtype=torch.float32, device=device)
    assert payload.numel() == sz[0] and scale_sp.numel() == sz[1] and scale_dn.numel() == sz[2]
    return PackedWeight(fmt, K, D, n_groups, payload, scale_sp, scale_dn, ts)


def empty_act(fmt: str, T: int, K: int, device="cuda") -> PreparedAct:
    sz = L.act_sizes(L.FORMATS[fmt], T, K)
    u8 = dict(dtype=torch.uint8, device=device)
    nv = fmt == "nvfp4"
    res_scale = torch.empty((T, K // 16 if nv else K // 32), **u8)
    ts = torch.empty(2, dtype=torch.float32, device=device) if nv else None
    ws = torch.empty(max(sz[6], 16), **u8) if sz[6] else None
    meta = torch.empty((T, K // 8 if fmt == "mxfp4_24" else K // 16), **u8)
    return PreparedAct(fmt, T, K, torch.empty((T, K // 4), **u8), meta,
                       torch.empty((T, K // 32), **u8), torch.empty((T, K // 2), **u8), res_scale, ts, ws)


def pack_weight(W: torch.Tensor, fmt: str = "mxfp4", out: Optional[PackedWeight] = None,
                stream=None) -> PackedWeight:
    """Pack W (K x D, or n_groups x K x D; fp32 or bf16, on the GPU)."""
    _dev_check(W)
    W3 = W if W.dim() == 3 else W.unsqueeze(0)
    if W3.stride(-1) != 1:
        raise ValueError("W must be contiguous along D")
    G, K, D = W3.shape
    out = out or empty_weight(fmt, K, D, G, W.device)
    ws_bytes = L.weight_sizes(L.FORMATS[fmt], K, D, G)[4]
    ws = torch.empty(max(ws_bytes, 16), dtype=torch.uint8, device=W.device) if ws_bytes else None
    st = out.struct()
    L.check(L.lib().sharq_pack_weight(W3.data_ptr(), _dtype_code(W3), K, D, G, W3.stride(1), W3.stride(0),
                                      st, _ptr(ws), ws_bytes, _stream_ptr(stream)))
    out._ws = ws        # keep the workspace alive until the stream has used it
    return out


def prepare(X: torch.Tensor, gamma: Optional[torch.Tensor], eps: float = 1e-6, fmt: str = "mxfp4",
            out: Optional[PreparedAct] = None, stream=None) -> PreparedAct:
    """Fused preparation of X (T x K, fp32 or bf16, rows contiguous)."""
    _dev_check(X, gamma)
    if X.dim() != 2 or X.stride(1) != 1:
        raise ValueError("X must be a 2-D tensor contiguous along K")
    T, K = X.shape
    out = out or empty_act(fmt, T, K, X.device)
    ws = out.workspace
    L.check(L.lib().sharq_prepare(X.data_ptr(), _dtype_code(X), T, K, X.stride(0), _ptr(gamma), eps,
                                  out.struct(), _ptr(ws), 0 if ws is None else ws.numel(), _stream_ptr(stream)))
    return out


def prepare_no_alloc(X: torch.Tensor, gamma: Optional[torch.Tensor], eps: float, out: PreparedAct,
                     stream=None) -> PreparedAct:
    """sharq_prepare_no_alloc: the preparation into caller-provided outputs,
    with the NVFP4 scratch in the library's static device array (no
    workspace; calls that overlap on one GPU race)."""
    _dev_check(X, gamma)
    if X.dim() != 2 or X.stride(1) != 1:
        raise ValueError("X must be a 2-D tensor contiguous along K")
    T, K = X.shape
    L.check(L.lib().sharq_prepare_no_alloc(X.data_ptr(), _dtype_code(X), T, K, X.stride(0), _ptr(gamma), eps,
                                           out.struct(), _stream_ptr(stream)))
    return out


def linear(act: PreparedAct, w: PackedWeight, group_offsets: Optional[torch.Tensor] = None,
           row_index: Optional[torch.Tensor] = None, total_rows: Optional[int] = None,
           out: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """Dual-path FP4 GEMM: Y = X~_sp W~ + R~ W~ (fp32, total_rows x D)."""
    _dev_check(group_offsets, row_index, out)
    if total_rows is None:
        total_rows = row_index.numel() if row_index is not None else act.T
    if out is None:
        out = torch.empty((total_rows, w.D), dtype=torch.float32, device=act.bb_codes.device)
    for t in (group_offsets, row_index):
        if t is not None and (t.dtype != torch.int32 or not t.is_contiguous()):
            raise ValueError("group_offsets / row_index must be contiguous int32")
    L.check(L.lib().sharq_linear(act.struct(), w.struct(), _ptr(group_offsets), _ptr(row_index), total_rows,
                                 out.data_ptr(), out.stride(0), _stream_ptr(stream)))
    return out


# default prepare_linear workspaces (16 bytes, zero before first use), one
# per (device, stream): calls that share a workspace must not overlap, and
# calls on one stream never do
_PL_WS: dict = {}


def _prepare_linear_ws(device: torch.device, stream=None) -> torch.Tensor:
    dev = device.index if device.index is not None else torch.cuda.current_device()
    key = (device.type, dev, _stream_ptr(stream))
    ws = _PL_WS.get(key)
    if ws is None:
        ws = torch.zeros(16, dtype=torch.uint8, device=device)
        _PL_WS[key] = ws
    return ws


def prepare_linear_status(workspace: torch.Tensor, stream=None) -> None:
    """Raise SharqError if a single-launch decode on ``workspace`` gave up
    waiting for its prepared rows (its Y was written as NaN).  Synchronizes
    the stream."""
    _dev_check(workspace)
    L.check(L.lib().sharq_prepare_linear_status(workspace.data_ptr(), workspace.numel(), _stream_ptr(stream)))


def prepare_linear(X: torch.Tensor, gamma: Optional[torch.Tensor], w: PackedWeight, eps: float = 1e-6,
                   act: Optional[PreparedAct] = None, out: Optional[torch.Tensor] = None,
                   workspace: Optional[torch.Tensor] = None, stream=None):
    """Preparation of X and the plain MXFP4 linear on it, in one launch for
    decode shapes (T <= 8); returns (prepared activations, Y fp32 T x D)."""
    _dev_check(X, gamma, out, workspace)
    if X.dim() != 2 or X.stride(1) != 1:
        raise ValueError("X must be a 2-D tensor contiguous along K")
    T, K = X.shape
    act = act or empty_act(w.fmt, T, K, X.device)
    if out is None:
        out = torch.empty((T, w.D), dtype=torch.float32, device=X.device)
    ws = workspace if workspace is not None else _prepare_linear_ws(X.device, stream)
    L.check(L.lib().sharq_prepare_linear(X.data_ptr(), _dtype_code(X), T, K, X.stride(0), _ptr(gamma), eps,
                                         act.struct(), w.struct(), out.data_ptr(), out.stride(0), ws.data_ptr(),
                                         ws.numel(), _stream_ptr(stream)))
    return act, out


# ----------------------------------------------------------------------------
# plain baseline: RMSNorm, plain MXFP4 quantization, dense MXFP4 GEMM
# ----------------------------------------------------------------------------
def rmsnorm(X: torch.Tensor, gamma: Optional[torch.Tensor], eps: float = 1e-6,
            out: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """RMSNorm of X (T x K, fp32 or bf16) into fp32 y (T x K), the fused
    preparation's pinned order."""
    _dev_check(X, gamma, out)
    if X.dim() != 2 or X.stride(1) != 1:
        raise ValueError("X must be a 2-D tensor contiguous along K")
    T, K = X.shape
    if out is None:
        out = torch.empty((T, K), dtype=torch.float32, device=X.device)
    L.check(L.lib().sharq_rmsnorm(X.data_ptr(), _dtype_code(X), T, K, X.stride(0), _ptr(gamma), eps,
                                  out.data_ptr(), out.stride(0), _stream_ptr(stream)))
    return out


def quantize_mx(Y: torch.Tensor, codes: Optional[torch.Tensor] = None, scales: Optional[torch.Tensor] = None,
                stream=None):
    """Plain MXFP4 quantization of fp32 rows: (codes T x K/2, E8M0 scales T x K/32)."""
    _dev_check(Y, codes, scales)
    if Y.dim() != 2 or Y.stride(1) != 1 or Y.dtype != torch.float32:
        raise ValueError("Y must be a 2-D float32 tensor contiguous along K")
    T, K = Y.shape
    if codes is None:
        codes = torch.empty((T, K // 2), dtype=torch.uint8, device=Y.device)
    if scales is None:
        scales = torch.empty((T, K // 32), dtype=torch.uint8, device=Y.device)
    L.check(L.lib().sharq_quantize_mx(Y.data_ptr(), T, K, Y.stride(0), codes.data_ptr(), scales.data_ptr(),
                                      _stream_ptr(stream)))
    return codes, scales


def linear_dense(codes: torch.Tensor, scales: torch.Tensor, w: PackedWeight, out: Optional[torch.Tensor] = None,
                 stream=None) -> torch.Tensor:
    """Dense one-operand MXFP4 GEMM Y = X~ W~ (fp32, T x D)."""
    _dev_check(codes, scales, out)
    T = codes.shape[0]
    if out is None:
        out = torch.empty((T, w.D), dtype=torch.float32, device=codes.device)
    L.check(L.lib().sharq_linear_dense(codes.data_ptr(), scales.data_ptr(), T, w.struct(), out.data_ptr(),
                                       out.stride(0), _stream_ptr(stream)))
    return out
