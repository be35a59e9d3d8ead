"""CPU oracle -- the SharQ linear-layer hot path (TEST INFRASTRUCTURE ONLY).

A plain, slow, step-by-step CPU implementation of what the SharQ hot path
computes, used to check the GPU library.  Only ``tests/``,
``__graft_entry__.smoke()`` and ``bench.py``'s cpu_baseline leg may import
this package; the product path never does.  It shares no code with the GPU
path: the two meet only in the byte layouts of their outputs.

Sources (pages about "SharQ: Bridging Activation Sparsity and FP4 Quantization
for LLM Inference"):

* review = the xllm-io paper review (xllm-io.github.io/paper-review):
  §3.1 objective Y = XW (X in R^{T x K}, W in R^{K x D}) and group-symmetric
  block scales; §3.2 sparse backbone X_sp = M(X) ⊙ X with an input-adaptive
  N:M mask; §3.3 quantized backbone X~_sp = D_sp(Q_sp(X_sp)) and residual
  R = X - X~_sp; §3.4 dual-path output GEMM_sp + GEMM_dn; §3.5 kernel design
  (one fused preparation: RMSNorm/PTS, pair-top-k 4:8 in-pairs mask, sparse
  compression, dense residual; one shared FP4 weight payload with a sparse
  group-32 scale view and a dense group-16 duplicated scale view; the dense
  branch accumulates into the sparse branch's output); §3.6 error merge
  X - (X~_sp + R~) = R - R~ and ||X W - (X~_sp + R~) W||_F <= ||R - R~||_F ||W||_2.
* explainer = the kasblo.com explainer: 4:8 in-pairs treats 8 contiguous
  values as 4 pairs and keeps 2 pairs (4 values), choosing pairs that hold
  large values; method steps 1-4 (mask, FP4 backbone, residual against the
  quantized backbone, two FP4 GEMMs summed); per-tensor scaling and layer
  normalization are part of the fused preparation; NVFP4 activation global
  scales are computed without calibration.

Readings taken where the pages leave a step open:

* "X" of the decomposition is the RMSNorm output y, kept in fp32.  RMSNorm is
  y_k = (x_k * (1 / sqrt(mean(x^2) + eps))) * gamma_k, every operation an fp32
  round-to-nearest-even operation without fused multiply-add; the sum of
  squares is a pairwise tree over the row in index order (zero-padded to a
  power of two).  The floating-point order must be pinned because the FP4
  codes are compared bit for bit.
* Pair score = max |y| of the pair's two values; the 2 pairs with the highest
  scores are kept, ties going to the lower pair index.
* MXFP4: E2M1 values with one E8M0 scale per 32 K-positions (the backbone's
  block is 32 logical positions = 16 kept values).  NVFP4 (emulated): E4M3
  block scales (backbone: per 32 logical positions; residual: per 16) and an
  fp32 tensor scale s_T = amax / (6 * 448) computed online ("PTS").
* Weights are scaled once per 32 along K, so both paths share the codes; the
  dense view repeats each scale for its two 16-value halves.

Byte layouts (the GPU library's layouts; row-major, K contiguous):

* element codes: two E2M1 codes per byte, the even K index in the low nibble;
* backbone ``bb_codes`` (T x K/4): per group of 8, the bytes of the two kept
  pairs in ascending pair order; ``bb_meta`` (T x K/16): per group the nibble
  i0 | i1 << 2 (i0 < i1 the kept pair indices), even group in the low nibble;
* scales: one byte per block, blocks in K order;
* weight ``payload`` (D x K/2): row d holds column d of W.
"""
from __future__ import annotations

import numpy as np

from .formats import (E2M1_MAX, E4M3_MAX, e2m1_decode, e2m1_encode, e4m3_decode, e4m3_encode,
                      e8m0_decode_exponent, e8m0_encode_exponent, e8m0_exponent)

F32 = np.float32
MX_BLOCK = 32
NV_BB_BLOCK = 32
NV_RES_BLOCK = 16
NV_W_BLOCK = 32
NV_TENSOR_DIV = F32(E2M1_MAX * E4M3_MAX)        # 2688


# ----------------------------------------------------------------------------
# RMSNorm (review §3.5 "RMSNorm/PTS" inside the fused preparation)
# ----------------------------------------------------------------------------
def pairwise_sum_f32(a: np.ndarray) -> np.ndarray:
    """Sum along the last axis as a pairwise tree in index order: zero-pad to a
    power of two, then repeatedly add neighbours (0,1), (2,3), ... in fp32."""
    a = np.asarray(a, dtype=F32)
    n = a.shape[-1]
    width = 1
    while width < n:
        width *= 2
    if width != n:
        pad = np.zeros(a.shape[:-1] + (width - n,), dtype=F32)
        a = np.concatenate([a, pad], axis=-1)
    while a.shape[-1] > 1:
        a = a[..., 0::2] + a[..., 1::2]
    return a[..., 0]


def rmsnorm(x: np.ndarray, gamma, eps: float) -> np.ndarray:
    """y = (x * inv_rms) * gamma in fp32; gamma None means no normalization.

    Input domain: every x_k * x_k and the row's sum of squares must be finite
    in fp32 (one value of magnitude above about 1.8e19 already overflows).
    Outside it S = +inf, inv = 1 / inf = 0 and the row comes out as signed
    zeros; this is what fp32 arithmetic in the stated order gives, and it is
    the documented behaviour of the library, not a supported use."""
    x = np.asarray(x, dtype=F32)
    if gamma is None:
        return x.copy()
    K = x.shape[-1]
    with np.errstate(over="ignore"):
        S = pairwise_sum_f32(x * x)
    ms = S / F32(K)
    r = np.sqrt(ms + F32(eps))
    inv = F32(1.0) / r
    return (x * inv[..., None]) * np.asarray(gamma, dtype=F32)


# ----------------------------------------------------------------------------
# 4:8 in-pairs mask (review §3.2, §3.5; explainer, 4:8 section)
# ----------------------------------------------------------------------------
def pair_scores(y: np.ndarray) -> np.ndarray:
    """score[t, g, p] = max(|y[t, 8g+2p]|, |y[t, 8g+2p+1]|)."""
    T, K = y.shape
    pairs = np.abs(y.reshape(T, K // 8, 4, 2))
    return pairs.max(axis=-1)


def pair_top2(y: np.ndarray):
    """Kept pair indices (i0 < i1) per group of 8: the two highest-scoring
    pairs, ties to the lower pair index.  Pair p is kept when fewer than two
    other pairs beat it; q beats p if its score is larger, or equal with q < p."""
    s = pair_scores(y)                                    # (T, G, 4)
    sp = s[..., :, None]                                  # score of p
    sq = s[..., None, :]                                  # score of q
    idx = np.arange(4)
    beats = (sq > sp) | ((sq == sp) & (idx[None, :] < idx[:, None]))
    kept = beats.sum(axis=-1) < 2                         # (T, G, 4)
    order = np.argsort(~kept, axis=-1, kind="stable")     # kept pairs first, ascending
    return order[..., 0].astype(np.uint8), order[..., 1].astype(np.uint8)


def mask_from_pairs(i0: np.ndarray, i1: np.ndarray) -> np.ndarray:
    """Element mask M (T x K, bool) of the kept pairs."""
    T, G = i0.shape
    keep = np.zeros((T, G, 4), dtype=bool)
    t, g = np.indices((T, G))
    keep[t, g, i0] = True
    keep[t, g, i1] = True
    return np.repeat(keep, 2, axis=-1).reshape(T, G * 8)


def nm_keep(y: np.ndarray, N: int, M: int, unit: int = 1) -> np.ndarray:
    """Element mask of the general N:M rule (review §3.2, input-adaptive N:M
    mask; explainer, 4:8 in-pairs section): each group of M contiguous values
    is cut into M / unit units of ``unit`` contiguous values, a unit scores
    the max |y| of its values, and the N / unit highest-scoring units are
    kept, ties to the lower unit index.  unit = 2 with 4:8 is the in-pairs
    pattern of ``pair_top2``; unit = 1 with 2:4 is the element-wise pattern
    the pages pair with MXFP4."""
    T, K = y.shape
    U, n = M // unit, N // unit
    s = np.abs(y.reshape(T, K // M, U, unit)).max(axis=-1)          # (T, G, U)
    sp, sq = s[..., :, None], s[..., None, :]
    idx = np.arange(U)
    beats = (sq > sp) | ((sq == sp) & (idx[None, :] < idx[:, None]))
    kept = beats.sum(axis=-1) < n
    return np.repeat(kept, unit, axis=-1).reshape(T, K)


def top2_of4_indices(M: np.ndarray):
    """Kept positions i0 < i1 of every group of 4 of a 2:4 mask (T x K)."""
    T, K = M.shape
    order = np.argsort(~M.reshape(T, K // 4, 4), axis=-1, kind="stable")
    return order[..., 0].astype(np.uint8), order[..., 1].astype(np.uint8)


def compact_24(codes: np.ndarray, i0: np.ndarray, i1: np.ndarray) -> np.ndarray:
    """2:4 backbone bytes (T x K/4): per group of 4 the codes at i0 (low
    nibble) and i1 (high nibble)."""
    T, K = codes.shape
    c = codes.reshape(T, K // 4, 4)
    t, g = np.indices(i0.shape)
    return (c[t, g, i0] | (c[t, g, i1] << 4)).astype(np.uint8)


def expand_24(bb_codes: np.ndarray, i0: np.ndarray, i1: np.ndarray) -> np.ndarray:
    """Inverse of compact_24: element codes (T x K) with 0 at dropped positions."""
    T, G = i0.shape
    c = np.zeros((T, G, 4), dtype=np.uint8)
    t, g = np.indices((T, G))
    c[t, g, i0] = bb_codes & 0xF
    c[t, g, i1] = bb_codes >> 4
    return c.reshape(T, G * 4)


def meta_bytes(i0: np.ndarray, i1: np.ndarray) -> np.ndarray:
    nib = (i0.astype(np.uint8) | (i1.astype(np.uint8) << 2))
    return (nib[:, 0::2] | (nib[:, 1::2] << 4)).astype(np.uint8)


def meta_unpack(meta: np.ndarray):
    T = meta.shape[0]
    nib = np.empty((T, meta.shape[1] * 2), dtype=np.uint8)
    nib[:, 0::2] = meta & 0xF
    nib[:, 1::2] = meta >> 4
    return nib & 3, nib >> 2


# ----------------------------------------------------------------------------
# packing helpers
# ----------------------------------------------------------------------------
def pack_nibbles(codes: np.ndarray) -> np.ndarray:
    """(…, 2n) codes -> (…, n) bytes, even index in the low nibble."""
    return (codes[..., 0::2] | (codes[..., 1::2] << 4)).astype(np.uint8)


def unpack_nibbles(b: np.ndarray) -> np.ndarray:
    out = np.empty(b.shape[:-1] + (b.shape[-1] * 2,), dtype=np.uint8)
    out[..., 0::2] = b & 0xF
    out[..., 1::2] = b >> 4
    return out


def compact_pairs(codes: np.ndarray, i0: np.ndarray, i1: np.ndarray) -> np.ndarray:
    """Keep the two chosen pair bytes of every group of 8 (ascending pair)."""
    T, K = codes.shape
    pair_bytes = pack_nibbles(codes).reshape(T, K // 8, 4)
    t, g = np.indices(i0.shape)
    out = np.stack([pair_bytes[t, g, i0], pair_bytes[t, g, i1]], axis=-1)
    return out.reshape(T, K // 4)


def expand_pairs(bb_codes: np.ndarray, i0: np.ndarray, i1: np.ndarray) -> np.ndarray:
    """Inverse of compact_pairs: element codes (T x K) with 0 in dropped pairs."""
    T = bb_codes.shape[0]
    G = i0.shape[1]
    kept = bb_codes.reshape(T, G, 2)
    pair_bytes = np.zeros((T, G, 4), dtype=np.uint8)
    t, g = np.indices((T, G))
    pair_bytes[t, g, i0] = kept[..., 0]
    pair_bytes[t, g, i1] = kept[..., 1]
    return unpack_nibbles(pair_bytes.reshape(T, G * 4))


# ----------------------------------------------------------------------------
# MXFP4 block quantizer (review §3.1, §5.3)
# ----------------------------------------------------------------------------
def mx_quantize(v: np.ndarray):
    """Quantize fp32 ``v`` (… x K) per 32-block: e = E8M0 exponent of the
    block amax, codes = E2M1(v / 2**e) (power-of-two scaling is exact).
    Returns (codes … x K uint8, exponents … x K/32 int32)."""
    v = np.asarray(v, dtype=F32)
    shp = v.shape
    vb = v.reshape(shp[:-1] + (shp[-1] // MX_BLOCK, MX_BLOCK))
    amax = np.abs(vb).max(axis=-1)
    e = e8m0_exponent(amax)
    scaled = vb.astype(np.float64) * np.exp2(-e.astype(np.float64))[..., None]
    codes = e2m1_encode(scaled)          # a signed zero keeps its sign bit
    return codes.reshape(shp), e


def mx_dequant_f32(codes: np.ndarray, e: np.ndarray) -> np.ndarray:
    """fp32 value q * 2**e of each code (exact)."""
    shp = codes.shape
    q = e2m1_decode(codes).reshape(shp[:-1] + (shp[-1] // MX_BLOCK, MX_BLOCK))
    return (q * np.exp2(e.astype(np.float64))[..., None]).reshape(shp).astype(F32)


def mx_dequant_f64(codes, e):
    shp = codes.shape
    q = e2m1_decode(codes).reshape(shp[:-1] + (shp[-1] // MX_BLOCK, MX_BLOCK))
    return (q * np.exp2(e.astype(np.float64))[..., None]).reshape(shp)


# ----------------------------------------------------------------------------
# NVFP4 block quantizer, emulated (review §3.1; explainer, block-scale section)
# ----------------------------------------------------------------------------
def nv_tensor_scale(amax) -> np.float32:
    """s_T = amax / (6 * 448) in fp32; an all-zero tensor gets s_T = 1."""
    amax = F32(amax)
    return F32(1.0) if amax == 0 else F32(amax / NV_TENSOR_DIV)


def nv_quantize(v: np.ndarray, block: int, s_T: np.float32):
    """Quantize fp32 ``v`` (… x K) per ``block`` with E4M3 block scales under
    the tensor scale s_T: u = (amax_b / 6) / s_T -> E4M3 code (dec = its value),
    d = dec * s_T, element code = E2M1(x / d); dec == 0 gives signed zeros.
    Every floating-point step is one fp32 operation.
    Returns (codes … x K uint8, scale codes … x K/block uint8)."""
    v = np.asarray(v, dtype=F32)
    s_T = F32(s_T)
    shp = v.shape
    vb = v.reshape(shp[:-1] + (shp[-1] // block, block))
    amax = np.abs(vb).max(axis=-1)
    u = (amax / F32(E2M1_MAX)) / s_T
    sc = e4m3_encode(u)
    dec = e4m3_decode(sc).astype(F32)
    d = (dec * s_T)[..., None]
    with np.errstate(divide="ignore", invalid="ignore"):
        t = np.where(d > 0, vb / np.where(d > 0, d, F32(1.0)), vb * F32(0.0))
    codes = e2m1_encode(t)
    return codes.reshape(shp), sc


def nv_dequant_f32(codes, sc, block: int, s_T) -> np.ndarray:
    """fp32 dequantized value fl(fl(q * dec) * s_T)."""
    shp = codes.shape
    q = e2m1_decode(codes).astype(F32).reshape(shp[:-1] + (shp[-1] // block, block))
    dec = e4m3_decode(sc).astype(F32)[..., None]
    return ((q * dec) * F32(s_T)).reshape(shp)


def nv_dequant_f64(codes, sc, block: int, s_T) -> np.ndarray:
    """Exact dequantized value q * dec * s_T (fp64)."""
    shp = codes.shape
    q = e2m1_decode(codes).reshape(shp[:-1] + (shp[-1] // block, block))
    dec = e4m3_decode(sc)[..., None]
    return (q * dec * np.float64(s_T)).reshape(shp)


# ----------------------------------------------------------------------------
# prepare: the fused activation preparation (review §3.2-§3.5)
# ----------------------------------------------------------------------------
def prepare(x: np.ndarray, gamma, eps: float = 1e-6, fmt: str = "mxfp4", mask: str = "4:8") -> dict:
    """Online sparse-dense decomposition of the activation rows ``x`` (T x K,
    fp32 values of the stored inputs).

    1. y = RMSNorm(x) (fp32).
    2. mask M(y): per group of 8, keep the 2 pairs with the largest max|y|.
    3. X_sp = M ⊙ y; Q_sp quantizes X_sp per block, D_sp dequantizes:
       X~_sp = D_sp(Q_sp(X_sp)).
    4. R = y - X~_sp (fp32; zero-cost at dropped positions where R = y).
    5. Q_dn quantizes R per block.
    ``mask``: "4:8" (in pairs, groups of 8: metadata nibble = kept pair
    indices) or "2:4" (element-wise, MXFP4 only, groups of 4: metadata nibble
    = kept element indices, backbone byte = their two codes).
    Returns the layouts of the GPU library plus the fp32 intermediates."""
    y = rmsnorm(x, gamma, eps)
    T, K = y.shape
    if mask == "4:8":
        i0, i1 = pair_top2(y)
        M = mask_from_pairs(i0, i1)
    elif mask == "2:4" and fmt == "mxfp4":
        M = nm_keep(y, 2, 4)
        i0, i1 = top2_of4_indices(M)
    else:
        raise ValueError(f"mask {mask} with {fmt}")
    X_sp = np.where(M, y, F32(0.0))
    out = {"y": y, "mask": M, "i0": i0, "i1": i1, "fmt": fmt, "T": T, "K": K, "mask_kind": mask}
    if fmt == "mxfp4":
        sp_codes, sp_e = mx_quantize(X_sp)
        Xt_sp = np.where(M, mx_dequant_f32(sp_codes, sp_e), F32(0.0))
        R = y - Xt_sp
        res_codes, res_e = mx_quantize(R)
        out.update(bb_scale=e8m0_encode_exponent(sp_e), res_scale=e8m0_encode_exponent(res_e),
                   tensor_scales=None)
    elif fmt == "nvfp4":
        s_sp = nv_tensor_scale(np.abs(y).max() if y.size else 0.0)
        sp_codes, sp_sc = nv_quantize(X_sp, NV_BB_BLOCK, s_sp)
        Xt_sp = np.where(M, nv_dequant_f32(sp_codes, sp_sc, NV_BB_BLOCK, s_sp), F32(0.0))
        R = y - Xt_sp
        s_dn = nv_tensor_scale(np.abs(R).max() if R.size else 0.0)
        res_codes, res_sc = nv_quantize(R, NV_RES_BLOCK, s_dn)
        out.update(bb_scale=sp_sc, res_scale=res_sc, tensor_scales=np.array([s_sp, s_dn], dtype=F32))
    else:
        raise ValueError(fmt)
    bb = compact_pairs(sp_codes, i0, i1) if mask == "4:8" else compact_24(sp_codes, i0, i1)
    out.update(X_sp=X_sp, Xt_sp=Xt_sp, R=R,
               bb_codes=bb, bb_meta=meta_bytes(i0, i1),
               res_codes=pack_nibbles(res_codes), sp_codes_full=sp_codes, res_codes_full=res_codes)
    return out


# ----------------------------------------------------------------------------
# weight packer: one payload, two scale views (review §3.5)
# ----------------------------------------------------------------------------
def pack_weight(w: np.ndarray, fmt: str = "mxfp4", tensor_amax=None) -> dict:
    """Quantize W (K x D, fp32 values) column by column, 32 K-values per block,
    into one shared payload (D x K/2) and the sparse (per 32) and dense (per 16,
    each per-32 scale repeated twice) scale views.  NVFP4: ``tensor_amax``
    overrides amax|W| when only some columns of a larger weight are packed."""
    w = np.asarray(w, dtype=F32)
    Wt = np.ascontiguousarray(w.T)                      # D x K
    if fmt == "mxfp4":
        codes, e = mx_quantize(Wt)
        sp = e8m0_encode_exponent(e)
        return {"fmt": fmt, "payload": pack_nibbles(codes), "scale_sp": sp, "scale_dn": sp.copy(),
                "tensor_scale": None, "codes": codes}
    if fmt == "nvfp4":
        if tensor_amax is None:
            tensor_amax = np.abs(w).max() if w.size else 0.0
        s_w = nv_tensor_scale(tensor_amax)
        codes, sc = nv_quantize(Wt, NV_W_BLOCK, s_w)
        return {"fmt": fmt, "payload": pack_nibbles(codes), "scale_sp": sc,
                "scale_dn": np.repeat(sc, 2, axis=-1), "tensor_scale": np.array([s_w], dtype=F32),
                "codes": codes}
    raise ValueError(fmt)


# ----------------------------------------------------------------------------
# dequantized operands
# ----------------------------------------------------------------------------
def act_dequant(act: dict):
    """(X~_sp, R~) as exact fp64 values from the stored layouts."""
    fmt = act["fmt"]
    i0, i1 = meta_unpack(act["bb_meta"])
    if act.get("mask_kind", "4:8") == "2:4":
        sp_codes = expand_24(act["bb_codes"], i0, i1)
        t, g = np.indices(i0.shape)
        keep = np.zeros(i0.shape + (4,), dtype=bool)
        keep[t, g, i0] = True
        keep[t, g, i1] = True
        M = keep.reshape(i0.shape[0], -1)
    else:
        sp_codes = expand_pairs(act["bb_codes"], i0, i1)
        M = mask_from_pairs(i0, i1)
    res_codes = unpack_nibbles(act["res_codes"])
    if fmt == "mxfp4":
        Xt = mx_dequant_f64(sp_codes, e8m0_decode_exponent(act["bb_scale"]))
        Rt = mx_dequant_f64(res_codes, e8m0_decode_exponent(act["res_scale"]))
    else:
        s_sp, s_dn = act["tensor_scales"]
        Xt = nv_dequant_f64(sp_codes, act["bb_scale"], NV_BB_BLOCK, s_sp)
        Rt = nv_dequant_f64(res_codes, act["res_scale"], NV_RES_BLOCK, s_dn)
    return np.where(M, Xt, 0.0), Rt


def weight_dequant(wp: dict, view: str = "sp") -> np.ndarray:
    """W~ (K x D, fp64) from the payload and one scale view."""
    codes = unpack_nibbles(wp["payload"])               # D x K
    if wp["fmt"] == "mxfp4":
        Wt = mx_dequant_f64(codes, e8m0_decode_exponent(wp["scale_" + view]))
    else:
        blk = NV_W_BLOCK if view == "sp" else NV_W_BLOCK // 2
        Wt = nv_dequant_f64(codes, wp["scale_" + view], blk, wp["tensor_scale"][0])
    return Wt.T


# ----------------------------------------------------------------------------
# dual-path GEMM (review §3.4, §3.5 residual accumulation)
# ----------------------------------------------------------------------------
def sharq_linear(act: dict, wp: dict, rows=None):
    """Y^ = GEMM_sp(Q_sp(X_sp), Q_w,sp(W)) + GEMM_dn(Q_dn(R), Q_w,dn(W)) in fp64
    from exact dequantized operands.  Also returns the per-element tolerance
    scale sum_k |x~_k w~_k| with x~ = X~_sp + R~.  ``rows`` optionally gathers
    activation rows (MoE up-projection)."""
    Xt, Rt = act_dequant(act)
    if rows is not None:
        Xt, Rt = Xt[rows], Rt[rows]
    W_sp = weight_dequant(wp, "sp")
    W_dn = weight_dequant(wp, "dn")
    Y = Xt @ W_sp + Rt @ W_dn
    scale = np.abs(Xt + Rt) @ np.abs(W_sp)
    return Y, scale


ACT_ROW_KEYS = ("bb_codes", "bb_meta", "bb_scale", "res_codes", "res_scale")
W_ROW_KEYS = ("payload", "scale_sp", "scale_dn")


def act_rows(act: dict, rows) -> dict:
    """The prepared activation restricted to the given rows."""
    return {k: (v[rows] if k in ACT_ROW_KEYS else v) for k, v in act.items()}


def weight_cols(wp: dict, cols) -> dict:
    """The packed weight restricted to the given output columns."""
    return {k: (v[cols] if k in W_ROW_KEYS else v) for k, v in wp.items()}


def sharq_linear_sampled(act: dict, wp: dict, out_rows, out_cols, rows=None):
    """Y^[out_rows[n], out_cols[n]] and its tolerance scale, for large shapes.
    ``rows`` optionally maps output rows to activation rows (gather)."""
    out_rows = np.asarray(out_rows)
    a_rows = out_rows if rows is None else np.asarray(rows)[out_rows]
    ua, ia = np.unique(a_rows, return_inverse=True)
    uc, ic = np.unique(np.asarray(out_cols), return_inverse=True)
    Xt, Rt = act_dequant(act_rows(act, ua))
    sub = weight_cols(wp, uc)
    W_sp, W_dn = weight_dequant(sub, "sp"), weight_dequant(sub, "dn")
    Y = np.einsum("nk,kn->n", Xt[ia], W_sp[:, ic]) + np.einsum("nk,kn->n", Rt[ia], W_dn[:, ic])
    scale = np.einsum("nk,kn->n", np.abs(Xt[ia] + Rt[ia]), np.abs(W_sp[:, ic]))
    return Y, scale


def grouped_linear(act: dict, wps: list, group_offsets: np.ndarray, row_index=None):
    """MoE: routed row r of expert e (group_offsets[e] <= r < group_offsets[e+1])
    is activation row row_index[r] (or r) times expert e's weights."""
    total = int(group_offsets[-1])
    D = wps[0]["payload"].shape[0]
    Y = np.zeros((total, D))
    S = np.zeros((total, D))
    Xt, Rt = act_dequant(act)
    for e, wp in enumerate(wps):
        a, b = int(group_offsets[e]), int(group_offsets[e + 1])
        if a == b:
            continue
        rows = np.arange(a, b) if row_index is None else row_index[a:b]
        W_sp = weight_dequant(wp, "sp")
        W_dn = weight_dequant(wp, "dn")
        Y[a:b] = Xt[rows] @ W_sp + Rt[rows] @ W_dn
        S[a:b] = np.abs(Xt[rows] + Rt[rows]) @ np.abs(W_sp)
    return Y, S


# ----------------------------------------------------------------------------
# comparison baselines and error report
# ----------------------------------------------------------------------------
def plain_quantized(y: np.ndarray, fmt: str = "mxfp4") -> np.ndarray:
    """Plain (no sparse-dense split) FP4 quantization of y, dequantized (fp64):
    MXFP4 per 32, or NVFP4 per 16 under its tensor scale."""
    if fmt == "mxfp4":
        c, e = mx_quantize(y)
        return mx_dequant_f64(c, e)
    s = nv_tensor_scale(np.abs(y).max())
    c, sc = nv_quantize(y, 16, s)
    return nv_dequant_f64(c, sc, 16, s)


def plain_prepare_mx(x: np.ndarray, gamma, eps: float = 1e-6) -> dict:
    """The unfused pipeline that the fused preparation replaces (review §5,
    kernel latency breakdown): RMSNorm (the pinned order of ``rmsnorm``), then
    plain MXFP4 of y per 32-block (review §3.1, scale rounded up to a power of
    two).  Returns y, the packed codes (T x K/2) and the E8M0 scale bytes
    (T x K/32)."""
    y = rmsnorm(x, gamma, eps)
    c, e = mx_quantize(y)
    return {"y": y, "codes": pack_nibbles(c), "scales": e8m0_encode_exponent(e)}


def plain_linear_mx(codes: np.ndarray, scales: np.ndarray, wp: dict):
    """Plain FP4 GEMM Y = X~ W~ in fp64 from the exact dequantized operand and
    the weight's dense scale view, with the tolerance scale sum_k |x~_k w~_k|."""
    Xt = mx_dequant_f64(unpack_nibbles(codes), e8m0_decode_exponent(scales))
    W = weight_dequant(wp, "dn")
    return Xt @ W, np.abs(Xt) @ np.abs(W)


def plain_linear_mx_sampled(codes: np.ndarray, scales: np.ndarray, wp: dict, out_rows, out_cols):
    """Y[out_rows[n], out_cols[n]] of ``plain_linear_mx`` for large shapes."""
    ur, ir = np.unique(np.asarray(out_rows), return_inverse=True)
    uc, ic = np.unique(np.asarray(out_cols), return_inverse=True)
    Xt = mx_dequant_f64(unpack_nibbles(codes[ur]), e8m0_decode_exponent(scales[ur]))
    W = weight_dequant(weight_cols(wp, uc), "dn")
    Y = np.einsum("nk,kn->n", Xt[ir], W[:, ic])
    S = np.einsum("nk,kn->n", np.abs(Xt[ir]), np.abs(W[:, ic]))
    return Y, S


def _sparse_quantized(v: np.ndarray, fmt: str, f64: bool = False, mask: str = "4:8") -> np.ndarray:
    """4:8 in-pairs sparsification of ``v`` (the pair-top-2 rule of
    ``pair_top2``) and backbone-style quantization of the kept values
    (MXFP4 per 32; NVFP4 E4M3 per 32 logical positions under the tensor scale
    of amax(v)), dequantized (fp32 as the preparation rounds it, or the exact
    fp64 value the GEMM multiplies) with zeros at dropped positions."""
    M = mask_from_pairs(*pair_top2(v)) if mask == "4:8" else nm_keep(v, 2, 4)
    vs = np.where(M, v, F32(0.0))
    if fmt == "mxfp4":
        c, e = mx_quantize(vs)
        q = mx_dequant_f64(c, e) if f64 else mx_dequant_f32(c, e)
    else:
        s = nv_tensor_scale(np.abs(v).max() if v.size else 0.0)
        c, sc = nv_quantize(vs, NV_BB_BLOCK, s)
        q = nv_dequant_f64(c, sc, NV_BB_BLOCK, s) if f64 else nv_dequant_f32(c, sc, NV_BB_BLOCK, s)
    return np.where(M, q, 0.0)


def _dense_quantized(v: np.ndarray, fmt: str, f64: bool = False) -> np.ndarray:
    """Dense quantization of ``v`` as the residual path does it (MXFP4 per 32;
    NVFP4 E4M3 per 16 under the tensor scale of amax(v)), dequantized in fp32
    or exactly in fp64."""
    if fmt == "mxfp4":
        c, e = mx_quantize(v)
        return mx_dequant_f64(c, e) if f64 else mx_dequant_f32(c, e)
    s = nv_tensor_scale(np.abs(v).max() if v.size else 0.0)
    c, sc = nv_quantize(v, NV_RES_BLOCK, s)
    return nv_dequant_f64(c, sc, NV_RES_BLOCK, s) if f64 else nv_dequant_f32(c, sc, NV_RES_BLOCK, s)


def decomposition_pieces(x: np.ndarray, gamma, fmt: str = "mxfp4", eps: float = 1e-6) -> dict:
    """The quantized pieces of the review's Table 5 path combinations
    (review §5.3) for the activation rows x: y = RMSNorm(x) and, each as
    the exact fp64 values the GEMM multiplies,
      sparse_first   X~_sp: the 4:8 in-pairs backbone of ``prepare``
      sparse_second  Q_sp(M'(R) ⊙ R): the pair-top-2 rule applied again to
                     R = y - X~_sp and quantized like a backbone
      dense_residual Q_dn(R): SharQ's dense residual path
      dense_first    Q(y): y quantized densely
      dense_second   Q(y - Q(y)): the residual of the dense first path,
                     quantized densely
    plus the fp32 inputs of the second paths (R and y - Q(y), exact by
    Sterbenz as for R) and, for MXFP4, the 2:4 element-wise backbone and its
    dense residual.  Every residual is taken against the quantized first path
    (review §3.3)."""
    prep = prepare(x, gamma, eps, fmt)
    y, R = prep["y"], prep["R"]
    q1 = _dense_quantized(y, fmt)                       # fp32, the dense residual's reference
    out = {"y": y, "prep": prep, "R": R, "y_minus_q": y - q1,
           "sparse_first": _sparse_quantized(y, fmt, f64=True),
           "sparse_second": _sparse_quantized(R, fmt, f64=True),
           "dense_residual": _dense_quantized(R, fmt, f64=True),
           "dense_first": _dense_quantized(y, fmt, f64=True),
           "dense_second": _dense_quantized(y - q1, fmt, f64=True)}
    if fmt == "mxfp4":                                  # the pages' MXFP4 pattern, 2:4 element-wise
        sp24 = _sparse_quantized(y, fmt, mask="2:4")
        out["sparse_first_24"] = _sparse_quantized(y, fmt, f64=True, mask="2:4")
        out["dense_residual_24"] = _dense_quantized(y - sp24, fmt, f64=True)
    return out


def decomposition_study(x: np.ndarray, gamma, w: np.ndarray, fmt: str = "mxfp4", eps: float = 1e-6,
                        wp: dict = None) -> dict:
    """Operator-level analogue of the review's Table 5 (sparse / dense path
    combinations): relative Frobenius error against the unquantized y W
    (fp64) of X^ W~ (packed FP4 weights, "weights_fp4") and of X^ W
    ("activation_only") for the activation approximations
      sparse_only   X~_sp                    (the residual dropped)
      sparse_sparse X~_sp + Q_sp(M'(R) ⊙ R)  (the residual also 4:8-sparse)
      dense_dense   Q(y) + Q(y - Q(y))       (both paths dense)
      sharq         X~_sp + Q_dn(R)          (sparse backbone, dense residual)
      plain         Q(y)                     (one dense FP4 path)
    and, for MXFP4, sparse_only_2:4 and sharq_2:4 with a 2:4 element-wise
    backbone mask instead of 4:8 in pairs, built from the pieces of
    ``decomposition_pieces``.  W~ is the packed weight.  ``wp``: W already
    packed (``pack_weight(w, fmt)``), to skip packing it again."""
    pc = decomposition_pieces(x, gamma, fmt, eps)
    y = pc["y"]
    W = weight_dequant(wp if wp is not None else pack_weight(w, fmt), "dn")
    ref = y.astype(np.float64) @ np.asarray(w, dtype=np.float64)
    approx = {
        "sparse_only": pc["sparse_first"],
        "sparse_sparse": pc["sparse_first"] + pc["sparse_second"],
        "dense_dense": pc["dense_first"] + pc["dense_second"],
        "sharq": pc["sparse_first"] + pc["dense_residual"],
        "plain": plain_quantized(y, fmt),
    }
    if fmt == "mxfp4":
        approx["sparse_only_2:4"] = pc["sparse_first_24"]
        approx["sharq_2:4"] = pc["sparse_first_24"] + pc["dense_residual_24"]
    Wf = np.asarray(w, dtype=np.float64)
    return {"weights_fp4": {k: rel_frobenius(v @ W, ref) for k, v in approx.items()},
            "activation_only": {k: rel_frobenius(v @ Wf, ref) for k, v in approx.items()}}


def rel_frobenius(Y_hat: np.ndarray, Y_ref: np.ndarray) -> float:
    return float(np.linalg.norm(Y_hat - Y_ref) / np.linalg.norm(Y_ref))


def error_bound_terms(act: dict, prep: dict, wp: dict):
    """(lhs, rhs) of review §3.6: ||y W~ - (X~_sp + R~) W~||_F and
    ||R - R~||_F * ||W~||_2 (fp64, spectral norm by SVD)."""
    Xt, Rt = act_dequant(act)
    W = weight_dequant(wp, "sp")
    y = prep["y"].astype(np.float64)
    lhs = np.linalg.norm(y @ W - (Xt + Rt) @ W)
    rhs = np.linalg.norm(prep["R"].astype(np.float64) - Rt) * np.linalg.norm(W, 2)
    return lhs, rhs
