"""Python binding of libmoe_fp8.so, the gfx950 DeepSeekMoE layer-forward library.

Argument marshalling only: every function below checks tensor placement, dtype and
shape, then calls the C entry point of the same name (declared in include/moe_fp8.h)
on the current HIP stream. All arithmetic happens in the library's HIP kernels; torch
only provides device memory and streams. A missing or unloadable library raises at
import time — there is no fallback.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmoe_fp8.so")

if not os.path.exists(LIB_PATH):
    raise ImportError(
        f"{LIB_PATH} is missing: build it with `python deepseekmoe_routing_fp8_amd/build.py`")
_lib = ctypes.CDLL(LIB_PATH)

MOE_F32, MOE_BF16 = 0, 1

ENTRY_POINTS = (
    "moe_status_string", "moe_quantize_1x128", "moe_quantize_128x128", "moe_quantize_1x128_pow2",
    "moe_quantize_128x128_pow2", "moe_pack_fp8_weights",
    "moe_pack_router_weights", "moe_router_weights_elems", "moe_route", "moe_route_workspace_bytes",
    "moe_permute", "moe_permute_workspace_bytes", "moe_grouped_ffn_workspace_bytes", "moe_grouped_ffn_fp8",
    "moe_grouped_ffn_fp8_gate_up", "moe_grouped_ffn_fp8_down", "moe_combine",
    "moe_update_bias", "moe_seq_balance", "moe_seq_balance_workspace_bytes",
    "moe_combine_backward", "moe_route_backward", "moe_route_backward_workspace_bytes",
    "moe_unpermute_sum", "moe_transpose_fp8_blocks", "moe_grouped_ffn_fp8_backward",
    "moe_grouped_ffn_backward_workspace_bytes", "moe_grouped_ffn_intermediate_offsets",
    "moe_grouped_ffn_fp8_noalloc", "moe_grouped_ffn_fp8_gate_up_train",
)
MOE_ERR_SCRATCH = 7
NOALLOC_SCRATCH_BYTES = 32 << 20   # MOE_NOALLOC_SCRATCH_BYTES


class moe_config(ctypes.Structure):
    _fields_ = [
        ("hidden", ctypes.c_int32), ("inter", ctypes.c_int32),
        ("n_routed", ctypes.c_int32), ("n_shared", ctypes.c_int32),
        ("top_k", ctypes.c_int32), ("n_group", ctypes.c_int32),
        ("topk_group", ctypes.c_int32), ("group_topn", ctypes.c_int32),
        ("routed_scaling", ctypes.c_float), ("bias_gamma", ctypes.c_float),
        ("scale_mode", ctypes.c_int32),
    ]

SCALE_FP32, SCALE_POW2 = 0, 1


def make_config(cfg, scale_mode: int = SCALE_FP32) -> moe_config:
    """moe_config from any object with the synth.MoEConfig field names. ``scale_mode``:
    SCALE_FP32 (the pages' FP32 group scales) or SCALE_POW2 (the opt-in variant)."""
    return moe_config(cfg.hidden_size, cfg.moe_intermediate_size, cfg.num_experts,
                      cfg.num_shared_experts, cfg.num_experts_per_tok, cfg.n_group,
                      cfg.topk_group, cfg.group_score_topn, cfg.routed_scaling_factor,
                      cfg.expert_bias_update_rate, scale_mode)


_P, _I64, _I32, _SZ = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_size_t
_CFG = ctypes.POINTER(moe_config)
_sig = {
    "moe_status_string": ([ctypes.c_int], ctypes.c_char_p),
    "moe_quantize_1x128": ([_P, ctypes.c_int, _I64, _I64, _P, _P, _P], ctypes.c_int),
    "moe_quantize_128x128": ([_P, _I64, _I64, _I64, _P, _P, _P], ctypes.c_int),
    "moe_quantize_1x128_pow2": ([_P, ctypes.c_int, _I64, _I64, _P, _P, _P], ctypes.c_int),
    "moe_quantize_128x128_pow2": ([_P, _I64, _I64, _I64, _P, _P, _P], ctypes.c_int),
    "moe_pack_fp8_weights": ([_P, _I64, _I64, _I64, _P, _P], ctypes.c_int),
    "moe_pack_router_weights": ([_P, _I64, _I64, _P, _P], ctypes.c_int),
    "moe_router_weights_elems": ([_I64, _I64], _SZ),
    "moe_route": ([_CFG, _P, ctypes.c_int, _I64, _P, _P, _P, _P, _P, _P, _P, _SZ, _P], ctypes.c_int),
    "moe_route_workspace_bytes": ([_CFG, _I64, ctypes.c_int], _SZ),
    "moe_permute": ([_CFG, _I64, _P, _P, _P, _P, _P, _SZ, _P], ctypes.c_int),
    "moe_permute_workspace_bytes": ([_CFG, _I64], _SZ),
    "moe_grouped_ffn_workspace_bytes": ([_CFG, _I32, _I64], _SZ),
    "moe_grouped_ffn_fp8": ([_CFG, _I32, _I64, _I64, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P,
                             _P, ctypes.c_int, _P, _SZ, _P], ctypes.c_int),
    "moe_grouped_ffn_intermediate_offsets": ([_CFG, _I32, _I64, ctypes.POINTER(_SZ),
                                              ctypes.POINTER(_SZ)], ctypes.c_int),
    "moe_grouped_ffn_fp8_noalloc": ([_CFG, _I32, _I64, _I64, _P, _P, _P, _P, _P, _P, _P, _P, _P,
                                     _P, _P, ctypes.c_int, _P], ctypes.c_int),
    "moe_grouped_ffn_fp8_gate_up": ([_CFG, _I32, _I64, _I64, _P, _P, _P, _P, _P, _P, _P, _P,
                                     _P, _SZ, _P], ctypes.c_int),
    "moe_grouped_ffn_fp8_gate_up_train": ([_CFG, _I32, _I64, _I64, _P, _P, _P, _P, _P, _P, _P,
                                           _P, _P, _P, _P, _SZ, _P], ctypes.c_int),
    "moe_grouped_ffn_fp8_down": ([_CFG, _I32, _I64, _P, _P, _P, ctypes.c_int, _P, _SZ, _P],
                                 ctypes.c_int),
    "moe_combine": ([_CFG, _I64, _P, ctypes.c_int, _P, _P, _P, _P, _P], ctypes.c_int),
    "moe_update_bias": ([_CFG, _I64, _P, _P, _P], ctypes.c_int),
    "moe_seq_balance": ([_CFG, _I64, _I64, _P, _P, ctypes.c_float, _P, _P, _P, _SZ, _P],
                        ctypes.c_int),
    "moe_seq_balance_workspace_bytes": ([_CFG, _I64, _I64], _SZ),
    "moe_combine_backward": ([_CFG, _I64, _P, _P, ctypes.c_int, _P, _P, _P, _P, _P], ctypes.c_int),
    "moe_route_backward_workspace_bytes": ([_CFG, _I64], _SZ),
    "moe_route_backward": ([_CFG, _I64, _P, ctypes.c_int, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P,
                            _SZ, _P], ctypes.c_int),
    "moe_unpermute_sum": ([_CFG, _I64, _P, ctypes.c_int, _P, _P, _P, _P], ctypes.c_int),
    "moe_transpose_fp8_blocks": ([_I64, _I64, _I64, _P, _P, _P, _P, _I64, _I64, _P], ctypes.c_int),
    "moe_grouped_ffn_backward_workspace_bytes": ([_CFG, _I32, _I64], _SZ),
    "moe_grouped_ffn_fp8_backward": ([_CFG, _I32, _I64, _I64, _P, _P, _P, ctypes.c_int, _P, _P, _P,
                                      _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, ctypes.c_int,
                                      _P, _P, _P, ctypes.c_int, _P, _SZ, _P], ctypes.c_int),
}
for _name, (_args, _res) in _sig.items():
    _f = getattr(_lib, _name)
    _f.argtypes = _args
    _f.restype = _res


class MoEError(RuntimeError):
    pass


def _check(status: int, what: str):
    if status != 0:
        raise MoEError(f"{what}: {_lib.moe_status_string(status).decode()} (status {status})")


def _stream(stream) -> Optional[int]:
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream


def _dev(t: torch.Tensor, dtype, name: str, shape=None):
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise MoEError(f"{name} must be a device tensor")
    if t.dtype != dtype:
        raise MoEError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise MoEError(f"{name} must be contiguous")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise MoEError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    return ctypes.c_void_p(t.data_ptr())


def _opt(t: Optional[torch.Tensor], dtype, name: str, shape=None):
    """_dev, or a NULL pointer for None."""
    return ctypes.c_void_p(0) if t is None else _dev(t, dtype, name, shape)


def _xdtype(x: torch.Tensor) -> int:
    if x.dtype == torch.bfloat16:
        return MOE_BF16
    if x.dtype == torch.float32:
        return MOE_F32
    raise MoEError(f"unsupported activation dtype {x.dtype}")


def moe_quantize_1x128(x: torch.Tensor, q: torch.Tensor = None, scales: torch.Tensor = None,
                       stream=None, pow2: bool = False):
    """1x128 E4M3 quantisation of x [rows, cols] -> (q uint8 [rows, cols], scales f32).
    ``pow2``: power-of-two scales (moe_quantize_1x128_pow2)."""
    rows, cols = x.shape
    q = torch.empty((rows, cols), dtype=torch.uint8, device=x.device) if q is None else q
    if scales is None:
        scales = torch.empty((rows, max(cols // 128, 0)), dtype=torch.float32, device=x.device)
    name = "moe_quantize_1x128_pow2" if pow2 else "moe_quantize_1x128"
    _check(getattr(_lib, name)(_dev(x, x.dtype, "x"), _xdtype(x), rows, cols,
                               _dev(q, torch.uint8, "q", (rows, cols)),
                               _dev(scales, torch.float32, "scales"), _stream(stream)), name)
    return q, scales


def moe_quantize_128x128(w: torch.Tensor, q: torch.Tensor = None, scales: torch.Tensor = None,
                         stream=None, pow2: bool = False):
    """128x128-block E4M3 quantisation of w [mats, rows, cols] (or [rows, cols]) float32.
    ``pow2``: power-of-two scales (moe_quantize_128x128_pow2)."""
    squeeze = w.dim() == 2
    w3 = w.unsqueeze(0) if squeeze else w
    mats, rows, cols = w3.shape
    if q is None:
        q = torch.empty(w.shape, dtype=torch.uint8, device=w.device)
    if scales is None:
        sshape = (rows // 128, cols // 128) if squeeze else (mats, rows // 128, cols // 128)
        scales = torch.empty(sshape, dtype=torch.float32, device=w.device)
    name = "moe_quantize_128x128_pow2" if pow2 else "moe_quantize_128x128"
    _check(getattr(_lib, name)(_dev(w, torch.float32, "w"), mats, rows, cols,
                               _dev(q, torch.uint8, "q", w.shape),
                               _dev(scales, torch.float32, "scales"), _stream(stream)), name)
    return q, scales


def moe_pack_fp8_weights(q: torch.Tensor, packed: torch.Tensor = None, stream=None):
    """Re-lay E4M3 codes q [mats, rows, cols] (or [rows, cols]) into the fragment-packed
    layout the grouped FFN reads; returns a tensor of q's shape holding the packed bytes."""
    q3 = q.unsqueeze(0) if q.dim() == 2 else q
    mats, rows, cols = q3.shape
    packed = torch.empty_like(q) if packed is None else packed
    _check(_lib.moe_pack_fp8_weights(_dev(q, torch.uint8, "q"), mats, rows, cols,
                                     _dev(packed, torch.uint8, "packed", q.shape), _stream(stream)),
           "moe_pack_fp8_weights")
    return packed


def moe_router_weights_elems(n_routed: int, hidden: int) -> int:
    return int(_lib.moe_router_weights_elems(n_routed, hidden))


def moe_pack_router_weights(w_router: torch.Tensor, out: torch.Tensor = None, stream=None):
    """FP32 router weight [N_r, H] -> packed bf16 planes (hi + mid + lo == W_r) in the MFMA
    fragment order moe_route reads (a flat tensor of moe_router_weights_elems elements)."""
    N, H = w_router.shape
    n = moe_router_weights_elems(N, H)
    if n == 0:
        raise MoEError("moe_pack_router_weights: unsupported shape")
    out = torch.empty((n,), dtype=torch.bfloat16, device=w_router.device) if out is None else out
    _check(_lib.moe_pack_router_weights(_dev(w_router, torch.float32, "w_router", (N, H)), N, H,
                                        _dev(out, torch.bfloat16, "w_split", (n,)),
                                        _stream(stream)), "moe_pack_router_weights")
    return out


def moe_route_workspace_bytes(cfg: moe_config, T: int, xt: int) -> int:
    return int(_lib.moe_route_workspace_bytes(ctypes.byref(cfg), T, xt))


def moe_route(cfg: moe_config, x: torch.Tensor, w_router: torch.Tensor, bias: torch.Tensor,
              scores: torch.Tensor = None, topk_idx: torch.Tensor = None,
              topk_gate: torch.Tensor = None, counts: torch.Tensor = None,
              ws: torch.Tensor = None, stream=None):
    """Router: -> (scores [T,N_r] f32, topk_idx [T,k] i32, topk_gate [T,k] f32, counts i32).

    ``w_router`` is the packed split from moe_pack_router_weights; ``ws`` a workspace of
    moe_route_workspace_bytes bytes (allocated here when None)."""
    T = x.shape[0]
    N, k = cfg.n_routed, cfg.top_k
    dev = x.device
    scores = torch.empty((T, N), dtype=torch.float32, device=dev) if scores is None else scores
    topk_idx = torch.empty((T, k), dtype=torch.int32, device=dev) if topk_idx is None else topk_idx
    topk_gate = torch.empty((T, k), dtype=torch.float32, device=dev) if topk_gate is None else topk_gate
    counts = torch.empty((N,), dtype=torch.int32, device=dev) if counts is None else counts
    need = moe_route_workspace_bytes(cfg, T, _xdtype(x))
    if ws is None:
        ws = torch.empty((max(need, 1),), dtype=torch.uint8, device=dev)
    _check(_lib.moe_route(ctypes.byref(cfg), _dev(x, x.dtype, "x", (T, cfg.hidden)), _xdtype(x), T,
                          _dev(w_router, torch.bfloat16, "w_router_split",
                               (moe_router_weights_elems(N, cfg.hidden),)),
                          _dev(bias, torch.float32, "bias", (N,)),
                          _dev(scores, torch.float32, "scores", (T, N)),
                          _dev(topk_idx, torch.int32, "topk_idx", (T, k)),
                          _dev(topk_gate, torch.float32, "topk_gate", (T, k)),
                          _dev(counts, torch.int32, "counts", (N,)),
                          _dev(ws, torch.uint8, "ws"), ws.numel(), _stream(stream)),
           "moe_route")
    return scores, topk_idx, topk_gate, counts


def moe_permute_workspace_bytes(cfg: moe_config, T: int) -> int:
    return int(_lib.moe_permute_workspace_bytes(ctypes.byref(cfg), T))


def moe_permute(cfg: moe_config, topk_idx: torch.Tensor, offsets: torch.Tensor = None,
                row_token: torch.Tensor = None, row_of: torch.Tensor = None,
                ws: torch.Tensor = None, stream=None):
    """-> (offsets [N_r+N_s+1], row_token [T*(k+N_s)], row_of [T,k]), all int32. The
    shared experts follow the routed ones as segments of T rows in token order."""
    T, k = topk_idx.shape
    S = cfg.n_shared
    dev = topk_idx.device
    if offsets is None:
        offsets = torch.empty((cfg.n_routed + S + 1,), dtype=torch.int32, device=dev)
    if row_token is None:
        row_token = torch.empty((T * (k + S),), dtype=torch.int32, device=dev)
    row_of = torch.empty((T, k), dtype=torch.int32, device=dev) if row_of is None else row_of
    if ws is None:
        ws = torch.empty((max(moe_permute_workspace_bytes(cfg, T), 1),), dtype=torch.uint8, device=dev)
    _check(_lib.moe_permute(ctypes.byref(cfg), T, _dev(topk_idx, torch.int32, "topk_idx", (T, cfg.top_k)),
                            _dev(offsets, torch.int32, "offsets", (cfg.n_routed + S + 1,)),
                            _dev(row_token, torch.int32, "row_token", (T * (k + S),)),
                            _dev(row_of, torch.int32, "row_of", (T, k)),
                            _dev(ws, torch.uint8, "ws"), ws.numel(), _stream(stream)),
           "moe_permute")
    return offsets, row_token, row_of


def moe_grouped_ffn_workspace_bytes(cfg: moe_config, n_experts: int, n_rows: int) -> int:
    return int(_lib.moe_grouped_ffn_workspace_bytes(ctypes.byref(cfg), n_experts, n_rows))


def _ffn_ws(cfg, n_experts, n_rows, ws, dev):
    need = moe_grouped_ffn_workspace_bytes(cfg, n_experts, n_rows)
    if ws is None:
        ws = torch.empty((max(need, 1),), dtype=torch.uint8, device=dev)
    return ws


def _gate_up_args(cfg, n_experts, n_rows, xq, xs, row_token, offsets, w1, w1s, w3, w3s):
    H, I, E = cfg.hidden, cfg.inter, n_experts
    n_tokens = xq.shape[0]
    rt = ctypes.c_void_p(0) if row_token is None else _dev(row_token, torch.int32, "row_token")
    return (E, n_rows, n_tokens, _dev(xq, torch.uint8, "xq", (n_tokens, H)),
            _dev(xs, torch.float32, "xs", (n_tokens, H // 128)), rt,
            _dev(offsets, torch.int32, "offsets", (E + 1,)),
            _dev(w1, torch.uint8, "w1", (E, I, H)), _dev(w1s, torch.float32, "w1s", (E, I // 128, H // 128)),
            _dev(w3, torch.uint8, "w3", (E, I, H)), _dev(w3s, torch.float32, "w3s", (E, I // 128, H // 128)))


def _down_args(cfg, n_experts, n_rows, w2, w2s, y):
    H, I, E = cfg.hidden, cfg.inter, n_experts
    yt = MOE_BF16 if y.dtype == torch.bfloat16 else MOE_F32
    return (_dev(w2, torch.uint8, "w2", (E, H, I)), _dev(w2s, torch.float32, "w2s", (E, H // 128, I // 128)),
            _dev(y, y.dtype, "y", (n_rows, H)), yt)


def moe_grouped_ffn_fp8(cfg: moe_config, n_experts: int, n_rows: int, xq: torch.Tensor,
                        xs: torch.Tensor, row_token: Optional[torch.Tensor], offsets: torch.Tensor,
                        w1, w1s, w3, w3s, w2, w2s, y: torch.Tensor = None,
                        ws: torch.Tensor = None, y_dtype=torch.bfloat16, stream=None):
    """Grouped SwiGLU FP8 experts -> y [n_rows, H] (bf16 or f32)."""
    dev = xq.device
    if y is None:
        y = torch.empty((n_rows, cfg.hidden), dtype=y_dtype, device=dev)
    ws = _ffn_ws(cfg, n_experts, n_rows, ws, dev)
    _check(_lib.moe_grouped_ffn_fp8(
        ctypes.byref(cfg), *_gate_up_args(cfg, n_experts, n_rows, xq, xs, row_token, offsets,
                                          w1, w1s, w3, w3s),
        *_down_args(cfg, n_experts, n_rows, w2, w2s, y), _dev(ws, torch.uint8, "ws"), ws.numel(),
        _stream(stream)), "moe_grouped_ffn_fp8")
    return y


def moe_grouped_ffn_fp8_noalloc(cfg: moe_config, n_experts: int, n_rows: int, xq: torch.Tensor,
                                xs: torch.Tensor, row_token: Optional[torch.Tensor],
                                offsets: torch.Tensor, w1, w1s, w3, w3s, w2, w2s,
                                y: torch.Tensor = None, y_dtype=torch.bfloat16, stream=None):
    """moe_grouped_ffn_fp8 on the library's static scratch array (no workspace, no
    allocation inside the call when ``y`` is given) -> y [n_rows, H]."""
    if y is None:
        y = torch.empty((n_rows, cfg.hidden), dtype=y_dtype, device=xq.device)
    _check(_lib.moe_grouped_ffn_fp8_noalloc(
        ctypes.byref(cfg), *_gate_up_args(cfg, n_experts, n_rows, xq, xs, row_token, offsets,
                                          w1, w1s, w3, w3s),
        *_down_args(cfg, n_experts, n_rows, w2, w2s, y), _stream(stream)), "moe_grouped_ffn_fp8_noalloc")
    return y


def moe_grouped_ffn_intermediate_offsets(cfg: moe_config, n_experts: int, n_rows: int):
    """Byte offsets (hq, hs) of the quantised intermediate inside a grouped-FFN workspace."""
    hq, hs = _SZ(0), _SZ(0)
    _check(_lib.moe_grouped_ffn_intermediate_offsets(ctypes.byref(cfg), n_experts, n_rows,
                                                     ctypes.byref(hq), ctypes.byref(hs)),
           "moe_grouped_ffn_intermediate_offsets")
    return int(hq.value), int(hs.value)


def grouped_ffn_intermediate(cfg: moe_config, n_experts: int, n_rows: int, ws: torch.Tensor):
    """Views of the quantised intermediate in a grouped-FFN workspace: hq [n_rows, I] uint8
    codes and hs [I/128, n_rows] float32 scales (chunk-major)."""
    hq_off, hs_off = moe_grouped_ffn_intermediate_offsets(cfg, n_experts, n_rows)
    I = cfg.inter
    hq = ws[hq_off:hq_off + n_rows * I].view(n_rows, I)
    hs = ws[hs_off:hs_off + n_rows * (I // 128) * 4].view(torch.float32).view(I // 128, n_rows)
    return hq, hs


def moe_grouped_ffn_fp8_gate_up(cfg: moe_config, n_experts: int, n_rows: int, xq: torch.Tensor,
                                xs: torch.Tensor, row_token: Optional[torch.Tensor],
                                offsets: torch.Tensor, w1, w1s, w3, w3s, ws: torch.Tensor = None,
                                stream=None):
    """First half of the grouped FFN; returns the workspace holding the tile plan and the
    quantised intermediate for moe_grouped_ffn_fp8_down."""
    ws = _ffn_ws(cfg, n_experts, n_rows, ws, xq.device)
    _check(_lib.moe_grouped_ffn_fp8_gate_up(
        ctypes.byref(cfg), *_gate_up_args(cfg, n_experts, n_rows, xq, xs, row_token, offsets,
                                          w1, w1s, w3, w3s),
        _dev(ws, torch.uint8, "ws"), ws.numel(), _stream(stream)), "moe_grouped_ffn_fp8_gate_up")
    return ws


def moe_grouped_ffn_fp8_gate_up_train(cfg: moe_config, n_experts: int, n_rows: int,
                                      xq: torch.Tensor, xs: torch.Tensor,
                                      row_token: Optional[torch.Tensor], offsets: torch.Tensor,
                                      w1, w1s, w3, w3s, a: torch.Tensor = None,
                                      b: torch.Tensor = None, ws: torch.Tensor = None, stream=None):
    """moe_grouped_ffn_fp8_gate_up that also keeps the SwiGLU inputs -> (ws, a, b), with
    a, b [n_rows, I] float32 for moe_grouped_ffn_fp8_backward."""
    dev = xq.device
    ws = _ffn_ws(cfg, n_experts, n_rows, ws, dev)
    a = torch.empty((n_rows, cfg.inter), dtype=torch.float32, device=dev) if a is None else a
    b = torch.empty((n_rows, cfg.inter), dtype=torch.float32, device=dev) if b is None else b
    _check(_lib.moe_grouped_ffn_fp8_gate_up_train(
        ctypes.byref(cfg), *_gate_up_args(cfg, n_experts, n_rows, xq, xs, row_token, offsets,
                                          w1, w1s, w3, w3s),
        _dev(a, torch.float32, "a", (n_rows, cfg.inter)), _dev(b, torch.float32, "b", (n_rows, cfg.inter)),
        _dev(ws, torch.uint8, "ws"), ws.numel(), _stream(stream)), "moe_grouped_ffn_fp8_gate_up_train")
    return ws, a, b


def moe_grouped_ffn_fp8_down(cfg: moe_config, n_experts: int, n_rows: int, w2, w2s,
                             ws: torch.Tensor, y: torch.Tensor = None, y_dtype=torch.bfloat16,
                             stream=None):
    """Second half of the grouped FFN, from the workspace of the gate_up call -> y."""
    if y is None:
        y = torch.empty((n_rows, cfg.hidden), dtype=y_dtype, device=w2.device)
    _check(_lib.moe_grouped_ffn_fp8_down(
        ctypes.byref(cfg), n_experts, n_rows, *_down_args(cfg, n_experts, n_rows, w2, w2s, y),
        _dev(ws, torch.uint8, "ws"), ws.numel(), _stream(stream)), "moe_grouped_ffn_fp8_down")
    return y


def moe_combine(cfg: moe_config, y_rows: torch.Tensor, row_of: torch.Tensor,
                topk_gate: torch.Tensor, y_shared: Optional[torch.Tensor],
                out: torch.Tensor = None, stream=None):
    """-> out [T, H] bf16 = sum of shared outputs + sum_j gate_j * y_rows[row_of[:, j]]."""
    T, k = row_of.shape
    H = cfg.hidden
    out = torch.empty((T, H), dtype=torch.bfloat16, device=row_of.device) if out is None else out
    yt = MOE_BF16 if y_rows.dtype == torch.bfloat16 else MOE_F32
    ys = ctypes.c_void_p(0)
    if y_shared is not None:
        ys = _dev(y_shared, y_rows.dtype, "y_shared")
        if y_shared.numel() != cfg.n_shared * T * H:
            raise MoEError("y_shared must hold [N_s, T, H]")
    _check(_lib.moe_combine(ctypes.byref(cfg), T, _dev(y_rows, y_rows.dtype, "y_rows"), yt,
                            _dev(row_of, torch.int32, "row_of", (T, cfg.top_k)),
                            _dev(topk_gate, torch.float32, "topk_gate", (T, cfg.top_k)), ys,
                            _dev(out, torch.bfloat16, "out", (T, H)), _stream(stream)),
           "moe_combine")
    return out


def moe_update_bias(cfg: moe_config, T: int, counts: torch.Tensor, bias: torch.Tensor, stream=None):
    """In-place sign-based update of bias [N_r] from counts [N_r]."""
    _check(_lib.moe_update_bias(ctypes.byref(cfg), T,
                                _dev(counts, torch.int32, "counts", (cfg.n_routed,)),
                                _dev(bias, torch.float32, "bias", (cfg.n_routed,)), _stream(stream)),
           "moe_update_bias")
    return bias


def moe_seq_balance_workspace_bytes(cfg: moe_config, T: int, seq_len: int) -> int:
    return int(_lib.moe_seq_balance_workspace_bytes(ctypes.byref(cfg), T, seq_len))


def moe_seq_balance(cfg: moe_config, scores: torch.Tensor, topk_idx: torch.Tensor, seq_len: int,
                    alpha: float = 0.001, loss: torch.Tensor = None, entropy: torch.Tensor = None,
                    with_entropy: bool = True, ws: torch.Tensor = None, stream=None):
    """Per-sequence balance loss and allocation entropy over sequences of seq_len
    consecutive tokens -> (loss [T/seq_len], entropy [T/seq_len] or None), float32."""
    T = scores.shape[0]
    dev = scores.device
    nseq = T // seq_len if seq_len > 0 else 0
    if loss is None:
        loss = torch.empty((nseq,), dtype=torch.float32, device=dev)
    if entropy is None and with_entropy:
        entropy = torch.empty((nseq,), dtype=torch.float32, device=dev)
    if ws is None:
        ws = torch.empty((max(moe_seq_balance_workspace_bytes(cfg, T, seq_len), 1),),
                         dtype=torch.uint8, device=dev)
    _check(_lib.moe_seq_balance(
        ctypes.byref(cfg), T, seq_len, _dev(scores, torch.float32, "scores", (T, cfg.n_routed)),
        _dev(topk_idx, torch.int32, "topk_idx", (T, cfg.top_k)), alpha,
        _dev(loss, torch.float32, "loss", (nseq,)),
        _dev(entropy, torch.float32, "entropy", (nseq,)) if entropy is not None else None,
        _dev(ws, torch.uint8, "ws"), ws.numel(), _stream(stream)), "moe_seq_balance")
    return loss, entropy


# ---------------------------------------------------------------------------------------
# Backward
# ---------------------------------------------------------------------------------------
def _dt(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return MOE_BF16
    if t.dtype == torch.float32:
        return MOE_F32
    raise MoEError(f"unsupported dtype {t.dtype}")


def moe_combine_backward(cfg: moe_config, dout: torch.Tensor, y_rows: torch.Tensor,
                         row_of: torch.Tensor, topk_gate: torch.Tensor,
                         row_gate: torch.Tensor = None, dgate: torch.Tensor = None, stream=None):
    """-> (row_gate [T*(k+N_s)] f32, dgate [T, k] f32) from dout [T, H] bf16. The rows'
    upstream gradient is row_gate[r] * dout[token(r)], formed by the FFN backward."""
    T, H = dout.shape
    k, S = cfg.top_k, cfg.n_shared
    dev = dout.device
    row_gate = torch.empty((T * (k + S),), dtype=torch.float32, device=dev) if row_gate is None else row_gate
    dgate = torch.empty((T, k), dtype=torch.float32, device=dev) if dgate is None else dgate
    _check(_lib.moe_combine_backward(
        ctypes.byref(cfg), T, _dev(dout, torch.bfloat16, "dout", (T, cfg.hidden)),
        _dev(y_rows, y_rows.dtype, "y_rows", (T * (k + S), H)), _dt(y_rows),
        _dev(row_of, torch.int32, "row_of", (T, k)), _dev(topk_gate, torch.float32, "topk_gate", (T, k)),
        _dev(row_gate, torch.float32, "row_gate", (T * (k + S),)), _dev(dgate, torch.float32, "dgate", (T, k)),
        _stream(stream)), "moe_combine_backward")
    return row_gate, dgate


def moe_route_backward_workspace_bytes(cfg: moe_config, T: int) -> int:
    return int(_lib.moe_route_backward_workspace_bytes(ctypes.byref(cfg), T))


def moe_route_backward(cfg: moe_config, x: torch.Tensor, w_router: torch.Tensor, scores: torch.Tensor,
                       topk_idx: torch.Tensor, dgate: torch.Tensor, offsets: torch.Tensor,
                       row_token: torch.Tensor, row_of: torch.Tensor, dx: torch.Tensor = None,
                       dw_router: torch.Tensor = None, ws: torch.Tensor = None, stream=None):
    """-> (dx [T, H] f32, dw_router [N_r, H] f32): the gates' gradient through the router."""
    T, H = x.shape
    N, k = cfg.n_routed, cfg.top_k
    dev = x.device
    dx = torch.empty((T, H), dtype=torch.float32, device=dev) if dx is None else dx
    dw_router = torch.empty((N, H), dtype=torch.float32, device=dev) if dw_router is None else dw_router
    if ws is None:
        ws = torch.empty((max(moe_route_backward_workspace_bytes(cfg, T), 1),), dtype=torch.uint8, device=dev)
    _check(_lib.moe_route_backward(
        ctypes.byref(cfg), T, _dev(x, x.dtype, "x", (T, cfg.hidden)), _dt(x),
        _dev(w_router, torch.float32, "w_router", (N, H)), _dev(scores, torch.float32, "scores", (T, N)),
        _dev(topk_idx, torch.int32, "topk_idx", (T, k)), _dev(dgate, torch.float32, "dgate", (T, k)),
        _dev(offsets, torch.int32, "offsets"), _dev(row_token, torch.int32, "row_token"),
        _dev(row_of, torch.int32, "row_of", (T, k)), _dev(dx, torch.float32, "dx", (T, H)),
        _dev(dw_router, torch.float32, "dw_router", (N, H)), _dev(ws, torch.uint8, "ws"), ws.numel(),
        _stream(stream)), "moe_route_backward")
    return dx, dw_router


def moe_unpermute_sum(cfg: moe_config, rows: torch.Tensor, row_of: torch.Tensor,
                      extra: torch.Tensor = None, out: torch.Tensor = None, stream=None):
    """-> out [T, H] bf16 = sum of each token's rows (shared, then slots) + extra."""
    T, k = row_of.shape
    H = cfg.hidden
    out = torch.empty((T, H), dtype=torch.bfloat16, device=rows.device) if out is None else out
    _check(_lib.moe_unpermute_sum(
        ctypes.byref(cfg), T, _dev(rows, rows.dtype, "rows", (T * (k + cfg.n_shared), H)), _dt(rows),
        _dev(row_of, torch.int32, "row_of", (T, k)),
        _dev(extra, torch.float32, "extra", (T, H)) if extra is not None else None,
        _dev(out, torch.bfloat16, "out", (T, H)), _stream(stream)), "moe_unpermute_sum")
    return out


def moe_transpose_fp8_blocks(q: torch.Tensor, scales: torch.Tensor, dst: torch.Tensor,
                             dst_scales: torch.Tensor, col0: int = 0, stream=None):
    """dst[e][c][col0 + r] = q[e][r][c] (codes [E, R, C] -> [E, C, dst_cols]) with the block
    scales moved along."""
    E, R, C = q.shape
    dst_cols = dst.shape[2]
    _check(_lib.moe_transpose_fp8_blocks(
        E, R, C, _dev(q, torch.uint8, "q"), _dev(scales, torch.float32, "scales", (E, R // 128, C // 128)),
        _dev(dst, torch.uint8, "dst", (E, C, dst_cols)),
        _dev(dst_scales, torch.float32, "dst_scales", (E, C // 128, dst_cols // 128)), dst_cols, col0,
        _stream(stream)), "moe_transpose_fp8_blocks")
    return dst, dst_scales


def moe_grouped_ffn_backward_workspace_bytes(cfg: moe_config, n_experts: int, n_rows: int) -> int:
    return int(_lib.moe_grouped_ffn_backward_workspace_bytes(ctypes.byref(cfg), n_experts, n_rows))


def moe_grouped_ffn_fp8_backward(cfg: moe_config, n_experts: int, xq, xs, x, row_token, offsets,
                                 w1, w1s, w3, w3s, w2t, w2ts, w13t, w13ts, dout,
                                 row_gate: Optional[torch.Tensor] = None,
                                 dx_rows: torch.Tensor = None, dx_dtype=torch.float32,
                                 dw1: torch.Tensor = None, dw3: torch.Tensor = None,
                                 dw2: torch.Tensor = None, dw_dtype=torch.float32,
                                 ws: torch.Tensor = None, a_saved: torch.Tensor = None,
                                 b_saved: torch.Tensor = None, stream=None):
    """-> (dx_rows [n_rows, H], dw1 [E, I, H], dw3 [E, I, H], dw2 [E, H, I]) for the rows'
    upstream gradient dy_r = row_gate[r] * dout[row_token[r]] (dout [T, H] bf16; row_gate
    None: every gate 1). ``a_saved``, ``b_saved``: the SwiGLU inputs kept by
    moe_grouped_ffn_fp8_gate_up_train (both or neither; without them they are recomputed
    from xq, xs)."""
    n_rows = row_token.shape[0]
    T = x.shape[0]
    H, I, E = cfg.hidden, cfg.inter, n_experts
    dev = x.device
    if dx_rows is None:
        dx_rows = torch.empty((n_rows, H), dtype=dx_dtype, device=dev)
    dw1 = torch.empty((E, I, H), dtype=dw_dtype, device=dev) if dw1 is None else dw1
    dw3 = torch.empty((E, I, H), dtype=dw_dtype, device=dev) if dw3 is None else dw3
    dw2 = torch.empty((E, H, I), dtype=dw_dtype, device=dev) if dw2 is None else dw2
    if ws is None:
        ws = torch.empty((max(moe_grouped_ffn_backward_workspace_bytes(cfg, E, n_rows), 1),),
                         dtype=torch.uint8, device=dev)
    _check(_lib.moe_grouped_ffn_fp8_backward(
        ctypes.byref(cfg), E, n_rows, T, _opt(xq, torch.uint8, "xq", (T, H)),
        _opt(xs, torch.float32, "xs", (T, H // 128)), _dev(x, x.dtype, "x", (T, H)), _dt(x),
        _dev(row_token, torch.int32, "row_token", (n_rows,)), _dev(offsets, torch.int32, "offsets", (E + 1,)),
        _dev(w1, torch.uint8, "w1"), _dev(w1s, torch.float32, "w1s"), _dev(w3, torch.uint8, "w3"),
        _dev(w3s, torch.float32, "w3s"), _dev(w2t, torch.uint8, "w2t"), _dev(w2ts, torch.float32, "w2ts"),
        _dev(w13t, torch.uint8, "w13t"), _dev(w13ts, torch.float32, "w13ts"),
        _opt(a_saved, torch.float32, "a_saved", (n_rows, I)), _opt(b_saved, torch.float32, "b_saved", (n_rows, I)),
        _dev(dout, torch.bfloat16, "dout", (T, H)), _opt(row_gate, torch.float32, "row_gate", (n_rows,)),
        _dev(dx_rows, dx_rows.dtype, "dx_rows", (n_rows, H)),
        _dt(dx_rows), _dev(dw1, dw1.dtype, "dw1", (E, I, H)), _dev(dw3, dw1.dtype, "dw3", (E, I, H)),
        _dev(dw2, dw1.dtype, "dw2", (E, H, I)), _dt(dw1), _dev(ws, torch.uint8, "ws"), ws.numel(),
        _stream(stream)), "moe_grouped_ffn_fp8_backward")
    return dx_rows, dw1, dw3, dw2


from .layer import MoELayer  # noqa: E402,F401
