"""MoE layer driver: device-resident weights and buffers, and the call sequence of one
forward step through the C entry points (quantise -> route -> permute -> routed experts
-> shared experts -> combine -> bias update).

Weights arrive as float32 host arrays (from the seeded generators), are quantised to
E4M3 128x128 blocks on the device by moe_quantize_128x128 and re-laid by
moe_pack_fp8_weights into the layout the grouped FFN streams. ``w1``/``w3``/``w2`` hold
the packed codes of the N_r routed experts followed by the N_s shared experts (index
N_r + s), so that one grouped-FFN call over N_r + N_s segments (moe_permute appends the
shared segments) evaluates both; ``unpack`` recovers the row-major codes of one matrix.
"""
from __future__ import annotations

from typing import Callable, Optional

import numpy as np
import torch

from . import (MOE_F32, make_config, moe_combine, moe_combine_backward,
               moe_grouped_ffn_backward_workspace_bytes, moe_grouped_ffn_fp8_backward,
               moe_grouped_ffn_fp8_down, moe_grouped_ffn_fp8_gate_up,
               moe_grouped_ffn_fp8_gate_up_train,
               moe_grouped_ffn_workspace_bytes, moe_pack_fp8_weights, moe_pack_router_weights,
               moe_permute, moe_permute_workspace_bytes, moe_quantize_1x128, moe_quantize_128x128,
               moe_route, moe_route_backward, moe_route_backward_workspace_bytes, moe_route_workspace_bytes,
               moe_seq_balance, moe_seq_balance_workspace_bytes, moe_transpose_fp8_blocks,
               moe_unpermute_sum, moe_update_bias)


class MoELayer:
    """One DeepSeekMoE layer on one GPU.

    ``cfg`` carries the synth.MoEConfig field names. Call ``load_weights`` (or
    ``load_from_synth``) once, then ``forward(x)`` per step.
    """

    def __init__(self, cfg, device="cuda", y_dtype=torch.bfloat16, scale_mode: int = 0,
                 backward: bool = False, dw_dtype=torch.float32, keep_swiglu_inputs: bool = True):
        """``scale_mode`` 0: the pages' FP32 group scales; 1: the power-of-two variant
        (weights and activations quantised with power-of-two scales, applied by the MFMA).
        ``backward``: also keep what ``backward`` needs (the transposed packed weights for
        the dgrad GEMMs and the FP32 router weight); weight gradients come in ``dw_dtype``.
        ``keep_swiglu_inputs`` (with ``backward``): the forward keeps the SwiGLU inputs a, b
        (FP32, [rows, I] each) so that the backward recomputes only h from them; False
        recomputes a and b by the gate/up GEMMs in the backward instead (same values)."""
        self.cfg = cfg
        self.scale_mode = scale_mode
        self.c = make_config(cfg, scale_mode)
        self.dev = torch.device(device)
        self.y_dtype = y_dtype
        H, I, E, S = cfg.hidden_size, cfg.moe_intermediate_size, cfg.num_experts, cfg.num_shared_experts
        u8, f32 = torch.uint8, torch.float32
        d = self.dev
        EA = E + S   # routed experts, then shared experts
        self.w1 = torch.empty((EA, I, H), dtype=u8, device=d)
        self.w3 = torch.empty((EA, I, H), dtype=u8, device=d)
        self.w2 = torch.empty((EA, H, I), dtype=u8, device=d)
        self.w1s = torch.empty((EA, I // 128, H // 128), dtype=f32, device=d)
        self.w3s = torch.empty((EA, I // 128, H // 128), dtype=f32, device=d)
        self.w2s = torch.empty((EA, H // 128, I // 128), dtype=f32, device=d)
        self.w_router = None
        self.bias = None
        self._T = None
        self._graph = None
        self.backward_enabled = backward
        # (the backward runs on the FP32 group scales only)
        self.keep_ab = backward and keep_swiglu_inputs and scale_mode == 0
        self.dw_dtype = dw_dtype
        if backward:
            # dgrad operands: W2^T [I, H] and [W1^T | W3^T] [H, 2I] per expert, packed
            self.w2t = torch.empty((EA, I, H), dtype=u8, device=d)
            self.w2ts = torch.empty((EA, I // 128, H // 128), dtype=f32, device=d)
            self.w13t = torch.empty((EA, H, 2 * I), dtype=u8, device=d)
            self.w13ts = torch.empty((EA, H // 128, 2 * I // 128), dtype=f32, device=d)
            self.w_router_f32 = None
            self._bT = None

    # -- weights -------------------------------------------------------------------
    def _quant_into(self, w: np.ndarray, q: torch.Tensor, s: torch.Tensor):
        """Quantise and pack one matrix; returns its row-major codes."""
        t = torch.from_numpy(np.ascontiguousarray(w, dtype=np.float32)).to(self.dev)
        rowmajor, _ = moe_quantize_128x128(t, scales=s, pow2=self.scale_mode == 1)
        moe_pack_fp8_weights(rowmajor, q)
        return rowmajor

    def _transposed_into(self, e: int, q1, q3, q2):
        """Pack expert e's dgrad operands from its row-major codes."""
        H, I = self.cfg.hidden_size, self.cfg.moe_intermediate_size
        u8, f32, d = torch.uint8, torch.float32, self.dev
        t2 = torch.empty((1, I, H), dtype=u8, device=d)
        moe_transpose_fp8_blocks(q2.unsqueeze(0), self.w2s[e:e + 1], t2, self.w2ts[e:e + 1])
        moe_pack_fp8_weights(t2[0], self.w2t[e])
        t13 = torch.empty((1, H, 2 * I), dtype=u8, device=d)
        moe_transpose_fp8_blocks(q1.unsqueeze(0), self.w1s[e:e + 1], t13, self.w13ts[e:e + 1], col0=0)
        moe_transpose_fp8_blocks(q3.unsqueeze(0), self.w3s[e:e + 1], t13, self.w13ts[e:e + 1], col0=I)
        moe_pack_fp8_weights(t13[0], self.w13t[e])

    @staticmethod
    def unpack(packed: np.ndarray) -> np.ndarray:
        """Row-major codes of one packed [rows, cols] matrix (inverse of the packing)."""
        rows, cols = packed.shape
        nkc = cols // 128
        # fragment n16 = 2m + p, lane = 16g + 4a + b holds row 32m + 8a + 4p + b
        f = packed.reshape(rows // 32, 2, nkc, 2, 4, 4, 4, 16)   # m, p, kc, half, g, a, b, byte
        return np.ascontiguousarray(f.transpose(0, 5, 1, 6, 2, 3, 4, 7)).reshape(rows, cols)

    def load_weights(self, w_router: np.ndarray, bias: np.ndarray,
                     routed: Callable[[Callable], None], shared: Callable[[Callable], None]):
        """``routed(put)`` / ``shared(put)`` call put(e, (w1, w3, w2)) for every expert."""
        self.w_router = moe_pack_router_weights(
            torch.from_numpy(np.ascontiguousarray(w_router, np.float32)).to(self.dev))
        self.bias = torch.from_numpy(np.ascontiguousarray(bias, np.float32)).to(self.dev)
        if self.backward_enabled:
            self.w_router_f32 = torch.from_numpy(np.ascontiguousarray(w_router, np.float32)).to(self.dev)

        def put_routed(e, w):
            q1 = self._quant_into(w[0], self.w1[e], self.w1s[e])
            q3 = self._quant_into(w[1], self.w3[e], self.w3s[e])
            q2 = self._quant_into(w[2], self.w2[e], self.w2s[e])
            if self.backward_enabled:
                self._transposed_into(e, q1, q3, q2)

        def put_shared(s, w):
            put_routed(self.cfg.num_experts + s, w)
        routed(put_routed)
        shared(put_shared)
        torch.cuda.synchronize(self.dev)

    def load_from_synth(self, threads: Optional[int] = None):
        import synth
        cfg = self.cfg
        self.load_weights(
            synth.router_weight(cfg), synth.expert_bias(cfg),
            lambda put: synth.map_experts(cfg, put, range(cfg.num_experts), threads=threads),
            lambda put: synth.map_experts(cfg, put, range(cfg.num_shared_experts), shared=True,
                                          threads=threads))

    # -- buffers -------------------------------------------------------------------
    def _buffers(self, T: int):
        if self._T == T:
            return
        cfg, d = self.cfg, self.dev
        H, I, N, k, S = (cfg.hidden_size, cfg.moe_intermediate_size, cfg.num_experts,
                         cfg.num_experts_per_tok, cfg.num_shared_experts)
        i32, f32 = torch.int32, torch.float32
        self._graph = None   # a captured step holds the old buffers' addresses
        self.xq = torch.empty((T, H), dtype=torch.uint8, device=d)
        self.xs = torch.empty((T, H // 128), dtype=f32, device=d)
        self.scores = torch.empty((T, N), dtype=f32, device=d)
        self.topk_idx = torch.empty((T, k), dtype=i32, device=d)
        self.topk_gate = torch.empty((T, k), dtype=f32, device=d)
        self.counts = torch.empty((N,), dtype=i32, device=d)
        self.offsets = torch.empty((N + S + 1,), dtype=i32, device=d)
        self.row_token = torch.empty((T * (k + S),), dtype=i32, device=d)
        self.row_of = torch.empty((T, k), dtype=i32, device=d)
        self.y_rows = torch.empty((T * (k + S), H), dtype=self.y_dtype, device=d)
        if self.keep_ab:   # the SwiGLU inputs of the last forward, for the backward
            self.a_saved = torch.empty((T * (k + S), I), dtype=f32, device=d)
            self.b_saved = torch.empty((T * (k + S), I), dtype=f32, device=d)
        self.ws = torch.empty((max(moe_grouped_ffn_workspace_bytes(self.c, N + S, T * (k + S)), 1),),
                              dtype=torch.uint8, device=d)
        self.y_shared = self.y_rows[T * k:] if S > 0 else None
        self.perm_ws = torch.empty((max(moe_permute_workspace_bytes(self.c, T), 1),),
                                   dtype=torch.uint8, device=d)
        self.out = torch.empty((T, H), dtype=torch.bfloat16, device=d)
        # sized for FP32 input, the larger of the two
        self.route_ws = torch.empty((max(moe_route_workspace_bytes(self.c, T, MOE_F32), 1),),
                                    dtype=torch.uint8, device=d)
        self._T = T

    # -- forward -------------------------------------------------------------------
    STAGES = ("quantize", "route", "permute", "ffn_gate_up", "ffn_down", "combine", "bias_update")

    def forward(self, x: torch.Tensor, update_bias: bool = True, events=None) -> torch.Tensor:
        """One layer step on x [T, H] (bf16 or f32, on the device). Returns out [T, H] bf16
        (a buffer reused by the next call); routing results stay in the attributes.

        ``events``: optional list of len(STAGES)+1 torch.cuda.Event recorded on the current
        stream around each stage (per-stage timing without extra synchronisation)."""
        cfg, c = self.cfg, self.c
        T = x.shape[0]
        self._buffers(T)
        k, N, S = cfg.num_experts_per_tok, cfg.num_experts, cfg.num_shared_experts
        EA, rows = N + S, T * (k + S)
        mark = (lambda i: events[i].record()) if events is not None else (lambda i: None)
        mark(0)
        self.x = x
        moe_quantize_1x128(x, self.xq, self.xs, pow2=self.scale_mode == 1)
        mark(1)
        moe_route(c, x, self.w_router, self.bias, self.scores, self.topk_idx, self.topk_gate,
                  self.counts, ws=self.route_ws)
        mark(2)
        moe_permute(c, self.topk_idx, self.offsets, self.row_token, self.row_of, ws=self.perm_ws)
        mark(3)
        if self.keep_ab:
            moe_grouped_ffn_fp8_gate_up_train(c, EA, rows, self.xq, self.xs, self.row_token,
                                              self.offsets, self.w1, self.w1s, self.w3, self.w3s,
                                              a=self.a_saved, b=self.b_saved, ws=self.ws)
        else:
            moe_grouped_ffn_fp8_gate_up(c, EA, rows, self.xq, self.xs, self.row_token, self.offsets,
                                        self.w1, self.w1s, self.w3, self.w3s, ws=self.ws)
        mark(4)
        moe_grouped_ffn_fp8_down(c, EA, rows, self.w2, self.w2s, self.ws, y=self.y_rows)
        mark(5)
        moe_combine(c, self.y_rows, self.row_of, self.topk_gate, self.y_shared, self.out)
        mark(6)
        if update_bias:
            moe_update_bias(c, T, self.counts, self.bias)
        mark(7)
        return self.out

    # -- graph capture ---------------------------------------------------------------
    def capture(self, x: torch.Tensor, update_bias: bool = True) -> "torch.cuda.CUDAGraph":
        """Captures one forward step on x into a HIP graph and keeps it for replay().

        The graph holds the addresses of x and of the layer's buffers: write the next input
        into x in place, then replay(); the outputs land in self.out and the routing
        attributes as with forward(). A step is library kernel launches only (no host
        synchronisation, no allocation, no memset nodes), so a replay runs the eager step's
        kernels on the same buffers and gives bit-identical results, without the per-launch
        host overhead that dominates the small kernels of a decode step."""
        self._buffers(x.shape[0])
        side = torch.cuda.Stream(device=self.dev)
        side.wait_stream(torch.cuda.current_stream(self.dev))
        with torch.cuda.stream(side):   # settle lazy state before capturing
            self.forward(x, update_bias=False)
        torch.cuda.current_stream(self.dev).wait_stream(side)
        torch.cuda.synchronize(self.dev)
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            self.forward(x, update_bias=update_bias)
        self._graph = g
        return g

    def replay(self) -> torch.Tensor:
        """Runs the captured step on torch's current stream; returns self.out."""
        if getattr(self, "_graph", None) is None:
            raise RuntimeError("replay(): no captured step (call capture() first)")
        self._graph.replay()
        return self.out

    # -- backward ------------------------------------------------------------------
    BWD_STAGES = ("combine_bwd", "ffn_bwd", "route_bwd", "unpermute")

    def _bwd_buffers(self, T: int):
        if self._bT == T:
            return
        cfg, d = self.cfg, self.dev
        H, I, N, k, S = (cfg.hidden_size, cfg.moe_intermediate_size, cfg.num_experts,
                         cfg.num_experts_per_tok, cfg.num_shared_experts)
        EA, rows, f32 = N + S, T * (k + S), torch.float32
        self.row_gate = torch.empty((rows,), dtype=f32, device=d)
        self.dgate = torch.empty((T, k), dtype=f32, device=d)
        self.dx_rows = torch.empty((rows, H), dtype=f32, device=d)
        self.dx_route = torch.empty((T, H), dtype=f32, device=d)
        self.dx = torch.empty((T, H), dtype=torch.bfloat16, device=d)
        self.dw1 = torch.empty((EA, I, H), dtype=self.dw_dtype, device=d)
        self.dw3 = torch.empty((EA, I, H), dtype=self.dw_dtype, device=d)
        self.dw2 = torch.empty((EA, H, I), dtype=self.dw_dtype, device=d)
        self.dw_router = torch.empty((N, H), dtype=f32, device=d)
        self.bwd_ws = torch.empty((max(moe_grouped_ffn_backward_workspace_bytes(self.c, EA, rows), 1),),
                                  dtype=torch.uint8, device=d)
        self.route_bwd_ws = torch.empty((max(moe_route_backward_workspace_bytes(self.c, T), 1),),
                                        dtype=torch.uint8, device=d)
        self._bT = T

    def backward(self, dout: torch.Tensor, events=None) -> torch.Tensor:
        """Gradients of the last forward for upstream gradient dout [T, H] (bf16): returns
        dx [T, H] bf16 (a reused buffer); weight gradients land in dw1, dw3 [E, I, H],
        dw2 [E, H, I] (routed experts, then shared) and dw_router [N_r, H]."""
        if not self.backward_enabled:
            raise RuntimeError("MoELayer was built without backward=True")
        cfg, c = self.cfg, self.c
        T = dout.shape[0]
        assert T == self._T, "backward needs the forward of the same batch"
        self._bwd_buffers(T)
        EA = cfg.num_experts + cfg.num_shared_experts
        mark = (lambda i: events[i].record()) if events is not None else (lambda i: None)
        mark(0)
        moe_combine_backward(c, dout, self.y_rows, self.row_of, self.topk_gate, row_gate=self.row_gate,
                             dgate=self.dgate)
        mark(1)
        moe_grouped_ffn_fp8_backward(c, EA, self.xq, self.xs, self.x, self.row_token, self.offsets,
                                     self.w1, self.w1s, self.w3, self.w3s, self.w2t, self.w2ts,
                                     self.w13t, self.w13ts, dout, row_gate=self.row_gate,
                                     dx_rows=self.dx_rows,
                                     dw1=self.dw1, dw3=self.dw3, dw2=self.dw2, ws=self.bwd_ws,
                                     a_saved=self.a_saved if self.keep_ab else None,
                                     b_saved=self.b_saved if self.keep_ab else None)
        mark(2)
        moe_route_backward(c, self.x, self.w_router_f32, self.scores, self.topk_idx, self.dgate,
                           self.offsets, self.row_token, self.row_of, dx=self.dx_route,
                           dw_router=self.dw_router, ws=self.route_bwd_ws)
        mark(3)
        moe_unpermute_sum(c, self.dx_rows, self.row_of, extra=self.dx_route, out=self.dx)
        mark(4)
        return self.dx

    def seq_balance(self, seq_len: int, alpha: float = 0.001, with_entropy: bool = True):
        """Per-sequence balance loss and allocation entropy of the last forward's routing
        (sequences of seq_len consecutive tokens) -> (loss, entropy or None), float32."""
        T = self._T
        key = (T, seq_len)
        if getattr(self, "_sb_key", None) != key:
            nseq = T // seq_len
            self.sb_loss = torch.empty((nseq,), dtype=torch.float32, device=self.dev)
            self.sb_entropy = torch.empty((nseq,), dtype=torch.float32, device=self.dev)
            self.sb_ws = torch.empty((max(moe_seq_balance_workspace_bytes(self.c, T, seq_len), 1),),
                                     dtype=torch.uint8, device=self.dev)
            self._sb_key = key
        return moe_seq_balance(self.c, self.scores, self.topk_idx, seq_len, alpha, loss=self.sb_loss,
                               entropy=self.sb_entropy if with_entropy else None,
                               with_entropy=with_entropy, ws=self.sb_ws)
