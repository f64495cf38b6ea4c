"""The layer step driven through the C ABI alone (needs an MI355X).

No Python wrapper of the library is used: every call goes through ctypes with plain
device pointers and sizes, exactly as a C caller would make it, on row-major inputs —
the weight preparation (moe_quantize_128x128, moe_pack_fp8_weights,
moe_pack_router_weights), then the six calls of one step (moe_quantize_1x128,
moe_route, moe_permute, moe_grouped_ffn_fp8, moe_combine, moe_update_bias). torch only
provides device memory. The result is compared with the oracle's layer forward and bias
update on the tiny layer (T = 64, H = 256, 16 routed + 1 shared experts, top-4).
"""
import ctypes
import os
import sys

import numpy as np
import pytest
import torch

import oracle
import synth
from routing_check import assert_routing_valid

pytestmark = pytest.mark.gpu
ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


class Cfg(ctypes.Structure):
    """moe_config as declared in include/moe_fp8.h."""
    _fields_ = [("hidden", ctypes.c_int32), ("inter", ctypes.c_int32), ("n_routed", ctypes.c_int32),
                ("n_shared", ctypes.c_int32), ("top_k", ctypes.c_int32), ("n_group", ctypes.c_int32),
                ("topk_group", ctypes.c_int32), ("group_topn", ctypes.c_int32),
                ("routed_scaling", ctypes.c_float), ("bias_gamma", ctypes.c_float),
                ("scale_mode", ctypes.c_int32)]


def test_six_calls_through_ctypes_match_oracle():
    lib = ctypes.CDLL(os.path.join(ROOT, "deepseekmoe_routing_fp8_amd", "libmoe_fp8.so"))
    P, I64, I32, SZ = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_size_t
    for name, res in (("moe_router_weights_elems", SZ), ("moe_route_workspace_bytes", SZ),
                      ("moe_permute_workspace_bytes", SZ), ("moe_grouped_ffn_workspace_bytes", SZ),
                      ("moe_status_string", ctypes.c_char_p)):
        getattr(lib, name).restype = res
    lib.moe_router_weights_elems.argtypes = [I64, I64]
    lib.moe_route_workspace_bytes.argtypes = [P, I64, ctypes.c_int]
    lib.moe_permute_workspace_bytes.argtypes = [P, I64]
    lib.moe_grouped_ffn_workspace_bytes.argtypes = [P, I32, I64]

    cfg = synth.PRESETS["tiny"]
    T, H, I = cfg.tokens, cfg.hidden_size, cfg.moe_intermediate_size
    N, S, k = cfg.num_experts, cfg.num_shared_experts, cfg.num_experts_per_tok
    E, rows = N + S, T * (k + S)
    c = Cfg(H, I, N, S, k, cfg.n_group, cfg.topk_group, cfg.group_score_topn,
            cfg.routed_scaling_factor, cfg.expert_bias_update_rate, 0)
    cp = ctypes.byref(c)
    MOE_F32, MOE_BF16 = 0, 1

    def ok(st, what):
        assert st == 0, f"{what}: {lib.moe_status_string(st).decode()}"

    def buf(shape, dtype):
        return torch.empty(shape, dtype=dtype, device="cuda")

    def ptr(t):
        return P(t.data_ptr())

    # inputs, row-major, as a C caller holds them
    x = synth.hidden_states(cfg)                       # fp32 [T, H]
    wr = synth.router_weight(cfg)                      # fp32 [N, H]
    b0 = synth.expert_bias(cfg)
    experts = [synth.routed_expert_weights(cfg, e) for e in range(N)] + \
              [synth.shared_expert_weights(cfg, s) for s in range(S)]
    w1 = torch.from_numpy(np.stack([w[0] for w in experts])).cuda()   # [E, I, H]
    w3 = torch.from_numpy(np.stack([w[1] for w in experts])).cuda()
    w2 = torch.from_numpy(np.stack([w[2] for w in experts])).cuda()   # [E, H, I]
    xd, wrd, bias = (torch.from_numpy(a).cuda() for a in (x, wr, b0.copy()))

    say("ABI chain: weight preparation")
    q = {}
    for name, w, r_, c_ in (("w1", w1, I, H), ("w3", w3, I, H), ("w2", w2, H, I)):
        codes, sc, packed = buf((E, r_, c_), torch.uint8), buf((E, r_ // 128, c_ // 128), torch.float32), \
            buf((E, r_, c_), torch.uint8)
        ok(lib.moe_quantize_128x128(ptr(w), I64(E), I64(r_), I64(c_), ptr(codes), ptr(sc), None), name)
        ok(lib.moe_pack_fp8_weights(ptr(codes), I64(E), I64(r_), I64(c_), ptr(packed), None), name)
        q[name] = (codes, sc, packed)
    wsplit = buf((lib.moe_router_weights_elems(N, H),), torch.int16)
    ok(lib.moe_pack_router_weights(ptr(wrd), I64(N), I64(H), ptr(wsplit), None), "pack router")

    say("ABI chain: the six calls of one step")
    xq, xs = buf((T, H), torch.uint8), buf((T, H // 128), torch.float32)
    ok(lib.moe_quantize_1x128(ptr(xd), MOE_F32, I64(T), I64(H), ptr(xq), ptr(xs), None), "quantize")
    scores, idx = buf((T, N), torch.float32), buf((T, k), torch.int32)
    gate, counts = buf((T, k), torch.float32), buf((N,), torch.int32)
    rws_n = lib.moe_route_workspace_bytes(cp, T, MOE_F32)
    rws = buf((max(rws_n, 1),), torch.uint8)
    ok(lib.moe_route(cp, ptr(xd), MOE_F32, I64(T), ptr(wsplit), ptr(bias), ptr(scores), ptr(idx),
                     ptr(gate), ptr(counts), ptr(rws), SZ(rws_n), None), "route")
    offsets, row_token, row_of = buf((E + 1,), torch.int32), buf((rows,), torch.int32), buf((T, k), torch.int32)
    pws_n = lib.moe_permute_workspace_bytes(cp, T)
    pws = buf((max(pws_n, 1),), torch.uint8)
    ok(lib.moe_permute(cp, I64(T), ptr(idx), ptr(offsets), ptr(row_token), ptr(row_of), ptr(pws),
                       SZ(pws_n), None), "permute")
    y = buf((rows, H), torch.bfloat16)
    fws_n = lib.moe_grouped_ffn_workspace_bytes(cp, E, rows)
    fws = buf((fws_n,), torch.uint8)
    ok(lib.moe_grouped_ffn_fp8(cp, I32(E), I64(rows), I64(T), ptr(xq), ptr(xs), ptr(row_token),
                               ptr(offsets), ptr(q["w1"][2]), ptr(q["w1"][1]), ptr(q["w3"][2]),
                               ptr(q["w3"][1]), ptr(q["w2"][2]), ptr(q["w2"][1]), ptr(y), MOE_BF16,
                               ptr(fws), SZ(fws_n), None), "grouped ffn")
    out = buf((T, H), torch.bfloat16)
    ok(lib.moe_combine(cp, I64(T), ptr(y), MOE_BF16, ptr(row_of), ptr(gate), P(y[T * k:].data_ptr()),
                       ptr(out), None), "combine")
    ok(lib.moe_update_bias(cp, I64(T), ptr(counts), ptr(bias), None), "update bias")
    torch.cuda.synchronize()

    # the oracle on the same inputs
    rq = [tuple(v for m in w for v in oracle.quantize_128x128(m)) for w in experts]
    for e in (0, N - 1, N):
        assert np.array_equal(q["w1"][0][e].cpu().numpy(), rq[e][0])
        assert np.array_equal(q["w2"][1][e].cpu().numpy(), rq[e][5])
    rxq, rxs = oracle.quantize_1x128(x)
    assert np.array_equal(xq.cpu().numpy(), rxq) and np.array_equal(xs.cpu().numpy(), rxs)
    g_idx = idx.cpu().numpy()
    ref = oracle.layer_forward(x, wr, b0, cfg, lambda e: rq[e], lambda s: rq[N + s])
    assert_routing_valid(ref["route"], g_idx, cfg)
    if np.any(g_idx != ref["route"]["idx"]):
        ref = oracle.layer_forward(x, wr, b0, cfg, lambda e: rq[e], lambda s: rq[N + s], force_idx=g_idx)
    g_counts = counts.cpu().numpy()
    assert np.array_equal(g_counts, np.bincount(g_idx.ravel(), minlength=N))
    o = out.float().cpu().numpy()
    err = float(np.linalg.norm(o - ref["out"]) / np.linalg.norm(ref["out"]))
    say(f"ABI chain: normwise error {err:.3e}")
    assert err < 5e-3
    nb = oracle.bias_update(b0, g_counts, T, k, cfg.expert_bias_update_rate)
    assert np.array_equal(bias.cpu().numpy().view(np.uint32), nb.view(np.uint32))
