"""moe_grouped_ffn_fp8_noalloc against moe_grouped_ffn_fp8 (needs an MI355X; collected last).

The no-allocation entry point runs the same kernels on the library's static scratch
array instead of a caller's workspace, so its output must equal the workspace entry
point's bit for bit. Two calls in a row, the second smaller, check that a call is not
disturbed by what the previous one left in the shared array; an oversized request is
refused on the host.
"""
import ctypes
import sys

import numpy as np
import pytest
import torch

import oracle

pytestmark = pytest.mark.gpu


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def _rand_codes(rng, shape):
    c = rng.integers(0, 0x7F, shape).astype(np.uint8)
    return c | (rng.integers(0, 2, shape).astype(np.uint8) << 7)


def _case(lib, rng, H, I, E, loads, T):
    rows = int(sum(loads))
    x = rng.standard_normal((T, H)).astype(np.float32)
    xq, xs = oracle.quantize_1x128(x)
    offsets = np.concatenate([[0], np.cumsum(loads)]).astype(np.int32)
    row_token = rng.integers(0, T, rows).astype(np.int32)
    f = lambda n, k: rng.uniform(0.5, 2.0, (E, n // 128, k // 128)).astype(np.float32) / 448
    w = [_rand_codes(rng, (E, I, H)), f(I, H), _rand_codes(rng, (E, I, H)), f(I, H),
         _rand_codes(rng, (E, H, I)), f(H, I)]
    dw = [lib.moe_pack_fp8_weights(torch.from_numpy(a).cuda()) if i % 2 == 0 else torch.from_numpy(a).cuda()
          for i, a in enumerate(w)]
    dv = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()
    return rows, (dv(xq), dv(xs), dv(row_token), dv(offsets)), dw


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr())


def test_noalloc_matches_workspace_call_twice():
    import dataclasses

    import synth
    import deepseekmoe_routing_fp8_amd as lib
    rng = np.random.default_rng(2024)
    # first call: a decode-like mix (several M tiles, empty experts); second: smaller
    for H, I, E, loads, T in ((1024, 512, 9, [300, 0, 17, 161, 5, 0, 90, 200, 33], 500),
                              (512, 256, 3, [40, 0, 7], 60)):
        cfg = dataclasses.replace(synth.PRESETS["tiny"], hidden_size=H, moe_intermediate_size=I,
                                  num_experts=max(E, 4), num_experts_per_tok=1, tokens=T)
        c = lib.make_config(cfg)
        rows, (xq, xs, rt, off), w = _case(lib, rng, H, I, E, loads, T)
        say(f"noalloc H={H} I={I} E={E} rows={rows}")
        for yt, ytc in ((torch.bfloat16, lib.MOE_BF16), (torch.float32, lib.MOE_F32)):
            y_ref = lib.moe_grouped_ffn_fp8(c, E, rows, xq, xs, rt, off, *w, y_dtype=yt)
            y = torch.full((rows, H), float("nan"), dtype=yt, device="cuda")
            torch.cuda.synchronize()
            # through the C ABI itself: no workspace argument
            st = lib._lib.moe_grouped_ffn_fp8_noalloc(
                ctypes.byref(c), E, rows, T, _ptr(xq), _ptr(xs), _ptr(rt), _ptr(off),
                *[_ptr(t) for t in w], _ptr(y), ytc, ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
            assert st == 0, lib._lib.moe_status_string(st).decode()
            torch.cuda.synchronize()
            assert torch.equal(y.view(torch.int16 if yt == torch.bfloat16 else torch.int32),
                               y_ref.view(torch.int16 if yt == torch.bfloat16 else torch.int32))
        # the binding's wrapper gives the same
        y2 = lib.moe_grouped_ffn_fp8_noalloc(c, E, rows, xq, xs, rt, off, *w)
        torch.cuda.synchronize()
        assert torch.equal(y2.view(torch.int16), lib.moe_grouped_ffn_fp8(c, E, rows, xq, xs, rt, off, *w).view(torch.int16))
    # a request larger than the static array: refused before any launch
    c = lib.make_config(synth.PRESETS["v3_prefill"])
    st = lib._lib.moe_grouped_ffn_fp8_noalloc(ctypes.byref(c), 257, 36864, 4096, *[_ptr(xq)] * 10,
                                              _ptr(xq), lib.MOE_BF16, None)
    assert st == lib.MOE_ERR_SCRATCH
