"""C-ABI checks that need no GPU: the library loads, exports every symbol that
include/moe_fp8.h declares, and rejects invalid arguments on the host with the
documented status codes before any launch."""
import ctypes
import os
import re

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "moe_fp8.h")


def _lib():
    import __graft_entry__
    b = __graft_entry__._builder()
    if not os.path.exists(b.LIB):
        b.build()
    import deepseekmoe_routing_fp8_amd as m
    return m


def _declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(moe_[a-z0-9_]+)\s*\(", text)))


def test_header_declares_the_six_calls():
    names = _declared()
    for n in ("moe_quantize_1x128", "moe_route", "moe_permute", "moe_grouped_ffn_fp8",
              "moe_grouped_ffn_fp8_gate_up", "moe_grouped_ffn_fp8_down", "moe_combine",
              "moe_update_bias", "moe_seq_balance", "moe_combine_backward", "moe_route_backward",
              "moe_unpermute_sum", "moe_grouped_ffn_fp8_backward"):
        assert n in names


def test_library_exports_every_declared_symbol():
    m = _lib()
    lib = ctypes.CDLL(m.LIB_PATH)
    for n in _declared():
        assert hasattr(lib, n), n
    assert set(_declared()) == set(m.ENTRY_POINTS)


def test_status_strings():
    m = _lib()
    for s in range(8):
        assert m._lib.moe_status_string(s).decode()
    assert "scratch" in m._lib.moe_status_string(7).decode()
    assert m._lib.moe_status_string(0).decode() == "ok"


def _cfg(m, **kw):
    base = dict(hidden=256, inter=128, n_routed=16, n_shared=1, top_k=4, n_group=1, topk_group=1,
                group_topn=2, routed_scaling=2.5, bias_gamma=0.001, scale_mode=0)
    base.update(kw)
    return m.moe_config(*[base[f] for f, _ in m.moe_config._fields_])


def test_host_validation_status_codes():
    m = _lib()
    L = m._lib
    P = ctypes.c_void_p
    fake = P(0x1000)  # never dereferenced: every call below fails validation first
    # NULL pointers
    assert L.moe_quantize_1x128(None, 0, 4, 128, fake, fake, None) == 1
    # shapes
    assert L.moe_quantize_1x128(fake, 0, 4, 100, fake, fake, None) == 2
    assert L.moe_quantize_1x128(fake, 0, -1, 128, fake, fake, None) == 2
    assert L.moe_quantize_128x128(fake, 1, 128, 130, fake, fake, None) == 2
    # dtype
    assert L.moe_quantize_1x128(fake, 7, 4, 128, fake, fake, None) == 3
    # config checks
    bad = [dict(hidden=200), dict(inter=0), dict(n_routed=0), dict(n_routed=1024),
           dict(top_k=17), dict(top_k=20, n_routed=16), dict(n_group=3),
           dict(n_group=4, topk_group=5), dict(n_group=4, topk_group=1, top_k=5),
           dict(n_group=4, topk_group=2, group_topn=5), dict(n_shared=17), dict(n_shared=-1)]
    for b in bad:
        c = _cfg(m, **b)
        assert L.moe_route(ctypes.byref(c), fake, 1, 4, fake, fake, fake, fake, fake, fake, fake,
                           1 << 30, None) == 2, b
        assert L.moe_permute(ctypes.byref(c), 4, fake, fake, fake, fake, fake, 1 << 30, None) == 2, b
    # an unknown scale mode is unsupported (4)
    c = _cfg(m, scale_mode=2)
    assert L.moe_route(ctypes.byref(c), fake, 1, 4, fake, fake, fake, fake, fake, fake, fake,
                       1 << 30, None) == 4
    # the power-of-two quantisers validate like the others
    assert L.moe_quantize_1x128_pow2(None, 0, 4, 128, fake, fake, None) == 1
    assert L.moe_quantize_1x128_pow2(fake, 0, 4, 100, fake, fake, None) == 2
    assert L.moe_quantize_128x128_pow2(fake, 1, 128, 130, fake, fake, None) == 2
    c = _cfg(m)
    big = 1 << 30
    assert L.moe_route(None, fake, 1, 4, fake, fake, fake, fake, fake, fake, fake, big, None) == 1
    assert L.moe_route(ctypes.byref(c), fake, 1, 4, fake, None, fake, fake, fake, fake, fake, big, None) == 1
    assert L.moe_route(ctypes.byref(c), fake, 5, 4, fake, fake, fake, fake, fake, fake, fake, big, None) == 3
    need_r = L.moe_route_workspace_bytes(ctypes.byref(c), 4, 1)
    assert need_r > 0
    assert L.moe_route(ctypes.byref(c), fake, 1, 4, fake, fake, fake, fake, fake, fake, None, 0, None) == 6
    assert L.moe_route(ctypes.byref(c), fake, 1, 4, fake, fake, fake, fake, fake, fake, fake,
                       need_r - 1, None) == 6
    assert L.moe_route(ctypes.byref(c), P(0x1008), 1, 4, fake, fake, fake, fake, fake, fake, fake,
                       need_r, None) == 4   # misaligned x
    # FP32 input needs room for its three bf16 planes
    assert L.moe_route_workspace_bytes(ctypes.byref(c), 4, 0) > need_r
    assert L.moe_router_weights_elems(20, 256) == 3 * 32 * 256
    assert L.moe_router_weights_elems(20, 100) == 0
    assert L.moe_permute(ctypes.byref(c), -2, fake, fake, fake, fake, fake, 1 << 30, None) == 2
    need_p = L.moe_permute_workspace_bytes(ctypes.byref(c), 1000)
    assert need_p == 4 * 16 * 4     # 4 blocks of 256 tokens x 16 experts
    assert L.moe_permute(ctypes.byref(c), 1000, fake, fake, fake, fake, fake, need_p - 1, None) == 6
    assert L.moe_permute(ctypes.byref(c), 1000, fake, fake, fake, fake, None, 0, None) == 6
    assert L.moe_combine(ctypes.byref(c), 4, fake, 1, fake, fake, None, fake, None) == 1  # N_s=1 needs y_shared
    assert L.moe_update_bias(ctypes.byref(c), 4, None, fake, None) == 1
    # grouped FFN: workspace too small, bad expert count
    need = L.moe_grouped_ffn_workspace_bytes(ctypes.byref(c), 16, 256)
    assert need > 256 * 128
    args = [fake] * 10
    assert L.moe_grouped_ffn_fp8(ctypes.byref(c), 16, 256, 64, fake, fake, None, *args[:7], fake, 1,
                                 fake, need - 1, None) == 6
    assert L.moe_grouped_ffn_fp8(ctypes.byref(c), 0, 256, 64, fake, fake, None, *args[:7], fake, 1,
                                 fake, need, None) == 2
    assert L.moe_grouped_ffn_fp8(ctypes.byref(c), 16, 256, 64, fake, fake, None, *args[:7], fake, 9,
                                 fake, need, None) == 3
    # the two halves
    assert L.moe_grouped_ffn_fp8_gate_up(ctypes.byref(c), 16, 256, 64, fake, fake, None, *args[:5],
                                         fake, need - 1, None) == 6
    assert L.moe_grouped_ffn_fp8_gate_up(ctypes.byref(c), 16, 256, 64, fake, fake, None, fake, None,
                                         fake, fake, fake, fake, need, None) == 1
    assert L.moe_grouped_ffn_fp8_gate_up(ctypes.byref(c), 2000, 256, 64, fake, fake, None, *args[:5],
                                         fake, need, None) == 2
    assert L.moe_grouped_ffn_fp8_down(ctypes.byref(c), 16, 256, fake, fake, fake, 1, fake, need - 1,
                                      None) == 6
    assert L.moe_grouped_ffn_fp8_down(ctypes.byref(c), 16, 256, fake, fake, fake, 4, fake, need,
                                      None) == 3
    assert L.moe_grouped_ffn_fp8_down(ctypes.byref(c), 16, 256, fake, None, fake, 1, fake, need,
                                      None) == 1
    # sequence balance statistics
    need_s = L.moe_seq_balance_workspace_bytes(ctypes.byref(c), 1000, 100)
    assert need_s == 10 * 4 * 16 * 12      # 10 sequences x 4 chunks x 16 experts x (f64 + i32)
    assert L.moe_seq_balance_workspace_bytes(ctypes.byref(c), 1000, 300) == 0
    sb = L.moe_seq_balance
    assert sb(ctypes.byref(c), 1000, 0, fake, fake, 0.001, fake, None, fake, need_s, None) == 2
    assert sb(ctypes.byref(c), 1000, 300, fake, fake, 0.001, fake, None, fake, need_s, None) == 2
    assert sb(ctypes.byref(c), -4, 2, fake, fake, 0.001, fake, None, fake, need_s, None) == 2
    assert sb(ctypes.byref(c), 1000, 100, None, fake, 0.001, fake, None, fake, need_s, None) == 1
    assert sb(ctypes.byref(c), 1000, 100, fake, fake, 0.001, None, fake, fake, need_s, None) == 1
    assert sb(ctypes.byref(c), 1000, 100, fake, fake, 0.001, fake, None, fake, need_s - 1, None) == 6
    assert sb(ctypes.byref(c), 1000, 100, fake, fake, 0.001, fake, None, None, need_s, None) == 6
    assert sb(ctypes.byref(c), 1000, 100, fake, fake, 0.001, fake, None, P(0x1004), need_s, None) == 4
    assert sb(ctypes.byref(c), 0, 100, None, None, 0.001, None, None, None, 0, None) == 0
    assert sb(ctypes.byref(c), 1 << 30, 1, fake, fake, 0.001, fake, None, fake, 1 << 62, None) == 2
    # backward entry points
    assert L.moe_combine_backward(ctypes.byref(c), 4, None, fake, 1, fake, fake, fake, fake, None) == 1
    assert L.moe_combine_backward(ctypes.byref(c), 4, fake, fake, 7, fake, fake, fake, fake, None) == 3
    assert L.moe_combine_backward(ctypes.byref(c), -1, fake, fake, 1, fake, fake, fake, fake, None) == 2
    assert L.moe_combine_backward(ctypes.byref(c), 0, None, None, 1, None, None, None, None, None) == 0
    need_rb = L.moe_route_backward_workspace_bytes(ctypes.byref(c), 10)
    assert need_rb >= 2 * 10 * 4 * 4
    rb = L.moe_route_backward
    assert rb(ctypes.byref(c), 10, fake, 1, fake, fake, fake, fake, fake, fake, fake, fake, None, None, 0,
              None) == 1
    assert rb(ctypes.byref(c), 10, fake, 1, fake, fake, fake, fake, fake, fake, fake, fake, fake, fake,
              need_rb - 1, None) == 6
    assert rb(ctypes.byref(c), 10, fake, 5, fake, fake, fake, fake, fake, fake, fake, fake, fake, fake,
              need_rb, None) == 3
    assert L.moe_unpermute_sum(ctypes.byref(c), 4, fake, 1, None, None, fake, None) == 1
    assert L.moe_unpermute_sum(ctypes.byref(c), 4, fake, 9, fake, None, fake, None) == 3
    tr = L.moe_transpose_fp8_blocks
    assert tr(2, 128, 100, fake, fake, fake, fake, 128, 0, None) == 2
    assert tr(2, 128, 128, fake, fake, fake, fake, 128, 128, None) == 2      # col0 + R > dst_cols
    assert tr(2, 128, 128, None, fake, fake, fake, 256, 128, None) == 1
    assert tr(0, 128, 128, None, None, None, None, 256, 0, None) == 0
    need_fb = L.moe_grouped_ffn_backward_workspace_bytes(ctypes.byref(c), 4, 100)
    assert need_fb > 100 * 256
    fb = L.moe_grouped_ffn_fp8_backward
    w10 = [fake] * 10   # row_token, offsets, w1, w1s, w3, w3s, w2t, w2ts, w13t, w13ts

    def fbc(cfg, E, dxt, dx_rows, ws_bytes, ab=(None, None), xq=fake, dout=fake):
        return fb(ctypes.byref(cfg), E, 100, 10, xq, fake, fake, 1, *w10, *ab, dout, None, dx_rows,
                  dxt, fake, fake, fake, 0, fake, ws_bytes, None)
    assert fbc(c, 4, 0, fake, need_fb - 1) == 6
    assert fbc(c, 0, 0, fake, need_fb) == 2
    assert fbc(c, 4, 5, fake, need_fb) == 3
    assert fbc(c, 4, 0, None, need_fb) == 1
    # the SwiGLU inputs come in pairs; without them the forward's codes are needed
    assert fbc(c, 4, 0, fake, need_fb, ab=(fake, None)) == 1
    assert fbc(c, 4, 0, fake, need_fb, ab=(None, fake)) == 1
    assert fbc(c, 4, 0, fake, need_fb, xq=None) == 1
    assert fbc(c, 4, 0, fake, need_fb, dout=None) == 1
    # the upstream gradient is read in 16-byte pieces
    assert fbc(c, 4, 0, fake, need_fb, dout=P(0x1008)) == 4
    p2 = _cfg(m, scale_mode=1)
    assert fbc(p2, 4, 0, fake, need_fb) == 4
    # the training gate/up: both outputs, FP32 group scales only
    tu = L.moe_grouped_ffn_fp8_gate_up_train
    assert tu(ctypes.byref(c), 16, 256, 64, fake, fake, None, *args[:5], None, fake, fake, need,
              None) == 1
    assert tu(ctypes.byref(c), 16, 256, 64, fake, fake, None, *args[:5], fake, fake, fake, need - 1,
              None) == 6
    assert tu(ctypes.byref(p2), 16, 256, 64, fake, fake, None, *args[:5], fake, fake, fake, need,
              None) == 4
    # too large for 32-bit operand offsets
    big = _cfg(m, hidden=16384, inter=16384)
    assert L.moe_grouped_ffn_fp8_gate_up(ctypes.byref(big), 16, 1 << 18, 64, fake, fake, None,
                                         *args[:5], fake, 1 << 62, None) == 4
    assert L.moe_grouped_ffn_fp8_gate_up(ctypes.byref(c), 16, 256, 1 << 25, fake, fake, None,
                                         *args[:5], fake, need, None) == 4


def test_workspace_size_grows_with_rows():
    m = _lib()
    c = _cfg(m)
    a = m._lib.moe_grouped_ffn_workspace_bytes(ctypes.byref(c), 16, 256)
    b = m._lib.moe_grouped_ffn_workspace_bytes(ctypes.byref(c), 16, 4096)
    assert 0 < a < b
    assert m._lib.moe_grouped_ffn_workspace_bytes(ctypes.byref(c), 0, 256) == 0


def test_unpack_inverts_documented_pack_map():
    """MoELayer.unpack against the packed layout written out from its documented index
    map (byte b of lane l, half h of fragment (n16, kc) holds code
    [32*(n16/2) + 8*(j/4) + 4*(n16%2) + j%4][128*kc + 64*h + 16*(l/16) + b], j = l%16)."""
    import numpy as np
    from deepseekmoe_routing_fp8_amd import MoELayer
    rows, cols = 96, 384
    W = np.random.default_rng(5).integers(0, 256, (rows, cols)).astype(np.uint8)
    packed = np.empty(rows * cols, np.uint8)
    nkc = cols // 128
    for n16 in range(rows // 16):
        for kc in range(nkc):
            for h in range(2):
                for l in range(64):
                    j = l % 16
                    r = 32 * (n16 // 2) + 8 * (j // 4) + 4 * (n16 % 2) + j % 4
                    c = 128 * kc + 64 * h + 16 * (l // 16)
                    o = ((n16 * nkc + kc) * 2 + h) * 1024 + l * 16
                    packed[o:o + 16] = W[r, c:c + 16]
    assert np.array_equal(MoELayer.unpack(packed.reshape(rows, cols)), W)
    # every row of a 32-row group appears exactly once across its two fragments
    js = np.arange(16)
    for m in range(rows // 32):
        got = sorted([32 * m + 8 * (j // 4) + 4 * p + j % 4 for p in range(2) for j in js])
        assert got == list(range(32 * m, 32 * m + 32))


def test_intermediate_offsets_and_noalloc_limit():
    """The intermediate's offsets follow the workspace's documented contents (hq after the
    tile plan, hs after hq), and the no-allocation grouped FFN rejects, on the host, a
    request larger than its static scratch array with MOE_ERR_SCRATCH, before any HIP call."""
    m = _lib()
    L = m._lib
    P = ctypes.c_void_p
    fake = P(0x1000)
    c = _cfg(m, hidden=7168, inter=2048, n_routed=256, n_shared=1, top_k=8)
    hq, hs = ctypes.c_size_t(0), ctypes.c_size_t(0)
    rows = 1152
    assert L.moe_grouped_ffn_intermediate_offsets(ctypes.byref(c), 257, rows, ctypes.byref(hq),
                                                  ctypes.byref(hs)) == 0
    assert hq.value % 256 == 0 and hs.value >= hq.value + rows * 2048 and hs.value % 256 == 0
    need = L.moe_grouped_ffn_workspace_bytes(ctypes.byref(c), 257, rows)
    assert hs.value + rows * 16 * 4 <= need
    assert L.moe_grouped_ffn_intermediate_offsets(ctypes.byref(c), 0, rows, ctypes.byref(hq),
                                                  ctypes.byref(hs)) == 2
    assert L.moe_grouped_ffn_intermediate_offsets(ctypes.byref(c), 257, rows, None, ctypes.byref(hs)) == 1
    # the limit: the largest row count that fits, and one 16-row unit more
    assert need <= m.NOALLOC_SCRATCH_BYTES
    big = 4096 * 9
    assert L.moe_grouped_ffn_workspace_bytes(ctypes.byref(c), 257, big) > m.NOALLOC_SCRATCH_BYTES
    args = [fake] * 10
    assert L.moe_grouped_ffn_fp8_noalloc(ctypes.byref(c), 257, big, 4096, *args, fake, 1, None) == 7
    # ordinary validation still comes first
    bad = _cfg(m, hidden=200)
    assert L.moe_grouped_ffn_fp8_noalloc(ctypes.byref(bad), 257, 16, 16, *args, fake, 1, None) == 2
    assert L.moe_grouped_ffn_fp8_noalloc(ctypes.byref(c), 0, 16, 16, *args, fake, 1, None) == 2
