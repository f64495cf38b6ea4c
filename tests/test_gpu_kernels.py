"""Per-kernel parity of the HIP library against the CPU oracle (needs an MI355X).

Both sides see identical seeded inputs; integer and byte outputs must match exactly,
floating outputs within the stated tolerances.
"""
import sys

import numpy as np
import pytest
import torch

import oracle
import synth
from oracle import e4m3
from routing_check import NEAR_TIE, assert_routing_valid

pytestmark = pytest.mark.gpu


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def lib():
    import deepseekmoe_routing_fp8_amd as m
    assert torch.cuda.is_available()
    return m


DEV = "cuda"


def dev(a, dtype=None):
    t = torch.from_numpy(np.ascontiguousarray(a))
    if dtype is not None:
        t = t.to(dtype)
    return t.to(DEV)


def host(t):
    return t.cpu().numpy()


# ---------------------------------------------------------------------------------------
# 1x128 activation quantisation: bit-exact codes and scales
# ---------------------------------------------------------------------------------------
@pytest.mark.parametrize("name,rows", [("tiny", None), ("reduced", None), ("v3_prefill", None),
                                       ("v3_prefill", 1), ("reduced", 3)])
def test_quantize_1x128_matches_oracle(lib, name, rows):
    cfg = synth.PRESETS[name]
    if rows is not None:
        cfg = cfg.with_tokens(rows)
    say(f"quantize_1x128 {name} T={cfg.tokens} H={cfg.hidden_size} {cfg.x_dtype}")
    x = synth.hidden_states(cfg)
    xd = dev(x, torch.bfloat16 if cfg.x_dtype == "bf16" else torch.float32)
    q, s = lib.moe_quantize_1x128(xd)
    torch.cuda.synchronize()
    rq, rs = oracle.quantize_1x128(x)
    assert np.array_equal(host(s).view(np.uint32), rs.view(np.uint32))
    assert np.array_equal(host(q), rq)


def _edge_tiles():
    rng = np.random.default_rng(7)
    tiles = []
    tiles.append(np.zeros(128))                                   # all zero -> s = 1
    t = rng.standard_normal(128); t[5] = 1e4; tiles.append(t)      # one outlier
    tiles.append(np.full(128, -3.25))                              # constant
    t = np.zeros(128); t[0] = -0.0; t[1] = 1e-30; tiles.append(t)  # -0 and a tiny value
    tiles.append(rng.standard_normal(128) * 1e-38)                 # float32 subnormal range
    tiles.append(rng.standard_normal(128) * 5e37)                  # near float32 max
    # amax 448 -> s = 1 exactly: every E4M3 value, midpoint and +-1 ulp neighbour
    pos = e4m3.finite_values()
    mids = (pos[:-1] + pos[1:]) / 2
    pts = np.concatenate([pos, mids]).astype(np.float32)
    nb = np.concatenate([pts, np.nextafter(pts, np.float32(0)), np.nextafter(pts, np.float32(1e9))])
    nb = np.concatenate([nb, -nb])
    nb = nb[np.abs(nb) <= 448]
    n = (len(nb) + 126) // 127
    for i in range(n):
        chunk = nb[i * 127:(i + 1) * 127]
        t = np.zeros(128, np.float32)
        t[:len(chunk)] = chunk
        t[127] = 448.0
        tiles.append(t)
    return np.stack(tiles).astype(np.float32)


def test_quantize_1x128_edge_cases(lib):
    x = _edge_tiles()
    say(f"quantize_1x128 edge tiles {x.shape}")
    q, s = lib.moe_quantize_1x128(dev(x))
    torch.cuda.synchronize()
    rq, rs = oracle.quantize_1x128(x)
    assert np.array_equal(host(s).view(np.uint32), rs.view(np.uint32))
    assert np.array_equal(host(q), rq)


def _midpoint_tiles():
    """Tiles whose quotients v / s sit on, and one float32 ulp either side of, every E4M3
    rounding midpoint, under scales away from 1 (codes are decided on fl32(v / s), so an
    error of one ulp in the division shows as a different code). Scales cover both sides
    of 2^-80 and 2^80, and values below 2^-100 of both signs."""
    rng = np.random.default_rng(11)
    pos = e4m3.finite_values().astype(np.float64)
    mids = (pos[:-1] + pos[1:]) / 2
    targets = list(rng.uniform(0.5, 2.0, 12)) + list(np.exp2(rng.uniform(-60, 60, 12))) + \
        [2.0 ** -79, 2.0 ** -81, 7e23, 2e24, 1e-30, 1e30]
    tiles = []
    for st in targets:
        amax = np.float32(448.0 * st)
        s = np.float32(amax / np.float32(448.0))
        base = (mids * np.float64(s)).astype(np.float32)
        cand = np.concatenate([base, np.nextafter(base, np.float32(0)), np.nextafter(base, np.float32(3e38))])
        cand = np.concatenate([cand, -cand, np.float32([2.0 ** -101, -2.0 ** -101, 1e-35, -1e-35, 0.0, -0.0])])
        cand = cand[np.abs(cand) <= amax]
        for i in range(0, len(cand), 127):
            t = np.zeros(128, np.float32)
            chunk = cand[i:i + 127]
            t[:len(chunk)] = chunk
            t[127] = amax
            tiles.append(t)
    return np.stack(tiles)


def test_quantize_1x128_midpoints_non_unit_scales(lib):
    x = _midpoint_tiles()
    say(f"quantize_1x128 midpoint tiles {x.shape}")
    q, s = lib.moe_quantize_1x128(dev(x))
    torch.cuda.synchronize()
    rq, rs = oracle.quantize_1x128(x)
    assert np.array_equal(host(s).view(np.uint32), rs.view(np.uint32))
    assert np.array_equal(host(q), rq)


def test_quantize_1x128_bf16_sweep(lib):
    """Every finite bf16 bit pattern, 127 per tile next to a fixed amax of 448."""
    b = np.arange(0, 1 << 16, dtype=np.uint32)
    v = (b << 16).view(np.float32)
    v = v[np.isfinite(v) & (np.abs(v) <= 448)]
    n = (len(v) + 126) // 127
    x = np.zeros((n, 128), np.float32)
    x[:, 127] = 448.0
    flat = x[:, :127].reshape(-1)
    flat[:len(v)] = v
    x[:, :127] = flat.reshape(n, 127)
    say(f"quantize_1x128 bf16 sweep {x.shape}")
    xd = dev(x, torch.bfloat16)
    q, s = lib.moe_quantize_1x128(xd)
    torch.cuda.synchronize()
    rq, rs = oracle.quantize_1x128(x)
    assert np.all(host(s) == 1.0) and np.array_equal(host(s), rs)
    assert np.array_equal(host(q), rq)


# ---------------------------------------------------------------------------------------
# 128x128 weight quantisation: bit-exact
# ---------------------------------------------------------------------------------------
def test_quantize_128x128_matches_oracle(lib):
    rng = np.random.default_rng(8)
    w = (rng.standard_normal((3, 256, 384)) * np.exp2(rng.integers(-8, 8, (3, 1, 1)))).astype(np.float32)
    w[1, :128, :128] = 0.0
    w[2, 5, 300] = 1e6
    say("quantize_128x128 random [3,256,384]")
    q, s = lib.moe_quantize_128x128(dev(w))
    torch.cuda.synchronize()
    for i in range(3):
        rq, rs = oracle.quantize_128x128(w[i])
        assert np.array_equal(host(s[i]).view(np.uint32), rs.view(np.uint32))
        assert np.array_equal(host(q[i]), rq)
    cfg = synth.PRESETS["reduced"]
    for e in (0, 63):
        say(f"quantize_128x128 reduced expert {e}")
        for wm in synth.routed_expert_weights(cfg, e):
            q, s = lib.moe_quantize_128x128(dev(wm))
            torch.cuda.synchronize()
            rq, rs = oracle.quantize_128x128(wm)
            assert np.array_equal(host(s).view(np.uint32), rs.view(np.uint32))
            assert np.array_equal(host(q), rq)


# ---------------------------------------------------------------------------------------
# Router
# ---------------------------------------------------------------------------------------
def check_routing(cfg, x, wr, b, g_scores, g_idx, g_gate, g_counts):
    """Indices exact outside declared near-ties; gates and scores within tolerance."""
    r = oracle.route(x, wr, b, cfg.num_experts_per_tok, cfg.n_group, cfg.topk_group,
                     cfg.group_score_topn, cfg.routed_scaling_factor)
    assert np.max(np.abs(g_scores - r["s"])) < 5e-7
    # the same set as the oracle's outside declared near-ties; inside them, every substituted
    # expert or group within the band; slots in descending score outside the band
    assert_routing_valid(r, g_idx, cfg)
    tie = (r["kth_gap"] < NEAR_TIE) | (r["group_gap"] < NEAR_TIE)
    k = cfg.num_experts_per_tok
    assert np.array_equal(g_counts, np.bincount(g_idx.ravel(), minlength=cfg.num_experts))
    if not np.any(tie):
        assert np.array_equal(g_counts, r["counts"])
    # gates from the oracle's affinities at the GPU's selection
    rf = oracle.route(x, wr, b, k, cfg.n_group, cfg.topk_group, cfg.group_score_topn,
                      cfg.routed_scaling_factor, force_idx=g_idx)
    assert np.allclose(g_gate, rf["gate"], rtol=2e-6, atol=0)
    assert np.allclose(g_gate.sum(1), cfg.routed_scaling_factor, rtol=1e-5)
    return int(tie.sum())


@pytest.mark.parametrize("name", ["tiny", "reduced", "v3_prefill", "v3_decode"])
def test_route_matches_oracle(lib, name):
    cfg = synth.PRESETS[name]
    say(f"route {name} T={cfg.tokens}")
    x = synth.hidden_states(cfg)
    wr = synth.router_weight(cfg)
    b = synth.expert_bias(cfg)
    xd = dev(x, torch.bfloat16 if cfg.x_dtype == "bf16" else torch.float32)
    c = lib.make_config(cfg)
    s, idx, gate, counts = lib.moe_route(c, xd, lib.moe_pack_router_weights(dev(wr)), dev(b))
    torch.cuda.synchronize()
    nt = check_routing(cfg, x, wr, b, host(s), host(idx), host(gate), host(counts))
    say(f"  near-tie tokens: {nt}")


def test_route_group_limit_binds_with_bias(lib):
    """V3 grouping with a large random bias, so that the group choice decides."""
    cfg = synth.PRESETS["v3_decode"]
    x = synth.hidden_states(cfg)
    wr = synth.router_weight(cfg)
    b = np.random.default_rng(9).uniform(-0.3, 0.3, cfg.num_experts).astype(np.float32)
    say("route v3_decode shapes, large bias")
    c = lib.make_config(cfg)
    s, idx, gate, counts = lib.moe_route(c, dev(x, torch.bfloat16), lib.moe_pack_router_weights(dev(wr)), dev(b))
    torch.cuda.synchronize()
    check_routing(cfg, x, wr, b, host(s), host(idx), host(gate), host(counts))
    free = oracle.route(x, wr, b, 8)
    assert np.any(free["idx"] != host(idx))  # the limit changed some selection


def test_route_general_shapes(lib):
    """Groups of uneven use, k = 1, N_r not a multiple of 64, fp32 input."""
    import dataclasses
    base = synth.PRESETS["tiny"]
    for kw in [dict(num_experts=48, num_experts_per_tok=1, n_group=4, topk_group=2, group_score_topn=3),
               dict(num_experts=96, num_experts_per_tok=5, n_group=6, topk_group=3),
               dict(num_experts=16, num_experts_per_tok=16),
               dict(tokens=1), dict(tokens=130, num_experts=32, num_experts_per_tok=3),
               dict(tokens=300, num_experts=20, num_experts_per_tok=3, n_group=4, topk_group=2),
               dict(tokens=700, hidden_size=1024, num_experts=200, num_experts_per_tok=6, n_group=8,
                    topk_group=3, group_score_topn=2),
               # the largest configuration the library accepts: N_r = 512, k = 16, G = 64
               dict(tokens=257, num_experts=512, num_experts_per_tok=16, n_group=64, topk_group=4,
                    group_score_topn=2),
               dict(tokens=100, hidden_size=512, num_experts=512, num_experts_per_tok=16)]:
        cfg = dataclasses.replace(base, **kw)
        say(f"route general {kw}")
        x = synth.hidden_states(cfg)
        rng = np.random.default_rng(11)
        wr = (rng.standard_normal((cfg.num_experts, cfg.hidden_size)) / 16).astype(np.float32)
        b = rng.uniform(-0.05, 0.05, cfg.num_experts).astype(np.float32)
        s, idx, gate, counts = lib.moe_route(lib.make_config(cfg), dev(x), lib.moe_pack_router_weights(dev(wr)), dev(b))
        torch.cuda.synchronize()
        check_routing(cfg, x, wr, b, host(s), host(idx), host(gate), host(counts))


def _unpack_router(flat, N, H):
    """Packed router planes -> [3, N, H] by the documented index map (re-indexing only)."""
    nb16 = (N + 15) // 16
    f = flat.reshape(3, nb16, H // 32, 4, 16, 8)            # q, block, K step, lane/16, lane%16, j
    full = f.transpose(0, 1, 4, 2, 3, 5).reshape(3, nb16 * 16, H)
    return full[:, :N], full[:, N:]


def test_pack_router_weights_exact(lib):
    """hi + mid + lo reproduces every FP32 weight exactly; hi is the RNE bf16 of W_r; rows
    past N_r are zero."""
    rng = np.random.default_rng(13)
    N, H = 60, 512
    w = (rng.standard_normal((N, H)) * np.exp2(rng.integers(-30, 30, (N, H)))).astype(np.float32)
    w[0, :4] = [0.0, -0.0, 1.0, -3.0e-38]
    say("pack router weights")
    flat = lib.moe_pack_router_weights(dev(w))
    assert flat.numel() == lib.moe_router_weights_elems(N, H) == 3 * 64 * H
    sp, pad = _unpack_router(flat.float().cpu().numpy().astype(np.float64), N, H)
    assert np.all(pad == 0)
    total = sp[0] + sp[1] + sp[2]
    exact = (np.abs(w) >= 2.0 ** -110) | (w == 0)
    assert np.array_equal(total[exact], w.astype(np.float64)[exact])
    # below 2^-110 the last piece is limited by bf16's subnormal grid (2^-133)
    assert np.all(np.abs(total - w.astype(np.float64))[~exact] <= 2.0 ** -133)
    hi = torch.from_numpy(w).to(torch.bfloat16).float().numpy()
    assert np.array_equal(sp[0].astype(np.float32), hi)


# ---------------------------------------------------------------------------------------
# Permutation: bit-exact
# ---------------------------------------------------------------------------------------
def _idx(rng, T, N, k, skew=None):
    if skew is None:
        return np.stack([rng.permutation(N)[:k] for _ in range(T)]).astype(np.int32)
    p = np.arange(1, N + 1) ** (-skew)
    p /= p.sum()
    return np.stack([rng.choice(N, k, replace=False, p=p) for _ in range(T)]).astype(np.int32)


def _check_permute(idx, N, S, off, rt, ro):
    """Routed part bit-exact against the oracle; shared segments by their closed form."""
    T, k = idx.shape
    off, rt, ro = host(off), host(rt), host(ro)
    valid = (idx >= 0) & (idx < N)
    if valid.all():
        r_off, r_rt, r_ro = oracle.permute(idx, N)
        assert np.array_equal(off[:N + 1], r_off)
        assert np.array_equal(rt[:T * k], r_rt)
        assert np.array_equal(ro, r_ro)
    V = int(valid.sum())
    assert off[N] == V
    assert np.array_equal(off[N + 1:], T * k + T * np.arange(1, S + 1))
    assert np.all(rt[V:T * k] == -1)
    assert np.array_equal(rt[T * k:], np.tile(np.arange(T), S))
    return off, rt, ro


@pytest.mark.parametrize("T,N,k,skew,S", [(64, 16, 4, None, 1), (4096, 256, 8, None, 1),
                                          (16384, 256, 8, 1.1, 1), (1, 256, 8, None, 1),
                                          (1500, 512, 16, None, 0), (3000, 64, 6, 2.0, 2),
                                          # one block of tokens (the one-launch path)
                                          (128, 256, 8, None, 1), (256, 512, 16, None, 2),
                                          (200, 256, 8, 1.1, 1), (256, 64, 6, 2.0, 0),
                                          (257, 256, 8, None, 1)])
def test_permute_matches_oracle(lib, T, N, k, skew, S):
    import dataclasses
    cfg = dataclasses.replace(synth.PRESETS["tiny"], num_experts=N, num_experts_per_tok=k, tokens=T,
                              num_shared_experts=S)
    rng = np.random.default_rng(T + N)
    idx = _idx(rng, T, N, k, skew)
    say(f"permute T={T} N={N} k={k} skew={skew} S={S}")
    off, rt, ro = lib.moe_permute(lib.make_config(cfg), dev(idx))
    torch.cuda.synchronize()
    _check_permute(idx, N, S, off, rt, ro)


@pytest.mark.parametrize("T", [500, 200])
def test_permute_invalid_entries(lib, T):
    """Entries naming no routed expert are skipped; the rows they leave free read token -1
    (T = 200: the one-launch path of a single token block)."""
    import dataclasses
    N, k, S = 64, 6, 2
    cfg = dataclasses.replace(synth.PRESETS["tiny"], num_experts=N, num_experts_per_tok=k, tokens=T,
                              num_shared_experts=S)
    rng = np.random.default_rng(5)
    idx = _idx(rng, T, N, k)
    idx[rng.random((T, k)) < 0.05] = -1
    idx[7, 2] = N + 3
    say(f"permute with invalid entries T={T}")
    off, rt, ro = lib.moe_permute(lib.make_config(cfg), dev(idx))
    torch.cuda.synchronize()
    off, rt, ro = _check_permute(idx, N, S, off, rt, ro)
    valid = (idx >= 0) & (idx < N)
    assert np.all(ro[~valid] == -1)
    # every valid pair has its own row, inside its expert's segment, naming its token
    rows = ro[valid]
    assert len(set(rows.tolist())) == rows.size
    e = idx[valid]
    assert np.all((off[e] <= rows) & (rows < off[e + 1]))
    assert np.array_equal(rt[rows], np.nonzero(valid)[0])


def test_permute_collapse_and_empty(lib):
    import dataclasses
    cfg = dataclasses.replace(synth.PRESETS["v3_prefill"], tokens=2048)
    c = lib.make_config(cfg)
    idx = np.tile(np.arange(200, 208, dtype=np.int32), (2048, 1))
    say("permute collapse")
    off, rt, ro = lib.moe_permute(c, dev(idx))
    torch.cuda.synchronize()
    off, _, _ = _check_permute(idx, 256, 1, off, rt, ro)
    cnt = np.diff(off[:257])
    assert np.all(cnt[200:208] == 2048) and cnt.sum() == 2048 * 8
    say("permute collapse, one token block")
    off, rt, ro = lib.moe_permute(lib.make_config(dataclasses.replace(cfg, tokens=256)), dev(idx[:256]))
    torch.cuda.synchronize()
    off, _, _ = _check_permute(idx[:256], 256, 1, off, rt, ro)
    assert np.all(np.diff(off[:257])[200:208] == 256)
    say("permute T=0")
    off, rt, ro = lib.moe_permute(c, torch.empty((0, 8), dtype=torch.int32, device=DEV))
    torch.cuda.synchronize()
    assert np.all(host(off) == 0)


# ---------------------------------------------------------------------------------------
# Grouped FP8 SwiGLU experts
# ---------------------------------------------------------------------------------------
def _rand_codes(rng, shape):
    c = rng.integers(0, 0x7F, shape).astype(np.uint8)
    return c | (rng.integers(0, 2, shape).astype(np.uint8) << 7)


def _expert_set(rng, E, H, I):
    f = lambda n, k: rng.uniform(0.5, 2.0, (E, n // 128, k // 128)).astype(np.float32) / 448
    w1 = _rand_codes(rng, (E, I, H)); w3 = _rand_codes(rng, (E, I, H)); w2 = _rand_codes(rng, (E, H, I))
    return w1, f(I, H), w3, f(I, H), w2, f(H, I)


def _device_weights(lib, w):
    """Row-major codes and scales -> device tensors, codes in the packed FFN layout."""
    out = []
    for i, a in enumerate(w):
        t = dev(a)
        out.append(lib.moe_pack_fp8_weights(t) if i % 2 == 0 else t)
    return out


def _pack_reference(W):
    """The packed layout by its documented index map (pure re-indexing, no arithmetic)."""
    rows, cols = W.shape
    nkc = cols // 128
    n16, kc, h, l, b = np.meshgrid(np.arange(rows // 16), np.arange(nkc), np.arange(2),
                                   np.arange(64), np.arange(16), indexing="ij")
    j = l % 16
    src = W[32 * (n16 // 2) + 8 * (j // 4) + 4 * (n16 % 2) + j % 4, 128 * kc + 64 * h + 16 * (l // 16) + b]
    return src.reshape(-1)


@pytest.mark.parametrize("mats,rows,cols", [(1, 32, 128), (3, 96, 384), (2, 2048, 1024)])
def test_pack_fp8_weights_layout(lib, mats, rows, cols):
    rng = np.random.default_rng(rows + cols)
    W = rng.integers(0, 256, (mats, rows, cols)).astype(np.uint8)
    say(f"pack {mats}x{rows}x{cols}")
    got = host(lib.moe_pack_fp8_weights(dev(W))).reshape(mats, -1)
    from deepseekmoe_routing_fp8_amd import MoELayer
    for i in range(mats):
        assert np.array_equal(got[i], _pack_reference(W[i]))
        assert np.array_equal(MoELayer.unpack(got[i].reshape(rows, cols)), W[i])


def _relerr(a, b):
    return np.linalg.norm(a - b) / max(np.linalg.norm(b), 1e-300)


@pytest.mark.parametrize("H,I,E,loads,identity", [
    (256, 128, 4, [0, 17, 64, 3], False),
    (512, 256, 3, [193, 1, 400], False),          # several M tiles, tiny tail
    (384, 256, 2, [16, 33], True),                 # identity token map, H % 256 == 128
    # identity token map over many segments, empty ones first, last and between: each
    # row's token comes from the segment that holds it, found without the tile plan
    (256, 128, 12, [0, 5, 17, 0, 33, 1, 0, 0, 64, 3, 160, 0], True),
    (1024, 512, 5, [130, 0, 0, 7, 250], False),
    # every tile height the kernel specialises (2, 4, 6, 8, 9, 10 16-row tiles) on both
    # sides of its boundary, and the 160-row split into two tiles
    (256, 256, 12, [160, 161, 16, 17, 48, 80, 112, 113, 128, 129, 144, 145], False),
    # K chunk counts of 5, 7 (gate/up) and 3, 5 (down): blocks end in padding steps
    # inside a pair of steps, with several n-blocks per workgroup
    (640, 384, 3, [150, 9, 200], False),
    (896, 640, 2, [77, 161], True),
    # the V3 expert shape (H = 7168, I = 2048): a full 160-row tile, a ragged one, one row
    (7168, 2048, 3, [160, 137, 1], False),
    # segments averaging >= 256 rows get 192-row tiles (12 16-row tiles: 380 -> 192 + 188,
    # 370 -> 192 + 178) beside shorter ones (200 -> 112 + 96)
    (1024, 512, 3, [380, 370, 200], False),
    (768, 384, 2, [384, 191], True),
    # tall tiles with one n-block per gate/up workgroup: 8 and 16 workgroups per tile, the
    # shared-weight XCD layout for the multi-tile experts (600 -> 4 tiles, 520 -> 3)
    (512, 1024, 2, [600, 300], False),
    (256, 2048, 2, [520, 100], False),
    # the largest contraction the kernel takes: K = 16384 in each phase
    (16384, 256, 2, [40, 7], False),
    (256, 16384, 2, [33, 0], False),
])
@pytest.mark.parametrize("ydt", ["float32", "bfloat16"])   # the two down-projection layouts
def test_grouped_ffn_matches_oracle(lib, H, I, E, loads, identity, ydt):
    import dataclasses
    rng = np.random.default_rng(H + I + E)
    rows = int(sum(loads))
    T = rows if identity else 300
    cfg = dataclasses.replace(synth.PRESETS["tiny"], hidden_size=H, moe_intermediate_size=I,
                              num_experts=max(E, 4), num_experts_per_tok=1, tokens=T)
    x = rng.standard_normal((T, H)).astype(np.float32)
    xq, xs = oracle.quantize_1x128(x)
    offsets = np.concatenate([[0], np.cumsum(loads)]).astype(np.int32)
    row_token = (np.arange(rows) - np.repeat(offsets[:-1], loads)).astype(np.int32) if identity \
        else rng.integers(0, T, rows).astype(np.int32)
    w = _expert_set(rng, E, H, I)
    say(f"grouped_ffn H={H} I={I} E={E} loads={loads} identity={identity} y={ydt}")
    y = lib.moe_grouped_ffn_fp8(lib.make_config(cfg), E, rows, dev(xq), dev(xs),
                                None if identity else dev(row_token), dev(offsets),
                                *_device_weights(lib, w), y_dtype=getattr(torch, ydt))
    torch.cuda.synchronize()
    y = y.float().cpu().numpy()
    for e in range(E):
        lo, hi = offsets[e], offsets[e + 1]
        if hi == lo:
            continue
        toks = row_token[lo:hi]
        ref = oracle.expert_ffn(xq[toks], xs[toks], w[0][e], w[1][e], w[2][e], w[3][e], w[4][e], w[5][e])[0]
        err = _relerr(y[lo:hi], ref)
        assert err < 5e-3, (e, err)


@pytest.mark.parametrize("ydt", ["float32", "bfloat16"])
def test_grouped_ffn_halves_equal_fused_call(lib, ydt):
    """gate_up + down on one workspace gives the fused call's output bit for bit (a load
    mix with several M tiles per expert, so the tile order differs from expert order)."""
    import dataclasses
    rng = np.random.default_rng(77)
    H, I, E = 768, 384, 6
    loads = [5, 400, 0, 193, 64, 250]
    rows, T = int(sum(loads)), 333
    cfg = dataclasses.replace(synth.PRESETS["tiny"], hidden_size=H, moe_intermediate_size=I,
                              num_experts=8, num_experts_per_tok=1, tokens=T)
    c = lib.make_config(cfg)
    x = rng.standard_normal((T, H)).astype(np.float32)
    xq, xs = oracle.quantize_1x128(x)
    offsets = np.concatenate([[0], np.cumsum(loads)]).astype(np.int32)
    row_token = rng.integers(0, T, rows).astype(np.int32)
    w = _device_weights(lib, _expert_set(rng, E, H, I))
    args = (dev(xq), dev(xs), dev(row_token), dev(offsets))
    say(f"grouped_ffn halves vs fused, y={ydt}")
    y_fused = lib.moe_grouped_ffn_fp8(c, E, rows, *args, *w, y_dtype=getattr(torch, ydt))
    ws = lib.moe_grouped_ffn_fp8_gate_up(c, E, rows, *args, *w[:4])
    y_split = lib.moe_grouped_ffn_fp8_down(c, E, rows, w[4], w[5], ws, y_dtype=getattr(torch, ydt))
    torch.cuda.synchronize()
    assert torch.equal(y_fused.view(torch.uint8), y_split.view(torch.uint8))


@pytest.mark.parametrize("H,I,loads", [
    (512, 256, [5, 400, 0, 193, 64, 250]),     # 160-row tiles, ragged tails
    (1024, 512, [380, 370, 200]),              # 192-row tiles (12 16-row tiles) beside shorter
    (7168, 2048, [160, 137, 1]),               # the V3 expert shape
])
def test_gate_up_train_keeps_swiglu_inputs(lib, H, I, loads):
    """The training gate/up launch leaves the same (hq, hs) as the plain one, bit for bit,
    and its a = G, b = U (FP32 rows) are the FP64 products of the oracle within the FP32
    promotion of the MFMA's partial sums (rows without a token: zeros)."""
    import dataclasses
    rng = np.random.default_rng(H + len(loads))
    E, rows, T = len(loads), int(sum(loads)), 301
    cfg = dataclasses.replace(synth.PRESETS["tiny"], hidden_size=H, moe_intermediate_size=I,
                              num_experts=max(E, 4), num_experts_per_tok=1, tokens=T)
    c = lib.make_config(cfg)
    x = rng.standard_normal((T, H)).astype(np.float32)
    xq, xs = oracle.quantize_1x128(x)
    offsets = np.concatenate([[0], np.cumsum(loads)]).astype(np.int32)
    row_token = rng.integers(0, T, rows).astype(np.int32)
    row_token[rng.choice(rows, 3, replace=False)] = -1
    w = _expert_set(rng, E, H, I)
    wd = _device_weights(lib, w)
    args = (dev(xq), dev(xs), dev(row_token), dev(offsets))
    say(f"gate_up_train H={H} I={I} loads={loads}")
    ws_plain = lib.moe_grouped_ffn_fp8_gate_up(c, E, rows, *args, *wd[:4])
    ws_train, a, b = lib.moe_grouped_ffn_fp8_gate_up_train(c, E, rows, *args, *wd[:4])
    torch.cuda.synchronize()
    hq0, hs0 = lib.grouped_ffn_intermediate(c, E, rows, ws_plain)
    hq1, hs1 = lib.grouped_ffn_intermediate(c, E, rows, ws_train)
    assert torch.equal(hq0, hq1) and torch.equal(hs0, hs1)
    a, b = a.cpu().numpy(), b.cpu().numpy()
    dead = row_token < 0
    assert not np.any(a[dead]) and not np.any(b[dead])
    for e in range(E):
        lo, hi = offsets[e], offsets[e + 1]
        live = np.nonzero(~dead[lo:hi])[0] + lo
        if len(live) == 0:
            continue
        act = oracle.dequant_1x128(xq[row_token[live]], xs[row_token[live]])
        g = act @ oracle.dequant_128x128(w[0][e], w[1][e]).T
        u = act @ oracle.dequant_128x128(w[2][e], w[3][e]).T
        e_a, e_b = _relerr(a[live], g), _relerr(b[live], u)
        say(f"  expert {e} ({len(live)} rows): a {e_a:.2e}, b {e_b:.2e}")
        # measured 5.4-5.5e-5 with these random codes
        assert e_a < 3e-4 and e_b < 3e-4, (e, e_a, e_b)


def test_grouped_ffn_bf16_output_and_bad_tokens(lib):
    import dataclasses
    rng = np.random.default_rng(21)
    H, I, E = 256, 256, 2
    loads = [40, 24]
    rows, T = 64, 50
    cfg = dataclasses.replace(synth.PRESETS["tiny"], hidden_size=H, moe_intermediate_size=I,
                              num_experts=4, num_experts_per_tok=1, tokens=T)
    x = rng.standard_normal((T, H)).astype(np.float32)
    xq, xs = oracle.quantize_1x128(x)
    offsets = np.array([0, 40, 64], np.int32)
    row_token = rng.integers(0, T, rows).astype(np.int32)
    row_token[3] = -1
    row_token[50] = T + 5        # out of range -> y row is 0
    w = _expert_set(rng, E, H, I)
    say("grouped_ffn bf16 output, invalid tokens")
    y = lib.moe_grouped_ffn_fp8(lib.make_config(cfg), E, rows, dev(xq), dev(xs), dev(row_token),
                                dev(offsets), *_device_weights(lib, w), y_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    y = y.float().cpu().numpy()
    assert np.all(y[3] == 0) and np.all(y[50] == 0)
    for e in range(E):
        lo, hi = offsets[e], offsets[e + 1]
        ok = [r for r in range(lo, hi) if 0 <= row_token[r] < T]
        ref = oracle.expert_ffn(xq[row_token[ok]], xs[row_token[ok]], *[a[e] for a in w])[0]
        assert _relerr(y[ok], ref) < 5e-3


# ---------------------------------------------------------------------------------------
# Combine and bias update
# ---------------------------------------------------------------------------------------
@pytest.mark.parametrize("T,H,k,S", [(64, 256, 4, 1), (300, 2048, 6, 2), (17, 7168, 8, 1), (5, 128, 2, 0),
                                     (40, 512, 16, 16)])   # k and N_s at their maxima
def test_combine_matches_oracle(lib, T, H, k, S):
    import dataclasses
    rng = np.random.default_rng(T * H)
    cfg = dataclasses.replace(synth.PRESETS["tiny"], hidden_size=H, num_experts=max(16, k),
                              num_experts_per_tok=k, num_shared_experts=S, tokens=T)
    y_rows = synth.to_bf16_exact(rng.standard_normal((T * k, H)).astype(np.float32))
    y_sh = synth.to_bf16_exact(rng.standard_normal((max(S, 1) * T, H)).astype(np.float32))
    row_of = rng.permutation(T * k).reshape(T, k).astype(np.int32)
    gate = rng.uniform(0, 1, (T, k)).astype(np.float32)
    say(f"combine T={T} H={H} k={k} S={S}")
    out = lib.moe_combine(lib.make_config(cfg), dev(y_rows, torch.bfloat16), dev(row_of), dev(gate),
                          dev(y_sh[:S * T], torch.bfloat16) if S else None)
    torch.cuda.synchronize()
    got = out.float().cpu().numpy().astype(np.float64)
    ref = oracle.combine(y_rows, row_of, gate, [y_sh[s * T:(s + 1) * T] for s in range(S)])
    # one bf16 rounding of an FP32 sum: |err| <= 2^-8 |ref| + FP32 summation error
    bound = np.abs(ref) * 2.0 ** -8 + 1e-5 * (np.abs(y_rows[row_of]).sum(1) + S * 4)
    assert np.all(np.abs(got - ref) <= bound)


def test_update_bias_matches_oracle_over_trajectory(lib):
    cfg = synth.PRESETS["v3_prefill"]
    c = lib.make_config(cfg)
    N, T, k = cfg.num_experts, cfg.tokens, cfg.num_experts_per_tok
    rng = np.random.default_rng(12)
    b = np.zeros(N, np.float32)
    bd = dev(b)
    say("update_bias 100 steps")
    for step in range(100):
        counts = rng.multinomial(T * k, np.ones(N) / N).astype(np.int32)
        counts[step % N] = T * k // N   # exactly on target -> unchanged
        lib.moe_update_bias(c, T, dev(counts), bd)
        b = oracle.bias_update(b, counts, T, k, cfg.expert_bias_update_rate)
    torch.cuda.synchronize()
    assert np.array_equal(host(bd).view(np.uint32), b.view(np.uint32))


# ---------------------------------------------------------------------------------------
# Power-of-two scale variant (scale_mode 1)
# ---------------------------------------------------------------------------------------
def test_quantize_pow2_matches_oracle(lib):
    rng = np.random.default_rng(21)
    x = (rng.standard_normal((67, 384)) * np.exp(rng.uniform(-20, 20, (67, 1)))).astype(np.float32)
    x[3, :128] = 0.0
    x[5, 7] = np.float32(448.0 * 2.0 ** -3)            # amax exactly 448 * 2^k
    x[6, 130] = np.nextafter(np.float32(448.0), np.float32(1e9))
    x[8, 260] = np.float32(1e-42)                      # subnormal-only tile
    x[8, 256:260] = 0.0
    xb = synth.to_bf16_exact(x)
    for arr, dt in ((x, torch.float32), (xb, torch.bfloat16)):
        say(f"quantize_1x128_pow2 {dt}")
        q, s = lib.moe_quantize_1x128(dev(arr, dt), pow2=True)
        torch.cuda.synchronize()
        rq, rs = oracle.quantize_1x128_pow2(arr)
        assert np.array_equal(host(q), rq)
        assert np.array_equal(host(s).view(np.uint32), rs.view(np.uint32))
    w = (rng.standard_normal((2, 256, 384)) * 0.05).astype(np.float32)
    w[1, :128, 128:256] *= 1e-30
    say("quantize_128x128_pow2")
    q, s = lib.moe_quantize_128x128(dev(w), pow2=True)
    torch.cuda.synchronize()
    for m in range(2):
        rq, rs = oracle.quantize_128x128_pow2(w[m])
        assert np.array_equal(host(q)[m], rq)
        assert np.array_equal(host(s)[m].view(np.uint32), rs.view(np.uint32))


@pytest.mark.parametrize("H,I,E,loads", [(256, 128, 4, [0, 17, 64, 3]),
                                         (384, 256, 3, [160, 161, 33]),
                                         (1024, 512, 5, [130, 0, 7, 250, 16])])
def test_grouped_ffn_pow2_matches_oracle(lib, H, I, E, loads):
    import dataclasses
    rng = np.random.default_rng(H * 7 + E)
    rows, T = int(sum(loads)), 200
    cfg = dataclasses.replace(synth.PRESETS["tiny"], hidden_size=H, moe_intermediate_size=I,
                              num_experts=max(E, 4), num_experts_per_tok=1, tokens=T)
    x = rng.standard_normal((T, H)).astype(np.float32)
    xq, xs = oracle.quantize_1x128_pow2(x)
    offsets = np.concatenate([[0], np.cumsum(loads)]).astype(np.int32)
    row_token = rng.integers(0, T, rows).astype(np.int32)
    w = []
    for n, k in ((I, H), (I, H), (H, I)):
        q = np.empty((E, n, k), np.uint8)
        sc = np.empty((E, n // 128, k // 128), np.float32)
        for e in range(E):
            q[e], sc[e] = oracle.quantize_128x128_pow2((rng.standard_normal((n, k)) / np.sqrt(k)).astype(np.float32))
        w += [q, sc]
    say(f"grouped_ffn pow2 H={H} I={I} E={E} loads={loads}")
    c = lib.make_config(cfg, lib.SCALE_POW2)
    for yt in (torch.float32, torch.bfloat16):
        y = lib.moe_grouped_ffn_fp8(c, E, rows, dev(xq), dev(xs), dev(row_token), dev(offsets),
                                    *_device_weights(lib, w), y_dtype=yt)
        torch.cuda.synchronize()
        y = host(y.float()).astype(np.float64)
        for e in range(E):
            lo, hi = offsets[e], offsets[e + 1]
            if hi == lo:
                continue
            toks = row_token[lo:hi]
            ref = oracle.expert_ffn(xq[toks], xs[toks], w[0][e], w[1][e], w[2][e], w[3][e], w[4][e],
                                    w[5][e], pow2=True)[0]
            err = _relerr(y[lo:hi], ref)
            assert err < 5e-3, (yt, e, err)


# ---------------------------------------------------------------------------------------
# Per-sequence balance loss and allocation entropy
# ---------------------------------------------------------------------------------------
@pytest.mark.parametrize("T,N,k,L,skew", [(64, 16, 4, 64, None), (300, 64, 6, 100, None),
                                          (4096, 256, 8, 4096, None), (4096, 256, 8, 1024, 1.1),
                                          (17, 512, 16, 1, None), (16384, 256, 8, 4096, 1.1)])
def test_seq_balance_matches_oracle(lib, T, N, k, L, skew):
    import dataclasses
    cfg = dataclasses.replace(synth.PRESETS["tiny"], num_experts=N, num_experts_per_tok=k, tokens=T)
    rng = np.random.default_rng(T + L)
    idx = _idx(rng, T, N, k, skew)
    s = rng.uniform(0.0, 1.0, (T, N)).astype(np.float32)
    say(f"seq_balance T={T} N={N} k={k} L={L} skew={skew}")
    loss, ent = lib.moe_seq_balance(lib.make_config(cfg), dev(s), dev(idx), L, alpha=0.001)
    torch.cuda.synchronize()
    rl = oracle.seq_balance_loss(s, idx, L, 0.001)
    rh = oracle.seq_assignment_entropy(idx, N, L)
    # FP64 sums on both sides, one FP32 rounding of the result: |err| <= 2^-24 |ref| (+ slack)
    assert np.all(np.abs(host(loss) - rl) <= 1.2e-7 * np.abs(rl) + 1e-30)
    assert np.all(np.abs(host(ent) - rh) <= 1.2e-7 * np.abs(rh) + 1e-12)


def test_seq_balance_collapse_invalid_entries_and_empty(lib):
    import dataclasses
    N, k, L = 32, 4, 40
    cfg = dataclasses.replace(synth.PRESETS["tiny"], num_experts=N, num_experts_per_tok=k, tokens=2 * L)
    c = lib.make_config(cfg)
    rng = np.random.default_rng(4)
    s = rng.uniform(0.0, 1.0, (2 * L, N)).astype(np.float32)
    # sequence 0: every token on experts 0..3 (entropy ln 4); sequence 1: some entries -1 or N
    idx = np.tile(np.arange(k, dtype=np.int32), (2 * L, 1))
    idx[L:] = _idx(rng, L, N, k)
    idx[L + 3, 1] = -1
    idx[L + 7, 0] = N
    say("seq_balance collapse / invalid entries")
    loss, ent = lib.moe_seq_balance(c, dev(s), dev(idx), L, alpha=0.5)
    torch.cuda.synchronize()
    rl = oracle.seq_balance_loss(s, idx, L, 0.5)
    rh = oracle.seq_assignment_entropy(idx, N, L)
    assert np.all(np.abs(host(loss) - rl) <= 1.2e-7 * np.abs(rl))
    assert np.all(np.abs(host(ent) - rh) <= 1.2e-7 * np.abs(rh) + 1e-12)
    assert abs(host(ent)[0] - np.log(k)) < 1e-6
    # entropy optional; T = 0 launches nothing
    loss2, none = lib.moe_seq_balance(c, dev(s), dev(idx), L, alpha=0.5, with_entropy=False)
    torch.cuda.synchronize()
    assert none is None and np.array_equal(host(loss2), host(loss))
    e_loss, _ = lib.moe_seq_balance(c, dev(s[:0]), dev(idx[:0]), L)
    assert e_loss.numel() == 0
