"""Whole-layer parity of the HIP path against the CPU oracle (needs an MI355X).

tiny and reduced run in full. The DeepSeek-V3 shapes (prefill T=4096, decode T=128,
skewed T=16384) run the full layer on the GPU in the configuration the benchmark times;
the oracle checks the routing of every token and the outputs of a few sampled tokens
(it quantises only the experts those tokens reach, and those codes must equal the GPU's).
"""
import sys

import numpy as np
import pytest
import torch

import oracle
import synth
from routing_check import NEAR_TIE, assert_routing_valid

pytestmark = pytest.mark.gpu
TOL = 5e-3


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def relerr(a, b):
    return float(np.linalg.norm(a - b) / np.linalg.norm(b))


def q3(w):
    w1, w3, w2 = w
    return (*oracle.quantize_128x128(w1), *oracle.quantize_128x128(w3), *oracle.quantize_128x128(w2))


def q3_pow2(w):
    w1, w3, w2 = w
    return (*oracle.quantize_128x128_pow2(w1), *oracle.quantize_128x128_pow2(w3),
            *oracle.quantize_128x128_pow2(w2))


def x_device(cfg, x):
    dt = torch.bfloat16 if cfg.x_dtype == "bf16" else torch.float32
    return torch.from_numpy(x).to(dt).cuda()


def routing_ties(r):
    return (r["kth_gap"] < NEAR_TIE) | (r["group_gap"] < NEAR_TIE)


@pytest.mark.parametrize("name", ["tiny", "reduced"])
def test_layer_pow2_matches_oracle(name):
    """The power-of-two scale variant end to end (scale_mode 1)."""
    from deepseekmoe_routing_fp8_amd import MoELayer
    cfg = synth.PRESETS[name]
    say(f"layer pow2 {name}: loading weights")
    layer = MoELayer(cfg, scale_mode=1)
    layer.load_from_synth()
    x = synth.hidden_states(cfg)
    b0 = synth.expert_bias(cfg)
    say(f"layer pow2 {name}: forward T={cfg.tokens}")
    out = layer.forward(x_device(cfg, x)).float().cpu().numpy()
    g_idx = layer.topk_idx.cpu().numpy()
    wr = synth.router_weight(cfg)
    routed = [q3_pow2(synth.routed_expert_weights(cfg, e)) for e in range(cfg.num_experts)]
    shared = [q3_pow2(synth.shared_expert_weights(cfg, s)) for s in range(cfg.num_shared_experts)]
    assert np.array_equal(layer.w2s[0].cpu().numpy(), routed[0][5])
    assert np.array_equal(MoELayer.unpack(layer.w1[1].cpu().numpy()), routed[1][0])
    ref = oracle.layer_forward(x, wr, b0, cfg, lambda e: routed[e], lambda s: shared[s], pow2=True)
    r = ref["route"]
    assert_routing_valid(r, g_idx, cfg)
    if np.any(g_idx != r["idx"]):
        ref = oracle.layer_forward(x, wr, b0, cfg, lambda e: routed[e], lambda s: shared[s],
                                   force_idx=g_idx, pow2=True)
    err = relerr(out, ref["out"])
    say(f"layer pow2 {name}: normwise error {err:.3e}")
    assert err < TOL


@pytest.mark.parametrize("name", ["tiny", "reduced"])
def test_layer_matches_oracle(name):
    _check_layer(synth.PRESETS[name], name)


@pytest.mark.parametrize("T", [1, 17, 129])
def test_layer_ragged_token_counts(T):
    """One token (a decode step of one sequence), a count below one 16-row tile per
    expert, and one past a multiple of 128 (a ragged last block in every token-axis pass)."""
    import dataclasses
    _check_layer(dataclasses.replace(synth.PRESETS["tiny"], tokens=T), f"tiny T={T}")


def _check_layer(cfg, name):
    from deepseekmoe_routing_fp8_amd import MoELayer
    say(f"layer {name}: loading weights")
    layer = MoELayer(cfg)
    layer.load_from_synth()
    x = synth.hidden_states(cfg)
    b0 = synth.expert_bias(cfg)
    say(f"layer {name}: forward T={cfg.tokens}")
    out = layer.forward(x_device(cfg, x)).float().cpu().numpy()
    g_idx = layer.topk_idx.cpu().numpy()
    g_counts = layer.counts.cpu().numpy()
    g_bias = layer.bias.cpu().numpy()
    wr = synth.router_weight(cfg)
    routed = [q3(synth.routed_expert_weights(cfg, e)) for e in range(cfg.num_experts)]
    shared = [q3(synth.shared_expert_weights(cfg, s)) for s in range(cfg.num_shared_experts)]
    # the device-quantised weights equal the oracle's codes and scales
    for e in (0, cfg.num_experts - 1):
        assert np.array_equal(MoELayer.unpack(layer.w1[e].cpu().numpy()), routed[e][0])
        assert np.array_equal(MoELayer.unpack(layer.w2[e].cpu().numpy()), routed[e][4])
        assert np.array_equal(layer.w2s[e].cpu().numpy(), routed[e][5])
    for s_ in range(cfg.num_shared_experts):   # shared experts follow the routed ones
        assert np.array_equal(MoELayer.unpack(layer.w1[cfg.num_experts + s_].cpu().numpy()), shared[s_][0])
        assert np.array_equal(layer.w3s[cfg.num_experts + s_].cpu().numpy(), shared[s_][3])
    ref = oracle.layer_forward(x, wr, b0, cfg, lambda e: routed[e], lambda s: shared[s])
    r = ref["route"]
    tie = routing_ties(r)
    assert_routing_valid(r, g_idx, cfg)
    if np.any(g_idx != r["idx"]):   # re-evaluate the oracle on the GPU's (equally valid) choice
        ref = oracle.layer_forward(x, wr, b0, cfg, lambda e: routed[e], lambda s: shared[s],
                                   force_idx=g_idx)
    err = relerr(out, ref["out"])
    say(f"layer {name}: normwise error {err:.3e}, near-tie tokens {int(tie.sum())}")
    assert err < TOL
    assert np.array_equal(g_counts, ref["route"]["counts"])
    nb = oracle.bias_update(b0, g_counts, cfg.tokens, cfg.num_experts_per_tok, cfg.expert_bias_update_rate)
    assert np.array_equal(g_bias.view(np.uint32), nb.view(np.uint32))


@pytest.mark.parametrize("name", ["tiny", "reduced"])
def test_graph_replay_matches_eager(name):
    """A captured step replays the eager step bit for bit: outputs and routing, with the
    program's own eager work and synchronisations between replays; with the bias update
    inside the graph, several replays give the same biases and outputs as as many eager
    steps of a second layer."""
    from deepseekmoe_routing_fp8_amd import MoELayer
    cfg = synth.PRESETS[name]
    say(f"graph {name}: loading two layers")
    a, b = MoELayer(cfg), MoELayer(cfg)
    a.load_from_synth()
    b.load_from_synth()
    x = x_device(cfg, synth.hidden_states(cfg))
    out0 = a.forward(x, update_bias=False).clone()
    idx0, gate0 = a.topk_idx.clone(), a.topk_gate.clone()
    say(f"graph {name}: capture without the bias update, 3 replays")
    a.capture(x, update_bias=False)
    for rep in range(3):
        a.out.zero_()
        a.topk_idx.fill_(-1)
        a.y_rows.zero_()
        torch.cuda.synchronize()
        a.replay()
        torch.cuda.synchronize()
        assert torch.equal(a.out, out0), rep
        assert torch.equal(a.topk_idx, idx0) and torch.equal(a.topk_gate, gate0), rep
    say(f"graph {name}: capture with the bias update, 3 replays against 3 eager steps")
    b.capture(x, update_bias=True)
    bias_ref = b.bias.clone()
    for rep in range(3):
        ref = a.forward(x, update_bias=True).clone()
        torch.cuda.synchronize()
        b.replay()
        torch.cuda.synchronize()
        assert torch.equal(b.out, ref), rep
        assert torch.equal(b.bias.view(torch.int32), a.bias.view(torch.int32)), rep
    assert not torch.equal(b.bias, bias_ref)   # the replays did update the bias


@pytest.fixture(scope="module")
def v3_layer():
    from deepseekmoe_routing_fp8_amd import MoELayer
    cfg = synth.PRESETS["v3_prefill"]
    say("V3 layer: generating and quantising 257 experts on the device")
    layer = MoELayer(cfg)
    layer.load_from_synth()
    return layer


def _sampled_parity(layer, cfg, x, bias, n_sample, seed):
    wr = synth.router_weight(cfg)
    g_idx = layer.topk_idx.cpu().numpy()
    # routing of every token
    r = oracle.route(x, wr, bias, cfg.num_experts_per_tok, cfg.n_group, cfg.topk_group,
                     cfg.group_score_topn, cfg.routed_scaling_factor)
    nt = assert_routing_valid(r, g_idx, cfg)
    say(f"  routing ok, near-tie tokens {nt}")
    # outputs of sampled tokens
    rng = np.random.default_rng(seed)
    toks = np.sort(rng.choice(cfg.tokens, n_sample, replace=False))
    experts = sorted(set(g_idx[toks].ravel().tolist()))
    say(f"  sampled tokens {toks.tolist()} reach {len(experts)} experts")
    cache = {}

    def put(e, w):
        cache[e] = q3(w)
    synth.map_experts(cfg, put, experts)
    from deepseekmoe_routing_fp8_amd import MoELayer
    for e in experts[:3]:
        assert np.array_equal(MoELayer.unpack(layer.w3[e].cpu().numpy()), cache[e][2])
        assert np.array_equal(layer.w1s[e].cpu().numpy(), cache[e][1])
    sh = {}
    synth.map_experts(cfg, lambda s, w: sh.__setitem__(s, q3(w)), range(cfg.num_shared_experts), shared=True)
    ref = oracle.layer_forward(x[toks], wr, bias, cfg, lambda e: cache[e], lambda s: sh[s],
                               force_idx=g_idx[toks])
    out = layer.out[torch.from_numpy(toks).cuda()].float().cpu().numpy()
    err = relerr(out, ref["out"])
    say(f"  sampled normwise error {err:.3e}")
    assert err < TOL
    return g_idx


def _full_checks(layer, cfg, x, bias, g_idx, inter_rows=640):
    """Checks at full size wherever the oracle can follow: every token's gates, the
    permutation, the combine of every token from the GPU's own expert rows and gates, the
    whole output segments of the shared expert and of the most loaded routed expert, and
    their quantised intermediate (hq, hs; the first ``inter_rows`` rows of a segment)."""
    import deepseekmoe_routing_fp8_amd as lib
    from intermediate_check import check_intermediate, h_band
    T, H, k, N, S = cfg.tokens, cfg.hidden_size, cfg.num_experts_per_tok, cfg.num_experts, cfg.num_shared_experts
    assert np.array_equal(layer.counts.cpu().numpy(), np.bincount(g_idx.ravel(), minlength=N))
    # gates of every token at the GPU's selection; they sum to rho
    wr = synth.router_weight(cfg)
    rf = oracle.route(x, wr, bias, k, cfg.n_group, cfg.topk_group, cfg.group_score_topn,
                      cfg.routed_scaling_factor, force_idx=g_idx)
    g_gate = layer.topk_gate.cpu().numpy()
    assert np.allclose(g_gate, rf["gate"], rtol=2e-6, atol=0)
    assert np.allclose(g_gate.sum(1), cfg.routed_scaling_factor, rtol=1e-5)
    # permutation bit-exact, shared segment in token order
    off, rt, ro = oracle.permute(g_idx, N)
    g_off = layer.offsets.cpu().numpy()
    g_rt = layer.row_token.cpu().numpy()
    assert np.array_equal(g_off[:N + 1], off) and g_off[N + 1] == T * (k + 1)
    assert np.array_equal(g_rt[:T * k], rt) and np.array_equal(g_rt[T * k:], np.arange(T))
    assert np.array_equal(layer.row_of.cpu().numpy(), ro)
    # combine of all tokens from the GPU's own rows and gates (one bf16 rounding of an FP32 sum)
    y_rows = layer.y_rows.float().cpu().numpy()
    ref = oracle.combine(y_rows[:T * k], ro, g_gate, [y_rows[T * k:]])
    got = layer.out.float().cpu().numpy().astype(np.float64)
    mag = np.abs(y_rows[T * k:]).astype(np.float64)
    for j in range(k):
        mag += np.abs(g_gate[:, j:j + 1]) * np.abs(y_rows[ro[:, j]])
    bound = np.abs(ref) * 2.0 ** -8 + 1e-5 * mag
    assert np.all(np.abs(got - ref) <= bound)
    del ref, got, mag
    say(f"  combine of all {T} tokens ok")
    # whole segments: the shared expert and the most loaded routed expert
    xq, xs = oracle.quantize_1x128(x)
    assert np.array_equal(layer.xq.cpu().numpy(), xq)
    heavy = int(np.argmax(np.diff(off)))
    cache = {}
    synth.map_experts(cfg, lambda e, w: cache.__setitem__(e, q3(w)), [heavy])
    sh = q3(synth.shared_expert_weights(cfg, 0))
    c = lib.make_config(cfg)
    hq_all, hs_all = lib.grouped_ffn_intermediate(c, N + S, T * (k + S), layer.ws)
    hq_all, hs_all = hq_all.cpu().numpy(), hs_all.cpu().numpy()
    for name, w, lo, hi, toks in (("shared", sh, T * k, T * k + T, np.arange(T)),
                                  (f"routed {heavy}", cache[heavy], int(off[heavy]), int(off[heavy + 1]),
                                   rt[off[heavy]:off[heavy + 1]])):
        y_ref = oracle.expert_ffn(xq[toks], xs[toks], *w)[0]
        err = relerr(y_rows[lo:hi], y_ref)
        say(f"  {name} expert, {hi - lo} rows: normwise error {err:.3e}")
        assert err < TOL
        m = min(hi - lo, inter_rows)
        h, dh = h_band(xq[toks[:m]], xs[toks[:m]], *w[:4])
        st = check_intermediate(hq_all[lo:lo + m], hs_all[:, lo:lo + m].T, h, dh)
        say(f"  {name} expert intermediate ({m} rows): {st}")


@pytest.mark.timeout(900)
def test_v3_prefill_full(v3_layer):
    """The V3 prefill step (T = 4096) in the benchmark's launch configuration, at full
    size wherever the oracle can follow (see _full_checks), and three sampled tokens end
    to end (all their experts re-evaluated by the oracle)."""
    cfg = synth.PRESETS["v3_prefill"]
    x = synth.hidden_states(cfg)
    bias = v3_layer.bias.cpu().numpy()
    say("V3 prefill forward T=4096")
    v3_layer.forward(x_device(cfg, x), update_bias=False)
    torch.cuda.synchronize()
    g_idx = _sampled_parity(v3_layer, cfg, x, bias, 3, 0)
    _full_checks(v3_layer, cfg, x, bias, g_idx)


@pytest.mark.timeout(900)
def test_v3_decode_sampled(v3_layer):
    cfg = synth.PRESETS["v3_decode"]
    x = synth.hidden_states(cfg)
    bias = v3_layer.bias.cpu().numpy()
    say("V3 decode forward T=128")
    v3_layer.forward(x_device(cfg, x), update_bias=False)
    torch.cuda.synchronize()
    g_idx = _sampled_parity(v3_layer, cfg, x, bias, 3, 1)
    _full_checks(v3_layer, cfg, x, bias, g_idx)


@pytest.mark.timeout(900)
def test_v3_single_token(v3_layer):
    """One token through the V3 layer: 8 routed rows in 8 one-row segments + the shared
    row; every check of the decode case at its smallest size."""
    import dataclasses
    cfg = dataclasses.replace(synth.PRESETS["v3_decode"], tokens=1)
    x = synth.hidden_states(cfg)
    bias = v3_layer.bias.cpu().numpy()
    say("V3 forward T=1")
    v3_layer.forward(x_device(cfg, x), update_bias=False)
    torch.cuda.synchronize()
    g_idx = _sampled_parity(v3_layer, cfg, x, bias, 1, 2)
    _full_checks(v3_layer, cfg, x, bias, g_idx)


@pytest.mark.timeout(900)
def test_v3_decode_graph_replay(v3_layer):
    """The V3 decode step (T=128) captured into a HIP graph, as the benchmark times it,
    replays the eager step bit for bit, twice, with eager work between the replays."""
    cfg = synth.PRESETS["v3_decode"]
    x = x_device(cfg, synth.hidden_states(cfg))
    ref = v3_layer.forward(x, update_bias=False).clone()
    idx = v3_layer.topk_idx.clone()
    v3_layer.capture(x, update_bias=False)
    for rep in range(2):
        v3_layer.out.zero_()
        v3_layer.y_rows.zero_()
        torch.cuda.synchronize()
        v3_layer.replay()
        torch.cuda.synchronize()
        assert torch.equal(v3_layer.out, ref), rep
        assert torch.equal(v3_layer.topk_idx, idx), rep
    v3_layer._graph = None


@pytest.mark.timeout(900)
def test_v3_skewed_steps(v3_layer):
    """Forward + bias update on the skewed workload: every step's bias follows the
    oracle's update of the GPU's own counts, and its routing matches the oracle."""
    cfg = synth.PRESETS["v3_skewed"]
    b = np.zeros(cfg.num_experts, np.float32)
    v3_layer.bias.copy_(torch.from_numpy(b))
    loads = []
    for step in range(3):
        x = synth.hidden_states(cfg, step=step)
        say(f"V3 skewed step {step} T={cfg.tokens}")
        v3_layer.forward(x_device(cfg, x), update_bias=True)
        torch.cuda.synchronize()
        counts = v3_layer.counts.cpu().numpy()
        loads.append(counts.max() / counts.mean())
        if step == 0:
            _sampled_parity(v3_layer, cfg, x, b, 2, 2)
        else:   # every step's routing; at the last, the heaviest segment (many M tiles) in full
            r = oracle.route(x, synth.router_weight(cfg), b, cfg.num_experts_per_tok, cfg.n_group,
                             cfg.topk_group, cfg.group_score_topn, cfg.routed_scaling_factor)
            g_idx = v3_layer.topk_idx.cpu().numpy()
            assert_routing_valid(r, g_idx, cfg)
            if step == 2:
                _full_checks(v3_layer, cfg, x, b, g_idx, inter_rows=320)
        b = oracle.bias_update(b, counts, cfg.tokens, cfg.num_experts_per_tok, cfg.expert_bias_update_rate)
        assert np.array_equal(v3_layer.bias.cpu().numpy().view(np.uint32), b.view(np.uint32))
    say(f"  max/mean load per step: {[round(float(v), 2) for v in loads]}")
    assert loads[0] > 2.0   # the clustered input is skewed
