"""Writes tests/golden/tiny_layer_oracle.npz: the oracle's result on the tiny preset.

Calls only ``synth`` (inputs) and ``oracle`` (arithmetic). The stored file is a
regression fixture: it catches unintended changes to the oracle's arithmetic.
Run from the repository root:  python tests/golden/make_tiny_layer_oracle.py
"""
import os
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

import oracle  # noqa: E402
import synth  # noqa: E402


def main():
    cfg = synth.PRESETS["tiny"]
    x = synth.hidden_states(cfg)
    wr = synth.router_weight(cfg)
    b = synth.expert_bias(cfg)

    def q(w):
        w1, w3, w2 = w
        return (*oracle.quantize_128x128(w1), *oracle.quantize_128x128(w3), *oracle.quantize_128x128(w2))
    routed = [q(synth.routed_expert_weights(cfg, e)) for e in range(cfg.num_experts)]
    shared = [q(synth.shared_expert_weights(cfg, s)) for s in range(cfg.num_shared_experts)]
    res = oracle.layer_forward(x, wr, b, cfg, lambda e: routed[e], lambda s: shared[s])
    out = os.path.join(os.path.dirname(os.path.abspath(__file__)), "tiny_layer_oracle.npz")
    np.savez_compressed(out, idx=res["route"]["idx"], counts=res["route"]["counts"],
                        xq=res["xq"], xs=res["xs"], out=res["out"])
    print("wrote", out)


if __name__ == "__main__":
    main()
