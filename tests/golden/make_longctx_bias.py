"""Writes longctx_bal_bias.txt: balancing biases for the long-context workload (32768
tokens, window 4096) such that top-1 counts follow a Zipf(1.2) law over the 16 experts
(expert id = rank) for 85% of the tokens and the skip class takes 15%.

Only the CPU oracle and the seeded input generator are used. The router's class
probabilities of the workload's first 2048 tokens are computed by the oracle (the
inputs are i.i.d. over positions, so their statistics stand for the whole sequence);
then a fixed, deterministic iteration b_j += eta (target_j - share_j) moves the biases,
each finally rounded to bfloat16 (the buffer holds bf16-representable values).

Run: python tests/golden/make_longctx_bias.py
"""
import os
import sys

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(os.path.dirname(HERE)))

from oracle import zaya_oracle as O  # noqa: E402
from zaya_synth import CONFIGS, block_inputs, block_weights  # noqa: E402


def targets(E=16, s=1.2, skip=0.15):
    z = 1.0 / np.arange(1, E + 1) ** s
    return np.concatenate([(1 - skip) * z / z.sum(), [skip]])


def main(n_cal=2048, iters=4000):
    cfg = CONFIGS["longctx"]
    w = {k: v.float().numpy() for k, v in block_weights(cfg, bal_bias=np.zeros(cfg.num_experts + 1)).items()}
    inp = block_inputs(cfg)
    c = cfg.replace(seq=n_cal)
    x = inp["x"][:, :n_cal].numpy().astype(np.float64)
    s = inp["s_in"][:, :n_cal].float().numpy()
    out = O.block_forward(c, w, x, s, None)
    p = O.rnd_f32(O.softmax(O.rnd_f32(out["router_logits"])))  # [n_cal, E+1]
    t = targets(cfg.num_experts)
    b = np.zeros(cfg.num_experts + 1)
    for it in range(iters):
        eta = 0.02 * (1.0 - it / iters) + 1e-4
        cls = np.argmax(O.rnd_f32(p + b), axis=-1)
        share = np.bincount(cls, minlength=len(t)) / n_cal
        b = b + eta * (t - share)
    b = O.rnd_bf16(b - b.max())  # only differences matter; keep values small
    cls = np.argmax(O.rnd_f32(p + b), axis=-1)
    share = np.bincount(cls, minlength=len(t)) / n_cal
    path = os.path.join(HERE, "longctx_bal_bias.txt")
    with open(path, "w") as f:
        f.write("# balancing biases (fp32 holding bf16 values) for the long-context workload;\n")
        f.write("# written by tests/golden/make_longctx_bias.py from the CPU oracle on the first\n")
        f.write(f"# {n_cal} tokens. target shares: {' '.join(f'{v:.4f}' for v in t)}\n")
        f.write(f"# realized shares on the calibration tokens: {' '.join(f'{v:.4f}' for v in share)}\n")
        for v in b:
            f.write(f"{v:.9g}\n")
    print("wrote", path)
    print("target  ", np.round(t, 4))
    print("realized", np.round(share, 4))


if __name__ == "__main__":
    main()
