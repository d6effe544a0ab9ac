"""Write synth/data/h_cfg{c}_seed{s}.npy: the normalised hidden state h of each
workload at its default seed, as computed by the CPU oracle (float64, stored
as float32).

The router shaping in synth/routing.py needs h.  Tests compute it with the
oracle directly; the benchmark's GPU leg may not run the oracle, so it loads
these files instead.  tests/test_synth.py re-derives every file from the
oracle and checks it.  Run from the repo root:  python -m synth.write_stored_h
"""
import os
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

from oracle import decode_layer_ref as ref  # noqa: E402
from synth import gen, routing  # noqa: E402


def oracle_h(raw) -> np.ndarray:
    r1 = ref.out_projection_residual(raw.attn, raw.w_o, raw.resid)
    h, _ = ref.rms_norm(r1, raw.gain)
    return h


def main():
    os.makedirs(routing._DATA, exist_ok=True)
    for cfg, seed in routing.STORED_H_SEEDS.items():
        raw = gen.draw(cfg, seed)
        h = oracle_h(raw).astype(np.float32)
        np.save(routing.stored_h_path(cfg), h, allow_pickle=False)
        print(cfg, h.shape, routing.stored_h_path(cfg))


if __name__ == "__main__":
    main()
