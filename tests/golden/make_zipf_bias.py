"""Writes the Zipf(1.1)-popularity selection biases of the 256-expert layers.

The workload asks for router biases under which expert popularity follows a
Zipf law with exponent 1.1.  The bias is found offline, with the oracle's
router only, by the bias-adjustment idea behind DeepSeek-V3's balancing
without an auxiliary loss ("25GB 内存跑 744B GLM-5.2 模型" page, section 四.3):
raise the bias of experts chosen less often than their target and lower it
for the others, here in log space:

    b_e <- b_e + eta * (log f*_e - log f_e)

where f_e is the fraction of calibration tokens that select e and f*_e is
the Zipf target for e's popularity rank (capped at 1 because a token picks
each expert at most once; the targets sum to k).  Ranks come from a seeded
permutation of the expert ids.  The calibration batch is a separate seeded
set of 4096 tokens, never used as a workload input.  The bias is then frozen
and stored as fp32 hex floats.  The biases are re-centred to mean 0 after
each update, which changes no selection.

Usage:  python tests/golden/make_zipf_bias.py   (about a minute on 8 cores)
"""
import os
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

from oracle import oracle  # noqa: E402
from routed_expert_ffn_sigmoid_amd import synth  # noqa: E402

N_CAL = 4096
ITERS = 800
ETA = 0.01


def calibrate(spec, layer, seed=0):
    W_r = synth.gen_router(spec, seed, layer)
    xc = synth.calibration_x(spec, N_CAL, seed, layer)
    z = oracle.router_logits(oracle.decode_act(xc, spec.act), W_r)
    order = synth.popularity_order(spec, seed, layer)
    target = np.empty(spec.E)
    target[order] = synth.zipf_target(spec.E, spec.k)
    b = np.zeros(spec.E)
    for it in range(ITERS):
        r = oracle.router_select(z, b.astype(np.float32), spec.k, spec.routed_scale)
        f = np.bincount(r.idx.reshape(-1), minlength=spec.E) / N_CAL
        b += ETA * (np.log(target) - np.log(np.maximum(f, 0.5 / N_CAL)))
        b -= b.mean()  # a common shift of every bias leaves the selection unchanged
    b32 = b.astype(np.float32)
    r = oracle.router_select(z, b32, spec.k, spec.routed_scale)
    f = np.bincount(r.idx.reshape(-1), minlength=spec.E) / N_CAL
    return b32, target, f, order


def main():
    spec = synth.CONFIGS["large_zipf"]
    for layer in range(4):
        b, target, f, order = calibrate(spec, layer)
        path = synth.zipf_bias_path(spec.E, spec.d, layer)
        rel = np.abs(f[order] - target[order]) / target[order]
        with open(path, "w") as fh:
            fh.write(f"# Zipf(s={synth.ZIPF_S}) selection bias, E={spec.E} k={spec.k} d={spec.d} seed=0 layer={layer}\n")
            fh.write(f"# written by tests/golden/make_zipf_bias.py: {ITERS} log-space bias updates, eta={ETA},\n")
            fh.write(f"# {N_CAL} seeded calibration tokens routed by the oracle.\n")
            fh.write(f"# achieved on the calibration batch: rank1 {f[order[0]]:.4f} (target {target[order[0]]:.4f}), "
                     f"rank2 {f[order[1]]:.4f} ({target[order[1]]:.4f}), rank10 {f[order[9]]:.4f} "
                     f"({target[order[9]]:.4f}), median rel err over ranks {np.median(rel):.3f}\n")
            fh.write("# one fp32 value per expert id, as a hex float\n")
            for v in b:
                fh.write(float(v).hex() + "\n")
        print(path, f"rank1 {f[order[0]]:.4f} rank2 {f[order[1]]:.4f} rank3 {f[order[2]]:.4f} "
              f"rank10 {f[order[9]]:.4f} rank256 {f[order[-1]]:.5f} median_rel_err {np.median(rel):.3f}", flush=True)


if __name__ == "__main__":
    main()
