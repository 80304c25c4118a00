"""The launch configuration bench.py times, checked against the oracle.

bench.py's pre27b prefill step (every rank's 28 shard products of one tp = 4
27B-class layer in one shard_linear_group call: column outputs written into
their blocks of full bf16 outputs, o and down as sum sets into bf16 rank
sums) and its dec7b decode step at M = 1, 4, 16 are built with bench.py's
own code and weights, run once, and every projection's full output is
compared on sampled rows with the oracle's product ([wiki] "Tensor parallel
processing", "Details" §1; [mlxcel] "Column Parallel", "Row Parallel",
"Communication patterns"): concat of the column shards' products, ordered
sum of the row shards' products.  Tolerance 2e-3 normwise plus half a bf16
ulp for the bf16 output rounding."""
import os
import sys

import numpy as np
import pytest

import oracle
from gpu_util import host, normwise, spec_dict, torch
from tensor_sharded_linear_plan_amd import binding as tsl
from tensor_sharded_linear_plan_amd import configs, synth

sys.path.insert(0, os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
import bench  # noqa: E402

pytestmark = pytest.mark.gpu
TOL = 2e-3 + 2.0 ** -9
SOURCE = {"q": "x", "k": "x", "v": "x", "gate": "x", "up": "x", "o": "attn", "down": "act"}


def weight(layer, pi, K, N):
    """The host copy of the weight bench.build_layer packs (same draws)."""
    seed = lambda t: synth.seed_of(layer.index, pi, t)  # noqa: E731
    return (synth.q4_codes(seed(synth.T_CODES), (K, N)),
            synth.uniform_bf16(seed(synth.T_SCALES), (K // 64, N), layer.scale_lo, layer.scale_hi),
            synth.normal_bf16(seed(synth.T_BIASES), (K // 64, N), layer.bias_std))


def bf16_rows(t, rows):
    return oracle.bf16_to_f64(t.view(torch().int16).cpu().numpy().view(np.uint16)[rows])


@pytest.mark.parametrize("layer,M", [(configs.PRE27B, 2048), (configs.DEC7B, 1),
                                     (configs.DEC7B, 4), (configs.DEC7B, 16)],
                         ids=["pre27b-M2048", "dec7b-M1", "dec7b-M4", "dec7b-M16"])
def test_bench_step_against_oracle(layer, M):
    t = torch()
    shards, packs, _, _ = bench.build_layer(layer, M, 1, tsl, t, synth, configs)
    bufs = {}
    run, _, _, _, nitems = bench.make_step(layer, M, shards, packs, tsl, t, configs, 31, bufs)
    assert nitems == 7 * layer.tp
    for Y in bufs["out"].values():
        Y.fill_(float("nan"))
    print("bench step %s M=%d: one grouped call" % (layer.name, M), flush=True)
    run(0, t.cuda.current_stream().cuda_stream)
    t.cuda.synchronize()
    rng = synth.rng(9100 + M)
    rows = (np.arange(M) if M <= 64 else
            np.unique(np.concatenate([np.arange(8), np.arange(M - 8, M),
                                      rng.choice(M, 16, replace=False)])))
    X = {k: bf16_rows(bufs[k], rows) for k in ("x", "attn", "act")}
    for pi, proj in enumerate(configs.PROJS):
        K, N = shards[pi].K, shards[pi].N
        codes, sc, bi = weight(layer, pi, K, N)
        Y = host(bufs["out"][proj])[rows]
        parts = []
        for r in range(layer.tp):
            s = spec_dict(shards[r * tsl.NPROJ + pi])
            W = oracle.dequant_q4(*oracle.slice_q4(codes, sc, bi, s))
            parts.append((s, oracle.gemm(oracle.slice_input(X[SOURCE[proj]], s), W)))
        if proj in ("o", "down"):
            ref = oracle.combine_sum([p for _, p in parts])
        else:
            ref = np.zeros((len(rows), N))
            for s, p in parts:
                ref[:, s["n_off"]:s["n_off"] + s["n_len"]] = p
        err = normwise(Y, ref)
        assert err <= TOL, (layer.name, M, proj, err)
