"""One rank's share of a transformer layer on the GPU against the oracle, at
the workloads' full sizes: every projection of rank 0 (q, k, v, o, gate,
up, down), and for the row layers (o, down) every rank's partial summed
on-device.  Random draws: max|y - r| / max|r| <= 2e-3 (bf16 and 4-bit
weights, binary32 accumulation); integer draws: bit-exact.  Outputs the
oracle would take minutes for are compared on a sample of whole rows
(first, last and random rows, every column)."""
import numpy as np
import pytest

import oracle
from gpu_util import Q4Weight, dev, host, host_bits, linear, normwise, spec_dict, torch
from tensor_sharded_linear_plan_amd import binding as tsl
from tensor_sharded_linear_plan_amd import configs, synth

pytestmark = pytest.mark.gpu
TOL = 2e-3
FULL_LIMIT = 1.5e9  # oracle multiply-adds before switching to a row sample


class LayerWeights:
    """Full logical weights of one projection, on host and device."""

    def __init__(self, layer, proj, variant):
        p = configs.PROJS.index(proj)
        self.layer, self.proj = layer, proj
        iv = 1 if variant == "integer" else 0
        sh = tsl.plan_shards(layer.hidden, layer.n_q_heads, layer.n_kv_heads, layer.head_dim,
                             layer.ffn, layer.tp, layer.group)[p]
        self.K, self.N = sh.K, sh.N
        seed = lambda t: synth.seed_of(layer.index, p, t, iv)
        if layer.wdtype == configs.Q4:
            self.q4 = Q4Weight(self.K, self.N, seed(synth.T_CODES), seed(synth.T_SCALES),
                               seed(synth.T_BIASES), integer=(variant == "integer"),
                               scale_lo=layer.scale_lo, scale_hi=layer.scale_hi,
                               bias_std=layer.bias_std)
            self.W = None
        else:
            self.q4 = None
            if variant == "integer":
                self.W = synth.small_int_bf16(seed(synth.T_W), (self.K, self.N))
            else:
                self.W = synth.normal_bf16(seed(synth.T_W), (self.K, self.N), layer.w_std)
            self.dW = dev(self.W)

    @property
    def wdtype(self):
        return tsl.Q4G64 if self.q4 else tsl.BF16

    def pack(self, shard):
        if self.q4:
            return self.q4.pack(shard)
        from gpu_util import pack
        return pack(shard, tsl.BF16, self.dW, self.N, 1)

    def shard_f64(self, s):
        if self.q4:
            return self.q4.shard_f64(s)
        return oracle.bf16_to_f64(oracle.slice_weight(self.W, s))


def activations(layer, proj, M, K, variant):
    p = configs.PROJS.index(proj)
    if variant == "integer":
        return synth.small_int_bf16(synth.seed_of(layer.index, p, synth.T_X, 1) + 7 * M, (M, K))
    return synth.normal_bf16(synth.seed_of(layer.index, p, synth.T_X, 0) + 7 * M, (M, K),
                             layer.x_std)


def sample_rows(M, K, N):
    if M * K * N <= FULL_LIMIT:
        return np.arange(M)
    rng = synth.rng(4242 + M)
    rows = np.concatenate([np.arange(16), np.arange(M - 16, M), rng.choice(M, 32, replace=False)])
    return np.unique(rows)


def check(y, ref, variant, what):
    if variant == "integer":
        assert np.array_equal(y, ref), what
    else:
        err = normwise(y, ref)
        assert err <= TOL, "%s: normwise error %.3g" % (what, err)


CASES = [(layer, M) for layer in (configs.LLAMA2K, configs.DEC7B, configs.GQA8, configs.PRE27B)
         for M in layer.ms]


@pytest.mark.parametrize("variant", ["random", "integer"])
@pytest.mark.parametrize("layer,M", CASES, ids=["%s-M%d" % (l.name, m) for l, m in CASES])
def test_rank0_projections(layer, M, variant):
    shards = tsl.plan_shards(layer.hidden, layer.n_q_heads, layer.n_kv_heads, layer.head_dim,
                             layer.ffn, layer.tp, layer.group)
    for pi, proj in enumerate(configs.PROJS):
        sh = shards[pi]
        s = spec_dict(sh)
        w = LayerWeights(layer, proj, variant)
        X = activations(layer, proj, M, sh.K, variant)
        dX = dev(X)
        buf, nb = w.pack(sh)
        # row shards read their block of X through a pointer and ldx
        Y = linear(sh, w.wdtype, buf, nb, tsl.BF16, dX[:, sh.k_off:], sh.K, M)
        rows = sample_rows(M, sh.k_len, sh.n_len)
        Xf = oracle.bf16_to_f64(X[rows])
        ref = oracle.gemm(oracle.slice_input(Xf, s), w.shard_f64(s))
        check(host(Y)[rows], ref, variant, "%s M=%d %s" % (layer.name, M, proj))
        if proj in ("gate", "o") and variant == "random":
            # bf16 output: one round-to-nearest-even of the same binary32 result
            Yb = linear(sh, w.wdtype, buf, nb, tsl.BF16, dX[:, sh.k_off:], sh.K, M,
                        ydtype=tsl.BF16)
            assert np.array_equal(host_bits(Yb), oracle.f64_to_bf16(host(Y))), proj
            assert normwise(host(Yb)[rows], ref) <= TOL + 2.0 ** -9


@pytest.mark.parametrize("variant", ["random", "integer"])
@pytest.mark.parametrize("layer,M", CASES, ids=["%s-M%d" % (l.name, m) for l, m in CASES])
def test_row_layers_all_ranks_summed(layer, M, variant):
    shards = tsl.plan_shards(layer.hidden, layer.n_q_heads, layer.n_kv_heads, layer.head_dim,
                             layer.ffn, layer.tp, layer.group)
    for proj in ("o", "down"):
        pi = configs.PROJS.index(proj)
        w = LayerWeights(layer, proj, variant)
        K, N = w.K, w.N
        X = activations(layer, proj, M, K, variant)
        dX = dev(X)
        parts = []
        rows = sample_rows(M, K // layer.tp, N)
        Xf = oracle.bf16_to_f64(X[rows])
        refs = []
        for r in range(layer.tp):
            sh = shards[r * tsl.NPROJ + pi]
            s = spec_dict(sh)
            assert s["strategy"] == oracle.ROW
            buf, nb = w.pack(sh)
            parts.append(linear(sh, w.wdtype, buf, nb, tsl.BF16, dX[:, sh.k_off:], K, M))
            refs.append(oracle.gemm(oracle.slice_input(Xf, s), w.shard_f64(s)))
            del buf
        Y = torch().full((M, N), float("nan"), dtype=torch().float32, device="cuda")
        tsl.combine_partials(tsl.COMBINE_SUM, parts, tsl.F32, M, N, N, tsl.F32, Y, N)
        ref = oracle.combine_sum(refs)
        check(host(Y)[rows], ref, variant, "%s M=%d %s sum" % (layer.name, M, proj))
