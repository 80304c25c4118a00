"""Helpers shared by the GPU parity tests: device upload through torch
(memory only), packing and calling the library through its C ABI, and the
error measures the tolerances are stated in."""
import numpy as np

import oracle
from tensor_sharded_linear_plan_amd import binding as tsl
from tensor_sharded_linear_plan_amd import synth

DEV = "cuda"


def torch():
    import torch as _t
    return _t


def dev(a):
    """numpy -> device tensor (uint16 arrays become bfloat16 tensors)."""
    t = torch()
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        return t.from_numpy(a.view(np.int16)).to(DEV).view(t.bfloat16)
    return t.from_numpy(a).to(DEV)


def host(t):
    """device tensor -> numpy float64 (bf16 widened exactly)."""
    tt = torch()
    if t.dtype == tt.bfloat16:
        return t.view(tt.int16).cpu().numpy().view(np.uint16).astype(np.uint32).__lshift__(16) \
            .view(np.float32).astype(np.float64)
    return t.cpu().numpy().astype(np.float64)


def host_bits(t):
    tt = torch()
    return t.view(tt.int16).cpu().numpy().view(np.uint16)


def empty_bytes(n):
    return torch().empty(max(int(n), 256), dtype=torch().uint8, device=DEV)


def pack(shard, wdtype, W, stride_k, stride_n, scales=None, biases=None, sb_g=0, sb_n=0):
    nb = tsl.pack_shard_size(shard, wdtype)
    buf = empty_bytes(nb)
    tsl.pack_shard(shard, wdtype, W, stride_k, stride_n, scales, biases, sb_g, sb_n, buf, nb)
    return buf, nb


def linear(shard, wdtype, packed, nb, xdtype, X, ldx, M, ydtype=tsl.F32, Y=None, ldy=None,
           accumulate=0):
    t = torch()
    if Y is None:
        ydt = t.float32 if ydtype == tsl.F32 else t.bfloat16
        Y = t.full((max(M, 1), shard.n_len), float("nan"), dtype=ydt, device=DEV)
        ldy = shard.n_len
    ws = tsl.shard_linear_workspace_size(shard, wdtype, M)
    wsbuf = empty_bytes(ws) if ws else None
    tsl.shard_linear(shard, wdtype, packed, nb, xdtype, X, ldx, M, ydtype, Y, ldy, accumulate,
                     wsbuf, ws)
    return Y


def spec_dict(shard):
    return dict(zip(tsl.Shard.FIELDS, shard.as_tuple()))


def normwise(y, r):
    """max |y - r| / max |r| over the whole tensor (the tolerance measure)."""
    y = np.asarray(y, dtype=np.float64)
    r = np.asarray(r, dtype=np.float64)
    den = np.max(np.abs(r)) if r.size else 0.0
    return float(np.max(np.abs(y - r)) / den) if den > 0 else float(np.max(np.abs(y - r), initial=0.0))


class Q4Weight:
    """A full logical 4-bit weight: codes [K][N] (bytes), bf16 scale and
    bias [K/64][N] (bits), and its device copies."""

    def __init__(self, K, N, seed_codes, seed_scales, seed_biases, integer=False,
                 scale_lo=0.005, scale_hi=0.02, bias_std=0.05):
        self.K, self.N = K, N
        self.codes = synth.q4_codes(seed_codes, (K, N))
        if integer:
            self.scales = synth.const_bf16((K // 64, N), 1.0)
            self.biases = synth.const_bf16((K // 64, N), -8.0)
        else:
            self.scales = synth.uniform_bf16(seed_scales, (K // 64, N), scale_lo, scale_hi)
            self.biases = synth.normal_bf16(seed_biases, (K // 64, N), bias_std)
        self.d_codes = dev(self.codes)
        self.d_scales = dev(self.scales)
        self.d_biases = dev(self.biases)

    def pack(self, shard):
        return pack(shard, tsl.Q4G64, self.d_codes, self.N, 1, self.d_scales, self.d_biases,
                    self.N, 1)

    def shard_f64(self, s):
        """The oracle's view of the shard: slice codes and groups, dequantise."""
        return oracle.dequant_q4(*oracle.slice_q4(self.codes, self.scales, self.biases, s))
