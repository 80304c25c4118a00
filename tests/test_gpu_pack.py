"""pack_shard on the GPU: the packed bytes, decoded with the layout the
header documents, hold exactly the oracle's slice of the full weight
(bit-exact), for both source memory orders, ragged shapes and every
strategy."""
import numpy as np
import pytest

import oracle
from gpu_util import Q4Weight, dev, pack, spec_dict, torch
from tensor_sharded_linear_plan_amd import binding as tsl
from tensor_sharded_linear_plan_amd import synth

pytestmark = pytest.mark.gpu


def decode_dense(buf, Ks, Ns, elems):
    """Undo the documented F32 (elems=4) / BF16 (elems=8) layout."""
    Nt = (Ns + 15) // 16
    ktile = 4 * elems
    KT = ((Ks + 63) // 64) * (64 // ktile)
    raw = buf.cpu().numpy()
    vals = raw.view(np.float32 if elems == 4 else np.uint16).reshape(Nt, KT, 64, elems)
    out = np.zeros((KT * ktile, Nt * 16), dtype=vals.dtype)
    for lane in range(64):
        n = np.arange(Nt)[:, None] * 16 + lane % 16
        for j in range(elems):
            k = np.arange(KT)[None, :] * ktile + (lane // 16) * elems + j
            out[k, n] = vals[:, :, lane, j]
    return out[:Ks, :Ns], out


def decode_q4(buf, Ks, Ns):
    Nt = (Ns + 15) // 16
    KB = (Ks + 127) // 128
    raw = buf.cpu().numpy()
    # records of 1152 bytes: codes [64][4] u32, then pairs [16][2] u32
    rec = raw[:Nt * KB * 1152].reshape(Nt, KB, 1152)
    words = np.ascontiguousarray(rec[:, :, :1024]).view(np.uint32).reshape(Nt, KB, 64, 4)
    codes = np.zeros((KB * 128, Nt * 16), dtype=np.uint8)
    for lane in range(64):
        n = np.arange(Nt)[:, None] * 16 + lane % 16
        for t in range(4):
            w = words[:, :, lane, t]
            for j in range(8):
                shift = 16 + 4 * (j // 2) if j % 2 else 4 * (j // 2)
                k = np.arange(KB)[None, :] * 128 + t * 32 + (lane // 16) * 8 + j
                codes[k, n] = (w >> shift) & 0xF
    # the two groups of a 128-k block side by side per column
    pairs = np.ascontiguousarray(rec[:, :, 1024:]).view(np.uint32).reshape(Nt, KB, 16, 2)
    sc = np.zeros((KB * 2, Nt * 16), dtype=np.uint16)
    bi = np.zeros_like(sc)
    for i in range(16):
        for h in range(2):
            sc[h::2, np.arange(Nt) * 16 + i] = (pairs[:, :, i, h] & 0xFFFF).T
            bi[h::2, np.arange(Nt) * 16 + i] = (pairs[:, :, i, h] >> 16).T
    return codes, sc, bi


def decode_q4_exponents(buf, Ks, Ns):
    """The column exponents after the records (records rounded up to 256 bytes)."""
    Nt = (Ns + 15) // 16
    KB = (Ks + 127) // 128
    at = (Nt * KB * 1152 + 255) // 256 * 256
    return buf.cpu().numpy()[at:at + Nt * 64].view(np.int32)


def column_exponents(sc, bi, Ns_pad):
    """Documented rule, in numpy: ilogb of the column's largest
    15 |s| + |b| (binary32, the product exact), minus 14; 0 for zero columns."""
    s = np.abs(oracle.bf16_to_f64(sc)).astype(np.float32)
    b = np.abs(oracle.bf16_to_f64(bi)).astype(np.float32)
    m = np.max(np.float32(15.0) * s + b, axis=0)
    e = np.where(m > 0, np.frexp(m)[1] - 1 - 14, 0).astype(np.int32)
    return np.concatenate([e, np.zeros(Ns_pad - e.size, dtype=np.int32)])


@pytest.mark.parametrize("wdtype", ["f32", "bf16"])
@pytest.mark.parametrize("K,N,tp,strategy", [(1024, 2048, 2, 0), (1024, 2048, 2, 1),
                                             (100, 30, 1, 0), (96, 80, 2, 1), (200, 48, 4, 2)])
def test_pack_dense_layout(wdtype, K, N, tp, strategy):
    if wdtype == "f32":
        W = synth.normal_f32(600, (K, N))
        code, elems = tsl.F32, 4
    else:
        W = synth.normal_bf16(600, (K, N))
        code, elems = tsl.BF16, 8
    dW = dev(W)
    dWt = dev(np.ascontiguousarray(W.T))  # [N][K] source order
    for shard in tsl.plan_linear(K, N, tp, strategy):
        s = spec_dict(shard)
        buf, nb = pack(shard, code, dW, N, 1)
        got, padded = decode_dense(buf, s["k_len"], s["n_len"], elems)
        assert np.array_equal(got, oracle.slice_weight(W, s))
        padded[:s["k_len"], :s["n_len"]] = 0
        assert not padded.any()  # padding is zero
        buf2, _ = pack(shard, code, dWt, 1, K)
        assert torch().equal(buf[:nb], buf2[:nb])


@pytest.mark.parametrize("K,N,tp,strategy", [(256, 64, 2, 1), (3584, 896, 1, 0), (192, 40, 1, 0),
                                             (4352, 128, 4, 1), (128, 48, 2, 0)])
def test_pack_q4_layout(K, N, tp, strategy):
    w = Q4Weight(K, N, 610, 611, 612)
    for shard in tsl.plan_linear(K, N, tp, strategy, 64):
        s = spec_dict(shard)
        buf, nb = w.pack(shard)
        codes, sc, bi = decode_q4(buf, s["k_len"], s["n_len"])
        c_want, s_want, b_want = oracle.slice_q4(w.codes, w.scales, w.biases, s)
        Ks, Ns = s["k_len"], s["n_len"]
        assert np.array_equal(codes[:Ks, :Ns], c_want)
        assert np.array_equal(sc[:Ks // 64, :Ns], s_want)
        assert np.array_equal(bi[:Ks // 64, :Ns], b_want)
        assert not codes[Ks:].any() and not codes[:, Ns:].any()
        assert not sc[Ks // 64:].any() and not sc[:, Ns:].any()
        want_e = column_exponents(s_want, b_want, (Ns + 15) // 16 * 16)
        assert np.array_equal(decode_q4_exponents(buf, Ks, Ns), want_e)


def test_pack_q4_column_exponents_wide_scales():
    # columns 10^+-30 apart, groups 2^+-20 apart within a column
    K, N = 640, 72
    w = Q4Weight(K, N, 620, 621, 622)
    w.scales = synth.wide_scales_bf16(623, (K // 64, N))
    w.biases = synth.wide_biases_bf16(624, w.scales)
    w.d_scales, w.d_biases = dev(w.scales), dev(w.biases)
    sh = tsl.plan_linear(K, N, 1, tsl.COLUMN, 64)[0]
    buf, nb = w.pack(sh)
    want = column_exponents(w.scales, w.biases, 80)
    assert np.array_equal(decode_q4_exponents(buf, K, N), want)
    assert want.min() < -100 and want.max() > 80
