"""The C-ABI library on the host: it loads, exports every entry point that
include/tsl.h declares, plans bit-exactly like the oracle, and rejects bad
arguments before anything reaches the GPU (no compute call is made here).
"""
import ctypes
import os
import re

import numpy as np
import pytest

import oracle
from conftest import ROOT
from tensor_sharded_linear_plan_amd import configs

HEADER = os.path.join(ROOT, "include", "tsl.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(\w+)\s*\(", text, flags=re.M)))


def test_library_exports_every_declared_symbol(tsl_lib):
    names = declared_functions()
    assert set(names) == {"plan_shards", "plan_linear", "pack_shard_size", "pack_shard",
                          "shard_linear_workspace_size", "shard_linear",
                          "shard_linear_group_workspace_size", "shard_linear_group",
                          "shard_linear_group_noalloc",
                          "combine_partials", "combine_to_ranks", "plan_vocab",
                          "embed_lookup", "plan_experts", "moe_dispatch", "moe_gather",
                          "moe_combine", "tsl_status_string", "tsl_last_hip_error_string"}
    lib = ctypes.CDLL(tsl_lib.LIBRARY)
    for n in names:
        assert hasattr(lib, n), n
    assert set(tsl_lib.EXPORTS) == set(names)


def test_library_exports_nothing_else(tsl_lib):
    # the kernels' C++ internals are hidden: the dynamic symbol table holds
    # the header's entry points and the HIP compiler's per-unit ids only
    import subprocess
    out = subprocess.run(["nm", "-D", "--defined-only", tsl_lib.LIBRARY], capture_output=True,
                         text=True, check=True).stdout
    defined = {l.split()[-1] for l in out.splitlines() if l.strip()}
    others = {n for n in defined if not n.startswith("__hip_cuid_")}
    assert others == set(declared_functions())


def test_shard_struct_layout_matches_header(tsl_lib):
    assert ctypes.sizeof(tsl_lib.Shard) == 72
    assert tsl_lib.Shard.K.offset == 16 and tsl_lib.Shard.head_off.offset == 64
    assert ctypes.sizeof(tsl_lib.Dims) == 28
    # tsl_linear_item: seven 8-byte fields, four int32, then the row index
    # pointer and x_rows
    assert ctypes.sizeof(tsl_lib.LinearItem) == 88
    assert tsl_lib.LinearItem.ldy.offset == 48 and tsl_lib.LinearItem.ydtype.offset == 56
    assert tsl_lib.LinearItem.sum_next.offset == 64 and tsl_lib.LinearItem.rows.offset == 68
    assert tsl_lib.LinearItem.row_index.offset == 72 and tsl_lib.LinearItem.x_rows.offset == 80


def _lib_plan(tsl_lib, hidden, hq, hkv, hd, ffn, tp, group=0):
    shards = tsl_lib.plan_shards(hidden, hq, hkv, hd, ffn, tp, group)
    return np.array([s.as_tuple() for s in shards], dtype=np.int64).reshape(tp, 7, 12)


@pytest.mark.parametrize("layer", configs.LAYERS, ids=lambda l: l.name)
def test_plan_shards_bit_exact_vs_oracle(tsl_lib, layer):
    args = (layer.hidden, layer.n_q_heads, layer.n_kv_heads, layer.head_dim, layer.ffn, layer.tp,
            layer.group)
    assert np.array_equal(_lib_plan(tsl_lib, *args), oracle.plan(*args))


def test_plan_shards_expected_rank0_shapes(tsl_lib):
    # rank-0 shards of the workloads: (K_s, N_s) per projection
    want = {
        "llama2k": [(2048, 512), (2048, 128), (2048, 128), (512, 2048), (2048, 2048),
                    (2048, 2048), (2048, 2048)],
        "dec7b": [(3584, 896), (3584, 128), (3584, 128), (896, 3584), (3584, 4736),
                  (3584, 4736), (4736, 3584)],
        "pre27b": [(5120, 2048), (5120, 256), (5120, 256), (2048, 5120), (5120, 4352),
                   (5120, 4352), (4352, 5120)],
        "gqa8": [(4096, 512), (4096, 512), (4096, 512), (512, 4096), (4096, 1792),
                 (4096, 1792), (1792, 4096)],
    }
    for layer in configs.LAYERS:
        shards = tsl_lib.plan_shards(layer.hidden, layer.n_q_heads, layer.n_kv_heads,
                                     layer.head_dim, layer.ffn, layer.tp, layer.group)
        got = [(s.k_len, s.n_len) for s in shards[:7]]
        assert got == want[layer.name], layer.name
    g = tsl_lib.plan_shards(4096, 32, 4, 128, 14336, 8)
    assert g[tsl_lib.K].strategy == tsl_lib.REPLICATED and g[tsl_lib.V].strategy == tsl_lib.REPLICATED


def test_plan_shards_grid_vs_oracle(tsl_lib):
    n = 0
    for tp in (1, 2, 4, 8, 16, 32):
        for hkv in (1, 2, 3, 4, 8, 12, 16):
            for ratio in (1, 2, 3, 4):
                for hd, ffn in ((64, 256), (128, 384), (8, 96)):
                    for group in (0, 64):
                        args = (512, hkv * ratio, hkv, hd, ffn, tp, group)
                        try:
                            want = oracle.plan(*args)
                        except oracle.OracleError as e:
                            with pytest.raises(tsl_lib.TslError) as got:
                                tsl_lib.plan_shards(*args)
                            assert got.value.status == e.code, args
                            continue
                        assert np.array_equal(_lib_plan(tsl_lib, *args), want), args
                        n += 1
    assert n > 100


def test_plan_shards_rejections(tsl_lib):
    ok = (2048, 32, 8, 64, 8192, 4, 0)
    tsl_lib.plan_shards(*ok)
    bad = [((2048, 32, 8, 64, 8192, 3, 0), tsl_lib.ERR_TP_NOT_POW2),
           ((2048, 32, 8, 64, 8192, 0, 0), tsl_lib.ERR_INVALID_ARG),
           ((0, 32, 8, 64, 8192, 4, 0), tsl_lib.ERR_INVALID_ARG),
           ((2048, 30, 8, 64, 8192, 4, 0), tsl_lib.ERR_NOT_DIVISIBLE),
           ((2048, 24, 12, 64, 8192, 8, 0), tsl_lib.ERR_NOT_DIVISIBLE),
           ((2048, 32, 8, 64, 8190, 4, 0), tsl_lib.ERR_NOT_DIVISIBLE),
           ((2048, 32, 8, 4, 8192, 4, 64), tsl_lib.ERR_GROUP_ALIGN),
           ((2048, 32, 8, 64, 8192, 4, 32), tsl_lib.ERR_INVALID_ARG)]
    for args, status in bad:
        with pytest.raises(tsl_lib.TslError) as e:
            tsl_lib.plan_shards(*args)
        assert e.value.status == status, args
    # short output buffer
    d = tsl_lib.Dims(*ok)
    out = (tsl_lib.Shard * 27)()
    assert tsl_lib._lib.plan_shards(ctypes.byref(d), out, 27) == tsl_lib.ERR_INVALID_ARG
    assert tsl_lib._lib.plan_shards(None, out, 28) == tsl_lib.ERR_INVALID_ARG


@pytest.mark.parametrize("strategy", [0, 1, 2])
def test_plan_linear_vs_oracle(tsl_lib, strategy):
    for K, N, tp, group in ((1024, 2048, 2, 0), (512, 2048, 2, 0), (192, 64, 2, 64),
                            (256, 48, 4, 64), (100, 30, 2, 0), (64, 64, 3, 0), (4096, 1, 1, 64)):
        try:
            want = oracle.plan_linear(K, N, tp, strategy, group)
        except oracle.OracleError as e:
            with pytest.raises(tsl_lib.TslError) as got:
                tsl_lib.plan_linear(K, N, tp, strategy, group)
            assert got.value.status == e.code
            continue
        got = np.array([s.as_tuple() for s in tsl_lib.plan_linear(K, N, tp, strategy, group)])
        assert np.array_equal(got, want), (K, N, tp, strategy, group)


def test_pack_shard_size_geometry(tsl_lib):
    s = tsl_lib.plan_linear(1024, 2048, 2, tsl_lib.COLUMN)[0]
    # f32: Nt=64 tiles, 64 k-tiles of 16, 64 lanes x 16 bytes
    assert tsl_lib.pack_shard_size(s, tsl_lib.F32) == 64 * 64 * 64 * 16
    assert tsl_lib.pack_shard_size(s, tsl_lib.BF16) == 64 * 32 * 64 * 16
    # Q4: records (codes + scale/bias pairs) of 64 tiles x 8 blocks, then the
    # column exponents, 64 x 16 int32
    assert tsl_lib.pack_shard_size(s, tsl_lib.Q4G64) == 64 * 8 * 1152 + 64 * 16 * 4
    # ragged: 100 x 30 bf16 -> 2 tiles of 16 columns, k padded to 128 (4 tiles of 32)
    r = tsl_lib.plan_linear(100, 30, 1, tsl_lib.COLUMN)[0]
    assert tsl_lib.pack_shard_size(r, tsl_lib.BF16) == 2 * 4 * 1024
    with pytest.raises(tsl_lib.TslError) as e:
        tsl_lib.pack_shard_size(r, tsl_lib.Q4G64)
    assert e.value.status == tsl_lib.ERR_GROUP_ALIGN


def test_shard_linear_rejections_before_launch(tsl_lib):
    s = tsl_lib.plan_linear(1024, 2048, 2, tsl_lib.COLUMN)[0]
    nb = tsl_lib.pack_shard_size(s, tsl_lib.BF16)
    P, X, Y = 1 << 20, 1 << 21, 1 << 22  # fake, aligned addresses: never dereferenced
    call = lambda **kw: tsl_lib.shard_linear(**dict(dict(
        shard=s, wdtype=tsl_lib.BF16, packed=P, packed_bytes=nb, xdtype=tsl_lib.BF16, X=X,
        ldx=1024, M=4, ydtype=tsl_lib.F32, Y=Y, ldy=1024), **kw))
    cases = [(dict(X=0), tsl_lib.ERR_INVALID_ARG),
             (dict(M=-1), tsl_lib.ERR_INVALID_ARG),
             (dict(xdtype=tsl_lib.F32), tsl_lib.ERR_UNSUPPORTED),
             (dict(wdtype=tsl_lib.F32, xdtype=tsl_lib.BF16, packed_bytes=1 << 30),
              tsl_lib.ERR_UNSUPPORTED),
             (dict(ydtype=tsl_lib.BF16, accumulate=1), tsl_lib.ERR_UNSUPPORTED),
             (dict(accumulate=2), tsl_lib.ERR_INVALID_ARG),
             (dict(packed_bytes=nb - 1), tsl_lib.ERR_BUFFER_TOO_SMALL),
             (dict(packed=P + 16), tsl_lib.ERR_MISALIGNED),
             (dict(X=X + 8), tsl_lib.ERR_MISALIGNED),
             (dict(ldx=1028), tsl_lib.ERR_MISALIGNED),
             (dict(ldx=1000), tsl_lib.ERR_INVALID_ARG),
             (dict(ldy=1000), tsl_lib.ERR_INVALID_ARG),
             (dict(Y=Y + 2), tsl_lib.ERR_MISALIGNED),
             # prefill path: 32-bit operand offsets bound the activation stride
             (dict(M=128, ldx=1 << 22), tsl_lib.ERR_UNSUPPORTED)]
    for kw, status in cases:
        with pytest.raises(tsl_lib.TslError) as e:
            call(**kw)
        assert e.value.status == status, kw
    # M == 0 enqueues nothing and succeeds
    call(M=0)
    bad = tsl_lib.Shard(*s.as_tuple())
    bad.n_len = 4000  # beyond W
    with pytest.raises(tsl_lib.TslError) as e:
        call(shard=bad)
    assert e.value.status == tsl_lib.ERR_INVALID_ARG


def test_pack_and_combine_rejections_before_launch(tsl_lib):
    s = tsl_lib.plan_linear(256, 128, 2, tsl_lib.ROW, 64)[0]
    nb = tsl_lib.pack_shard_size(s, tsl_lib.Q4G64)
    W, S, B, P = 1 << 20, 1 << 21, 1 << 22, 1 << 23
    with pytest.raises(tsl_lib.TslError) as e:
        tsl_lib.pack_shard(s, tsl_lib.Q4G64, W, 128, 1, None, B, 128, 1, P, nb)
    assert e.value.status == tsl_lib.ERR_INVALID_ARG
    with pytest.raises(tsl_lib.TslError) as e:
        tsl_lib.pack_shard(s, tsl_lib.Q4G64, W, 128, 1, S, B, 128, 1, P, nb - 1)
    assert e.value.status == tsl_lib.ERR_BUFFER_TOO_SMALL
    with pytest.raises(tsl_lib.TslError) as e:
        tsl_lib.pack_shard(s, tsl_lib.Q4G64, W, 128, 1, S, B, 128, 1, P + 64, nb)
    assert e.value.status == tsl_lib.ERR_MISALIGNED
    with pytest.raises(tsl_lib.TslError) as e:
        tsl_lib.pack_shard(s, tsl_lib.BF16, W, 128, 1, S, B, 128, 1, P, nb)
    assert e.value.status == tsl_lib.ERR_INVALID_ARG
    parts = [1 << 20, 1 << 21]
    Y = 1 << 22
    with pytest.raises(tsl_lib.TslError) as e:
        tsl_lib.combine_partials(tsl_lib.COMBINE_SUM, parts, tsl_lib.BF16, 4, 8, 8, tsl_lib.F32, Y, 8)
    assert e.value.status == tsl_lib.ERR_UNSUPPORTED
    with pytest.raises(tsl_lib.TslError) as e:
        tsl_lib.combine_partials(tsl_lib.COMBINE_CONCAT, parts, tsl_lib.F32, 4, 8, 8, tsl_lib.F32, Y, 8)
    assert e.value.status == tsl_lib.ERR_INVALID_ARG  # ldy < 2 * 8
    with pytest.raises(tsl_lib.TslError) as e:
        tsl_lib.combine_partials(tsl_lib.COMBINE_CONCAT, parts, tsl_lib.F32, 4, 8, 8, tsl_lib.BF16, Y, 16)
    assert e.value.status == tsl_lib.ERR_UNSUPPORTED
    with pytest.raises(tsl_lib.TslError) as e:
        tsl_lib.combine_partials(tsl_lib.COMBINE_SUM, [0, 1 << 21], tsl_lib.F32, 4, 8, 8, tsl_lib.F32, Y, 8)
    assert e.value.status == tsl_lib.ERR_INVALID_ARG
    with pytest.raises(tsl_lib.TslError) as e:
        tsl_lib.combine_partials(tsl_lib.COMBINE_SUM, [1 << 20] * 65, tsl_lib.F32, 4, 8, 8, tsl_lib.F32, Y, 8)
    assert e.value.status == tsl_lib.ERR_INVALID_ARG
    with pytest.raises(tsl_lib.TslError) as e:
        tsl_lib.combine_partials(7, parts, tsl_lib.F32, 4, 8, 8, tsl_lib.F32, Y, 8)
    assert e.value.status == tsl_lib.ERR_INVALID_ARG
    # outputs overlapping a part are rejected, except F32 SUM into part 0 itself
    overlap = [
        (tsl_lib.COMBINE_SUM, parts[0], tsl_lib.BF16, 8),       # in place, but bf16
        (tsl_lib.COMBINE_SUM, parts[0], tsl_lib.F32, 16),       # in place, other stride
        (tsl_lib.COMBINE_SUM, parts[1] + 64, tsl_lib.F32, 8),   # inside part 1
        (tsl_lib.COMBINE_CONCAT, parts[1] - 64, tsl_lib.F32, 16),  # runs into part 1
    ]
    for mode, Yo, yd, ldy in overlap:
        with pytest.raises(tsl_lib.TslError) as e:
            tsl_lib.combine_partials(mode, parts, tsl_lib.F32, 4, 8, 8, yd, Yo, ldy)
        assert e.value.status == tsl_lib.ERR_INVALID_ARG, (mode, Yo, yd, ldy)
    # empty work succeeds without a launch
    tsl_lib.combine_partials(tsl_lib.COMBINE_SUM, parts, tsl_lib.F32, 0, 8, 8, tsl_lib.F32, Y, 8)
    tsl_lib.combine_partials(tsl_lib.COMBINE_SUM, parts, tsl_lib.F32, 0, 8, 8, tsl_lib.BF16, parts[0], 8)


def test_status_strings(tsl_lib):
    for st in range(0, -9, -1):
        assert tsl_lib.tsl_status_string(st) not in ("", "unknown status")
    assert tsl_lib.tsl_status_string(-99) == "unknown status"
    assert tsl_lib.tsl_last_hip_error_string() == "no error"


def test_one_hip_runtime_in_process(tsl_lib):
    # the binding loads torch's HIP runtime before libtsl.so: one runtime only
    maps = open("/proc/self/maps").read().splitlines()
    runtimes = {l.split()[-1] for l in maps if "libamdhip64" in l}
    assert len(runtimes) == 1, runtimes


def test_group_rejections_and_workspace(tsl_lib):
    sh = tsl_lib.plan_linear(1024, 512, 2, tsl_lib.COLUMN, 64)
    nb = tsl_lib.pack_shard_size(sh[0], tsl_lib.Q4G64)
    P0, P1, X = 1 << 24, 1 << 25, 1 << 26          # fake, aligned: never dereferenced
    Y0, Y1 = 1 << 27, (1 << 27) + (1 << 22)
    M = 256

    def item(s, P, Y, **kw):
        return dict(dict(shard=s, packed=P, packed_bytes=nb, X=X, ldx=1024, Y=Y, ldy=256), **kw)

    good = [item(sh[0], P0, Y0), item(sh[1], P1, Y1)]
    # the group's workspace is the sum of its items' (4-bit prefill: a
    # binary16 copy of the activations and its row exponents, padded to whole
    # 256-row tiles -- a size query sees no X pointers, so it never counts a
    # copy as shared -- and, the launch being far too small to fill the chip,
    # the binary32 partials of two k-splits of 8 stages each; the weights are
    # read from their 4-bit records)
    w = [tsl_lib.shard_linear_workspace_size(s, tsl_lib.Q4G64, M) for s in sh]
    assert w[0] == M * 1024 * 2 + M * 4 + 2 * M * 256 * 4
    assert tsl_lib.shard_linear_group_workspace_size(good, tsl_lib.Q4G64, M) == sum(w)
    assert tsl_lib.shard_linear_group_workspace_size(good[:1], tsl_lib.Q4G64, 4) == \
        tsl_lib.shard_linear_workspace_size(sh[0], tsl_lib.Q4G64, 4)
    call = lambda items, **kw: tsl_lib.shard_linear_group(
        items, **dict(dict(wdtype=tsl_lib.Q4G64, xdtype=tsl_lib.BF16, M=M), **kw))
    cases = [([item(sh[0], P0, Y0), item(sh[1], P1, Y0 + 512)], {}, tsl_lib.ERR_INVALID_ARG),
             ([item(sh[0], P0, X + 64), item(sh[1], P1, Y1)], {}, tsl_lib.ERR_INVALID_ARG),
             ([item(sh[0], P0, Y0, ydtype=tsl_lib.Q4G64)], {}, tsl_lib.ERR_INVALID_ARG),
             ([item(sh[0], P0, Y0, ydtype=tsl_lib.BF16, accumulate=1)], {},
              tsl_lib.ERR_UNSUPPORTED),
             # bf16 Y0 column block beside f32 Y1: byte ranges of unequal strides
             ([item(sh[0], P0, Y0, ydtype=tsl_lib.BF16), item(sh[1], P1, Y0 + 512)], {},
              tsl_lib.ERR_INVALID_ARG),
             ([item(sh[0], P0, Y0, packed_bytes=nb - 1)], {}, tsl_lib.ERR_BUFFER_TOO_SMALL),
             ([item(sh[0], P0 + 16, Y0)], {}, tsl_lib.ERR_MISALIGNED),
             ([item(sh[0], P0, Y0, ldx=1 << 22)], {}, tsl_lib.ERR_UNSUPPORTED),
             (good, dict(xdtype=tsl_lib.F32), tsl_lib.ERR_UNSUPPORTED),
             (good, dict(M=-1), tsl_lib.ERR_INVALID_ARG),
             (good, {}, tsl_lib.ERR_BUFFER_TOO_SMALL),  # no workspace for the activation copy
             ([], {}, tsl_lib.ERR_INVALID_ARG)]
    for items, kw, status in cases:
        with pytest.raises(tsl_lib.TslError) as e:
            call(items, **kw)
        assert e.value.status == status, (items, kw)
    # empty row count: validated, nothing enqueued
    call(good, M=0)


def test_row_index_rules(tsl_lib):
    """Items that read their rows through a row index: validation before
    launch, and their workspace -- none where the kernels read through the
    index (4-bit weights above 64 rows; a call of a few decode rows whose
    activations stay in LDS), else a gathered copy per indexed item
    (M x k_len, 2 bytes per element, rounded to 256 bytes)."""
    K, N, M = 1024, 512, 256
    sh = tsl_lib.plan_linear(K, N, 1, tsl_lib.COLUMN, 64)[0]
    P, X, Y, R = 1 << 24, 1 << 26, 1 << 27, 1 << 28  # fake, aligned: never dereferenced
    ws = tsl_lib.shard_linear_group_workspace_size

    def item(wdtype=tsl_lib.Q4G64, **kw):
        nb = tsl_lib.pack_shard_size(sh, wdtype)
        return dict(dict(shard=sh, packed=P, packed_bytes=nb, X=X, ldx=K, Y=Y, ldy=N,
                         row_index=R, x_rows=100), **kw)

    plain = lambda wd, m: ws([dict(item(wd), row_index=None)], wd, m)
    assert ws([item()], tsl_lib.Q4G64, M) == plain(tsl_lib.Q4G64, M)
    assert ws([item()], tsl_lib.Q4G64, 2) == plain(tsl_lib.Q4G64, 2)
    assert ws([item(tsl_lib.BF16)], tsl_lib.BF16, M) == plain(tsl_lib.BF16, M) + M * K * 2
    call = lambda items, wd=tsl_lib.Q4G64, m=M: tsl_lib.shard_linear_group(
        items, wd, tsl_lib.BF16, m)
    cases = [(item(row_index=R + 2), tsl_lib.ERR_MISALIGNED),
             (item(x_rows=0), tsl_lib.ERR_INVALID_ARG),
             (item(x_rows=1 << 31), tsl_lib.ERR_INVALID_ARG),
             (item(row_index=Y + 64), tsl_lib.ERR_INVALID_ARG),  # inside the output
             (item(X=Y + N * 2 * M), tsl_lib.ERR_INVALID_ARG),   # X's 100 rows meet Y
             (item(), tsl_lib.ERR_BUFFER_TOO_SMALL)]             # no workspace given
    for it, status in cases:
        with pytest.raises(tsl_lib.TslError) as e:
            call([it])
        assert e.value.status == status, it


def test_group_output_overlap_rule(tsl_lib):
    """Items may write disjoint column blocks of one output (same stride);
    any shared element is rejected.  Checked with a group whose workspace is
    missing, so an accepted layout reports BUFFER_TOO_SMALL before any
    launch."""
    sh = tsl_lib.plan_linear(1024, 512, 2, tsl_lib.COLUMN, 64)
    nb = tsl_lib.pack_shard_size(sh[0], tsl_lib.Q4G64)
    P0, P1, X, Y = 1 << 24, 1 << 25, 1 << 26, 1 << 27
    M, N = 256, 512

    def status(y0, y1, ldy0=N, ldy1=N):
        items = [dict(shard=sh[0], packed=P0, packed_bytes=nb, X=X, ldx=1024, Y=y0, ldy=ldy0),
                 dict(shard=sh[1], packed=P1, packed_bytes=nb, X=X, ldx=1024, Y=y1, ldy=ldy1)]
        try:
            tsl_lib.shard_linear_group(items, tsl_lib.Q4G64, tsl_lib.BF16, M)
        except tsl_lib.TslError as e:
            return e.status
        return tsl_lib.OK

    ok, bad = tsl_lib.ERR_BUFFER_TOO_SMALL, tsl_lib.ERR_INVALID_ARG
    assert status(Y, Y + 4 * 256) == ok                 # the two column halves of Y
    assert status(Y + 4 * 256, Y) == ok
    assert status(Y, Y + 4 * 252) == bad                # 4 shared columns per row
    assert status(Y, Y + 4 * N * M) == ok               # the next matrix
    assert status(Y, Y + 4 * (N * (M - 1) + 256)) == ok  # last row's free half
    assert status(Y, Y + 4 * (N * (M - 1) + 255)) == bad
    assert status(Y + 4 * N * M, Y + 4 * 256) == ok     # b before a
    assert status(Y + 4 * (N * (M - 1) + 255), Y) == bad  # a starts on the last element of b
    assert status(Y, Y + 4 * 256, ldy1=N + 4) == bad    # unequal strides: address ranges


def test_sum_set_rules(tsl_lib):
    """Sum sets: validation before launch and their workspace."""
    K, N, tp, M = 1024, 512, 4, 256
    sh = tsl_lib.plan_linear(K, N, tp, tsl_lib.ROW, 64)
    nb = tsl_lib.pack_shard_size(sh[0], tsl_lib.Q4G64)
    X, Y = 1 << 26, 1 << 27

    def items(changes=None):
        out = []
        for r, s in enumerate(sh):
            it = dict(shard=s, packed=(1 << 24) + r * (1 << 20), packed_bytes=nb,
                      X=X + 2 * s.k_off, ldx=K, Y=Y if r == 0 else None, ldy=N,
                      sum_next=1 if r < tp - 1 else 0)
            it.update((changes or {}).get(r, {}))
            out.append(it)
        return out

    # prefill, members of whole 128-k records: the set is one product over
    # the members' k-ranges end to end -- the workspace of the unsharded
    # product (its binary16 weights with the set's column exponents, the
    # activation copy with its row exponents, k-partials), no rank partials
    full = tsl_lib.plan_linear(K, N, 1, tsl_lib.ROW, 64)[0]
    assert tsl_lib.shard_linear_group_workspace_size(items(), tsl_lib.Q4G64, M) == \
        tsl_lib.shard_linear_workspace_size(full, tsl_lib.Q4G64, M)
    # prefill, 192-k members: the products go to binary32 partials in the
    # workspace first (M x N x 4 bytes each), then the binary16 weights
    sh192 = tsl_lib.plan_linear(768, N, tp, tsl_lib.ROW, 64)
    w = sum(tsl_lib.shard_linear_workspace_size(s, tsl_lib.Q4G64, M) for s in sh192)
    odd = [dict(it, shard=s) for it, s in zip(items(), sh192)]
    assert tsl_lib.shard_linear_group_workspace_size(odd, tsl_lib.Q4G64, M) == \
        w + tp * M * N * 4
    # decode: the same partials (the products themselves need no workspace
    # here) and, as the streaming launch adds the set up itself, a counter
    # of 8 bytes per 16-column tile (rounded up to 256 bytes)
    ctr = (N // 16 * 8 + 255) // 256 * 256
    assert tsl_lib.shard_linear_group_workspace_size(items(), tsl_lib.Q4G64, 4) == \
        tp * 4 * N * 4 + ctr
    # a set of 3-row items inside a 4-row call: partials of 3 rows
    rows3 = items({r: dict(rows=3) for r in range(tp)})
    assert tsl_lib.shard_linear_group_workspace_size(rows3, tsl_lib.Q4G64, 4) == \
        tp * ((3 * N * 4 + 255) // 256 * 256) + ctr
    call = lambda its, M=M: tsl_lib.shard_linear_group(its, tsl_lib.Q4G64, tsl_lib.BF16, M)
    bad = [items({3: dict(sum_next=1)}),                 # the last item links on
           items({1: dict(sum_next=2)}),
           items({2: dict(rows=1)}),                     # members' rows differ
           items({1: dict(rows=M + 1)}),                 # more rows than M
           items({1: dict(rows=-1)}),
           items({0: dict(accumulate=1)}),               # a set's output cannot accumulate
           items({0: dict(Y=None)})]
    for its in bad:
        with pytest.raises(tsl_lib.TslError) as e:
            call(its)
        assert e.value.status == tsl_lib.ERR_INVALID_ARG
    # members must share n_len
    other = tsl_lib.plan_linear(K, 2 * N, tp, tsl_lib.ROW, 64)[1]
    with pytest.raises(tsl_lib.TslError) as e:
        call(items({1: dict(shard=other, packed_bytes=1 << 30)}))
    assert e.value.status == tsl_lib.ERR_INVALID_ARG
    # a well-formed set passes validation (no workspace given -> too small)
    with pytest.raises(tsl_lib.TslError) as e:
        call(items())
    assert e.value.status == tsl_lib.ERR_BUFFER_TOO_SMALL


def test_bf16_sum_sets_join_in_the_gemm_regime(tsl_lib):
    """bf16 weights above 64 rows: a sum set whose members hold whole 64-k
    stages is one product over the members' k-ranges end to end -- the
    workspace of the unsharded product, no rank partials, whatever the
    members' activation row strides (the workspace query does not see
    them); a member read through a row index first has its rows gathered
    into the workspace (M x k_len x 2 bytes), and the set still joins."""
    K, N, tp, M = 2048, 512, 4, 256
    sh = tsl_lib.plan_linear(K, N, tp, tsl_lib.ROW, 64)
    nb = tsl_lib.pack_shard_size(sh[0], tsl_lib.BF16)
    X, Y = 1 << 26, 1 << 27

    def items(ldx0=K, **kw):
        return [dict(shard=s, packed=(1 << 24) + r * (1 << 20), packed_bytes=nb,
                     X=X + 2 * s.k_off, ldx=ldx0 if r == 0 else K, Y=Y if r == 0 else None,
                     ldy=N, sum_next=1 if r < tp - 1 else 0, **(kw if r == 1 else {}))
                for r, s in enumerate(sh)]

    full = tsl_lib.plan_linear(K, N, 1, tsl_lib.ROW, 64)[0]
    ws = tsl_lib.shard_linear_group_workspace_size
    joined = tsl_lib.shard_linear_workspace_size(full, tsl_lib.BF16, M)
    assert ws(items(), tsl_lib.BF16, M) == joined
    assert ws(items(K + 64), tsl_lib.BF16, M) == joined
    indexed = ws(items(row_index=1 << 28, x_rows=M), tsl_lib.BF16, M)
    assert indexed == joined + M * (K // tp) * 2
    # decode-sized calls never join: the rank partials are there
    assert ws(items(), tsl_lib.BF16, 16) >= tp * 16 * N * 4


def test_combine_to_ranks_rejections(tsl_lib):
    """Per-rank collectives: argument checks before any launch.  Accepted
    layouts are probed with M == 0 (validated, nothing enqueued) or via an
    unsupported type that is only reported after the layout passed."""
    n, M, N = 4, 10, 64
    parts = [(1 << 24) + r * (1 << 20) for r in range(n)]
    Y = 1 << 28
    call = lambda op, outs, **kw: tsl_lib.combine_to_ranks(
        op, parts, kw.get("pdtype", tsl_lib.F32), kw.get("M", M), N, N,
        kw.get("odtype", tsl_lib.F32), outs, kw.get("ldo", N))
    # reduce-scatter: the rank blocks of one [M][N] buffer side by side are fine
    rs_outs = [Y + 4 * N * ((r * M) // n) for r in range(n)]
    call(tsl_lib.REDUCE_SCATTER, rs_outs, M=0)
    bad = [
        (tsl_lib.ALL_REDUCE, rs_outs, {}),                        # full-size outputs overlap
        (tsl_lib.REDUCE_SCATTER, [Y] * n, {}),                    # the same block twice
        (tsl_lib.REDUCE_SCATTER, [parts[1] + 64] + rs_outs[1:], {}),  # output inside a part
        (tsl_lib.ALL_GATHER, [Y + r * 4 * N * n * M for r in range(n)], dict(ldo=N)),  # ldo < n N
        (7, rs_outs, {}),
    ]
    for op, outs, kw in bad:
        with pytest.raises(tsl_lib.TslError) as e:
            call(op, outs, **kw)
        assert e.value.status == tsl_lib.ERR_INVALID_ARG, (op, kw)
    with pytest.raises(tsl_lib.TslError) as e:  # sums need binary32 parts
        call(tsl_lib.ALL_REDUCE, [Y + r * 4 * N * M for r in range(n)], pdtype=tsl_lib.BF16)
    assert e.value.status == tsl_lib.ERR_UNSUPPORTED
    with pytest.raises(tsl_lib.TslError) as e:  # a gather copies: same types
        call(tsl_lib.ALL_GATHER, [Y + r * 4 * N * n * M for r in range(n)], ldo=n * N,
             odtype=tsl_lib.BF16)
    assert e.value.status == tsl_lib.ERR_UNSUPPORTED
    with pytest.raises(tsl_lib.TslError) as e:
        call(tsl_lib.ALL_REDUCE, [Y + 2] + [Y + r * 4 * N * M for r in range(1, n)])
    assert e.value.status == tsl_lib.ERR_MISALIGNED


@pytest.mark.parametrize("tp", [1, 2, 4, 8])
def test_plan_vocab_vs_oracle(tsl_lib, tp):
    for vocab, hidden, group in ((152064, 3584, 64), (32000, 4096, 0), (100, 64, 0),
                                 (96, 96, 64), (8, 128, 64)):
        try:
            want = oracle.plan_vocab(vocab, hidden, tp, group)
        except oracle.OracleError as e:
            with pytest.raises(tsl_lib.TslError) as got:
                tsl_lib.plan_vocab(vocab, hidden, tp, group)
            assert got.value.status == e.code
            continue
        got = np.array([s.as_tuple() for s in tsl_lib.plan_vocab(vocab, hidden, tp, group)])
        assert np.array_equal(got, want.reshape(2 * tp, -1)), (vocab, hidden, tp, group)
    with pytest.raises(tsl_lib.TslError) as e:
        tsl_lib.plan_vocab(96, 64, 3)
    assert e.value.status == tsl_lib.ERR_TP_NOT_POW2


def test_embed_lookup_rejections(tsl_lib):
    """Argument checks before any launch; accepted layouts are probed with
    M == 0 (validated, nothing enqueued)."""
    e_sh = tsl_lib.plan_vocab(1024, 64, 4)[2]  # rank 1's 256 x 64 slice
    table, tokens, Y = 1 << 24, 1 << 26, 1 << 28
    call = lambda **kw: tsl_lib.embed_lookup(
        kw.get("shard", e_sh), kw.get("tdtype", tsl_lib.BF16), kw.get("table", table),
        kw.get("ld_table", 64), kw.get("tokens", tokens), kw.get("M", 0),
        kw.get("ydtype", tsl_lib.F32), kw.get("Y", Y), kw.get("ldy", 64))
    call()
    call(tdtype=tsl_lib.F32, ydtype=tsl_lib.BF16, ld_table=65, ldy=70)
    bad = [
        (dict(table=None), tsl_lib.ERR_INVALID_ARG),
        (dict(tokens=None), tsl_lib.ERR_INVALID_ARG),
        (dict(Y=None), tsl_lib.ERR_INVALID_ARG),
        (dict(M=-1), tsl_lib.ERR_INVALID_ARG),
        (dict(tdtype=tsl_lib.Q4G64), tsl_lib.ERR_INVALID_ARG),
        (dict(ydtype=5), tsl_lib.ERR_INVALID_ARG),
        (dict(ld_table=63), tsl_lib.ERR_INVALID_ARG),
        (dict(ldy=32), tsl_lib.ERR_INVALID_ARG),
        (dict(table=table + 1), tsl_lib.ERR_MISALIGNED),
        (dict(tokens=tokens + 2), tsl_lib.ERR_MISALIGNED),
        (dict(Y=Y + 2), tsl_lib.ERR_MISALIGNED),
        (dict(M=4, Y=table + 128), tsl_lib.ERR_INVALID_ARG),       # output inside the table
        (dict(M=4, Y=tokens - 4 * 64 * 2), tsl_lib.ERR_INVALID_ARG),  # last row over the ids
    ]
    for kw, code in bad:
        with pytest.raises(tsl_lib.TslError) as e:
            call(**kw)
        assert e.value.status == code, kw
    broken = tsl_lib.plan_vocab(1024, 64, 4)[2]
    broken.k_len = 2000  # past the end of W
    with pytest.raises(tsl_lib.TslError) as e:
        call(shard=broken)
    assert e.value.status == tsl_lib.ERR_INVALID_ARG


@pytest.mark.parametrize("mode", [0, 1])
def test_plan_experts_vs_oracle(tsl_lib, mode):
    for ne, hidden, ffn, tp, group in ((128, 2048, 768, 4, 64), (8, 4096, 14336, 4, 0),
                                       (3, 64, 128, 8, 64), (4, 64, 100, 8, 0),
                                       (4, 64, 96, 2, 64), (5, 64, 128, 3, 0)):
        try:
            want = oracle.plan_experts(ne, hidden, ffn, tp, mode, group)
        except oracle.OracleError as e:
            with pytest.raises(tsl_lib.TslError) as got:
                tsl_lib.plan_experts(ne, hidden, ffn, tp, mode, group)
            assert got.value.status == e.code
            continue
        got = tsl_lib.plan_experts(ne, hidden, ffn, tp, mode, group)
        assert len(got) == len(want)
        for g, (e, r, sh) in zip(got, want):
            assert (g.expert, g.rank) == (e, r)
            for p in ("gate", "up", "down"):
                assert getattr(g, p).as_tuple() == tuple(sh[p][f] for f in oracle.FIELDS)
    with pytest.raises(tsl_lib.TslError) as e:
        tsl_lib.plan_experts(4, 64, 128, 2, 7)
    assert e.value.status == tsl_lib.ERR_INVALID_ARG


def test_moe_dispatch_vs_oracle(tsl_lib):
    rng = np.random.default_rng(9)
    cases = [(np.array([[0, 2], [2, 1], [0, 0]]), 3, [2, 0])]
    for T, k, E in ((0, 2, 4), (1, 1, 1), (37, 2, 8), (2048, 8, 128), (5, 3, 6)):
        topk = np.stack([rng.permutation(E)[:k] for _ in range(T)]) if T else \
            np.zeros((0, k), dtype=np.int64)
        for tp in (1, 4):
            for r in range(min(tp, 2)):
                cases.append((topk, E, [e for e in range(E) if e % tp == r]))
        cases.append((rng.integers(0, E, (T, k)), E, list(rng.permutation(E)[: E // 2])))
    for topk, E, held in cases:
        off, row_slot, slot_row = tsl_lib.moe_dispatch(topk, E, held)
        w_off, w_rs, w_sr = oracle.moe_dispatch(topk, held)
        assert np.array_equal(off, w_off)
        assert np.array_equal(row_slot, w_rs) and np.array_equal(slot_row, w_sr)
    bad = [(np.array([[0, 5]]), 4, [0]),      # routed to an expert that does not exist
           (np.array([[0, 1]]), 4, [1, 1]),   # an expert listed twice
           (np.array([[0, 1]]), 4, [4]),      # a held expert out of range
           (np.array([[0, -1]]), 4, [0])]
    for topk, E, held in bad:
        with pytest.raises(tsl_lib.TslError) as e:
            tsl_lib.moe_dispatch(topk, E, held)
        assert e.value.status == tsl_lib.ERR_INVALID_ARG


def test_moe_gather_and_combine_rejections(tsl_lib):
    src, idx, out = 1 << 24, 1 << 26, 1 << 28
    g = lambda **kw: tsl_lib.moe_gather(kw.get("src", src), kw.get("ld", 64), 100,
                                        kw.get("dt", tsl_lib.BF16), kw.get("idx", idx),
                                        kw.get("n", 0), 64, kw.get("out", out), kw.get("ldo", 64))
    g()
    for kw, code in ((dict(src=None), tsl_lib.ERR_INVALID_ARG), (dict(ld=32), tsl_lib.ERR_INVALID_ARG),
                     (dict(dt=tsl_lib.Q4G64), tsl_lib.ERR_INVALID_ARG),
                     (dict(ldo=8), tsl_lib.ERR_INVALID_ARG), (dict(out=out + 1), tsl_lib.ERR_MISALIGNED),
                     (dict(n=5, out=src + 256), tsl_lib.ERR_INVALID_ARG)):
        with pytest.raises(tsl_lib.TslError) as e:
            g(**kw)
        assert e.value.status == code, kw
    P, sr, w, Y = 1 << 24, 1 << 26, (1 << 26) + 4096, 1 << 28
    c = lambda **kw: tsl_lib.moe_combine(kw.get("P", P), 64, kw.get("rows", 10), kw.get("sr", sr),
                                         kw.get("w", w), kw.get("T", 0), kw.get("k", 2), 64,
                                         kw.get("yd", tsl_lib.F32), kw.get("Y", Y),
                                         kw.get("ldy", 64))
    c()
    c(P=None, rows=0)  # no rows held: every token gets -0.0
    for kw, code in ((dict(k=0), tsl_lib.ERR_INVALID_ARG), (dict(P=None), tsl_lib.ERR_INVALID_ARG),
                     (dict(ldy=63), tsl_lib.ERR_INVALID_ARG), (dict(yd=tsl_lib.Q4G64), tsl_lib.ERR_INVALID_ARG),
                     (dict(Y=Y + 2), tsl_lib.ERR_MISALIGNED),
                     (dict(T=4, Y=P + 256), tsl_lib.ERR_INVALID_ARG),
                     (dict(T=4, Y=w - 64), tsl_lib.ERR_INVALID_ARG)):
        with pytest.raises(tsl_lib.TslError) as e:
            c(**kw)
        assert e.value.status == code, kw


def test_plan_choices_are_remembered_per_geometry_and_thread_safe(tsl_lib):
    """The GEMM regime's tile-shape and k-split choices are cached per group
    geometry (weight type; each item's rows, k, columns and flags): queries
    from many threads at once give the sizes the same queries give one at a
    time, groups that differ only in rows, columns or a flag get their own
    plans, and the cache stays bounded past its 256 entries."""
    import concurrent.futures
    sh = tsl_lib.plan_linear(2048, 4096, 4, tsl_lib.COLUMN, 64)
    nb = tsl_lib.pack_shard_size(sh[0], tsl_lib.Q4G64)

    def group(M, rows=None, acc=0, n=4, wd=None):
        wd = wd or tsl_lib.Q4G64
        items = []
        for r in range(n):
            it = dict(shard=sh[r % 4], packed=(1 << 24) + r * (1 << 22), packed_bytes=nb,
                      X=(1 << 40) + r * (1 << 30), ldx=2048, Y=(1 << 42) + r * (1 << 30),
                      ldy=sh[0].n_len, ydtype=tsl_lib.F32, accumulate=acc)
            if rows is not None:
                it["rows"] = rows[r % len(rows)]
            items.append(it)
        return items, wd, M

    cases = [group(M) for M in (65, 100, 300, 1000, 2048)]
    cases += [group(300, rows=(300, 77)), group(300, acc=1), group(2048, n=17)]
    serial = [tsl_lib.shard_linear_group_workspace_size(*c) for c in cases]
    # each variant of the same base geometry is planned on its own
    assert len({(c[2], tuple(i.get("rows", -1) for i in c[0]), c[0][0]["accumulate"], len(c[0]))
                for c in cases}) == len(cases)
    with concurrent.futures.ThreadPoolExecutor(8) as ex:
        for _ in range(3):
            got = list(ex.map(lambda c: tsl_lib.shard_linear_group_workspace_size(*c),
                              cases * 8))
            assert got == serial * 8
    # more than 256 distinct geometries: the cache starts over, sizes unchanged
    for M in range(65, 65 + 300):
        tsl_lib.shard_linear_group_workspace_size(*group(M))
    assert [tsl_lib.shard_linear_group_workspace_size(*c) for c in cases] == serial
