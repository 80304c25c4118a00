"""shard_linear_group_noalloc: the grouped shard product with its workspace
in the library's fixed device array instead of a caller's buffer.

On the GPU its outputs must equal, bit for bit, those of
shard_linear_group with a caller workspace on the same items (the same
plan and kernels run; only the workspace address differs): a prefill-sized
call (binary16 activation copies, a joined sum set) followed by a smaller,
decode-sized call (k-partials and the in-launch rank-sum counters, in the
array the first call left behind), then the first again; and calls whose
products read their rows through a row index (gathered into the array,
or read by the activation pass).  On the CPU: a
call whose workspace would not fit the array is rejected before any device
work."""
import re

import numpy as np
import pytest

from tensor_sharded_linear_plan_amd import binding as tsl
from tensor_sharded_linear_plan_amd import synth


def test_scratch_size_matches_header():
    import os
    hdr = open(os.path.join(os.path.dirname(__file__), "..", "include", "tsl.h")).read()
    m = re.search(r"#define TSL_NOALLOC_SCRATCH_BYTES \(\(size_t\)(\d+) << (\d+)\)", hdr)
    assert m and int(m.group(1)) << int(m.group(2)) == tsl.NOALLOC_SCRATCH_BYTES


def test_rejects_calls_beyond_its_scratch():
    """M = 8192 rows over k_len = 8192 need a 128 MiB binary16 activation
    copy: TSL_ERR_BUFFER_TOO_SMALL, decided on the host (the device
    addresses below are never touched)."""
    K, N, M = 8192, 1024, 8192
    sh = tsl.plan_linear(K, N, 1, tsl.COLUMN, 64)[0]
    nb = tsl.pack_shard_size(sh, tsl.Q4G64)
    base = 1 << 40
    item = dict(shard=sh, packed=base, packed_bytes=nb, X=base + (1 << 32), ldx=K,
                Y=base + (2 << 32), ldy=N, ydtype=tsl.F32)
    assert tsl.shard_linear_group_workspace_size([item], tsl.Q4G64, M) > tsl.NOALLOC_SCRATCH_BYTES
    with pytest.raises(tsl.TslError) as e:
        tsl.shard_linear_group_noalloc([item], tsl.Q4G64, tsl.BF16, M)
    assert e.value.status == tsl.ERR_BUFFER_TOO_SMALL


def _calls(M, tag):
    """A group of 4-bit products: gate and up column shards reading one X,
    rank 1's o column block in bf16, and the two row shards of down as one
    sum set.  Returns the items for the no-alloc call, the same items
    writing to a second set of outputs, and both output lists."""
    from gpu_util import Q4Weight, dev, torch
    t = torch()
    H, F = 1024, 2048
    seed = 7100 + 10 * tag
    wg = Q4Weight(H, F, seed, seed + 1, seed + 2)
    wd = Q4Weight(F, H, seed + 3, seed + 4, seed + 5)
    X1 = dev(synth.normal_bf16(seed + 6, (M, H)))
    X2 = dev(synth.normal_bf16(seed + 7, (M, F)))
    col = tsl.plan_linear(H, F, 2, tsl.COLUMN, 64)
    row = tsl.plan_linear(F, H, 2, tsl.ROW, 64)
    packs = {("g", r): wg.pack(col[r]) for r in range(2)}
    packs.update({("d", r): wd.pack(row[r]) for r in range(2)})
    sets = []
    for _ in range(2):
        outs = [t.full((M, F // 2), float("nan"), dtype=t.float32, device="cuda"),
                t.full((M, F // 2), float("nan"), dtype=t.bfloat16, device="cuda"),
                t.full((M, H), float("nan"), dtype=t.float32, device="cuda")]
        items = [dict(shard=col[0], packed=packs[("g", 0)][0], packed_bytes=packs[("g", 0)][1],
                      X=X1, ldx=H, Y=outs[0], ldy=F // 2, ydtype=tsl.F32),
                 dict(shard=col[1], packed=packs[("g", 1)][0], packed_bytes=packs[("g", 1)][1],
                      X=X1, ldx=H, Y=outs[1], ldy=F // 2, ydtype=tsl.BF16)]
        for r in range(2):
            items.append(dict(shard=row[r], packed=packs[("d", r)][0],
                              packed_bytes=packs[("d", r)][1], X=X2[:, row[r].k_off:], ldx=F,
                              Y=outs[2] if r == 0 else None, ldy=H, ydtype=tsl.F32,
                              sum_next=int(r == 0)))
        sets.append((items, outs))
    keep = (wg, wd, X1, X2, packs)
    return sets, keep


def _check_call(M, tag):
    from gpu_util import empty_bytes, torch
    t = torch()
    sets, keep = _calls(M, tag)
    (items_n, outs_n), (items_w, outs_w) = sets
    ws = tsl.shard_linear_group_workspace_size(items_w, tsl.Q4G64, M)
    assert 0 < ws <= tsl.NOALLOC_SCRATCH_BYTES
    tsl.shard_linear_group(items_w, tsl.Q4G64, tsl.BF16, M, empty_bytes(ws), ws)
    tsl.shard_linear_group_noalloc(items_n, tsl.Q4G64, tsl.BF16, M)
    t.cuda.synchronize()
    for a, b in zip(outs_n, outs_w):
        assert not t.isnan(a.float()).any()
        assert t.equal(a.view(t.int16) if a.dtype == t.bfloat16 else a.view(t.int32),
                       b.view(t.int16) if b.dtype == t.bfloat16 else b.view(t.int32)), (M, tag)


@pytest.mark.gpu
def test_noalloc_matches_workspace_entry_point_on_consecutive_calls():
    print("noalloc: prefill-sized call M=300", flush=True)
    _check_call(300, 0)
    print("noalloc: smaller decode-sized call M=4", flush=True)
    _check_call(4, 1)
    print("noalloc: prefill-sized call again M=300", flush=True)
    _check_call(300, 2)


def _indexed_check(wdtype, M, seed):
    """Three column products reading X [150, 1024] through row indices
    (two share one): the no-alloc call against the workspace call."""
    from gpu_util import Q4Weight, dev, empty_bytes, pack, torch
    t = torch()
    K, N, x_rows = 1024, 256, 150
    X = dev(synth.normal_bf16(seed, (x_rows, K)))
    rng = np.random.default_rng(seed + 1)
    idx = [dev(rng.integers(-2, x_rows + 2, M).astype(np.int32)) for _ in range(2)]
    sh = tsl.plan_linear(K, N, 1, tsl.COLUMN, 64)[0]
    if wdtype == tsl.Q4G64:
        buf, nb = Q4Weight(K, N, seed + 2, seed + 3, seed + 4).pack(sh)
    else:
        buf, nb = pack(sh, tsl.BF16, dev(synth.normal_bf16(seed + 2, (K, N), 0.02)), N, 1)
    outs = [[t.full((M, N), float("nan"), dtype=t.float32, device="cuda") for _ in range(3)]
            for _ in range(2)]
    items = [[dict(shard=sh, packed=buf, packed_bytes=nb, X=X, ldx=K, Y=Y, ldy=N,
                   row_index=idx[w], x_rows=x_rows) for w, Y in zip((0, 0, 1), ys)]
             for ys in outs]
    ws = tsl.shard_linear_group_workspace_size(items[1], wdtype, M)
    assert 0 < ws <= tsl.NOALLOC_SCRATCH_BYTES
    tsl.shard_linear_group(items[1], wdtype, tsl.BF16, M, empty_bytes(ws), ws)
    tsl.shard_linear_group_noalloc(items[0], wdtype, tsl.BF16, M)
    t.cuda.synchronize()
    for a, b in zip(*outs):
        assert not t.isnan(a).any()
        assert t.equal(a.view(t.int32), b.view(t.int32)), (wdtype, M)


@pytest.mark.gpu
def test_noalloc_with_rows_read_through_an_index():
    """Row-indexed products (some indices out of range): a decode-sized
    bf16 call whose rows the call gathers into the fixed array, a
    prefill-sized 4-bit call whose activation pass reads through the index,
    then the first again -- each bit for bit the workspace entry point's
    outputs."""
    print("noalloc: row-indexed bf16 call M=24 (gathered)", flush=True)
    _indexed_check(tsl.BF16, 24, 9500)
    print("noalloc: row-indexed 4-bit call M=300", flush=True)
    _indexed_check(tsl.Q4G64, 300, 9510)
    print("noalloc: row-indexed bf16 call M=24 again", flush=True)
    _indexed_check(tsl.BF16, 24, 9520)
