#!/usr/bin/env python3
"""Throughput of the sharded-linear hot path on one MI355X.

One step is the in-process multi-rank pass the mlxcel manual describes
("Tensor parallelism", "Current runtime support": one process holds every
rank's shards and runs them in lockstep), here for one tp=4 layer of a
27B-class model with 4-bit weights at M = 2048 prefill tokens: for every
rank r and projection p, shard_linear(r, p) -- column outputs written
straight into their block of the full output (the concat), the 4 o and
the 4 down shards each a sum set (their on-device rank sum, which the
4-bit GEMM regime accumulates inside one product over the ranks' k-ranges
end to end) -- all 28 products in one shard_linear_group call.
The plan is recomputed each step (host only); packing is load-time work
and is timed separately.

value = algorithmic FLOP of the step / step time (inputs resident in HBM).
A decode figure (7B-class, 4-bit, M = 1, 4, 16, every rank of one layer,
HIP-graph replay over weight copies that together exceed the 256 MB
Infinity Cache) is reported beside it in GB/s.

Usage: python bench.py [--steps K] [--warmup W] [--gpus 1]
"""
import argparse
import ctypes
import json
import os
import sys
import time

METRIC = "shard-linear TFLOP/s (prefill) and HBM GB/s (decode) + % roofline, 1 MI355X"
ROOT = os.path.dirname(os.path.abspath(__file__))
# HBM bytes of the prefill step's grouped call, from rocprofv3 FETCH_SIZE /
# WRITE_SIZE runs scaled by a plain copy's readings; valid only for the
# kernel sources it was measured on (their SHA-256 is recorded with it)
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_pre27b.json")
TRAFFIC_SOURCES = ("tensor_sharded_linear_plan_amd/csrc/q4gemm.hip",
                   "tensor_sharded_linear_plan_amd/csrc/prefill.hip",
                   "tensor_sharded_linear_plan_amd/csrc/gemm_common.hpp",
                   "tensor_sharded_linear_plan_amd/csrc/device.hpp",
                   "tensor_sharded_linear_plan_amd/csrc/internal.hpp",
                   "tensor_sharded_linear_plan_amd/csrc/abi.cpp")
PEAK_MFMA_F16 = 2500.0  # TFLOP/s, dense fp16/bf16 MFMA, MI355X
PEAK_HBM = 8000.0       # GB/s, MI355X HBM3E


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def sources_digest():
    """SHA-256 of the kernel sources' code: comments and blank space do not
    count, so a documentation edit keeps a measurement valid."""
    import hashlib
    import re
    h = hashlib.sha256()
    for rel in TRAFFIC_SOURCES:
        with open(os.path.join(ROOT, rel)) as f:
            text = f.read()
        text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
        text = re.sub(r"//[^\n]*", " ", text)
        h.update(" ".join(text.split()).encode())
    return h.hexdigest()


def measured_traffic(kernel):
    """HBM bytes (fetched + written) per launch of the named kernel of the
    grouped call, from the committed counter runs, or None when the kernel
    sources have changed since they were taken."""
    try:
        with open(TRAFFIC_FILE) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    if rec.get("sources_sha256") != sources_digest():
        return None
    k = rec.get("kernels", {}).get(kernel)
    return None if k is None else k["fetch_bytes"] + k["write_bytes"]


def build_layer(layer, M, copies, tsl, torch, synth, configs):
    """Pack every rank's shard of every projection (copies times)."""
    shards = tsl.plan_shards(layer.hidden, layer.n_q_heads, layer.n_kv_heads, layer.head_dim,
                             layer.ffn, layer.tp, layer.group)
    packs = [dict() for _ in range(copies)]
    pack_s, pack_bytes = 0.0, 0
    for pi, proj in enumerate(configs.PROJS):
        K, N = shards[pi].K, shards[pi].N
        seed = lambda t: synth.seed_of(layer.index, pi, t)
        codes = torch.from_numpy(synth.q4_codes(seed(synth.T_CODES), (K, N))).cuda()
        sc = torch.from_numpy(synth.uniform_bf16(seed(synth.T_SCALES), (K // 64, N),
                                                 layer.scale_lo, layer.scale_hi).view("int16")).cuda()
        bi = torch.from_numpy(synth.normal_bf16(seed(synth.T_BIASES), (K // 64, N),
                                                layer.bias_std).view("int16")).cuda()
        for c in range(copies):
            for r in range(layer.tp):
                sh = shards[r * tsl.NPROJ + pi]
                nb = tsl.pack_shard_size(sh, tsl.Q4G64)
                buf = torch.empty(nb, dtype=torch.uint8, device="cuda")
                torch.cuda.synchronize()
                t0 = time.perf_counter()
                tsl.pack_shard(sh, tsl.Q4G64, codes, N, 1, sc, bi, N, 1, buf, nb)
                torch.cuda.synchronize()
                pack_s += time.perf_counter() - t0
                pack_bytes += sh.k_len * sh.n_len + (sh.k_len // 64) * sh.n_len * 4 + nb
                packs[c][(r, proj)] = (sh, buf, nb)
        del codes, sc, bi
    return shards, packs, pack_s, pack_bytes


def step_items(layer, M, pk, bufs, tsl, configs, sets=True):
    """The shard products of one multi-rank layer pass, as group items:
    column shards write their block of the full bf16 output (the concat);
    row shards form one sum set per projection (the rank sum, into the bf16
    output), or with sets=False write their own f32 partial."""
    items, flops, nbytes = [], 0.0, 0
    for proj in configs.PROJS:
        for r in range(layer.tp):
            sh, buf, nb = pk[(r, proj)]
            if proj in ("o", "down"):
                X = bufs["attn"] if proj == "o" else bufs["act"]
                if sets:
                    items.append(dict(shard=sh, packed=buf, packed_bytes=nb, X=X[:, sh.k_off:],
                                      ldx=X.shape[1], Y=bufs["out"][proj] if r == 0 else None,
                                      ldy=layer.hidden, ydtype=tsl.BF16,
                                      sum_next=int(r < layer.tp - 1)))
                else:
                    items.append(dict(shard=sh, packed=buf, packed_bytes=nb, X=X[:, sh.k_off:],
                                      ldx=X.shape[1], Y=bufs["parts"][proj][r], ldy=layer.hidden,
                                      ydtype=tsl.F32))
                # a set writes its bf16 sum once; separate partials are f32
                yb = (2 if r == 0 else 0) if sets else 4
            else:
                Y = bufs["out"][proj]
                items.append(dict(shard=sh, packed=buf, packed_bytes=nb, X=bufs["x"],
                                  ldx=layer.hidden, Y=Y[:, sh.n_off:], ldy=Y.shape[1],
                                  ydtype=tsl.BF16))
                yb = 2
            flops += 2.0 * M * sh.k_len * sh.n_len
            nbytes += (sh.k_len * sh.n_len // 2 + (sh.k_len // 64) * sh.n_len * 4
                       + M * sh.k_len * 2 + M * sh.n_len * yb)
    return items, flops, nbytes


def make_step(layer, M, shards, packs, tsl, torch, configs, seed_base, buffers=None):
    """Buffers and the calls of one multi-rank layer pass: one
    shard_linear_group over every rank's 7 projections, the rank sums of o
    and down included (sum sets).  `buffers`, a dict, receives the inputs
    and outputs (the parity test of this configuration reads them)."""
    hq_hd = layer.n_q_heads * layer.head_dim
    kv = layer.n_kv_heads * layer.head_dim
    g = torch.Generator(device="cuda")
    g.manual_seed(seed_base)
    bf = torch.bfloat16
    bufs = {"x": torch.randn((M, layer.hidden), generator=g, device="cuda").to(bf),   # input
            "attn": torch.randn((M, hq_hd), generator=g, device="cuda").to(bf),       # o input
            "act": torch.randn((M, layer.ffn), generator=g, device="cuda").to(bf),    # down input
            "out": {"q": torch.empty((M, hq_hd), dtype=bf, device="cuda"),
                    "k": torch.empty((M, kv), dtype=bf, device="cuda"),
                    "v": torch.empty((M, kv), dtype=bf, device="cuda"),
                    "gate": torch.empty((M, layer.ffn), dtype=bf, device="cuda"),
                    "up": torch.empty((M, layer.ffn), dtype=bf, device="cuda"),
                    "o": torch.empty((M, layer.hidden), dtype=bf, device="cuda"),
                    "down": torch.empty((M, layer.hidden), dtype=bf, device="cuda")},
            "parts": {p: [torch.empty((M, layer.hidden), dtype=torch.float32, device="cuda")
                          for _ in range(layer.tp)] for p in ("o", "down")}}
    if buffers is not None:
        buffers.update(bufs)
    steps = []
    ws_max = 0
    for pk in packs:
        items, flops, nbytes = step_items(layer, M, pk, bufs, tsl, configs)
        arr, n = tsl._items(items)
        ws_max = max(ws_max, tsl.shard_linear_group_workspace_size(items, tsl.Q4G64, M))
        sep, _, _ = step_items(layer, M, pk, bufs, tsl, configs, sets=False)
        for it in sep:
            ws_max = max(ws_max, tsl.shard_linear_workspace_size(it["shard"], tsl.Q4G64, M))
        steps.append((arr, n, sep))
    # the copies run one after another on one stream: one workspace serves all
    wsbuf = torch.empty(max(ws_max, 256), dtype=torch.uint8, device="cuda")

    def run(step_index, stream, timers=None):
        arr, n, _ = steps[step_index % len(steps)]
        # plan (host) each step, as a runtime would for a new topology check
        tsl.plan_shards(layer.hidden, layer.n_q_heads, layer.n_kv_heads, layer.head_dim,
                        layer.ffn, layer.tp, layer.group)
        if timers is not None:
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record()
        st = tsl._lib.shard_linear_group(n, arr, tsl.Q4G64, tsl.BF16, M, wsbuf.data_ptr(),
                                         ws_max, stream)
        if st != 0:
            raise tsl.TslError(st, "shard_linear_group")
        if timers is not None:
            e1.record()
            timers.append((e0, e1))

    def run_separate(step_index, stream):
        """The same pass as 28 separate shard_linear calls and two
        combine_partials (for comparison)."""
        _, _, items = steps[step_index % len(steps)]
        for it in items:
            tsl.shard_linear(it["shard"], tsl.Q4G64, it["packed"], it["packed_bytes"], tsl.BF16,
                             it["X"], it["ldx"], M, it["ydtype"], it["Y"], it["ldy"], 0, wsbuf,
                             ws_max, stream)
        for proj in ("o", "down"):
            tsl.combine_partials(tsl.COMBINE_SUM, bufs["parts"][proj], tsl.F32, M, layer.hidden,
                                 layer.hidden, tsl.BF16, bufs["out"][proj], layer.hidden, stream)

    _, flops, nbytes = step_items(layer, M, packs[0], bufs, tsl, configs)
    return run, run_separate, flops, nbytes, len(steps[0][2])


class _KernelNodeParams(ctypes.Structure):
    """hipKernelNodeParams (hip_runtime_api.h), with room to spare."""
    _fields_ = [("blockDim", ctypes.c_uint * 3), ("extra", ctypes.c_void_p),
                ("func", ctypes.c_void_p), ("gridDim", ctypes.c_uint * 3),
                ("kernelParams", ctypes.c_void_p), ("sharedMemBytes", ctypes.c_uint),
                ("_spare", ctypes.c_char * 64)]


def _hip_runtime():
    """The HIP runtime this process already loaded (torch's, which the
    library shares)."""
    with open("/proc/self/maps") as f:
        for line in f:
            if "libamdhip64" in line:
                return ctypes.CDLL(line.split()[-1])
    raise RuntimeError("no HIP runtime loaded")


def kernel_times(torch, call, reps):
    """Each kernel of one call, timed on its own: the call is captured into a
    HIP graph on a side stream; for each of its kernel nodes, in launch
    order, a copy of the graph that keeps only that node is replayed reps
    times between two HIP events recorded on that stream.  The replays read
    what the eager calls before them left in the workspace.  Returns
    [(kernel name, grid workgroups, average microseconds)]."""
    hip = _hip_runtime()
    vp = ctypes.c_void_p
    pvp, psz = ctypes.POINTER(vp), ctypes.POINTER(ctypes.c_size_t)
    sigs = {"hipStreamBeginCapture": [vp, ctypes.c_int], "hipStreamEndCapture": [vp, pvp],
            "hipGraphGetNodes": [vp, vp, psz], "hipGraphNodeGetType": [vp, ctypes.c_void_p],
            "hipGraphNodeGetDependencies": [vp, vp, psz],
            "hipGraphKernelNodeGetParams": [vp, ctypes.c_void_p], "hipGraphClone": [pvp, vp],
            "hipGraphNodeFindInClone": [pvp, vp, vp], "hipGraphDestroyNode": [vp],
            "hipGraphInstantiate": [pvp, vp, vp, ctypes.c_char_p, ctypes.c_size_t],
            "hipGraphLaunch": [vp, vp], "hipGraphExecDestroy": [vp], "hipGraphDestroy": [vp]}
    for f, a in sigs.items():
        getattr(hip, f).restype = ctypes.c_int
        getattr(hip, f).argtypes = a
    hip.hipKernelNameRefByPtr.restype = ctypes.c_char_p
    hip.hipKernelNameRefByPtr.argtypes = [vp, vp]

    def ok(e, what):
        if e != 0:
            raise RuntimeError("%s failed (HIP error %d)" % (what, e))

    side = torch.cuda.Stream()
    sp = vp(side.cuda_stream)
    torch.cuda.synchronize()
    graph = vp()
    ok(hip.hipStreamBeginCapture(sp, 2), "hipStreamBeginCapture")  # relaxed mode
    try:
        call(side.cuda_stream)
    finally:
        ok(hip.hipStreamEndCapture(sp, ctypes.byref(graph)), "hipStreamEndCapture")
    n = ctypes.c_size_t(0)
    ok(hip.hipGraphGetNodes(graph, None, ctypes.byref(n)), "hipGraphGetNodes")
    nodes = (vp * n.value)()
    ok(hip.hipGraphGetNodes(graph, nodes, ctypes.byref(n)), "hipGraphGetNodes")
    nodes = [vp(x) for x in nodes]
    depth = {}

    def node_depth(nd):
        if nd.value not in depth:
            m = ctypes.c_size_t(0)
            ok(hip.hipGraphNodeGetDependencies(nd, None, ctypes.byref(m)), "dependencies")
            deps = (vp * max(m.value, 1))()
            if m.value:
                ok(hip.hipGraphNodeGetDependencies(nd, deps, ctypes.byref(m)), "dependencies")
            depth[nd.value] = 1 + max([node_depth(vp(d)) for d in deps[:m.value]] or [0])
        return depth[nd.value]

    kernels = []
    for nd in nodes:
        t = ctypes.c_int(-1)
        ok(hip.hipGraphNodeGetType(nd, ctypes.byref(t)), "hipGraphNodeGetType")
        if t.value == 0:  # hipGraphNodeTypeKernel
            kernels.append(nd)
    kernels.sort(key=node_depth)
    out = []
    for k in kernels:
        prm = _KernelNodeParams()
        ok(hip.hipGraphKernelNodeGetParams(k, ctypes.byref(prm)), "hipGraphKernelNodeGetParams")
        name = hip.hipKernelNameRefByPtr(prm.func, sp)
        name = name.decode(errors="replace") if name else "?"
        wgs = prm.gridDim[0] * prm.gridDim[1] * prm.gridDim[2]
        clone = vp()
        ok(hip.hipGraphClone(ctypes.byref(clone), graph), "hipGraphClone")
        for other in nodes:
            if other.value != k.value:
                c = vp()
                ok(hip.hipGraphNodeFindInClone(ctypes.byref(c), other, clone), "FindInClone")
                ok(hip.hipGraphDestroyNode(c), "hipGraphDestroyNode")
        exe = vp()
        ok(hip.hipGraphInstantiate(ctypes.byref(exe), clone, None, None, 0), "hipGraphInstantiate")
        for _ in range(2):
            ok(hip.hipGraphLaunch(exe, sp), "hipGraphLaunch")
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(side)
        for _ in range(reps):
            ok(hip.hipGraphLaunch(exe, sp), "hipGraphLaunch")
        e1.record(side)
        torch.cuda.synchronize()
        out.append((name, wgs, e0.elapsed_time(e1) * 1e3 / reps))
        ok(hip.hipGraphExecDestroy(exe), "hipGraphExecDestroy")
        ok(hip.hipGraphDestroy(clone), "hipGraphDestroy")
    ok(hip.hipGraphDestroy(graph), "hipGraphDestroy")
    return out


def short_kernel_name(name):
    """q4_gemm_kernel<256, 256, 2, 4> from a mangled or demangled name."""
    import re
    m = re.search(r"(\w+_kernel)<([\d, ]+)>", name)  # demangled
    if m:
        return "%s<%s>" % (m.group(1), m.group(2))
    # mangled: <length><identifier>, integer template arguments as Li256E
    m = re.search(r"\d+([a-z][a-z0-9_]*_kernel)(I(?:Li-?\d+E)+E)?", name)
    if not m:
        m = re.search(r"(\w+_kernel)\b", name)  # demangled, no template arguments
        return m.group(1) if m else name
    args = re.findall(r"Li(-?\d+)E", m.group(2) or "")
    return "%s<%s>" % (m.group(1), ", ".join(args)) if args else m.group(1)


def prefill_bench(args, tsl, torch, synth, configs):
    layer = configs.PRE27B
    M = layer.ms[0]
    t0 = time.perf_counter()
    # two copies of every rank's packed weights (2 x 203.5 MB), alternated
    # step by step, so that no step finds its weights in the 256 MB
    # last-level cache
    shards, packs, pack_s, pack_bytes = build_layer(layer, M, 2, tsl, torch, synth, configs)
    log("prefill: packed %d shards x %d copies (%.1f s)" % (len(packs[0]), len(packs),
                                                           time.perf_counter() - t0))
    run, run_separate, flops, nbytes, nitems = make_step(layer, M, shards, packs, tsl, torch,
                                                         configs, 31)
    stream = torch.cuda.current_stream().cuda_stream
    for i in range(args.warmup):
        run(i, stream)
    torch.cuda.synchronize()
    log("prefill: warmup done")
    timers = []
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    w0 = time.perf_counter()
    start.record()
    for i in range(args.steps):
        run(i, stream, timers)
    end.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - w0
    ms = start.elapsed_time(end) / args.steps
    k_ms = sum(e0.elapsed_time(e1) for e0, e1 in timers) / len(timers)
    log("prefill: %.3f ms/step (%d shard products in one group call, %.3f ms), wall %.2f s"
        % (ms, nitems, k_ms, wall))
    # each kernel of the call on its own (HIP events around graph replays)
    kt = kernel_times(torch, lambda s: run(0, s), 10)
    for name, wgs, us in kt:
        log("prefill: kernel %s (%d workgroups): %.1f us" % (short_kernel_name(name), wgs, us))
    # context: the same pass as separate calls
    for i in range(2):
        run_separate(i, stream)
    start.record()
    for i in range(5):
        run_separate(i, stream)
    end.record()
    torch.cuda.synchronize()
    sep_ms = start.elapsed_time(end) / 5
    log("prefill: %.3f ms/step as %d separate shard_linear calls" % (sep_ms, nitems))
    per = per_projection(layer, M, packs, tsl, torch, configs, 5)
    lib = library_gemm(M, [sh for sh, _, _ in packs[0].values()], torch)
    log("prefill: the same %d products as torch.matmul, dense f16 operands: %.1f us, %.0f TFLOP/s"
        % (len(packs[0]), lib["us"], lib["TFLOP/s"]))
    return dict(ms=ms, flops=flops, bytes=nbytes, wall=wall, kernel_ms=k_ms,
                kernel_tflops=flops / (k_ms * 1e-3) / 1e12, pack_gbs=pack_bytes / pack_s / 1e9,
                nitems=nitems, separate_ms=sep_ms, per_projection=per, library=lib,
                kernels=kt)


def library_gemm(M, shards, torch, reps=5):
    """Context for the prefill figure: the step's shard products as plain
    torch.matmul calls (the vendor GEMM library) on dense random f16
    operands of the same shapes -- no 4-bit expansion, no rank sums."""
    g = torch.Generator(device="cuda")
    g.manual_seed(5)
    xs = {}
    ops = []
    for sh in shards:
        if sh.k_len not in xs:
            xs[sh.k_len] = torch.randn((M, sh.k_len), generator=g, device="cuda",
                                       dtype=torch.float16)
        ops.append((xs[sh.k_len], torch.randn((sh.k_len, sh.n_len), generator=g, device="cuda",
                                              dtype=torch.float16)))
    flops = sum(2.0 * M * b.shape[0] * b.shape[1] for _, b in ops)
    for _ in range(2):
        for a, b in ops:
            torch.matmul(a, b)
    torch.cuda.synchronize()
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    start.record()
    for _ in range(reps):
        for a, b in ops:
            torch.matmul(a, b)
    end.record()
    torch.cuda.synchronize()
    us = start.elapsed_time(end) * 1e3 / reps
    del xs, ops
    return {"what": "torch.matmul of the same shard products, dense random f16 operands",
            "us": round(us, 1), "TFLOP/s": round(flops / us / 1e6, 1)}


def per_projection(layer, M, packs, tsl, torch, configs, reps):
    """Rank 0's seven projections of a 4-bit layer, each as its own
    shard_linear call into an f32 output, HIP-graph replay over the weight
    copies in `packs`: time, TFLOP/s, GB/s of algorithmic bytes and the
    fraction of the product's own roofline."""
    g = torch.Generator(device="cuda")
    g.manual_seed(77 + M)
    out = []
    for proj in configs.PROJS:
        sh = packs[0][(0, proj)][0]
        X = torch.randn((M, sh.k_len), generator=g, device="cuda").to(torch.bfloat16)
        Y = torch.empty((M, sh.n_len), dtype=torch.float32, device="cuda")
        ws = tsl.shard_linear_workspace_size(sh, tsl.Q4G64, M)
        wsb = torch.empty(max(ws, 256), dtype=torch.uint8, device="cuda")

        def run(cp, stream):
            _, buf, nb = packs[cp][(0, proj)]
            tsl.shard_linear(sh, tsl.Q4G64, buf, nb, tsl.BF16, X, sh.k_len, M, tsl.F32, Y,
                             sh.n_len, 0, wsb, ws, stream)
        us = graph_time(torch, run, len(packs), reps)
        flops = 2.0 * M * sh.k_len * sh.n_len
        nbytes = (sh.k_len * sh.n_len // 2 + (sh.k_len // 64) * sh.n_len * 4 + M * sh.k_len * 2
                  + M * sh.n_len * 4)
        t_roof = max(flops / (PEAK_MFMA_F16 * 1e12), nbytes / (PEAK_HBM * 1e9)) * 1e6
        out.append({"proj": proj, "K": sh.k_len, "N": sh.n_len, "us": round(us, 2),
                    "flops": flops, "bytes": nbytes,
                    "TFLOP/s": round(flops / us / 1e6, 1),
                    "GB/s": round(nbytes / (us * 1e-6) / 1e9, 1),
                    "bound": "mfma" if flops / (PEAK_MFMA_F16 * 1e12) > nbytes / (PEAK_HBM * 1e9)
                    else "hbm", "roofline_frac": round(t_roof / us, 4)})
    log("%s M=%d rank 0 per projection: %s" % (layer.name, M, ", ".join(
        "%s %.1f us" % (r["proj"], r["us"]) for r in out)))
    return out


def collectives_bench(tsl, torch):
    """Every rank's result of the three collectives over the prefill
    layer's row-layer partials (4 ranks x [2048, 5120] fp32 -> bf16, or the
    bf16 concat for the gather), GB/s of algorithmic bytes."""
    R, M, n = 4, 2048, 5120
    g = torch.Generator(device="cuda")
    g.manual_seed(5)
    parts = [torch.randn((M, n), generator=g, device="cuda") for _ in range(R)]
    shards = [p.to(torch.bfloat16) for p in parts]
    full = [torch.empty((M, n), dtype=torch.bfloat16, device="cuda") for _ in range(R)]
    blocks = torch.empty((M, n), dtype=torch.bfloat16, device="cuda")
    rs_outs = [blocks[(r * M) // R:] for r in range(R)]
    gath = [torch.empty((M, R * n), dtype=torch.bfloat16, device="cuda") for _ in range(R)]
    cases = {
        "all_reduce": (lambda: tsl.combine_to_ranks(tsl.ALL_REDUCE, parts, tsl.F32, M, n, n,
                                                    tsl.BF16, full, n),
                       R * M * n * 4 + R * M * n * 2),
        "reduce_scatter": (lambda: tsl.combine_to_ranks(tsl.REDUCE_SCATTER, parts, tsl.F32, M, n,
                                                        n, tsl.BF16, rs_outs, n),
                           R * M * n * 4 + M * n * 2),
        "all_gather": (lambda: tsl.combine_to_ranks(tsl.ALL_GATHER, shards, tsl.BF16, M, n, n,
                                                    tsl.BF16, gath, R * n),
                       R * M * n * 2 + R * R * M * n * 2),
    }
    out = {"workload": "4 ranks x [2048, 5120] row-layer partials (fp32 in, bf16 out; bf16 "
                       "shards for the gather), every rank's buffer on one GPU",
           "unit": "GB/s", "peak": PEAK_HBM}
    for name, (fn, nbytes) in cases.items():
        for _ in range(3):
            fn()
        start = torch.cuda.Event(enable_timing=True)
        end = torch.cuda.Event(enable_timing=True)
        start.record()
        for _ in range(10):
            fn()
        end.record()
        torch.cuda.synchronize()
        us = start.elapsed_time(end) * 1e3 / 10
        out[name] = {"us": round(us, 1), "GB/s": round(nbytes / (us * 1e-6) / 1e9, 1),
                     "frac": round(nbytes / (us * 1e-6) / 1e9 / PEAK_HBM, 4), "bytes": nbytes}
        log("collective %s: %.1f us, %.0f GB/s" % (name, us, out[name]["GB/s"]))
    return out


def decode_bench(args, tsl, torch, synth, configs):
    layer = configs.DEC7B
    # weights of the whole layer (all ranks) are ~131 MB: 4 copies > 256 MB MALL + L2
    copies = 4
    t0 = time.perf_counter()
    shards, packs, _, _ = build_layer(layer, 16, copies, tsl, torch, synth, configs)
    log("decode: packed %d copies (%.1f s)" % (copies, time.perf_counter() - t0))
    res = []
    for M in layer.ms:
        run, _, flops, nbytes, nitems = make_step(layer, M, shards, packs, tsl, torch, configs,
                                                  41 + M)
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            for c in range(copies):  # eager warmup of every launch
                run(c, side.cuda_stream)
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            cap = torch.cuda.current_stream().cuda_stream
            for c in range(copies):
                run(c, cap)
        for _ in range(3):
            graph.replay()
        torch.cuda.synchronize()
        reps = max(5, args.steps)
        start = torch.cuda.Event(enable_timing=True)
        end = torch.cuda.Event(enable_timing=True)
        start.record()
        for _ in range(reps):
            graph.replay()
        end.record()
        torch.cuda.synchronize()
        us = start.elapsed_time(end) * 1e3 / (reps * copies)
        gbs = nbytes / (us * 1e-6) / 1e9
        res.append({"M": M, "us_per_step": round(us, 2), "GB/s": round(gbs, 1),
                    "frac": round(gbs / PEAK_HBM, 4), "shard_products_per_step": nitems,
                    "bytes_per_step": nbytes, "flops_per_step": flops})
        log("decode M=%d: %.1f us/step, %.0f GB/s" % (M, us, gbs))
        del graph
        if M == 1:
            res[-1]["rank0_per_projection"] = per_projection(layer, M, packs, tsl, torch,
                                                             configs, max(5, args.steps))
    return res


def vocab_bench(args, tsl, torch, synth, configs):
    """vocab7b: the 4-bit LM head at decode (every rank's vocabulary slice in
    one grouped call, writing its slice of the full f32 logits), HIP-graph
    replay over 2 weight copies; and the embedding lookup of 2048 ids
    (every rank's masked lookup into f32 partials, then their sum into bf16
    rows), GB/s of algorithmic bytes."""
    c = configs.VOCAB7B
    t0 = time.perf_counter()
    plan = tsl.plan_vocab(c.vocab, c.hidden, c.tp, 64)
    heads, embeds = plan[1::2], plan[0::2]
    seed = lambda tt: synth.seed_of(c.index, 1, tt)
    codes = torch.from_numpy(synth.q4_codes(seed(synth.T_CODES), (c.hidden, c.vocab))).cuda()
    sc = torch.from_numpy(synth.uniform_bf16(seed(synth.T_SCALES), (c.hidden // 64, c.vocab),
                                             c.scale_lo, c.scale_hi).view("int16")).cuda()
    bi = torch.from_numpy(synth.normal_bf16(seed(synth.T_BIASES), (c.hidden // 64, c.vocab),
                                            c.bias_std).view("int16")).cuda()
    copies = 2
    packs = []
    for _ in range(copies):
        row = []
        for sh in heads:
            nb = tsl.pack_shard_size(sh, tsl.Q4G64)
            buf = torch.empty(nb, dtype=torch.uint8, device="cuda")
            tsl.pack_shard(sh, tsl.Q4G64, codes, c.vocab, 1, sc, bi, c.vocab, 1, buf, nb)
            row.append((buf, nb))
        packs.append(row)
    del codes, sc, bi
    torch.cuda.synchronize()
    log("vocab: packed the LM head x%d (%.1f s)" % (copies, time.perf_counter() - t0))
    wbytes = c.hidden * c.vocab // 2 + (c.hidden // 64) * c.vocab * 4
    out = {"workload": "vocab7b: vocabulary 152064 split over tp=4 at hidden 3584; LM head 4-bit "
                       "g64 -> f32 logits (all 4 vocabulary slices in one shard_linear_group "
                       "call, HIP-graph replay over 2 weight copies); embedding bf16 table, 2048 "
                       "uniform ids, 4 masked lookups into f32 partials + their sum into bf16",
           "unit": "GB/s", "peak": PEAK_HBM, "lm_head": []}
    for M in c.head_ms:
        X = torch.from_numpy(synth.normal_bf16(seed(synth.T_X) + M, (M, c.hidden))
                             .view("int16")).cuda().view(torch.bfloat16)
        logits = torch.empty((M, c.vocab), dtype=torch.float32, device="cuda")
        groups = []
        for cp in range(copies):
            items = [dict(shard=sh, packed=buf, packed_bytes=nb, X=X, ldx=c.hidden,
                          Y=logits[:, sh.n_off:], ldy=c.vocab)
                     for sh, (buf, nb) in zip(heads, packs[cp])]
            arr = tsl._items(items)
            ws = tsl.shard_linear_group_workspace_size(items, tsl.Q4G64, M)
            wsb = torch.empty(max(ws, 256), dtype=torch.uint8, device="cuda")
            groups.append((arr, wsb, ws))

        def run(cp, stream):
            (arr, n), wsb, ws = groups[cp]
            tsl._check(tsl._lib.shard_linear_group(n, arr, tsl.Q4G64, tsl.BF16, M, wsb.data_ptr(),
                                                   ws, stream), "shard_linear_group")
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            for cp in range(copies):
                run(cp, side.cuda_stream)
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            cap = torch.cuda.current_stream().cuda_stream
            for cp in range(copies):
                run(cp, cap)
        for _ in range(3):
            graph.replay()
        torch.cuda.synchronize()
        reps = max(5, args.steps)
        start = torch.cuda.Event(enable_timing=True)
        end = torch.cuda.Event(enable_timing=True)
        start.record()
        for _ in range(reps):
            graph.replay()
        end.record()
        torch.cuda.synchronize()
        us = start.elapsed_time(end) * 1e3 / (reps * copies)
        nbytes = wbytes + M * c.hidden * 2 + M * c.vocab * 4
        gbs = nbytes / (us * 1e-6) / 1e9
        out["lm_head"].append({"M": M, "us_per_step": round(us, 2), "GB/s": round(gbs, 1),
                               "frac": round(gbs / PEAK_HBM, 4), "bytes_per_step": nbytes})
        log("vocab LM head M=%d: %.1f us/step, %.0f GB/s" % (M, us, gbs))
        del graph
    del packs
    # embedding lookup
    E = torch.from_numpy(synth.normal_bf16(synth.seed_of(c.index, 0, synth.T_W),
                                           (c.vocab, c.hidden), c.e_std).view("int16")).cuda()
    tokens = torch.from_numpy(synth.token_ids(synth.seed_of(c.index, 0, synth.T_X), c.lookup_m,
                                              c.vocab)).cuda()
    M, H = c.lookup_m, c.hidden
    parts = [torch.empty((M, H), dtype=torch.float32, device="cuda") for _ in embeds]
    Y = torch.empty((M, H), dtype=torch.bfloat16, device="cuda")

    def lookup():
        for sh, P in zip(embeds, parts):
            tsl.embed_lookup(sh, tsl.BF16, E[sh.k_off:], H, tokens, M, tsl.F32, P, H)
        tsl.combine_partials(tsl.COMBINE_SUM, parts, tsl.F32, M, H, H, tsl.BF16, Y, H)
    for _ in range(3):
        lookup()
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    start.record()
    for _ in range(10):
        lookup()
    end.record()
    torch.cuda.synchronize()
    us = start.elapsed_time(end) * 1e3 / 10
    R = len(embeds)
    nbytes = M * 4 + M * H * 2 + R * M * H * 4 + R * M * H * 4 + M * H * 2
    gbs = nbytes / (us * 1e-6) / 1e9
    out["embed"] = {"M": M, "us_per_step": round(us, 1), "GB/s": round(gbs, 1),
                    "frac": round(gbs / PEAK_HBM, 4), "bytes_per_step": nbytes,
                    "bytes": "ids + owned table rows + 4 f32 partials written and read + bf16 rows"}
    log("vocab embedding M=%d: %.1f us/step, %.0f GB/s" % (M, us, gbs))
    return out


def graph_time(torch, run, copies, reps):
    """Microseconds per call of run(copy, stream), replayed from a HIP graph
    over `copies` weight copies."""
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        for cp in range(copies):
            run(cp, side.cuda_stream)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        cap = torch.cuda.current_stream().cuda_stream
        for cp in range(copies):
            run(cp, cap)
    for _ in range(3):
        graph.replay()
    torch.cuda.synchronize()
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    start.record()
    for _ in range(reps):
        graph.replay()
    end.record()
    torch.cuda.synchronize()
    return start.elapsed_time(end) * 1e3 / (reps * copies)


def dense_bench(args, tsl, torch, configs):
    """The dense workloads, every rank of one layer per step as one
    shard_linear_group call (rank sums of the row shards as sum sets,
    column shards concat-free, replicated K/V into per-rank buffers): llama2k
    (bf16, tp=4) at M = 1, 16, 256, gqa8 (bf16, tp=8, K/V replicated) at
    M = 64, 512, and the wiki example (fp32, 1024 -> 2048 on 2 ranks, column
    and row) at M = 32.  Weights N(0, 0.02^2) from torch's seeded generator,
    HIP-graph replay over enough copies (at most 8) to exceed the 256 MB
    last-level cache -- the 8 MB example stays cache-resident; each row
    against its own roofline max(flops / 2.5 PF (fp32:
    157.3 TF), bytes / 8 TB/s)."""
    rows = []
    g = torch.Generator(device="cuda")
    cases = [(configs.LLAMA2K, tsl.BF16), (configs.GQA8, tsl.BF16), (configs.WORKED, tsl.F32)]
    for layer, wd in cases:
        dt = torch.bfloat16 if wd == tsl.BF16 else torch.float32
        eb = 2 if wd == tsl.BF16 else 4
        g.manual_seed(900 + layer.index)
        if layer is configs.WORKED:
            projs = [("col", tsl.plan_linear(layer.K, layer.N, layer.tp, tsl.COLUMN)),
                     ("row", tsl.plan_linear(layer.K, layer.N, layer.tp, tsl.ROW))]
            ms = (layer.M,)
            name = "worked: fp32 X[32, 1024] x W 1024 -> 2048 on 2 ranks, column (concat) and " \
                   "row (sum) shards"
        else:
            sh = tsl.plan_shards(layer.hidden, layer.n_q_heads, layer.n_kv_heads, layer.head_dim,
                                 layer.ffn, layer.tp, layer.group)
            projs = [(p, sh[i::tsl.NPROJ]) for i, p in enumerate(configs.PROJS)]
            ms = layer.ms
            name = "%s: every rank of one tp=%d layer (hidden %d, ffn %d, %d Q / %d KV heads of " \
                   "%d), bf16" % (layer.name, layer.tp, layer.hidden, layer.ffn, layer.n_q_heads,
                                  layer.n_kv_heads, layer.head_dim)
        full = {}
        wbytes = 0
        for p, shards in projs:
            s0 = shards[0]
            full[p] = (torch.randn((s0.K, s0.N), generator=g, device="cuda") * 0.02).to(dt)
            wbytes += sum(s.k_len * s.n_len * eb for s in shards)
        copies = min(8, max(2, int(-(-600e6 // max(wbytes, 1)))))
        packs = []
        for _ in range(copies):
            pk = {}
            for p, shards in projs:
                for s in shards:
                    nb = tsl.pack_shard_size(s, wd)
                    buf = torch.empty(nb, dtype=torch.uint8, device="cuda")
                    tsl.pack_shard(s, wd, full[p], s.N, 1, None, None, 0, 0, buf, nb)
                    pk[p, s.rank] = (buf, nb)
            packs.append(pk)
        del full
        for M in ms:
            X = {p: torch.randn((M, sh[0].K), generator=g, device="cuda").to(dt)
                 for p, sh in projs}
            outs, items_per_copy = {}, []
            flops, nbytes = 0.0, 0
            for cp in range(copies):
                items = []
                for p, shards in projs:
                    s0 = shards[0]
                    if s0.strategy == tsl.ROW:  # one sum set into the full f32/bf16 output
                        Y = outs.setdefault(p, torch.empty((M, s0.N), dtype=dt, device="cuda"))
                        for r, s in enumerate(shards):
                            buf, nb = packs[cp][p, s.rank]
                            items.append(dict(shard=s, packed=buf, packed_bytes=nb,
                                              X=X[p][:, s.k_off:], ldx=s.K,
                                              Y=Y if r == 0 else None, ldy=s.N,
                                              ydtype=wd, sum_next=int(r < len(shards) - 1)))
                    elif s0.strategy == tsl.COLUMN:  # concat-free into the full output
                        Y = outs.setdefault(p, torch.empty((M, s0.N), dtype=dt, device="cuda"))
                        for s in shards:
                            buf, nb = packs[cp][p, s.rank]
                            items.append(dict(shard=s, packed=buf, packed_bytes=nb, X=X[p],
                                              ldx=s.K, Y=Y[:, s.n_off:], ldy=s.N, ydtype=wd))
                    else:  # replicated: every rank its own full output
                        for s in shards:
                            Y = outs.setdefault((p, s.rank), torch.empty((M, s.N), dtype=dt,
                                                                         device="cuda"))
                            buf, nb = packs[cp][p, s.rank]
                            items.append(dict(shard=s, packed=buf, packed_bytes=nb, X=X[p],
                                              ldx=s.K, Y=Y, ldy=s.N, ydtype=wd))
                    if cp == 0:
                        for s in shards:
                            flops += 2.0 * M * s.k_len * s.n_len
                            nbytes += s.k_len * s.n_len * eb + M * s.k_len * eb
                        nbytes += M * s0.N * eb * (1 if s0.strategy != tsl.REPLICATED
                                                   else len(shards))
                ws = tsl.shard_linear_group_workspace_size(items, wd, M)
                items_per_copy.append((tsl._items(items),
                                       torch.empty(max(ws, 256), dtype=torch.uint8,
                                                   device="cuda"), ws))

            def run(cp, stream):
                (arr, n), wsb, ws = items_per_copy[cp]
                tsl._check(tsl._lib.shard_linear_group(n, arr, wd, wd, M, wsb.data_ptr(), ws,
                                                       stream), "shard_linear_group")
            us = graph_time(torch, run, copies, max(5, args.steps))
            peak = PEAK_MFMA_F16 if wd == tsl.BF16 else 157.3
            t_roof = max(flops / (peak * 1e12), nbytes / (PEAK_HBM * 1e9)) * 1e6
            rows.append({"workload": name, "M": M, "us_per_step": round(us, 2),
                         "TFLOP/s": round(flops / us / 1e6, 2),
                         "GB/s": round(nbytes / (us * 1e-6) / 1e9, 1),
                         "bound": "mfma" if flops / (peak * 1e12) > nbytes / (PEAK_HBM * 1e9)
                         else "hbm", "roofline_frac": round(t_roof / us, 4),
                         "flops": flops, "bytes": nbytes, "weight_copies": copies})
            log("dense %s M=%d: %.1f us/step, %.1f TFLOP/s, %.0f GB/s, %.0f%% of roofline"
                % (layer.name, M, us, flops / us / 1e6, nbytes / (us * 1e-6) / 1e9,
                   100 * t_roof / us))
        del packs
    return rows


def moe_bench(args, tsl, torch, synth, configs):
    """moe30b, expert parallel, every rank of the layer on one GPU: per
    step every held expert's gate and up products in one
    shard_linear_group call, the down products in another (each product
    reads its rows -- the tokens, or the per-slot down inputs, routed to
    its expert -- through moe_dispatch's row index, with no gather pass),
    each rank's moe_combine and the sum of the rank outputs.
    Routing (moe_dispatch) is host work on the router's output and is done
    before the timed region.  T = 2048: TFLOP/s of the expert products;
    T = 16: GB/s of the weights of the experts the step touches, HIP-graph
    replay over 2 weight copies."""
    import numpy as np
    c = configs.MOE30B
    t0 = time.perf_counter()
    plan = tsl.plan_experts(c.n_experts, c.hidden, c.expert_ffn, c.tp, tsl.MOE_EXPERT_PARALLEL, 64)
    by_expert = {x.expert: x for x in plan}
    copies = 2
    packs = [dict() for _ in range(copies)]
    for x in plan:
        for pi, p in enumerate(("gate", "up", "down")):
            sh = getattr(x, p)
            K, N = sh.K, sh.N
            sd = synth.seed_of(c.index, 10 * x.expert + pi, 0)
            codes = torch.from_numpy(synth.q4_codes(sd + synth.T_CODES, (K, N))).cuda()
            sc = torch.from_numpy(synth.uniform_bf16(sd + synth.T_SCALES, (K // 64, N), c.scale_lo,
                                                     c.scale_hi).view("int16")).cuda()
            bi = torch.from_numpy(synth.normal_bf16(sd + synth.T_BIASES, (K // 64, N),
                                                    c.bias_std).view("int16")).cuda()
            nb = tsl.pack_shard_size(sh, tsl.Q4G64)
            for cp in range(copies):
                buf = torch.empty(nb, dtype=torch.uint8, device="cuda")
                tsl.pack_shard(sh, tsl.Q4G64, codes, N, 1, sc, bi, N, 1, buf, nb)
                packs[cp][x.expert, p] = (buf, nb)
    torch.cuda.synchronize()
    log("moe: packed %d experts x3 x%d (%.1f s)" % (c.n_experts, copies, time.perf_counter() - t0))
    wbytes = lambda K, N: K * N // 2 + (K // 64) * N * 4
    out = {"workload": "moe30b: 128 experts of width 768, top-8, hidden 2048, expert parallel "
                       "over tp=4 (32 experts per rank), 4-bit g64, all ranks on one GPU; per "
                       "step: the gate+up and the down products of every held expert (two "
                       "shard_linear_group calls, rows read through the routing's row "
                       "index), 4 moe_combine and the rank sum",
           "rows": []}
    for T in c.tokens:
        xs = synth.seed_of(c.index, 0, synth.T_X) + T
        topk, w = synth.router(xs + 2, T, c.top_k, c.n_experts)
        k = c.top_k
        X = torch.from_numpy(synth.normal_bf16(xs, (T, c.hidden)).view("int16")).cuda() \
            .view(torch.bfloat16)
        H = torch.from_numpy(synth.normal_bf16(xs + 1, (T * k, c.expert_ffn)).view("int16")) \
            .cuda().view(torch.bfloat16)
        dw = torch.from_numpy(w.ravel()).cuda()
        ranks, tok_idx, slot_idx = [], [], []
        base = 0
        for r in range(c.tp):
            held = [x.expert for x in plan if x.rank == r]
            off, row_slot, slot_row = tsl.moe_dispatch(topk, c.n_experts, held)
            ranks.append((held, off + base, torch.from_numpy(slot_row).cuda(), base,
                          int(off[-1])))
            tok_idx.append(row_slot // k)
            slot_idx.append(row_slot)
            base += int(off[-1])
        R = base
        d_tok = torch.from_numpy(np.concatenate(tok_idx).astype(np.int32)).cuda()
        d_slot = torch.from_numpy(np.concatenate(slot_idx).astype(np.int32)).cuda()
        G = torch.empty((R, c.expert_ffn), dtype=torch.bfloat16, device="cuda")
        U = torch.empty((R, c.expert_ffn), dtype=torch.bfloat16, device="cuda")
        P = torch.empty((R, c.hidden), dtype=torch.float32, device="cuda")
        Yr = [torch.empty((T, c.hidden), dtype=torch.float32, device="cuda") for _ in ranks]
        Y = torch.empty((T, c.hidden), dtype=torch.bfloat16, device="cuda")
        calls, flops, touched = [], 0, 0
        counts = np.concatenate([np.diff(o) for _, o, _, _, _ in ranks])
        Mmax = int(counts.max())
        for cp in range(copies):
            gu, dn = [], []
            for held, off, _, _, _ in ranks:
                for i, e in enumerate(held):
                    rows = int(off[i + 1] - off[i])
                    if rows == 0:
                        continue
                    o = int(off[i])
                    x = by_expert[e]
                    for p, Yb in (("gate", G), ("up", U)):
                        buf, nb = packs[cp][e, p]
                        gu.append(dict(shard=getattr(x, p), packed=buf, packed_bytes=nb,
                                       X=X, ldx=c.hidden, Y=Yb[o:], ldy=c.expert_ffn,
                                       ydtype=tsl.BF16, rows=rows, row_index=d_tok[o:],
                                       x_rows=T))
                    buf, nb = packs[cp][e, "down"]
                    dn.append(dict(shard=x.down, packed=buf, packed_bytes=nb, X=H,
                                   ldx=c.expert_ffn, Y=P[o:], ldy=c.hidden, rows=rows,
                                   row_index=d_slot[o:], x_rows=T * k))
                    if cp == 0:
                        flops += 6 * rows * c.hidden * c.expert_ffn
                        touched += 3 * wbytes(c.hidden, c.expert_ffn)
            groups = []
            for items in (gu, dn):
                arr = tsl._items(items)
                ws = tsl.shard_linear_group_workspace_size(items, tsl.Q4G64, Mmax)
                groups.append((arr, torch.empty(max(ws, 256), dtype=torch.uint8, device="cuda"),
                               ws))
            calls.append(groups)

        def step(cp, stream):
            for (arr, n), wsb, ws in calls[cp]:
                tsl._check(tsl._lib.shard_linear_group(n, arr, tsl.Q4G64, tsl.BF16, Mmax,
                                                       wsb.data_ptr(), ws, stream),
                           "shard_linear_group")
            for (held, off, d_sr, b, rr), Yo in zip(ranks, Yr):
                tsl.moe_combine(P[b:], c.hidden, rr, d_sr, dw, T, k, c.hidden, tsl.F32, Yo,
                                c.hidden, stream)
            tsl.combine_partials(tsl.COMBINE_SUM, Yr, tsl.F32, T, c.hidden, c.hidden, tsl.BF16,
                                 Y, c.hidden, stream)
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            for cp in range(copies):
                step(cp, side.cuda_stream)
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            cap = torch.cuda.current_stream().cuda_stream
            for cp in range(copies):
                step(cp, cap)
        for _ in range(3):
            graph.replay()
        torch.cuda.synchronize()
        reps = max(5, args.steps)
        start = torch.cuda.Event(enable_timing=True)
        end = torch.cuda.Event(enable_timing=True)
        start.record()
        for _ in range(reps):
            graph.replay()
        end.record()
        torch.cuda.synchronize()
        us = start.elapsed_time(end) * 1e3 / (reps * copies)
        row = {"T": T, "us_per_step": round(us, 1), "TFLOP/s": round(flops / us / 1e6, 1),
               "mfma_frac": round(flops / us / 1e6 / PEAK_MFMA_F16, 4),
               "touched_weight_GB/s": round(touched / (us * 1e-6) / 1e9, 1),
               "hbm_frac": round(touched / (us * 1e-6) / 1e9 / PEAK_HBM, 4),
               "expert_rows": R, "experts_touched": int((counts > 0).sum()),
               "flops_per_step": flops, "weight_bytes_touched": touched}
        out["rows"].append(row)
        log("moe T=%d: %.1f us/step, %.1f TFLOP/s, %.0f GB/s of touched weights"
            % (T, us, row["TFLOP/s"], row["touched_weight_GB/s"]))
        del graph
    return out


def cpu_baseline(synth, configs):
    """The oracle, as it stands, on a bounded sample of the prefill workload:
    the layer's shards in plan order (rank 0's q, k, v, o, gate, up, down,
    then rank 1's, ...), each dequantised and multiplied over all 2048
    token rows, until about 10 s of host work have been spent."""
    import oracle
    layer = configs.PRE27B
    M = layer.ms[0]
    plan = oracle.plan(layer.hidden, layer.n_q_heads, layer.n_kv_heads, layer.head_dim,
                       layer.ffn, layer.tp, layer.group)
    flops, t, done = 0.0, 0.0, []
    for r in range(layer.tp):
        for pi, proj in enumerate(configs.PROJS):
            if t >= 10.0:
                break
            sh = oracle.spec(plan, r, proj)
            seed = lambda tt: synth.seed_of(layer.index, pi, tt)
            K, N = sh["K"], sh["N"]
            codes = synth.q4_codes(seed(synth.T_CODES), (K, N))
            sc = synth.uniform_bf16(seed(synth.T_SCALES), (K // 64, N), layer.scale_lo,
                                    layer.scale_hi)
            bi = synth.normal_bf16(seed(synth.T_BIASES), (K // 64, N), layer.bias_std)
            X = oracle.bf16_to_f64(synth.normal_bf16(seed(synth.T_X), (M, K)))
            Xr = oracle.slice_input(X, sh)
            t0 = time.perf_counter()
            W = oracle.dequant_q4(*oracle.slice_q4(codes, sc, bi, sh))
            oracle.gemm(Xr, W)
            t += time.perf_counter() - t0
            flops += 2.0 * M * sh["k_len"] * sh["n_len"]
            done.append("%d:%s" % (r, proj))
    threads = int(os.environ.get("OMP_NUM_THREADS", "0")) or os.cpu_count()
    return {"value": round(flops / t / 1e12, 5), "unit": "TFLOP/s", "cores": threads,
            "kind": "oracle",
            "sample": "%d of the prefill workload's 28 shards (%s; 4-bit g64, all %d token "
                      "rows): dequantise + naive fp64 GEMM, %.1f s" % (len(done), " ".join(done),
                                                                         M, t)}


def environment(torch):
    """The device and its current clock levels, read from the driver's sysfs
    files for its PCI address (best effort; no helper program is started, so
    nothing here forks or execs once the GPU is in use)."""
    props = torch.cuda.get_device_properties(0)
    env = {"device": props.name, "compute_units": props.multi_processor_count,
           "memory_GB": round(props.total_memory / 2**30, 1)}
    try:
        base = "/sys/bus/pci/devices/%04x:%02x:%02x.0" % (
            props.pci_domain_id, props.pci_bus_id, props.pci_device_id)
        clocks = {}
        for name in ("pp_dpm_sclk", "pp_dpm_mclk"):
            with open(os.path.join(base, name)) as f:
                cur = [ln.split(":", 1)[1].strip(" *\n") for ln in f if ln.rstrip().endswith("*")]
            clocks[name[-4:]] = cur[0] if cur else None
        env["clocks_at_start"] = clocks
    except Exception as e:  # the clocks are context only
        env["clocks_at_start"] = "unavailable (%s)" % type(e).__name__
    return env


def results_rows(line, layer_pre, layer_dec):
    """Per-row records in the survey's report format: one per measured row
    (cfg, row, M, shard shape, flops, bytes, time, rates, bound, fraction of
    the row's own roofline)."""
    rows = []

    def rec(cfg, row, M, K, N, dtype, flops, nbytes, us, bound=None):
        t_roof = max(flops / (PEAK_MFMA_F16 * 1e12), nbytes / (PEAK_HBM * 1e9)) * 1e6
        b = bound or ("mfma" if flops / (PEAK_MFMA_F16 * 1e12) > nbytes / (PEAK_HBM * 1e9)
                      else "hbm")
        rows.append({"cfg": cfg, "row": row, "M": M, "K_s": K, "N_s": N, "dtype": dtype,
                     "flops": flops, "bytes": nbytes, "t_gpu_us": round(us, 2),
                     "tflops": round(flops / us / 1e6, 2),
                     "gbs": round(nbytes / us / 1e3, 1) if nbytes else None, "bound": b,
                     "pct_roofline": round(100 * t_roof / us, 2)})

    pre = line["roofline"]
    rec("C3", "pre27b step, one grouped call", layer_pre.ms[0], None, None, "q4g64 x bf16",
        line["step_flops"], line["step_bytes"], line["ms_per_step"] * 1e3, "mfma")
    rec("C3", "pre27b fused GEMM launch", layer_pre.ms[0], None, None, "q4g64 x bf16",
        line["step_flops"], pre["traffic"] or 0, pre["avg_launch_us"], "mfma")
    for r in line["prefill_rank0_per_projection"]:
        rec("C3", "rank 0 %s" % r["proj"], layer_pre.ms[0], r["K"], r["N"], "q4g64 x bf16",
            r["flops"], r["bytes"], r["us"])
    for d in line["decode"]["rows"]:
        rec("C2", "dec7b step, one grouped call", d["M"], None, None, "q4g64 x bf16",
            d["flops_per_step"], d["bytes_per_step"], d["us_per_step"], "hbm")
        for r in d.get("rank0_per_projection", []):
            rec("C2", "rank 0 %s" % r["proj"], d["M"], r["K"], r["N"], "q4g64 x bf16",
                r["flops"], r["bytes"], r["us"])
    for r in line["dense"] or []:
        cfg = {"llama2k": "C1", "gqa8": "C4", "worked": "C0"}.get(r["workload"].split(":")[0])
        rec(cfg, r["workload"].split(":")[0] + " step, one grouped call", r["M"], None, None,
            "bf16" if cfg != "C0" else "f32", r["flops"], r["bytes"], r["us_per_step"], r["bound"])
    return rows


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawTextHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-decode", action="store_true")
    ap.add_argument("--copy-probe", type=int, default=0, metavar="MIB",
                    help="first run a plain device copy of MIB MiB five times (the reference "
                         "for scaling HBM byte counters)")
    ap.add_argument("--only", choices=("all", "decode", "moe", "dense"), default="all",
                    help="profiling aid: 'decode' runs the dec7b decode rows alone (value: GB/s "
                         "at M = 1), 'moe' the moe30b rows (value: TFLOP/s at T = 2048), 'dense' "
                         "the bf16 / fp32 layer rows (value: gqa8 M = 512 TFLOP/s), and prints "
                         "them as the line")
    ap.add_argument("--results", metavar="PATH",
                    help="also append one record per measured row to PATH (JSON lines)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: this library runs every rank's shard on a single "
              "MI355X and has no multi-GPU path; run with --gpus 1", file=sys.stderr)
        sys.exit(2)

    import torch
    from tensor_sharded_linear_plan_amd import binding as tsl
    from tensor_sharded_linear_plan_amd import configs, synth
    torch.cuda.set_device(0)
    log("device:", torch.cuda.get_device_name(0))
    if args.copy_probe:
        n = args.copy_probe << 20
        src = torch.ones(n, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        log("copy probe: %d MiB x 5" % args.copy_probe)
        del src, dst

    if args.only == "decode":
        dec = decode_bench(args, tsl, torch, synth, configs)
        print(json.dumps({"metric": "dec7b decode step, 4-bit shard GEMVs of every rank",
                          "value": dec[0]["GB/s"], "unit": "GB/s", "n_gpus": 1,
                          "steps": args.steps, "warmup": args.warmup,
                          "higher_is_better": True, "dtype": "bf16", "data": "synthetic",
                          "rows": dec}), flush=True)
        return
    if args.only == "dense":
        dense = dense_bench(args, tsl, torch, configs)
        g = [r for r in dense if r["workload"].startswith("gqa8") and r["M"] == 512]
        print(json.dumps({"metric": "dense bf16 / fp32 layer steps, every rank",
                          "value": g[0]["TFLOP/s"] if g else None, "unit": "TFLOP/s",
                          "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
                          "higher_is_better": True, "dtype": "bf16", "data": "synthetic",
                          "dense": dense}), flush=True)
        return
    if args.only == "moe":
        moe = moe_bench(args, tsl, torch, synth, configs)
        print(json.dumps({"metric": "moe30b step, 4-bit expert products of every rank",
                          "value": moe["rows"][0]["TFLOP/s"], "unit": "TFLOP/s", "n_gpus": 1,
                          "steps": args.steps, "warmup": args.warmup,
                          "higher_is_better": True, "dtype": "f16", "data": "synthetic",
                          "moe": moe}), flush=True)
        return
    pre = prefill_bench(args, tsl, torch, synth, configs)
    dec = [] if args.no_decode else decode_bench(args, tsl, torch, synth, configs)
    coll = None if args.no_decode else collectives_bench(tsl, torch)
    voc = None if args.no_decode else vocab_bench(args, tsl, torch, synth, configs)
    moe = None if args.no_decode else moe_bench(args, tsl, torch, synth, configs)
    dense = None if args.no_decode else dense_bench(args, tsl, torch, configs)
    cpu = None
    if not args.no_cpu_baseline:
        sys.path.insert(0, os.path.dirname(os.path.abspath(__file__)))
        cpu = cpu_baseline(synth, configs)
        log("cpu baseline:", cpu["sample"])

    value = pre["flops"] / (pre["ms"] * 1e-3) / 1e12
    # the dominant kernel: the longest launch of the grouped call; its time
    # inside the call is the call's (HIP events over the timed steps) less
    # the other kernels' (each replayed on its own), launch gaps included
    dom_full, _, dom_alone_us = max(pre["kernels"], key=lambda k: k[2])
    dom_name = short_kernel_name(dom_full)
    dom_us = pre["kernel_ms"] * 1e3 - sum(u for n, _, u in pre["kernels"] if n != dom_full)
    dom_tflops = pre["flops"] / (dom_us * 1e-6) / 1e12
    layer = configs.PRE27B
    line = {
        "metric": METRIC, "value": round(value, 2), "unit": "TFLOP/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(pre["ms"], 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f16",
        "data": "synthetic",
        "config": {"workload": "pre27b: every rank of one tp=4 27B-class layer on one GPU "
                               "(hidden 5120, ffn 17408, 64 Q / 8 KV heads of 128), 4-bit "
                               "affine g64 weights, bf16 activations, M=2048 prefill tokens; "
                               "%d shard GEMMs (f16 MFMA, f32 accumulate) and the rank sums of "
                               "o and down, all in one shard_linear_group call" % pre["nitems"],
                   "tp": layer.tp, "M": layer.ms[0], "weights": "q4g64", "activations": "bf16",
                   "parallelism": "tp4 in-process on 1 GPU"},
        "roofline": {"bound": "mfma", "achieved": round(dom_tflops, 2),
                     "peak": PEAK_MFMA_F16, "unit": "TFLOP/s",
                     "frac": round(dom_tflops / PEAK_MFMA_F16, 4),
                     "traffic": measured_traffic(dom_name),
                     "kernel": dom_name,
                     "what": "the fused 4-bit GEMM launch of the step's shard_linear_group "
                             "call: the 20 column-shard products and the o and down rank "
                             "sums (each as one GEMM over the ranks' k-ranges end to end), "
                             "codes expanded in registers, f16 MFMA, f32 accumulate; "
                             "algorithmic flops of the whole step / its duration in the call "
                             "(call time less the other kernels' own times)",
                     "avg_launch_us": round(dom_us, 2),
                     "alone_replay_us": round(dom_alone_us, 2),
                     "other_kernels_us": {short_kernel_name(n): round(u, 2)
                                          for n, _, u in pre["kernels"] if n != dom_full},
                     "call_us": round(pre["kernel_ms"] * 1e3, 2)},
        "cpu_baseline": cpu,
        "decode": {"workload": "dec7b: every rank of one tp=4 7B-class layer (hidden 3584, ffn "
                               "18944, 28 Q / 4 KV heads of 128), 4-bit g64, 28 shard GEMVs and "
                               "the o/down rank sums in one shard_linear_group call per step, "
                               "HIP-graph replay over 4 weight copies",
                   "unit": "GB/s", "peak": PEAK_HBM, "rows": dec},
        "collectives": coll,
        "vocab": voc,
        "moe": moe,
        "dense": dense,
        "pack_GBps": round(pre["pack_gbs"], 1),
        "prefill_separate_calls_ms_per_step": round(pre["separate_ms"], 4),
        "prefill_rank0_per_projection": pre["per_projection"],
        "prefill_library_gemm": pre["library"],
        "wall_s_timed": round(pre["wall"], 3),
        "step_flops": pre["flops"],
        "step_bytes": pre["bytes"],
        "env": environment(torch),
    }
    print(json.dumps(line), flush=True)
    if args.results:
        with open(args.results, "a") as f:
            for r in results_rows(line, configs.PRE27B, configs.DEC7B):
                f.write(json.dumps(r) + "\n")


if __name__ == "__main__":
    main()
