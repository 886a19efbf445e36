#!/usr/bin/env python3
"""One POET-X training step of a Llama-8B q_proj-shaped layer on one MI355X.

Workload: W0 4096 x 4096 bf16 ~ N(0, 0.02^2), block size b = 256 (16 blocks
per side), Neumann order k = 3, upper-triangle parameters float32 ~ N(0, 1e-3^2),
x bf16 ~ N(0, 1) of 1 x 2048 tokens, fast variant.  One step is

  poetx_cnp_fwd_save   (all 32 R and P blocks in one call; keeps Q and its
                        square for the backward)
  poetx_linear_fwd
  poetx_linear_bwd
  poetx_cnp_bwd_saved  (all 32 blocks in one call, reusing what the forward kept)

with every input already resident in HBM.  The timed region is bracketed by a
device synchronisation on both sides and measured with HIP events on the
stream the library launches on (torch's current stream).

Prints ONE JSON line.  Besides the step throughput it reports the time of every
stage (each stage re-run alone through the C ABI with the same launch
configuration), the aggregate MFMA efficiency of the block and dense GEMMs,
the roofline of the dominant kernel (the dense Wt GEMM), the float64 oracle
timed on the host cores as a baseline, and, as context outside the timed step,
the vendor library (torch.matmul, i.e. hipBLASLt) on the same dense shapes and a
plain device copy (`vendor_reference`), and the same step with every variant
of the linear (`variants`: fast, mem, all four permutations on the
activations, the original weight-centric POET with dense R and P, and mem on
the int8-stored weight).

The default line also nests, under "configs", the other Llama-shaped workloads
timed the same way (K steps after W warm-up steps): the up_proj-shaped linear in
the fast and mem variants, all 7 linears of a Llama-8B and of a Llama-13B
decoder layer (mem), and the 15280-block Cayley-Neumann launch; each with its
step time and the aggregate MFMA rate of its block and dense products
(--no-configs leaves them out).  The roofline object describes the longer of the
two dense products (the backward's, Wt read n-major) and lists both.

  --pmc-dir DIR   parse a rocprofv3 --pmc FETCH_SIZE / WRITE_SIZE run of this
                  script and record the two dense products' HBM traffic in
                  profiles/traffic_dense_gemm.json (scaled by a plain copy of
                  known size that every run performs); prints every kernel's
                  mean counter values per dispatch.
  --workload W    other workloads, same line format (the default is the one
                  the metric is quoted on): up_proj / up_proj_mem (Llama-8B
                  MLP up_proj shape, b=512, k=4, 4096 tokens), llama8b_layer
                  and llama13b_layer (all 7 linears of a decoder layer, mem
                  variant, one Cayley-Neumann forward and backward over all
                  the layer's blocks; both also time the AdamW update of all
                  the layer's q and the step with it, and the 8B line times
                  poetx_merge and the step with a merge every 400), cnp_13b (one
                  Cayley-Neumann forward + backward over the 15280 b=256
                  blocks of 40 Llama-13B layers).
"""
import argparse
import csv
import glob
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "POET-X linear fwd+bwd tokens/s + % bf16 MFMA peak, Llama-8B shapes, 1 GPU"
PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E
COPY_BYTES = 256 << 20      # plain copy every run performs (counter scale reference)
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_dense_gemm.json")
GEMM_SRC = os.path.join(ROOT, "orthogonal_equivalence_poet_amd", "csrc", "dense_gemm.hip")
COPY_KERNEL_TAG = "copyBuffer"   # the runtime's device-to-device copy kernel


def gemm_source_hash() -> str:
    with open(GEMM_SRC, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


FLUSH_BYTES = 512 << 20   # written before every "cold" launch, twice the last-level cache


def _time_cold(fn, reps, flush):
    """Mean microseconds of fn alone with the caches flushed before every launch
    (a 512 MB write between launches; only the launch itself is timed)."""
    import torch
    fn()
    tot = 0.0
    for _ in range(reps):
        flush.fill_(1)
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        a.record()
        fn()
        b.record()
        torch.cuda.synchronize()
        tot += a.elapsed_time(b)
    return tot / reps * 1e3


def _time_events(fn, reps, warm=3):
    import torch
    for _ in range(warm):
        fn()
    torch.cuda.synchronize()
    a = torch.cuda.Event(enable_timing=True)
    b = torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(reps):
        fn()
    b.record()
    torch.cuda.synchronize()
    return a.elapsed_time(b) / reps * 1e3   # microseconds per launch


def build_state(spec):
    import torch
    from orthogonal_equivalence_poet_amd import binding as B
    from orthogonal_equivalence_poet_amd import inputs as I

    inp = I.make_linear_inputs(spec)
    dev = "cuda"
    bf = torch.bfloat16

    def t(a, dt=torch.float32):
        return torch.from_numpy(a).to(dev).to(dt)

    S = {}
    S["x"] = t(inp["x"], bf)
    S["dy"] = t(inp["dy"], bf)
    S["W0"] = t(inp["W0"], bf)
    S["pi_R"] = torch.from_numpy(inp["pi_R"]).to(dev)
    S["pi_P"] = torch.from_numpy(inp["pi_P"]).to(dev)
    S["Wt"] = torch.empty_like(S["W0"])
    B.poetx_prepermute(S["W0"], S["Wt"], spec.m, spec.n, S["pi_R"], S["pi_P"])
    nR, nP, b = spec.nblk_R, spec.nblk_P, spec.b
    S["q"] = torch.cat([t(inp["q_R"]), t(inp["q_P"])]).contiguous()      # one flat batch of blocks
    if spec.q_block_norm is not None:
        # rescale every block's parameters so that its skew matrix has the given spectral norm
        Q = torch.empty((nR + nP, b, b), dtype=torch.float32, device=dev)
        B.poetx_skew_unpack(S["q"], Q, nR + nP, b)
        S["q"] *= (spec.q_block_norm / torch.linalg.matrix_norm(Q, ord=2))[:, None]
        del Q
    S["G"] = torch.empty((nR + nP, b, b), dtype=bf, device=dev)
    S["G_R"], S["G_P"] = S["G"][:nR], S["G"][nR:]
    S["dG"] = torch.empty((nR + nP, b, b), dtype=torch.float32, device=dev)
    S["dG_R"], S["dG_P"] = S["dG"][:nR], S["dG"][nR:]
    S["dq"] = torch.empty_like(S["q"])
    S["y"] = torch.empty((spec.T, spec.m), dtype=bf, device=dev)
    S["dx"] = torch.empty((spec.T, spec.n), dtype=bf, device=dev)
    var = B.POETX_MEM if spec.variant == "mem" else B.POETX_FAST
    S["desc"] = B.desc(spec.T, spec.m, spec.n, b, spec.k, B.POETX_BF16, var)
    S["saved"] = B.workspace(B.poetx_linear_saved_bytes(S["desc"])) if var == B.POETX_FAST else None
    ws = max(B.poetx_linear_fwd_workspace_bytes(S["desc"]), B.poetx_linear_bwd_workspace_bytes(S["desc"]),
             B.poetx_cnp_fwd_workspace_bytes(nR + nP, b, spec.k, B.POETX_BF16),
             B.poetx_cnp_bwd_workspace_bytes(nR + nP, b, spec.k, B.POETX_BF16))
    S["ws"] = B.workspace(ws)
    # the transform's forward keeps Q, its square and companions for the backward
    S["cnp_saved"] = B.workspace(B.poetx_cnp_saved_bytes(nR + nP, b, spec.k, B.POETX_BF16))
    return S, inp


def make_step(spec, S):
    from orthogonal_equivalence_poet_amd import binding as B
    nblk = spec.nblk_R + spec.nblk_P

    def step():
        B.poetx_cnp_fwd_save(S["q"], nblk, spec.b, spec.k, S["G"], S["cnp_saved"], S["ws"])
        B.poetx_linear_fwd(S["desc"], S["x"], S["Wt"], S["G_R"], S["G_P"], S["pi_R"], S["pi_P"], S["y"],
                           S["saved"], S["ws"])
        B.poetx_linear_bwd(S["desc"], S["dy"], S["x"], S["Wt"], S["G_R"], S["G_P"], S["pi_R"], S["pi_P"],
                           S["saved"], S["dx"], S["dG_R"], S["dG_P"], S["ws"])
        B.poetx_cnp_bwd_saved(S["q"], S["dG"], nblk, spec.b, spec.k, S["dq"], B.POETX_BF16, S["cnp_saved"],
                              S["ws"])
    return step


def stage_timings(spec, S, reps, gemm_only=False, only=None):
    """Every stage of the step alone, through the C ABI, same shapes and
    launch configurations as inside poetx_linear_fwd / _bwd (the mem variant
    repeats the input gather, the P-side block product and the dense forward in
    its backward; the fast variant keeps their outputs).  gemm_only: only the
    block, dense and block-gradient products, warm, for the nested records."""
    import torch
    from orthogonal_equivalence_poet_amd import binding as B
    T, m, n, b, k = spec.T, spec.m, spec.n, spec.b, spec.k
    bf = torch.bfloat16
    a = torch.empty((T, n), dtype=bf, device="cuda")
    h1 = torch.empty((T, n), dtype=bf, device="cuda")
    h2 = torch.empty((T, m), dtype=bf, device="cuda")
    z = torch.empty((T, m), dtype=bf, device="cuda")
    dG = torch.empty((max(m, n) // b, b, b), dtype=torch.float32, device="cuda")
    gws = B.workspace(max(B.poetx_block_grad_workspace_bytes(T, m, b, B.POETX_BF16),
                          B.poetx_block_grad_workspace_bytes(T, n, b, B.POETX_BF16)))
    nblk = spec.nblk_R + spec.nblk_P
    NT, NN = B.POETX_GEMM_NT, B.POETX_GEMM_NN

    def blk(layout, A, G, C, d):
        return lambda: B.poetx_block_apply(A, G, C, T, d, b, transpose_G=(layout == NT))

    st = {}
    # (name, fn, algorithmic flops, algorithmic HBM bytes)
    stages = [
        ("cnp_fwd", lambda: B.poetx_cnp_fwd_save(S["q"], nblk, b, k, S["G"], S["cnp_saved"], S["ws"]),
         _products(k)[0] * 2 * b ** 3 * nblk,
         4 * nblk * b * (b - 1) // 2 + 2 * nblk * b * b),
        ("perm_gather_x", lambda: B.poetx_permute(S["x"], a, T, n, None, S["pi_P"], False), 0, 2 * 2 * T * n),
        ("blk_fwd_P", blk(NT, a, S["G_P"], h1, n), 2 * T * n * b, 2 * (2 * T * n + n * b)),
    ]
    dense_fwd = ("dense_fwd", lambda: B.poetx_gemm(NT, h1, S["Wt"], h2, T, m, n, dense=True), 2 * T * m * n,
                 2 * (T * n + m * n + T * m))
    tiles = -(-T // 128) * (m // 256)
    if b == 256 and (tiles % 256 == 0 or tiles >= 1024):
        # the forward's dense product with the R-side block product folded in
        # (poetx_linear_fwd's path for b = 256 on such grids); FAST also writes h2
        keep = spec.variant != "mem"
        stages.append(("dense_fwd_fold_R",
                       lambda: B.poetx_dense_fold_r(h1, S["Wt"], S["G_R"], z, T, m, n, b, h2=h2 if keep else None),
                       2 * T * m * n + 2 * T * m * b,
                       2 * (T * n + m * n + T * m + m * b) + (2 * T * m if keep else 0)))
    else:
        stages += [dense_fwd,
                   ("blk_fwd_R", blk(NT, h2, S["G_R"], z, m), 2 * T * m * b, 2 * (2 * T * m + m * b))]
    stages += [
        ("perm_scatter_y", lambda: B.poetx_permute(z, S["y"], T, m, None, S["pi_R"], True), 0, 2 * 2 * T * m),
        ("perm_gather_dy", lambda: B.poetx_permute(S["dy"], z, T, m, None, S["pi_R"], False), 0, 2 * 2 * T * m),
        ("grad_R", lambda: B.poetx_block_grad(z, h2, dG, T, m, b, gws), 2 * T * m * b, 2 * 2 * T * m + 4 * m * b),
        ("blk_bwd_R", blk(NN, z, S["G_R"], h2, m), 2 * T * m * b, 2 * (2 * T * m + m * b)),
        ("dense_bwd", lambda: B.poetx_gemm(NN, h2, S["Wt"], h1, T, n, m, ldb=n, dense=True), 2 * T * m * n,
         2 * (T * n + m * n + T * m)),
        ("grad_P", lambda: B.poetx_block_grad(h1, a, dG, T, n, b, gws), 2 * T * n * b, 2 * 2 * T * n + 4 * n * b),
        ("blk_bwd_P", blk(NN, h1, S["G_P"], a, n), 2 * T * n * b, 2 * (2 * T * n + n * b)),
        ("perm_scatter_dx", lambda: B.poetx_permute(a, S["dx"], T, n, None, S["pi_P"], True), 0, 2 * 2 * T * n),
        ("cnp_bwd", lambda: B.poetx_cnp_bwd_saved(S["q"], S["dG"], nblk, b, k, S["dq"], B.POETX_BF16,
                                                  S["cnp_saved"], S["ws"]),
         _products(k)[1] * 2 * b ** 3 * nblk, 4 * nblk * b * b + 4 * nblk * b * (b - 1) // 2),
    ]
    if spec.variant == "mem":   # recomputed in the backward, same kernels (fast keeps a and h2)
        stages += [(nm + "_recompute", fn, fl, nb) for nm, fn, fl, nb in stages + [dense_fwd]
                   if nm in ("perm_gather_x", "blk_fwd_P", "dense_fwd")]
    # the standalone skew unpack (to bf16) and pack of the same blocks; not part of the
    # step (the fused forward unpacks on chip, the backward's pack is inside cnp_bwd)
    ntri = b * (b - 1) // 2
    Qb = torch.empty((nblk, b, b), dtype=bf, device="cuda")
    dQ = torch.zeros((nblk, b, b), dtype=torch.float32, device="cuda")
    # the optimizer update of the same parameters (outside the step): AdamW at the
    # POET-scaled rate on a copy of q, reading q, dq, m, v and writing q, m, v
    q_opt, m_opt, v_opt = S["q"].clone(), torch.zeros_like(S["q"]), torch.zeros_like(S["q"])
    opt_p = B.adamw_params(1e-6)
    stages += [
        ("aux_skew_unpack", lambda: B.poetx_skew_unpack(S["q"], Qb, nblk, b), 0, 4 * nblk * ntri + 2 * nblk * b * b),
        ("aux_skew_pack", lambda: B.poetx_skew_pack(dQ, S["dq"], nblk, b), 0, 4 * nblk * b * b + 4 * nblk * ntri),
        ("aux_adamw", lambda: B.poetx_adamw_step(q_opt, S["dq"], m_opt, v_opt, nblk * ntri, 1, opt_p), 0,
         28 * nblk * ntri),
    ]
    if gemm_only:
        stages = [st_ for st_ in stages if st_[0].startswith(GEMM_STAGES)]
    if only is not None:
        stages = [st_ for st_ in stages if st_[0] in only]
    quick = gemm_only or only is not None
    flush = None if quick else torch.empty(FLUSH_BYTES // 4, dtype=torch.float32, device="cuda")
    for name, fn, flops, nbytes in stages:
        us = _time_events(fn, reps)
        tf = flops / us / 1e6 if flops else None
        gbs = nbytes / us / 1e3
        # dense products are bound by MFMA; block products, gradients, permutations and the
        # b x b transform (at tens of blocks) by memory
        mfma = name.startswith("dense")
        st[name] = {"us": round(us, 2), "tflops": round(tf, 1) if tf else None, "gbs": round(gbs, 1),
                    "bound": "mfma" if mfma else "hbm",
                    "frac": round((tf / PEAK_BF16_TFLOPS) if mfma else (gbs / PEAK_HBM_GBS), 4)}
        if not mfma and flush is not None:   # memory-bound stages also cold: nothing left in L2 / MALL
            cold = _time_cold(fn, 5, flush)
            st[name]["cold_us"] = round(cold, 2)
            st[name]["cold_gbs"] = round(nbytes / cold / 1e3, 1)
        st[name]["_flops"] = flops
    return st


GEMM_STAGES = ("blk", "dense", "grad")   # the block, dense and block-gradient products


def gemm_aggregate(st):
    """Aggregate MFMA rate of the block and dense products of a stage table:
    their algorithmic FLOPs over the sum of their kernel times."""
    names = [nm for nm in st if nm.startswith(GEMM_STAGES)]
    flops = sum(st[nm]["_flops"] for nm in names)
    us = sum(st[nm]["us"] for nm in names)
    return flops, us


def cpu_baseline(spec, inp, budget_s=12.0, max_reps=3):
    """The float64 oracle as it stands, on the host cores: Cayley-Neumann
    blocks, dense forward and backward of the same batch."""
    from threadpoolctl import threadpool_info
    from oracle import poet_oracle as O
    reps, t0 = 0, time.perf_counter()
    while True:
        O.forward(inp["x"], inp["W0"], inp["q_R"], inp["q_P"], inp["pi_R"], inp["pi_P"], spec.b, spec.k)
        O.backward(inp["dy"], inp["x"], inp["W0"], inp["q_R"], inp["q_P"], inp["pi_R"], inp["pi_P"], spec.b,
                   spec.k)
        reps += 1
        el = time.perf_counter() - t0
        if el >= budget_s or reps >= max_reps:
            break
    blas = [p for p in threadpool_info() if p.get("user_api") == "blas"]
    threads = max([p.get("num_threads", 1) for p in blas] or [1])
    lib = f"{blas[0].get('internal_api', '?')} {blas[0].get('version', '')}".strip() if blas else "?"
    cpu = "?"
    try:
        with open("/proc/cpuinfo") as f:
            cpu = next((ln.split(":", 1)[1].strip() for ln in f if ln.startswith("model name")), "?")
    except OSError:
        pass
    return {"value": round(spec.T * reps / el, 1), "unit": "tokens/s", "cores": int(threads), "kind": "oracle",
            "sample": f"the full {spec.T}-token batch of the same layer, {reps} oracle step(s) "
                      f"(float64 numpy: Cayley-Neumann blocks, dense R W0 P forward, backward with block "
                      f"gradients and parameter gradients) in {el:.1f} s",
            "cpu": cpu, "blas": lib}


def read_traffic():
    try:
        with open(TRAFFIC_FILE) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    if rec.get("gemm_source_sha256_16") != gemm_source_hash():
        return None   # kernel changed since the counters were taken
    return rec


# The dense products of the q_proj-shaped step (2048 x 4096 x 4096): 256
# workgroups of 512 lanes, the forward on the 128 x 256 tile with the R-side
# block product folded in (Wt read k-major), the backward on the 256 x 128 tile
# (Wt read n-major).  Dispatches of the same kernel at other shapes (the
# comparison variants) are told apart by their grid size.
DENSE_KERNELS = {"dense_fwd_fold_R": ("pipe_gemm_kernel<128, 256, false, false, false, 3,", 256 * 512),
                 "dense_bwd": ("pipe_gemm_kernel<256, 128, false, true, false,", 256 * 512)}


def _pmc_rows(pmc_dir):
    """(kernel name, grid size, counter, value per dispatch) from every rocprofv3
    counter output under pmc_dir: CSV files or rocpd SQLite databases."""
    import sqlite3
    for path in glob.glob(os.path.join(pmc_dir, "**", "*counter_collection.csv"), recursive=True):
        with open(path) as f:
            for row in csv.DictReader(f):
                yield (row.get("Kernel_Name", ""), int(float(row.get("Grid_Size", "0") or 0)),
                       row.get("Counter_Name", ""), float(row.get("Counter_Value", "nan")))
    for path in glob.glob(os.path.join(pmc_dir, "**", "*_results.db"), recursive=True):
        con = sqlite3.connect(path)
        try:
            yield from con.execute("select kernel_name, grid_size, counter_name, value from counters_collection")
        finally:
            con.close()


def parse_pmc(pmc_dir):
    """Per-dispatch FETCH_SIZE / WRITE_SIZE (KiB) of the two dense products and
    of the reference copy, from rocprofv3 counter CSVs; writes TRAFFIC_FILE.
    Also prints every kernel's mean per dispatch (for the profile summaries)."""
    vals, every, copies = {}, {}, {}
    for name, grid, cn, v in _pmc_rows(pmc_dir):
        every.setdefault((name, grid, cn), []).append(v)
        key = None
        for nm, (tag, g) in DENSE_KERNELS.items():
            if tag in name and grid == g:
                key = nm
        if key:
            vals.setdefault((key, cn), []).append(v)
        if COPY_KERNEL_TAG in name:
            copies.setdefault((cn, grid), []).append(v)
    rec = {"gemm_source_sha256_16": gemm_source_hash(), "copy_bytes": COPY_BYTES}
    for cn in ("FETCH_SIZE", "WRITE_SIZE"):
        # the 256 MiB reference copy: the largest copy dispatch of the run (plus
        # any of at least a tenth of it, should the runtime split the copy);
        # the run's other copies are small, some with the same grid size
        c_all = [v for (c, g), vs in copies.items() if c == cn for v in vs]
        if not c_all:
            continue
        c = [v for v in c_all if v >= 0.1 * max(c_all)]
        c_kib = sum(c)
        scale = COPY_BYTES / (c_kib * 1024.0)
        for nm in DENSE_KERNELS:
            g = vals.get((nm, cn))
            if not g:
                continue
            g_kib = sum(g) / len(g)
            rec.setdefault(nm, {})[cn] = {"kib_per_dispatch": g_kib, "dispatches": len(g), "copy_kib": c_kib,
                                          "copy_dispatches": len(c), "scale": scale,
                                          "bytes_per_dispatch": g_kib * 1024.0 * scale}
    os.makedirs(os.path.dirname(TRAFFIC_FILE), exist_ok=True)
    with open(TRAFFIC_FILE, "w") as f:
        json.dump(rec, f, indent=1)
    print(json.dumps(rec))
    for (name, grid, cn), v in sorted(every.items()):
        print(f"{cn}\t{grid}\t{len(v)}\t{sum(v) / len(v):.1f}\t{name[:150]}")


def _products(k):
    """b x b products of one forward / one saved-state backward of the transform."""
    return {3: 2, 4: 3}.get(k, k), {3: 4, 4: 7}.get(k, 3 * k - 1)


def _time_steps(step, steps, warmup, per_step=None):
    """Mean ms per step over exactly `steps` steps after `warmup` untimed ones,
    bracketed by device synchronisation.  With a dict `per_step`, events between
    the steps (same stream, no synchronisation) also give the median and minimum."""
    import torch
    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
    ev[0].record()
    for i in range(steps):
        step()
        ev[i + 1].record()
    torch.cuda.synchronize()
    if per_step is not None:
        t = sorted(ev[i].elapsed_time(ev[i + 1]) for i in range(steps))
        per_step["median"] = t[len(t) // 2] if len(t) % 2 else 0.5 * (t[len(t) // 2 - 1] + t[len(t) // 2])
        per_step["min"] = t[0]
    return ev[0].elapsed_time(ev[steps]) / steps


def vendor_reference(spec, S, cs, cd, reps=20):
    """Context, not the product path: the vendor library (torch.matmul -> hipBLASLt)
    on the same dense shapes and weight, and a plain device copy of known size."""
    import torch
    import torch.nn.functional as F
    g = torch.Generator(device="cuda").manual_seed(1234)
    a = torch.randn(spec.T, spec.n, device="cuda", generator=g).to(torch.bfloat16)
    d = torch.randn(spec.T, spec.m, device="cuda", generator=g).to(torch.bfloat16)
    Wt = S["Wt"]

    def timed(fn):
        for _ in range(3):
            fn()
        torch.cuda.synchronize()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) * 1e3 / reps

    nt = timed(lambda: F.linear(a, Wt))          # a Wt^T, as the dense forward
    nn = timed(lambda: torch.matmul(d, Wt))      # d Wt, as the dense backward
    cp = timed(lambda: cd.copy_(cs))
    flops = 2.0 * spec.T * spec.m * spec.n
    return {"hipblaslt_dense_nt_us": round(nt, 2), "hipblaslt_dense_nt_tflops": round(flops / nt / 1e6, 1),
            "hipblaslt_dense_nn_us": round(nn, 2), "hipblaslt_dense_nn_tflops": round(flops / nn / 1e6, 1),
            "copy_bytes": 2 * COPY_BYTES, "copy_gbs": round(2 * COPY_BYTES / cp / 1e3, 1)}


def variant_steps(spec, S, steps=10, warmup=5):
    """Context, not the product path: the same step (transform forward, linear
    forward and backward, transform backward) with every variant of the linear:
    the fast and mem chains, the chain with all four permutations on the
    activations, and the original weight-centric POET (dense R and P, W_RP
    formed every step).  Mean ms per step over `steps` after `warmup`."""
    from orthogonal_equivalence_poet_amd import binding as B
    nblk = spec.nblk_R + spec.nblk_P
    out = {}
    Wq = B.workspace(B.poetx_qweight_bytes(spec.m, spec.n))
    B.poetx_quantize_weight(S["Wt"], spec.m, spec.n, Wq)
    for name, var in (("fast", B.POETX_FAST), ("mem", B.POETX_MEM), ("four_perm", B.POETX_FOUR_PERM),
                      ("weight_centric", B.POETX_WEIGHT_CENTRIC), ("mem_q8", B.POETX_MEM_Q8)):
        d = B.desc(spec.T, spec.m, spec.n, spec.b, spec.k, B.POETX_BF16, var)
        weight = {B.POETX_FAST: S["Wt"], B.POETX_MEM: S["Wt"], B.POETX_MEM_Q8: Wq}.get(var, S["W0"])
        saved = B.workspace(B.poetx_linear_saved_bytes(d)) if var not in (B.POETX_MEM, B.POETX_MEM_Q8) else None
        ws = B.workspace(max(B.poetx_linear_fwd_workspace_bytes(d), B.poetx_linear_bwd_workspace_bytes(d),
                             B.poetx_cnp_fwd_workspace_bytes(nblk, spec.b, spec.k, B.POETX_BF16),
                             B.poetx_cnp_bwd_workspace_bytes(nblk, spec.b, spec.k, B.POETX_BF16)))

        def step():
            B.poetx_cnp_fwd_save(S["q"], nblk, spec.b, spec.k, S["G"], S["cnp_saved"], ws)
            B.poetx_linear_fwd(d, S["x"], weight, S["G_R"], S["G_P"], S["pi_R"], S["pi_P"], S["y"], saved, ws)
            B.poetx_linear_bwd(d, S["dy"], S["x"], weight, S["G_R"], S["G_P"], S["pi_R"], S["pi_P"], saved,
                               S["dx"], S["dG_R"], S["dG_P"], ws)
            B.poetx_cnp_bwd_saved(S["q"], S["dG"], nblk, spec.b, spec.k, S["dq"], B.POETX_BF16, S["cnp_saved"],
                                  ws)
        out[f"{name}_ms"] = round(_time_steps(step, steps, warmup), 4)
    out["weight_centric_over_fast"] = round(out["weight_centric_ms"] / out["fast_ms"], 2)
    out["four_perm_over_fast"] = round(out["four_perm_ms"] / out["fast_ms"], 3)
    out["mem_q8_over_mem"] = round(out["mem_q8_ms"] / out["mem_ms"], 3)
    return out


def _base_line(args, value, unit, ms, workload, T):
    return {"metric": METRIC, "value": round(value, 1), "unit": unit, "n_gpus": 1,
            "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 4), "higher_is_better": True,
            "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
            "config": {"workload": workload, "global_batch": 1, "seq_len": T, "parallelism": "single GPU"}}


def run_linear(args, spec, label):
    """One linear: step throughput, every stage alone, dense roofline, oracle baseline."""
    import torch
    S, inp = build_state(spec)
    step = make_step(spec, S)

    # reference copy of known size (scale for the HBM counters)
    cs = torch.ones(COPY_BYTES // 2, dtype=torch.bfloat16, device="cuda")
    cd = torch.empty_like(cs)
    cd.copy_(cs)

    per = {}
    ms = _time_steps(step, args.steps, args.warmup, per)
    tok_s = spec.T / (ms / 1e3)
    # the same step captured in a HIP graph (the library allocates nothing and
    # records no memset nodes): its replays, timed the same way, as context
    graph = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    with torch.cuda.graph(graph):
        step()
    ms_graph = _time_steps(graph.replay, args.steps, args.warmup)

    st = stage_timings(spec, S, args.stage_reps)
    g_flops, g_us = gemm_aggregate(st)
    gemm_tflops = g_flops / g_us / 1e6
    traffic = read_traffic() if label == "q_proj" else None
    shapes = {"dense_fwd": f"dense Wt GEMM, forward, h2 = h1 Wt^T ({spec.T} x {spec.m} x {spec.n}, Wt read k-major)",
              "dense_fwd_fold_R": f"dense Wt GEMM with the R-side block product folded in, forward, "
                                  f"z = (h1 Wt^T) blockdiag(G_R)^T ({spec.T} x {spec.m} x {spec.n}, then "
                                  f"{spec.m // spec.b} blocks of {spec.b}; Wt read k-major)",
              "dense_bwd": f"dense Wt GEMM, backward, dh1 = dh2 Wt ({spec.T} x {spec.n} x {spec.m}, Wt read n-major)"}
    kernels = {}
    for nm in ("dense_fwd_fold_R" if "dense_fwd_fold_R" in st else "dense_fwd", "dense_bwd"):
        flops = st[nm]["_flops"]
        tr = None
        rec = (traffic or {}).get(nm)
        if rec and "FETCH_SIZE" in rec and "WRITE_SIZE" in rec:
            tr = round(rec["FETCH_SIZE"]["bytes_per_dispatch"] + rec["WRITE_SIZE"]["bytes_per_dispatch"])
        kernels[nm] = {"kernel": f"{shapes[nm]}, bf16, fp32 accumulate",
                       "achieved": round(flops / st[nm]["us"] / 1e6, 1),
                       "frac": round(flops / st[nm]["us"] / 1e6 / PEAK_BF16_TFLOPS, 4),
                       "traffic": tr, "avg_launch_us": st[nm]["us"], "algorithmic_flops_per_launch": flops}
    # the roofline object describes the longer of the two dense products (the
    # step's dominant kernel); both are listed under "kernels"
    dom = max(kernels, key=lambda nm: kernels[nm]["avg_launch_us"])
    roof = {"kernel": kernels[dom]["kernel"], "bound": "mfma", "achieved": kernels[dom]["achieved"],
            "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s", "frac": kernels[dom]["frac"],
            "traffic": kernels[dom]["traffic"], "avg_launch_us": kernels[dom]["avg_launch_us"],
            "algorithmic_flops_per_launch": kernels[dom]["algorithmic_flops_per_launch"], "stage": dom,
            "kernels": kernels}
    for v in st.values():
        v.pop("_flops", None)
    nR, nP = spec.nblk_R, spec.nblk_P
    workload = (f"llama8b_{label}: W0 {spec.m}x{spec.n} bf16, b={spec.b} ({nR}+{nP} blocks), k={spec.k}, "
                f"{spec.T // 2048} x 2048 tokens, {spec.variant} variant"
                + (f", every Q block at spectral norm {spec.q_block_norm}" if spec.q_block_norm else "")
                + "; step = cnp_fwd_save + linear_fwd + linear_bwd + cnp_bwd_saved")
    out = _base_line(args, tok_s, "tokens/s", ms, workload, spec.T)
    out["ms_per_step_median"] = round(per["median"], 4)
    out["ms_per_step_min"] = round(per["min"], 4)
    out["ms_per_step_graph"] = round(ms_graph, 4)
    out.update({
        "gemm_pct_peak": round(100 * gemm_tflops / PEAK_BF16_TFLOPS, 2),
        "gemm_tflops": round(gemm_tflops, 1),
        "gemm_gflop_per_step": round(g_flops / 1e9, 2),
        "stages": st,
        "roofline": roof,
    })
    out["vendor_reference"] = vendor_reference(spec, S, cs, cd)
    out["variants"] = variant_steps(spec, S)
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(spec, inp)
    return out


def nested_linear(args, spec, label):
    """A linear's step (as in the main line) and the aggregate MFMA rate of its
    block and dense products, each timed alone (warm), for the nested records."""
    S, _ = build_state(spec)
    step = make_step(spec, S)
    per = {}
    ms = _time_steps(step, args.steps, args.warmup, per)
    st = stage_timings(spec, S, 20, gemm_only=True)
    flops, us = gemm_aggregate(st)
    nR, nP = spec.nblk_R, spec.nblk_P
    rec = {"workload": f"llama8b_{label}: W0 {spec.m}x{spec.n} bf16, b={spec.b} ({nR}+{nP} blocks), k={spec.k}, "
                       f"{spec.T // 2048} x 2048 tokens, {spec.variant} variant"
                       + (f", every Q block at spectral norm {spec.q_block_norm}" if spec.q_block_norm else ""),
           "tokens_per_s": round(spec.T / (ms / 1e3), 1), "ms_per_step": round(ms, 4),
           "ms_per_step_median": round(per["median"], 4), "ms_per_step_min": round(per["min"], 4),
           "gemm_pct_peak": round(100 * flops / us / 1e6 / PEAK_BF16_TFLOPS, 2),
           "gemm_tflops": round(flops / us / 1e6, 1), "gemm_gflop_per_step": round(flops / 1e9, 2),
           "stages_us": {nm: v["us"] for nm, v in st.items()},
           "dense_frac": {nm: v["frac"] for nm, v in st.items() if nm.startswith("dense")}}
    return rec


_TOP_KEYS = ("metric", "n_gpus", "steps", "warmup", "higher_is_better", "scaling", "vs_baseline", "dtype", "data")


def _nest(line):
    """A workload's line as a nested record: without the keys the main line holds."""
    rec = {k: v for k, v in line.items() if k not in _TOP_KEYS}
    cfg = rec.pop("config", {})
    rec["workload"] = cfg.get("workload")
    return rec


def nested_configs(args):
    """The other Llama-8B / 13B workloads, each timed the same way as the main
    line (K steps after W warm-up steps) and nested in it."""
    import torch
    from orthogonal_equivalence_poet_amd import inputs as I
    out = {}
    jobs = [("up_proj_fast", lambda: nested_linear(args, I.llama8b_up_proj("fast"), "up_proj")),
            ("up_proj_mem", lambda: nested_linear(args, I.llama8b_up_proj("mem"), "up_proj")),
            ("llama8b_layer", lambda: _nest(run_layer(args, I.llama8b_layer(), "llama8b_layer", merge=True))),
            ("llama13b_layer", lambda: _nest(run_layer(args, I.llama13b_layer(), "llama13b_layer", merge=False))),
            ("cnp_13b", lambda: _nest(run_cnp_13b(args)))]
    for name, fn in jobs:
        t0 = time.perf_counter()
        out[name] = fn()
        torch.cuda.synchronize()
        torch.cuda.empty_cache()
        print(f"bench: {name} done in {time.perf_counter() - t0:.1f} s", file=sys.stderr, flush=True)
    return out


def run_layer(args, specs, label, merge):
    """All 7 linears of a decoder layer (mem variant): step throughput and the
    whole-step rate of the algorithmic GEMM work; optionally the merge."""
    import torch
    from orthogonal_equivalence_poet_amd import binding as B
    from orthogonal_equivalence_poet_amd import inputs as I
    states = [build_state(sp)[0] for sp in specs]
    # one Cayley-Neumann batch for the whole layer (every linear has b = 256 and
    # the same k): flat q, G, dG, dq; each linear's tensors are views into them
    b, k = specs[0].b, specs[0].k
    assert all(sp.b == b and sp.k == k for sp in specs)
    nbs = [sp.nblk_R + sp.nblk_P for sp in specs]
    nall = sum(nbs)
    q_all = torch.cat([S["q"] for S in states]).contiguous()
    G_all = torch.empty((nall, b, b), dtype=torch.bfloat16, device="cuda")
    dG_all = torch.empty((nall, b, b), dtype=torch.float32, device="cuda")
    dq_all = torch.empty_like(q_all)
    o = 0
    for sp, S, nb in zip(specs, states, nbs):
        S["q"], S["G"], S["dG"], S["dq"] = q_all[o:o + nb], G_all[o:o + nb], dG_all[o:o + nb], dq_all[o:o + nb]
        S["G_R"], S["G_P"] = S["G"][:sp.nblk_R], S["G"][sp.nblk_R:]
        S["dG_R"], S["dG_P"] = S["dG"][:sp.nblk_R], S["dG"][sp.nblk_R:]
        o += nb
    cnp_saved = B.workspace(B.poetx_cnp_saved_bytes(nall, b, k, B.POETX_BF16))
    cnp_ws = B.workspace(B.poetx_cnp_bwd_workspace_bytes(nall, b, k, B.POETX_BF16))

    def step():
        B.poetx_cnp_fwd_save(q_all, nall, b, k, G_all, cnp_saved, cnp_ws)
        for S in states:
            B.poetx_linear_fwd(S["desc"], S["x"], S["Wt"], S["G_R"], S["G_P"], S["pi_R"], S["pi_P"], S["y"],
                               S["saved"], S["ws"])
        for S in reversed(states):
            B.poetx_linear_bwd(S["desc"], S["dy"], S["x"], S["Wt"], S["G_R"], S["G_P"], S["pi_R"], S["pi_P"],
                               S["saved"], S["dx"], S["dG_R"], S["dG_P"], S["ws"])
        B.poetx_cnp_bwd_saved(q_all, dG_all, nall, b, k, dq_all, B.POETX_BF16, cnp_saved, cnp_ws)
    per = {}
    ms = _time_steps(step, args.steps, args.warmup, per)
    T = specs[0].T
    g_flops = 0
    for sp in specs:
        fwd = 2 * T * (sp.n * sp.b + sp.n * sp.m + sp.m * sp.b)
        bwd = 2 * T * (2 * sp.m * sp.b + sp.n * sp.m + 2 * sp.n * sp.b) + 2 * T * (sp.n * sp.b + sp.n * sp.m)
        g_flops += fwd + bwd
    out = _base_line(args, T / (ms / 1e3), "tokens/s", ms,
                     f"{label}: all 7 linears of one decoder layer, b=256, k=3, mem variant, "
                     f"{T // 2048} x 2048 tokens; step = cnp_fwd_save over the layer's {nall} blocks + 7 x "
                     "linear_fwd + 7 x linear_bwd + cnp_bwd_saved over the same blocks", T)
    out["ms_per_step_median"] = round(per["median"], 4)
    out["ms_per_step_min"] = round(per["min"], 4)
    # the block and dense products of every linear alone (warm, same launches
    # as inside the step): their algorithmic FLOPs over their kernel time
    kf, ku = 0, 0.0
    for sp, S in zip(specs, states):
        f_, u_ = gemm_aggregate(stage_timings(sp, S, 20, gemm_only=True))
        kf, ku = kf + f_, ku + u_
    out["gemm_pct_peak"] = round(100 * kf / ku / 1e6 / PEAK_BF16_TFLOPS, 2)
    out["gemm_tflops"] = round(kf / ku / 1e6, 1)
    out["gemm_kernel_us"] = round(ku, 1)
    out["step_gemm_tflops"] = round(g_flops / (ms * 1e-3) / 1e12, 1)
    out["step_pct_peak"] = round(100 * g_flops / (ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 2)
    out["gemm_gflop_per_step"] = round(g_flops / 1e9, 2)
    # the same step with q/k/v and gate/up as groups of linears sharing an input
    ms_grouped = grouped_layer_step(args, specs, states)
    out["grouped"] = {"ms_per_step": round(ms_grouped, 4), "tokens_per_s": round(T / (ms_grouped / 1e3), 1),
                      "groups": "q/k/v, o, gate/up, down", "over_ungrouped": round(ms_grouped / ms, 3)}
    # training-step closure: the AdamW update of every q of the layer in one call,
    # and the merge + optimizer reset that a reset gap of 400 updates amortizes
    count = q_all.numel()
    m_all, v_all = torch.zeros_like(q_all), torch.zeros_like(q_all)
    opt_p = B.adamw_params(1e-6)
    opt = lambda: B.poetx_adamw_step(q_all, dq_all, m_all, v_all, count, 1, opt_p)
    us_opt = _time_events(opt, 20, warm=3)
    out["adamw"] = {"params": count, "us": round(us_opt, 1), "gbs": round(28 * count / us_opt / 1e3, 1),
                    "frac_hbm": round(28 * count / us_opt / 1e3 / PEAK_HBM_GBS, 4)}
    ms_train = _time_steps(lambda: (step(), opt()), args.steps, max(3, args.warmup // 4))
    out["train_step_ms"] = round(ms_train, 4)
    us_reset = _time_events(lambda: B.poetx_adamw_reset(m_all, v_all, count), 10, warm=2)
    out["adamw_reset_us"] = round(us_reset, 1)
    if merge:
        merges = []
        for sp, S in zip(specs, states):
            pi_R2 = torch.from_numpy(I.permutation(sp.m, *sp.key, I.PIR2_ID)).cuda()
            pi_P2 = torch.from_numpy(I.permutation(sp.n, *sp.key, I.PIP2_ID)).cuda()
            ws = B.workspace(B.poetx_merge_workspace_bytes(S["desc"]))
            qR, qP = S["q"][:sp.nblk_R], S["q"][sp.nblk_R:]
            merges.append(lambda S=S, ws=ws, qR=qR, qP=qP, a=pi_R2, c=pi_P2:
                          B.poetx_merge(S["desc"], S["Wt"], qR, qP, S["pi_R"], S["pi_P"], a, c, ws))
        us = _time_events(lambda: [f() for f in merges], 5, warm=1)
        out["merge_all_7_us"] = round(us, 1)
        out["train_step_ms_reset_gap_400"] = round(ms_train + (us + us_reset) / 1e3 / 400, 4)
    return out


def grouped_layer_step(args, specs, states):
    """The same layer step with the linears that read the same input (q, k, v;
    gate, up) run as groups (poetx_group_fwd / _bwd: every stage one launch for
    the group), the others alone; one Cayley-Neumann batch ordered so that each
    group's R blocks and P blocks are contiguous.  Mean ms per step."""
    import torch
    from orthogonal_equivalence_poet_amd import binding as B
    b, k, T = specs[0].b, specs[0].k, specs[0].T
    names = [sp.name.split("_", 1)[1] for sp in specs]
    parts = [["q_proj", "k_proj", "v_proj"], ["o_proj"], ["gate_proj", "up_proj"], ["down_proj"]]
    qs, units, o = [], [], 0
    for part in parts:
        idx = [names.index(nm) for nm in part]
        sps, sts = [specs[i] for i in idx], [states[i] for i in idx]
        qR = [S["q"][:sp.nblk_R] for sp, S in zip(sps, sts)]
        qP = [S["q"][sp.nblk_R:] for sp, S in zip(sps, sts)]
        nR, nP = sum(sp.nblk_R for sp in sps), sum(sp.nblk_P for sp in sps)
        qs += qR + qP
        units.append(dict(sps=sps, sts=sts, r=(o, o + nR), p=(o + nR, o + nR + nP)))
        o += nR + nP
    nall = o
    q_all = torch.cat(qs).contiguous()
    G_all = torch.empty((nall, b, b), dtype=torch.bfloat16, device="cuda")
    dG_all = torch.empty((nall, b, b), dtype=torch.float32, device="cuda")
    dq_all = torch.empty_like(q_all)
    cnp_saved = B.workspace(B.poetx_cnp_saved_bytes(nall, b, k, B.POETX_BF16))
    cnp_ws = B.workspace(B.poetx_cnp_bwd_workspace_bytes(nall, b, k, B.POETX_BF16))
    calls = []
    for u in units:
        sps, sts = u["sps"], u["sts"]
        G_R, G_P = G_all[u["r"][0]:u["r"][1]], G_all[u["p"][0]:u["p"][1]]
        dG_R, dG_P = dG_all[u["r"][0]:u["r"][1]], dG_all[u["p"][0]:u["p"][1]]
        x = sts[0]["x"]
        M = sum(sp.m for sp in sps)
        if len(sps) == 1:
            S = sts[0]
            fwd = (lambda S=S, G_R=G_R, G_P=G_P: B.poetx_linear_fwd(S["desc"], S["x"], S["Wt"], G_R, G_P, S["pi_R"],
                                                                     S["pi_P"], S["y"], S["saved"], S["ws"]))
            bwd = (lambda S=S, G_R=G_R, G_P=G_P, dG_R=dG_R, dG_P=dG_P:
                   B.poetx_linear_bwd(S["desc"], S["dy"], S["x"], S["Wt"], G_R, G_P, S["pi_R"], S["pi_P"],
                                      S["saved"], S["dx"], dG_R, dG_P, S["ws"]))
        else:
            var = B.POETX_MEM if sps[0].variant == "mem" else B.POETX_FAST
            gd = B.group_desc(T, sps[0].n, b, k, B.POETX_BF16, var, [sp.m for sp in sps])
            Wt = torch.cat([S["Wt"] for S in sts]).contiguous()
            pi_R = torch.cat([S["pi_R"] for S in sts]).contiguous()
            pi_P = torch.cat([S["pi_P"] for S in sts]).contiguous()
            y = torch.empty((T, M), dtype=torch.bfloat16, device="cuda")
            dy = torch.cat([S["dy"] for S in sts], dim=1).contiguous()
            dx = torch.empty_like(x)
            saved = B.workspace(B.poetx_group_saved_bytes(gd)) if var == B.POETX_FAST else None
            ws = B.workspace(max(B.poetx_group_fwd_workspace_bytes(gd), B.poetx_group_bwd_workspace_bytes(gd)))
            fwd = (lambda gd=gd, x=x, Wt=Wt, G_R=G_R, G_P=G_P, pi_R=pi_R, pi_P=pi_P, y=y, saved=saved, ws=ws:
                   B.poetx_group_fwd(gd, x, Wt, G_R, G_P, pi_R, pi_P, y, saved, ws))
            bwd = (lambda gd=gd, dy=dy, x=x, Wt=Wt, G_R=G_R, G_P=G_P, pi_R=pi_R, pi_P=pi_P, saved=saved, dx=dx,
                   dG_R=dG_R, dG_P=dG_P, ws=ws:
                   B.poetx_group_bwd(gd, dy, x, Wt, G_R, G_P, pi_R, pi_P, saved, dx, dG_R, dG_P, ws))
        calls.append((fwd, bwd))

    def step():
        B.poetx_cnp_fwd_save(q_all, nall, b, k, G_all, cnp_saved, cnp_ws)
        for fwd, _ in calls:
            fwd()
        for _, bwd in reversed(calls):
            bwd()
        B.poetx_cnp_bwd_saved(q_all, dG_all, nall, b, k, dq_all, B.POETX_BF16, cnp_saved, cnp_ws)
    return _time_steps(step, args.steps, args.warmup)


def run_cnp_13b(args):
    """One Cayley-Neumann forward (saving) and backward over the b=256 blocks of
    every POET-X linear in 40 Llama-13B layers."""
    import torch
    from orthogonal_equivalence_poet_amd import binding as B
    from orthogonal_equivalence_poet_amd import inputs as I
    b, k = 256, 3
    nblk = I.llama13b_cnp_blocks()
    q = torch.from_numpy(I.cnp_params(nblk, b, 1e-3, 5, 1, 0)).cuda()
    gen = torch.Generator(device="cuda").manual_seed(5)
    dG = torch.randn((nblk, b, b), device="cuda", generator=gen)
    G = torch.empty((nblk, b, b), dtype=torch.bfloat16, device="cuda")
    dq = torch.empty_like(q)
    saved = B.workspace(B.poetx_cnp_saved_bytes(nblk, b, k, B.POETX_BF16))
    ws = B.workspace(B.poetx_cnp_bwd_workspace_bytes(nblk, b, k, B.POETX_BF16))
    fwd = lambda: B.poetx_cnp_fwd_save(q, nblk, b, k, G, saved, ws)
    bwd = lambda: B.poetx_cnp_bwd_saved(q, dG, nblk, b, k, dq, B.POETX_BF16, saved, ws)
    ms = _time_steps(lambda: (fwd(), bwd()), max(1, args.steps // 4), 2)
    us_f = _time_events(fwd, 5, warm=1)
    us_b = _time_events(bwd, 5, warm=1)
    pf, pb = _products(k)
    out = _base_line(args, nblk / (ms / 1e3), "blocks/s", ms,
                     f"cnp_13b: one Cayley-Neumann forward (saving) + backward over {nblk} blocks of 256 "
                     "(all POET-X linears of 40 Llama-13B layers), k=3, bf16 products", 0)
    ntri = b * (b - 1) // 2
    out["fwd_us"], out["bwd_us"] = round(us_f, 1), round(us_b, 1)
    out["fwd_tflops"] = round(pf * 2 * b ** 3 * nblk / us_f / 1e6, 1)
    out["bwd_tflops"] = round(pb * 2 * b ** 3 * nblk / us_b / 1e6, 1)
    out["fwd_gbs"] = round((4 * ntri + 2 * b * b) * nblk / us_f / 1e3, 1)
    # the standalone skew unpack (q -> bf16 Q) and pack (float32 dQ -> dq) over the
    # same blocks, in the buffers of the backward (not part of the step)
    del G
    Qb = torch.empty((nblk, b, b), dtype=torch.bfloat16, device="cuda")
    us_u = _time_events(lambda: B.poetx_skew_unpack(q, Qb, nblk, b), 5, warm=1)
    del Qb
    us_p = _time_events(lambda: B.poetx_skew_pack(dG, dq, nblk, b), 5, warm=1)
    out["skew_unpack_us"] = round(us_u, 1)
    out["skew_unpack_gbs"] = round((4 * ntri + 2 * b * b) * nblk / us_u / 1e3, 1)
    out["skew_pack_us"] = round(us_p, 1)
    out["skew_pack_gbs"] = round((4 * b * b + 4 * ntri) * nblk / us_p / 1e3, 1)
    return out


def profile_cnp_13b(args):
    """The 15280-block Cayley-Neumann forward and backward and the skew passes,
    each --stage-reps times, for counter passes (no timing of the whole step)."""
    import torch
    from orthogonal_equivalence_poet_amd import binding as B
    from orthogonal_equivalence_poet_amd import inputs as I
    b, k = 256, 3
    nblk = I.llama13b_cnp_blocks()
    q = torch.from_numpy(I.cnp_params(nblk, b, 1e-3, 5, 1, 0)).cuda()
    gen = torch.Generator(device="cuda").manual_seed(5)
    dG = torch.randn((nblk, b, b), device="cuda", generator=gen)
    G = torch.empty((nblk, b, b), dtype=torch.bfloat16, device="cuda")
    dq = torch.empty_like(q)
    saved = B.workspace(B.poetx_cnp_saved_bytes(nblk, b, k, B.POETX_BF16))
    ws = B.workspace(B.poetx_cnp_bwd_workspace_bytes(nblk, b, k, B.POETX_BF16))
    cs = torch.ones(COPY_BYTES // 2, dtype=torch.bfloat16, device="cuda")
    torch.empty_like(cs).copy_(cs)
    del cs
    for _ in range(args.stage_reps):
        B.poetx_cnp_fwd_save(q, nblk, b, k, G, saved, ws)
        B.poetx_cnp_bwd_saved(q, dG, nblk, b, k, dq, B.POETX_BF16, saved, ws)
    B.poetx_skew_unpack(q, G, nblk, b)
    B.poetx_skew_pack(dG, dq, nblk, b)
    torch.cuda.synchronize()
    print(json.dumps({"cnp_13b_profiled": nblk, "reps": args.stage_reps}))
    return 0


def profile_stages(args):
    """Only the named stages of the workload's step, each --stage-reps times
    (warm), through the same entry points and launch shapes as stage_timings."""
    from orthogonal_equivalence_poet_amd import inputs as I
    w = args.workload
    spec = (I.llama8b_q_proj() if w == "q_proj"
            else I.llama8b_up_proj("mem" if w == "up_proj_mem" else "fast") if w.startswith("up_proj") else None)
    if spec is None:
        print(f"--profile-stages supports the single-linear workloads, not {w}", file=sys.stderr)
        return 2
    import torch
    S, _ = build_state(spec)
    # a plain device copy of known size: the scale for the HBM byte counters
    cs = torch.ones(COPY_BYTES // 2, dtype=torch.bfloat16, device="cuda")
    torch.empty_like(cs).copy_(cs)
    want = [nm for nm in args.profile_stages.split(",") if nm]
    st = stage_timings(spec, S, args.stage_reps, only=want)
    missing = set(want) - set(st)
    if missing:
        print(f"unknown stages: {sorted(missing)}", file=sys.stderr)
        return 2
    print(json.dumps({nm: {"us": v["us"], "frac": v["frac"]} for nm, v in st.items()}))
    return 0


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=100)
    ap.add_argument("--stage-reps", type=int, default=50)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-configs", action="store_true",
                    help="skip the nested records of the other workloads in the default line")
    ap.add_argument("--pmc-dir", default=None)
    ap.add_argument("--profile-stages", default=None,
                    help="comma-separated stage names (see stage_timings): build the workload's state, "
                         "run only those stages --stage-reps times each and print their mean times "
                         "(for rocprofv3 counter and trace passes on chosen kernels)")
    ap.add_argument("--workload", default="q_proj",
                    choices=["q_proj", "up_proj", "up_proj_mem", "llama8b_layer", "llama13b_layer", "cnp_13b"])
    args = ap.parse_args()
    if args.pmc_dir:
        parse_pmc(args.pmc_dir)
        return 0
    if args.gpus != 1:
        print(f"bench.py: this build measures one GPU only (asked for --gpus {args.gpus}); the data-parallel "
              "sharding across GPUs is a design, not a launched path", file=sys.stderr)
        return 2

    import torch
    from orthogonal_equivalence_poet_amd import binding as B
    from orthogonal_equivalence_poet_amd import inputs as I

    B.load()
    torch.cuda.set_device(0)
    w = args.workload
    if args.profile_stages and w == "cnp_13b":
        return profile_cnp_13b(args)
    if args.profile_stages:
        return profile_stages(args)
    if w == "q_proj":
        out = run_linear(args, I.llama8b_q_proj(), "q_proj")
        print("bench: q_proj done", file=sys.stderr, flush=True)
        if not args.no_configs:
            out["configs"] = nested_configs(args)
    elif w in ("up_proj", "up_proj_mem"):
        spec = I.llama8b_up_proj("mem" if w == "up_proj_mem" else "fast")
        out = run_linear(args, spec, "up_proj")
    elif w == "llama8b_layer":
        out = run_layer(args, I.llama8b_layer(), "llama8b_layer", merge=True)
    elif w == "llama13b_layer":
        out = run_layer(args, I.llama13b_layer(), "llama13b_layer", merge=False)
    else:
        out = run_cnp_13b(args)
    print(json.dumps(out))
    return 0


if __name__ == "__main__":
    sys.exit(main())
