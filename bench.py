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
the roofline of the dominant kernel (the dense Wt GEMM) and the float64 oracle
timed on the host cores as a baseline.

  --pmc-dir DIR   parse a rocprofv3 --pmc FETCH_SIZE / WRITE_SIZE run of this
                  script and record the dense GEMM's HBM traffic in
                  profiles/traffic_dense_gemm.json (scaled by a plain copy of
                  known size that every run performs).
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
DENSE_KERNEL_TAG = "pipe_gemm_kernel<256, 128, false, false, false, false, 3>"   # dense NT (forward), demangled
COPY_KERNEL_TAG = "copyBuffer"   # the runtime's device-to-device copy kernel


def gemm_source_hash() -> str:
    with open(GEMM_SRC, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


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
    S["G"] = torch.empty((nR + nP, b, b), dtype=bf, device=dev)
    S["G_R"], S["G_P"] = S["G"][:nR], S["G"][nR:]
    S["dG"] = torch.empty((nR + nP, b, b), dtype=torch.float32, device=dev)
    S["dG_R"], S["dG_P"] = S["dG"][:nR], S["dG"][nR:]
    S["dq"] = torch.empty_like(S["q"])
    S["y"] = torch.empty((spec.T, spec.m), dtype=bf, device=dev)
    S["dx"] = torch.empty((spec.T, spec.n), dtype=bf, device=dev)
    S["desc"] = B.desc(spec.T, spec.m, spec.n, b, spec.k, B.POETX_BF16, B.POETX_FAST)
    S["saved"] = B.workspace(B.poetx_linear_saved_bytes(S["desc"]))
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


def stage_timings(spec, S, reps):
    """Every stage of the step alone, through the C ABI, same shapes and
    launch configurations as inside poetx_linear_fwd / _bwd."""
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
         2 * 2 * b ** 3 * nblk,
         4 * nblk * b * (b - 1) // 2 + 2 * nblk * b * b),
        ("perm_gather_x", lambda: B.poetx_permute(S["x"], a, T, n, None, S["pi_P"], False), 0, 2 * 2 * T * n),
        ("blk_fwd_P", blk(NT, a, S["G_P"], h1, n), 2 * T * n * b, 2 * (2 * T * n + n * b)),
        ("dense_fwd", lambda: B.poetx_gemm(NT, h1, S["Wt"], h2, T, m, n, dense=True), 2 * T * m * n,
         2 * (T * n + m * n + T * m)),
        ("blk_fwd_R", blk(NT, h2, S["G_R"], z, m), 2 * T * m * b, 2 * (2 * T * m + m * b)),
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
         4 * 2 * b ** 3 * nblk, 4 * nblk * b * b + 4 * nblk * b * (b - 1) // 2),
    ]
    for name, fn, flops, nbytes in stages:
        us = _time_events(fn, reps)
        st[name] = {"us": round(us, 2), "tflops": round(flops / us / 1e6, 1) if flops else None,
                    "gbs": round(nbytes / us / 1e3, 1)}
        st[name]["_flops"] = flops
    return st


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
    threads = max([p.get("num_threads", 1) for p in threadpool_info() if p.get("user_api") == "blas"] or [1])
    return {"value": round(spec.T * reps / el, 1), "unit": "tokens/s", "cores": int(threads), "kind": "oracle",
            "sample": f"the full {spec.T}-token batch of the same layer, {reps} oracle step(s) "
                      f"(float64 numpy: Cayley-Neumann blocks, dense R W0 P forward, backward with block "
                      f"gradients and parameter gradients) in {el:.1f} s"}


def read_traffic():
    try:
        with open(TRAFFIC_FILE) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    if rec.get("gemm_source_sha256_16") != gemm_source_hash():
        return None   # kernel changed since the counters were taken
    return rec


def parse_pmc(pmc_dir):
    """Per-dispatch FETCH_SIZE / WRITE_SIZE (KiB) of the dense NT GEMM and of the
    reference copy, from rocprofv3 counter CSVs; writes TRAFFIC_FILE."""
    vals = {}
    for path in glob.glob(os.path.join(pmc_dir, "**", "*counter_collection.csv"), recursive=True):
        with open(path) as f:
            for row in csv.DictReader(f):
                name = row.get("Kernel_Name", "")
                cn = row.get("Counter_Name", "")
                v = float(row.get("Counter_Value", "nan"))
                if DENSE_KERNEL_TAG in name:
                    key = "gemm"
                elif COPY_KERNEL_TAG in name:
                    key = "copy"
                else:
                    continue
                vals.setdefault((key, cn), []).append(v)
    rec = {"gemm_source_sha256_16": gemm_source_hash(), "copy_bytes": COPY_BYTES}
    for cn in ("FETCH_SIZE", "WRITE_SIZE"):
        g = vals.get(("gemm", cn))
        c = vals.get(("copy", cn))
        if not g or not c:
            continue
        g_kib = sum(g) / len(g)
        c_kib = max(c)   # the 256 MiB copy is the largest copy dispatch
        scale = COPY_BYTES / (c_kib * 1024.0)
        rec[cn] = {"gemm_kib_per_dispatch": g_kib, "copy_kib": c_kib, "scale": scale,
                   "gemm_bytes_per_dispatch": g_kib * 1024.0 * scale}
    os.makedirs(os.path.dirname(TRAFFIC_FILE), exist_ok=True)
    with open(TRAFFIC_FILE, "w") as f:
        json.dump(rec, f, indent=1)
    print(json.dumps(rec))


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=100)
    ap.add_argument("--stage-reps", type=int, default=50)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--pmc-dir", default=None)
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
    spec = I.llama8b_q_proj()
    S, inp = build_state(spec)
    step = make_step(spec, S)

    # reference copy of known size (scale for the HBM counters)
    cs = torch.ones(COPY_BYTES // 2, dtype=torch.bfloat16, device="cuda")
    cd = torch.empty_like(cs)
    cd.copy_(cs)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(args.steps):
        step()
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / args.steps
    tok_s = spec.T / (ms / 1e3)

    st = stage_timings(spec, S, args.stage_reps)
    gemm_names = ["blk_fwd_P", "dense_fwd", "blk_fwd_R", "grad_R", "blk_bwd_R", "dense_bwd", "grad_P", "blk_bwd_P"]
    g_flops = sum(st[nm]["_flops"] for nm in gemm_names)
    g_us = sum(st[nm]["us"] for nm in gemm_names)
    gemm_tflops = g_flops / g_us / 1e6
    dense = st["dense_fwd"]
    dense_flops = dense["_flops"]
    traffic = read_traffic()
    tr = None
    if traffic and "FETCH_SIZE" in traffic and "WRITE_SIZE" in traffic:
        tr = round(traffic["FETCH_SIZE"]["gemm_bytes_per_dispatch"] + traffic["WRITE_SIZE"]["gemm_bytes_per_dispatch"])
    roof = {"kernel": "dense Wt GEMM, forward (h2 = h1 Wt^T, 2048 x 4096 x 4096, bf16, fp32 accumulate)",
            "bound": "mfma", "achieved": round(dense_flops / dense["us"] / 1e6, 1),
            "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
            "frac": round(dense_flops / dense["us"] / 1e6 / PEAK_BF16_TFLOPS, 4),
            "traffic": tr, "avg_launch_us": dense["us"],
            "algorithmic_flops_per_launch": dense_flops}
    for v in st.values():
        v.pop("_flops", None)

    out = {
        "metric": METRIC, "value": round(tok_s, 1), "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 4), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": "llama8b_q_proj: W0 4096x4096 bf16, b=256 (16+16 blocks), k=3, "
                               "1 x 2048 tokens, fast variant; step = cnp_fwd_save + linear_fwd + linear_bwd + "
                               "cnp_bwd_saved",
                   "global_batch": 1, "seq_len": spec.T, "parallelism": "single GPU"},
        "gemm_pct_peak": round(100 * gemm_tflops / PEAK_BF16_TFLOPS, 2),
        "gemm_tflops": round(gemm_tflops, 1),
        "gemm_gflop_per_step": round(g_flops / 1e9, 2),
        "stages": st,
        "roofline": roof,
    }
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(spec, inp)
    print(json.dumps(out))
    return 0


if __name__ == "__main__":
    sys.exit(main())
