"""Benchmark of the mLSTM matrix-memory hot path on one MI355X.

A timed step is one chunkwise parallel forward (mlstm_fwd_prepare +
mlstm_fwd_scan, i.e. mlstm_fwd_parallel) over the 1.3B-class layer, lm_1_3b:
B=4, NH=4, S=2048, d_qk=d_v=1024, chunk 64, bf16 q/k/v, fp32 gate
pre-activations, inputs resident in HBM.  `value` is forward tokens/s (B*S
tokens per step) from the wall clock around exactly --steps steps.

The same run times, each under a key of its own:
  "workloads"  the forward on the 125M-class layer (lm_125m: B=8, NH=4, S=2048,
               d=384, chunk 64) and on the long-context stress (long_ctx: B=1,
               NH=8, S=32768, d=256, chunk 128), each with its own roofline;
  "decode"     128 consecutive one-token steps (mlstm_step, batch 256, NH=4,
               d=512, fp32 state);
  "backward"   mlstm_bwd_parallel (gradients with respect to q, k, v and the three
               gate pre-activations, given dh) on lm_125m and long_ctx;
  "epilogue"   mlstm_block_epilogue (per-head GroupNorm, learnable skip, external
               output gate) on lm_125m's h shape;
  "slstm"      slstm_fwd on slstm_125m (B=8, NH=4, S=2048, d_h=192).

Forward roofline.  Algorithmic FLOPs per forward are
    B*NH*S*((L+1)*(d_qk+d_v) + 4*d_qk*d_v)
with L the chunk the kernels execute (a 128-token chunk runs as two 64-token
chunks on the matrix cores, so long_ctx counts L = 64); algorithmic bytes are
    B*NH*S*(2*(2*d_qk + d_v) + 8 + 4*d_v + 2*d_v) + B*NH*(4*d_qk*d_v + 4*d_qk + 4)
(q, k, v and h in bf16, i~ and f~ and o~ in fp32, the final state in fp32; the
workspace the two stages exchange is not algorithmic).  "roofline" is the whole
forward call (all its kernels, timed with HIP events on the stream they run on):
the MFMA fraction is reported as "frac" with "bound": "mfma" where the MFMA
ceiling is within 10% of the HBM one (lm_1_3b sits at the ridge: 56.7 us at the
bf16 peak against 58.8 us at the HBM peak), else the HBM fraction with "bound":
"hbm"; both fractions are always given.  "traffic" is the sum over every forward
kernel of the HBM bytes the TCC counters measured (profiles/hbm_traffic.json),
filled only while the forward's kernel source is the one profiled; its ratio to
the algorithmic bytes is "traffic_ratio".  "scan_roofline" is the dominant
kernel, chunk_scan, alone.

cpu_baseline: the fp64 oracle (oracle/, plain C + OpenMP over heads) timed on the
host on a bounded sample of the headline workload.

Backward: sequences of 1024 tokens or more (bf16, d_qk, d_v <= 512, and not the
GEMM form that widths above 384 take up to 16384 tokens) run the two-level form
with superchunks of 256 tokens.  Its algorithmic FLOPs are, per
head, the causal (t, s) pairs inside each superchunk times 6 (d_qk + d_v) (scores
and numerator recomputed, then dA, dq, dk and dv, one multiply-add each per pair
and dimension), plus 2 d_v d_qk (+ 2 d_qk for the normalizer) per token for each
of the six state products: C~ q and C~^T dnum' for the queries after the first
superchunk, dC~^T v and dC~ k for the keys before the last, and the two
per-superchunk state sums.  Shorter sequences and the GEMM form run the
quadratic form over all S(S+1)/2 pairs.  The whole call is timed with HIP events on its stream; its
roofline is against the bf16 MFMA peak.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
BF16_PEAK_TFLOPS = 2500.0      # MI355X dense bf16 MFMA
METRIC = "mLSTM fwd tokens/s + TFLOP/s (% bf16 MFMA peak); step tokens/s (% HBM BW)"
SCAN_SOURCE = os.path.join(ROOT, "mlstm_matrix_memory_amd", "csrc", "fwd_mfma_kernel.hip")
STEP_SOURCE = os.path.join(ROOT, "mlstm_matrix_memory_amd", "csrc", "step_kernel.hip")
EPILOGUE_SOURCE = os.path.join(ROOT, "mlstm_matrix_memory_amd", "csrc", "epilogue_kernel.hip")
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "hbm_traffic.json")


def exec_chunk(w) -> int:
    """Chunk the kernels execute: a 128-token chunk runs as two 64-token chunks."""
    return 64 if (w.dtype == "bf16" and w.chunk == 128) else w.chunk


def fwd_alg_flops(w) -> float:
    return float(w.B * w.NH * w.S) * ((exec_chunk(w) + 1) * (w.dqk + w.dv) + 4.0 * w.dqk * w.dv)


def scan_alg_bytes(w) -> float:
    e = 2
    per_tok = e * (2 * w.dqk + w.dv) + 4 * w.dv + e * w.dv
    return float(w.B * w.NH * w.S) * per_tok + float(w.B * w.NH) * (4 * w.dqk * w.dv + 4 * w.dqk + 4)


def fwd_alg_bytes(w) -> float:
    return scan_alg_bytes(w) + float(w.B * w.NH * w.S) * 8  # + i~, f~ (fp32)


def fwd_roofline(w, ms: float, kernel: str, flops: float, nbytes: float, traffic=None) -> dict:
    """Roofline of one forward-shaped unit of work timed at ms per call."""
    tflops = flops / (ms / 1e3) / 1e12
    gbs = nbytes / (ms / 1e3) / 1e9
    t_mfma = flops / (BF16_PEAK_TFLOPS * 1e12)
    t_hbm = nbytes / (HBM_PEAK_GBS * 1e9)
    mfma_bound = t_mfma >= 0.9 * t_hbm
    r = {"kernel": kernel, "bound": "mfma" if mfma_bound else "hbm",
         "achieved": tflops if mfma_bound else gbs,
         "peak": BF16_PEAK_TFLOPS if mfma_bound else HBM_PEAK_GBS,
         "unit": "TFLOP/s" if mfma_bound else "GB/s",
         "frac": tflops / BF16_PEAK_TFLOPS if mfma_bound else gbs / HBM_PEAK_GBS,
         "mfma_frac": tflops / BF16_PEAK_TFLOPS, "hbm_frac": gbs / HBM_PEAK_GBS,
         "tflops_alg": tflops, "hbm_gbs_alg": gbs,
         "alg_flops_per_launch": flops, "alg_bytes_per_launch": nbytes,
         "traffic": None, "traffic_ratio": None}
    if traffic is not None:
        r["traffic"] = traffic["bytes"]
        r["traffic_ratio"] = traffic["bytes"] / nbytes
        r["traffic_kernels"] = traffic["kernels"]
    return r


BWD_SUPERCHUNK = 256            # the backward's superchunk length from 1024 tokens on


def bwd_alg_flops(w) -> float:
    S, LS = w.S, BWD_SUPERCHUNK
    pair = 6.0 * (w.dqk + w.dv)
    d = max(w.dqk, w.dv)
    gemm_form = w.dtype == "bf16" and d > 384 and S <= 16384
    if gemm_form or S < 1024 or d > 512 or w.dtype != "bf16":
        return float(w.B * w.NH) * S * (S + 1) / 2 * pair
    G = (S + LS - 1) // LS
    band = sum(n * (n + 1) / 2 for n in [LS] * (G - 1) + [S - (G - 1) * LS])
    prod = 2.0 * w.dv * w.dqk + 2.0 * w.dqk       # one state product for one token
    later, earlier = S - LS, (G - 1) * LS          # queries after the first / keys before the last superchunk
    per_head = band * pair + prod * (2 * later + 2 * earlier + earlier + later)
    return float(w.B * w.NH) * per_head


def epilogue_alg_bytes(w) -> float:
    e = 2
    return float(w.B * w.NH * w.S * w.dv) * 4 * e + float(w.NH * w.dv) * 12   # h, x, z, y + parameters


def slstm_alg_flops(w) -> float:
    return float(w.B * w.NH * w.S) * 4 * w.dqk * w.dqk * 2     # the four recurrent matrix-vector products


def step_alg_bytes(w) -> float:
    e = 2
    per_head = 8 * w.dqk * w.dv + 8 * w.dqk + 8 + e * (2 * w.dqk + w.dv) + 8 + 4 * w.dv + e * w.dv
    return float(w.B * w.NH) * per_head


def source_hash(path: str) -> str:
    return hashlib.sha256(open(path, "rb").read()).hexdigest()[:16]


def _traffic_records():
    if not os.path.exists(TRAFFIC_FILE):
        return {}
    try:
        return json.load(open(TRAFFIC_FILE))
    except (ValueError, OSError):
        return {}


def measured_traffic(kernel: str, source: str, workload: str):
    """HBM bytes per launch from committed counter runs, if taken on this exact source and workload."""
    rec = _traffic_records().get(f"{kernel}:{workload}")
    if not rec or rec.get("source_sha") != source_hash(source):
        return None
    return rec.get("bytes_per_launch")


def forward_traffic(workload: str):
    """HBM bytes of one whole forward (every kernel it launches), from committed counter
    runs taken on this exact forward source, or None."""
    rec = _traffic_records().get(f"forward:{workload}")
    if not rec or rec.get("source_sha") != source_hash(SCAN_SOURCE):
        return None
    return {"bytes": rec["bytes_per_call"], "kernels": rec["kernels"]}


def cpu_baseline(w, x, budget_s: float = 12.0):
    """Time the fp64 oracle on whole sequences of the workload (all heads of each)."""
    import numpy as np
    import oracle
    orc = oracle.Oracle()
    cores = orc.num_threads()

    def run(nb):
        sl = slice(0, nb)
        args = [x[k][sl] for k in ("q", "k", "v", "i_pre", "f_pre", "o_pre")]
        args = [np.ascontiguousarray(a, dtype=np.float64) for a in args]
        t = time.perf_counter()
        orc.fwd(*args)
        return time.perf_counter() - t

    t = run(1)
    nb = max(1, min(w.B, int(budget_s / max(t, 1e-3))))
    if nb > 1:
        t = run(nb)
    reps = 1
    if t < 0.5 * budget_s:
        # the whole workload is a short sample: repeat it, so that the figure rests on
        # about budget_s of work rather than on one short run
        reps = max(1, min(50, int(budget_s / max(t, 1e-3))))
        t = sum(run(nb) for _ in range(reps))
    tok_s = reps * nb * w.S / t
    times = f", {reps} times" if reps > 1 else ""
    return {"value": tok_s, "unit": "tokens/s", "cores": cores, "kind": "oracle",
            "sample": f"{nb} of {w.B} sequences (all {w.NH} heads, S={w.S}, d={w.dqk}){times} in {t:.1f} s"}


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=30,
                    help="untimed steps first (fewer leave the clocks below steady state)")
    ap.add_argument("--workload", default="lm_1_3b")
    ap.add_argument("--extra-workloads", default="lm_125m,long_ctx",
                    help="forward workloads timed besides the headline one (comma list, '' for none)")
    ap.add_argument("--bwd-workloads", default="lm_125m,long_ctx")
    ap.add_argument("--decode-steps", type=int, default=128)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-decode", action="store_true")
    ap.add_argument("--no-bwd", action="store_true")
    ap.add_argument("--no-epilogue", action="store_true")
    ap.add_argument("--no-block", action="store_true",
                    help="skip the forward + block epilogue leg (fused against two calls)")
    ap.add_argument("--no-slstm", action="store_true")
    ap.add_argument("--bwd-steps", type=int, default=5)
    ap.add_argument("--bwd-warmup", type=int, default=10,
                    help="untimed backward calls first (the GPU idles while dh is generated on the host, "
                         "and the first calls after that run slow)")
    ap.add_argument("--copy-calibration-mib", type=int, default=0,
                    help="also run one plain device copy of this size (for counter calibration)")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU only: the library runs on a single MI355X and has no "
              "multi-GPU path (heads would shard across GPUs with no communication). "
              "Run with --gpus 1.", file=sys.stderr)
        return 2

    import numpy as np
    import torch

    from mlstm_matrix_memory_amd import (MLSTM_BF16, MLSTM_GATE_SWISH, inputs, mlstm_block_epilogue, slstm_fwd,
                                         mlstm_bwd_parallel, mlstm_bwd_workspace_bytes,
                                         mlstm_fwd_prepare, mlstm_fwd_scan, mlstm_fwd_workspace_bytes, mlstm_step,
                                         mlstm_fwd_block_workspace_bytes, mlstm_fwd_parallel,
                                         mlstm_fwd_parallel_block)

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    def gpu(a, dt):
        t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(dev)
        return t.to(torch.bfloat16) if dt == "bf16" else t

    def describe(w):
        return (f"{w.name}: mLSTM fwd B={w.B} NH={w.NH} S={w.S} d_qk={w.dqk} d_v={w.dv} "
                f"chunk={w.chunk} bf16 q/k/v, fp32 gates")

    # ---------------- forward ------------------------------------------------
    def time_forward(w, x, steps, warmup):
        """Warm up, then time exactly `steps` forwards (prepare + scan) on the current stream."""
        d = {k: gpu(v, w.dtype if k in ("q", "k", "v") else "f32") for k, v in x.items()}
        ws = torch.empty(max(1, mlstm_fwd_workspace_bytes(w.B, w.NH, w.S, w.dqk, w.dv, w.chunk, MLSTM_BF16)),
                         dtype=torch.uint8, device=dev)
        h = torch.empty((w.B, w.NH, w.S, w.dv), dtype=torch.bfloat16, device=dev)
        C = torch.empty((w.B, w.NH, w.dv, w.dqk), dtype=torch.float32, device=dev)
        n = torch.empty((w.B, w.NH, w.dqk), dtype=torch.float32, device=dev)
        m = torch.empty((w.B, w.NH), dtype=torch.float32, device=dev)
        fa = (d["q"], d["k"], d["v"], d["i_pre"], d["f_pre"], d["o_pre"], w.chunk)
        for _ in range(warmup):
            mlstm_fwd_prepare(*fa, workspace=ws)
            mlstm_fwd_scan(*fa, h, C, n, m, workspace=ws)
        torch.cuda.synchronize()
        # events on the current stream, the one the binding launches every kernel on
        evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(steps)]
        torch.cuda.synchronize()
        t_start = time.perf_counter()
        for s in range(steps):
            evs[s][0].record()
            mlstm_fwd_prepare(*fa, workspace=ws)
            evs[s][1].record()
            mlstm_fwd_scan(*fa, h, C, n, m, workspace=ws)
            evs[s][2].record()
        torch.cuda.synchronize()
        wall = time.perf_counter() - t_start
        res = {"ms_per_step": wall * 1e3 / steps,
               "prepare_ms": sum(e[0].elapsed_time(e[1]) for e in evs) / steps,
               "scan_ms": sum(e[1].elapsed_time(e[2]) for e in evs) / steps,
               "event_ms": sum(e[0].elapsed_time(e[2]) for e in evs) / steps}
        del d, ws, h, C, n, m
        torch.cuda.empty_cache()
        return res

    def fwd_record(w, t):
        flops, nbytes = fwd_alg_flops(w), fwd_alg_bytes(w)
        rec = {"workload": describe(w), "ms_per_step": t["ms_per_step"],
               "tokens_per_s": w.B * w.S / (t["ms_per_step"] / 1e3),
               "event_ms": t["event_ms"], "prepare_ms": t["prepare_ms"], "scan_ms": t["scan_ms"],
               "executed_chunk": exec_chunk(w),
               "roofline": fwd_roofline(w, t["event_ms"], "forward (all kernels of mlstm_fwd_parallel)",
                                        flops, nbytes, forward_traffic(w.name)),
               "scan_roofline": fwd_roofline(w, t["scan_ms"], "chunk_scan", flops, scan_alg_bytes(w),
                                             None)}
        tr = measured_traffic("chunk_scan", SCAN_SOURCE, w.name)
        if tr is not None:
            rec["scan_roofline"]["traffic"] = tr
            rec["scan_roofline"]["traffic_ratio"] = tr / scan_alg_bytes(w)
        return rec

    w = inputs.WORKLOADS[args.workload]
    x = inputs.fwd_inputs(w)
    t = time_forward(w, x, args.steps, args.warmup)
    head = fwd_record(w, t)
    ms_per_step = t["ms_per_step"]
    out = {
        "metric": METRIC,
        "value": head["tokens_per_s"],
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": describe(w),
                   "B": w.B, "NH": w.NH, "S": w.S, "d_qk": w.dqk, "d_v": w.dv, "chunk": w.chunk},
        "fwd": {"tflops_alg": head["roofline"]["tflops_alg"], "mfma_frac": head["roofline"]["mfma_frac"],
                "hbm_gbs_alg": head["roofline"]["hbm_gbs_alg"], "hbm_frac": head["roofline"]["hbm_frac"],
                "event_ms": t["event_ms"], "prepare_ms": t["prepare_ms"], "scan_ms": t["scan_ms"],
                "executed_chunk": exec_chunk(w)},
        "roofline": head["roofline"],
        "scan_roofline": head["scan_roofline"],
    }
    head_x = x
    del x

    extra = [nm for nm in args.extra_workloads.split(",") if nm and nm != w.name]
    if extra:
        out["workloads"] = {}
        for nm in extra:
            we = inputs.WORKLOADS[nm]
            xe = inputs.fwd_inputs(we)
            te = time_forward(we, xe, args.steps, args.warmup)
            del xe
            out["workloads"][nm] = fwd_record(we, te)

    # ---------------- backward ------------------------------------------------
    if not args.no_bwd:
        out["backward"] = {}
        for nm in [b for b in args.bwd_workloads.split(",") if b]:
            wb = inputs.WORKLOADS[nm]
            xb = head_x if nm == w.name else inputs.fwd_inputs(wb)
            db = {k: gpu(v, wb.dtype if k in ("q", "k", "v") else "f32") for k, v in xb.items()}
            del xb
            fb = (db["q"], db["k"], db["v"], db["i_pre"], db["f_pre"], db["o_pre"])
            dh = gpu(inputs.bwd_dh(wb), wb.dtype)
            bws = torch.empty(max(1, mlstm_bwd_workspace_bytes(wb.B, wb.NH, wb.S, wb.dqk, wb.dv, MLSTM_BF16)),
                              dtype=torch.uint8, device=dev)
            grads = mlstm_bwd_parallel(*fb, dh, workspace=bws)
            for _ in range(max(0, args.bwd_warmup - 1)):
                mlstm_bwd_parallel(*fb, dh, grads=grads, workspace=bws)
            torch.cuda.synchronize()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            t_start = time.perf_counter()
            e0.record()
            for _ in range(args.bwd_steps):
                mlstm_bwd_parallel(*fb, dh, grads=grads, workspace=bws)
            e1.record()
            torch.cuda.synchronize()
            bwall = time.perf_counter() - t_start
            bwd_ms = e0.elapsed_time(e1) / args.bwd_steps
            bflops = bwd_alg_flops(wb)
            btf = bflops / (bwd_ms / 1e3) / 1e12
            out["backward"][nm] = {
                "workload": f"{wb.name}: mlstm_bwd_parallel B={wb.B} NH={wb.NH} S={wb.S} d_qk={wb.dqk} "
                            f"d_v={wb.dv} bf16 q/k/v/dh, fp32 gradients",
                "tokens_per_s": wb.B * wb.S * args.bwd_steps / bwall, "ms_per_call": bwd_ms,
                "roofline": {"kernel": "mlstm_bwd_parallel (whole call)", "bound": "mfma", "achieved": btf,
                             "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s", "frac": btf / BF16_PEAK_TFLOPS,
                             "traffic": None, "alg_flops_per_call": bflops},
            }
            del db, fb, dh, bws, grads
            torch.cuda.empty_cache()

    # ---------------- block epilogue ------------------------------------------
    if not args.no_epilogue:
        w = inputs.WORKLOADS["lm_125m"]
        ex = inputs.epilogue_inputs(w)
        de = {k: gpu(v, w.dtype if k in ("h", "x", "z") else "f32") for k, v in ex.items()}
        del ex
        y = torch.empty_like(de["h"])
        ea = (de["h"], de["x"], de["z"], de["gn_w"], de["gn_b"], de["skip_w"])
        for _ in range(3):
            mlstm_block_epilogue(*ea, eps=1e-5, act=MLSTM_GATE_SWISH, y_out=y)
        torch.cuda.synchronize()
        n_ep = 20
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(n_ep):
            mlstm_block_epilogue(*ea, eps=1e-5, act=MLSTM_GATE_SWISH, y_out=y)
        e1.record()
        torch.cuda.synchronize()
        ep_ms = e0.elapsed_time(e1) / n_ep
        ep_bytes = epilogue_alg_bytes(w)
        ep_gbs = ep_bytes / (ep_ms / 1e3) / 1e9
        out["epilogue"] = {
            "workload": f"{w.name}: mlstm_block_epilogue B={w.B} NH={w.NH} S={w.S} d_v={w.dv} bf16 h/x/z/y, "
                        "swish gate",
            "us_per_call": ep_ms * 1e3,
            "roofline": {"kernel": "epilogue_kernel", "bound": "hbm", "achieved": ep_gbs, "peak": HBM_PEAK_GBS,
                         "unit": "GB/s", "frac": ep_gbs / HBM_PEAK_GBS,
                         "traffic": measured_traffic("epilogue_kernel", EPILOGUE_SOURCE, w.name),
                         "alg_bytes_per_launch": ep_bytes},
        }
        del de, y, ea
        torch.cuda.empty_cache()

    # ---------------- forward + block epilogue --------------------------------
    # mlstm_fwd_parallel_block on a shape with one value tile per head, where the
    # scan applies the epilogue itself, against mlstm_fwd_parallel followed by
    # mlstm_block_epilogue on the same inputs (events over 10 calls each)
    if not args.no_block:
        wb = inputs.WORKLOADS["heads64"]
        xb = inputs.fwd_inputs(wb)
        eb = inputs.epilogue_inputs(wb)
        db = [gpu(xb[k], "bf16" if k in ("q", "k", "v") else "f32") for k in ("q", "k", "v", "i_pre", "f_pre", "o_pre")]
        xe, ze = gpu(eb["x"], "bf16"), gpu(eb["z"], "bf16")
        gw, gb, sw = (gpu(eb[k], "f32") for k in ("gn_w", "gn_b", "skip_w"))
        del xb, eb
        yb = torch.empty_like(xe)
        hb = torch.empty_like(xe)
        Cb = torch.empty((wb.B, wb.NH, wb.dv, wb.dqk), dtype=torch.float32, device=dev)
        nb = torch.empty((wb.B, wb.NH, wb.dqk), dtype=torch.float32, device=dev)
        mb = torch.empty((wb.B, wb.NH), dtype=torch.float32, device=dev)
        wsb = torch.empty(max(1, mlstm_fwd_block_workspace_bytes(wb.B, wb.NH, wb.S, wb.dqk, wb.dv, wb.chunk,
                                                                 MLSTM_BF16, 1)), dtype=torch.uint8, device=dev)
        wsb0 = torch.empty(max(1, mlstm_fwd_block_workspace_bytes(wb.B, wb.NH, wb.S, wb.dqk, wb.dv, wb.chunk,
                                                                  MLSTM_BF16, 0)), dtype=torch.uint8, device=dev)
        wsf = torch.empty(max(1, mlstm_fwd_workspace_bytes(wb.B, wb.NH, wb.S, wb.dqk, wb.dv, wb.chunk, MLSTM_BF16)),
                          dtype=torch.uint8, device=dev)

        def fused():
            mlstm_fwd_parallel_block(*db, xe, ze, gw, gb, sw, wb.chunk, eps=1e-5, act=MLSTM_GATE_SWISH, fuse=1,
                                     y_out=yb, C_final=Cb, n_final=nb, m_final=mb, workspace=wsb)

        def unfused():
            mlstm_fwd_parallel_block(*db, xe, ze, gw, gb, sw, wb.chunk, eps=1e-5, act=MLSTM_GATE_SWISH, fuse=0,
                                     y_out=yb, C_final=Cb, n_final=nb, m_final=mb, workspace=wsb0)

        def two_calls():
            mlstm_fwd_parallel(*db, wb.chunk, h_out=hb, C_final=Cb, n_final=nb, m_final=mb, workspace=wsf)
            mlstm_block_epilogue(hb, xe, ze, gw, gb, sw, eps=1e-5, act=MLSTM_GATE_SWISH, y_out=yb)

        def time_calls(fn, n=10):
            for _ in range(5):
                fn()
            torch.cuda.synchronize()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            for _ in range(n):
                fn()
            e1.record()
            torch.cuda.synchronize()
            return e0.elapsed_time(e1) / n

        t_two = time_calls(two_calls)
        t_fused = time_calls(fused)
        t_unfused = time_calls(unfused)
        out["block"] = {
            "workload": f"{describe(wb)}; block epilogue (swish gate) on h",
            "fuse1_ms": t_fused, "fuse0_ms": t_unfused, "two_calls_ms": t_two,
            "tokens_per_s_fuse0": wb.B * wb.S / (t_unfused / 1e3),
        }
        del db, xe, ze, gw, gb, sw, yb, hb, Cb, nb, mb, wsb, wsb0, wsf
        torch.cuda.empty_cache()

    # ---------------- sLSTM recurrence -----------------------------------------
    if not args.no_slstm:
        wsl = inputs.WORKLOADS["slstm_125m"]
        xs = inputs.slstm_inputs(wsl)
        xp, Rs = gpu(xs["x_pre"], "f32"), gpu(xs["R"], wsl.dtype)
        del xs
        so = slstm_fwd(xp, Rs)
        torch.cuda.synchronize()
        n_sl = 3
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        t_start = time.perf_counter()
        e0.record()
        for _ in range(n_sl):
            slstm_fwd(xp, Rs, 0, None, None, None, None, *so)
        e1.record()
        torch.cuda.synchronize()
        swall = time.perf_counter() - t_start
        sl_ms = e0.elapsed_time(e1) / n_sl
        sflops = slstm_alg_flops(wsl)
        stf = sflops / (sl_ms / 1e3) / 1e12
        out["slstm"] = {
            "workload": f"slstm_125m: slstm_fwd B={wsl.B} NH={wsl.NH} S={wsl.S} d_h={wsl.dqk} bf16 R, fp32 gates",
            "tokens_per_s": wsl.B * wsl.S * n_sl / swall, "ms_per_call": sl_ms,
            "us_per_step": sl_ms * 1e3 / wsl.S, "workgroups": wsl.NH * ((wsl.B + 3) // 4),
            "roofline": {"kernel": "slstm_kernel", "bound": "mfma", "achieved": stf, "peak": BF16_PEAK_TFLOPS,
                         "unit": "TFLOP/s", "frac": stf / BF16_PEAK_TFLOPS, "traffic": None,
                         "alg_flops_per_launch": sflops},
        }
        del xp, Rs, so
        torch.cuda.empty_cache()

    # ---------------- decode step ---------------------------------------------
    if not args.no_decode:
        wd = inputs.WORKLOADS["decode"]
        T = args.decode_steps
        st = inputs.step_state(wd)
        xs = inputs.step_inputs(wd, steps=T)
        C0 = gpu(st["C"], "f32")
        n0 = gpu(st["n"], "f32")
        m0 = gpu(st["m"], "f32")
        dx = {k: gpu(v, "bf16" if k in ("q", "k", "v") else "f32") for k, v in xs.items()}
        del xs, st
        Cw, nw, mw = C0.clone(), n0.clone(), m0.clone()
        hd = torch.empty((wd.B, wd.NH, wd.dv), dtype=torch.bfloat16, device=dev)

        def one(t):
            mlstm_step(dx["q"][t], dx["k"][t], dx["v"][t], dx["i_pre"][t], dx["f_pre"][t], dx["o_pre"][t],
                       Cw, nw, mw, hd)
        for t in range(min(8, T)):
            one(t)
        Cw.copy_(C0); nw.copy_(n0); mw.copy_(m0)   # pristine state, outside the timed region
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        t_start = time.perf_counter()
        e0.record()
        for t in range(T):
            one(t)
        e1.record()
        torch.cuda.synchronize()
        dwall = time.perf_counter() - t_start
        dev_ms = e0.elapsed_time(e1)
        step_bytes = step_alg_bytes(wd)
        step_gbs = step_bytes * T / (dev_ms / 1e3) / 1e9
        out["decode"] = {
            "workload": f"decode: mlstm_step batch={wd.B} NH={wd.NH} d_qk=d_v={wd.dqk} fp32 state, "
                        f"bf16 q/k/v, {T} consecutive steps",
            "tokens_per_s": wd.B * T / (dwall), "us_per_step": dev_ms * 1e3 / T,
            "roofline": {"kernel": "step_kernel", "bound": "hbm", "achieved": step_gbs, "peak": HBM_PEAK_GBS,
                         "unit": "GB/s", "frac": step_gbs / HBM_PEAK_GBS,
                         "traffic": measured_traffic("step_kernel", STEP_SOURCE, wd.name),
                         "alg_bytes_per_launch": step_bytes},
        }
        del C0, n0, m0, Cw, nw, mw, dx
        torch.cuda.empty_cache()

    if args.copy_calibration_mib > 0:
        nbytes = args.copy_calibration_mib * (1 << 20)
        src = torch.empty(nbytes // 4, dtype=torch.float32, device=dev).fill_(1.0)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        torch.neg(src, out=dst)   # one elementwise kernel: reads and writes nbytes each
        torch.cuda.synchronize()
        out["copy_calibration_bytes"] = nbytes

    # ---------------- CPU baseline (oracle) ------------------------------------
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(inputs.WORKLOADS[args.workload], head_x)

    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
