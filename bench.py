"""Benchmark: prefill tokens/s and decode state GB/s of the gated delta rule on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--decode-steps D] [--no-cpu-baseline]
    python bench.py --copy-calibration      (a plain 256 MiB device copy, for HBM counter scaling)
    python bench.py --prefill-only          (the headline prefill and its halves only, for profilers)
    python bench.py --fused-norm-only       (the prefill with the gated norm fused onto o, for profilers)

Prints ONE JSON line.  The timed step is one gdn_chunk_fwd call over the Qwen3-Next-shaped prefill
workload (B=1, T=4096, 16 q/k heads, 32 v heads, head dim 128, bf16 inputs, fp32 state and output),
inputs resident in HBM.  ``value`` is prefill tokens/s over K back-to-back steps.  The same run then
times the call's two halves on their own (gdn_chunk_fwd_prepare: every chunk's triangular solve;
gdn_chunk_fwd_scan: the in-order pass, the dominant kernel, which ``roofline`` describes), and the
decode workload (256 sequences, 2 MiB fp32 state each, D one-token steps of gdn_recurrent_step),
reported under ``decode``.

Roofline figures use algorithmic work only:
  prefill, per (token, v-head): bytes  = q,k (bf16, shared by Hv/Hk v-heads) + v (bf16) + g, beta
                                         (bf16) + o (fp32) = 1028 B at d = 128, G = 2;
                                         plus the fp32 initial/final state per (sequence, v-head).
                                         The scan kernel's share is the same without g and beta
                                         (1024 B), which its roofline uses.
                                 flops = 6 dk dv + C (3 dk + 2 dv)  (C = 64; the three d x d
                                         contractions per token and the lower-triangular intra-chunk
                                         products, the triangular solve not counted).
  decode, per step:              bytes = state read + write (2 B Hv dk dv 4) + q, k, v, g, beta, o.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

MI355X_HBM_GBS = 8000.0        # HBM3E peak, GB/s
MI355X_BF16_TFLOPS = 2500.0    # dense bf16 matrix peak, TFLOP/s
MI355X_F32_TFLOPS = 157.3      # fp32 peak (vector and dense matrix alike), TFLOP/s

# The chunked backward's products per 64-token chunk and v-head at dk = dv = 128, each counted once
# (not per state slice): K K^T, Q K^T (lower halves); the forward sweep's K S, T (beta X), K^T (f U);
# the reverse sweep's K S, T (beta X), K D, Q S, P^T dO, T^T dU, dY U^T, dO U^T (lower halves where
# triangular), the dq / dk terms dO S^T, U D^T, dY S^T, the state gradient's Q^T dO, K^T dY, and the
# three C x C x dk products of dq and dk: 13.37 M multiply-adds, 2 flops each, per 64 tokens.
BWD_FLOPS_PER_TOKEN_VHEAD = 2 * (64 * 64 * 128 + 10 * 64 * 128 * 128 + 6 * 64 * 64 * 128 // 2
                                 + 3 * 64 * 64 * 128 // 2) // 64
CHUNK = 64

METRIC = "prefill tokens/s + decode state GB/s, gated delta rule, Qwen3-Next shape, 1 GPU"

# Counter readings per launch from rocprofv3 (profiles/): HBM bytes from FETCH_SIZE and WRITE_SIZE, each
# scaled by what the same counter reads on a plain copy of known size, and the matrix-core work from
# SQ_INSTS_VALU_MFMA_MOPS_* (units of 512 flops).  Each reading was taken at the version of its
# kernel's source file whose hash it names; when the file has changed since, it is reported as null.
# (chunk_mfma.hip's HBM readings were taken at sha16 538da900da46eea7, since when only a comment
# changed; its matrix-core reading at the current source.
# chunk_bwd.hip's readings were taken at sha16 04610cae2a836398; since then only comments changed.)
COUNTERS = {
    "scan": {"source": "gated_deltanet_delta_amd/csrc/chunk_mfma.hip", "sha16": "f5f86e9959c219d4",
             "traffic": 160440667, "mfma_exec_flops": (80740352 + 7274496) * 512},
    "solve": {"source": "gated_deltanet_delta_amd/csrc/chunk_mfma.hip", "sha16": "f5f86e9959c219d4",
              "traffic": 43558845},
    "scan_norm": {"source": "gated_deltanet_delta_amd/csrc/chunk_mfma.hip", "sha16": "f5f86e9959c219d4",
                  "traffic": 169155707, "prepare_traffic": 47753149},
    "decode": {"source": "gated_deltanet_delta_amd/csrc/recurrent.hip", "sha16": "df00f8ca898a19e2",
               "traffic": 1085280816},
    "conv": {"source": "gated_deltanet_delta_amd/csrc/conv1d.hip", "sha16": "592040b86d906439",
             "traffic": 134710246},
    "norm": {"source": "gated_deltanet_delta_amd/csrc/norm.hip", "sha16": "e94d82c291e7fd2c",
             "traffic": 134250675},
    "bwd": {"source": "gated_deltanet_delta_amd/csrc/chunk_bwd.hip", "sha16": "4bbae852a1b2b7dc",
            "mfma_exec_f32_flops": (10485760 + 36700160 + 327680) * 512,
            "mfma_exec_bf16_flops": 176160768 * 512,
            "traffic": round((207879.1875 + 312944.875 + 16956.25) * 1.9998 * 1024
                             + (477808.71875 + 67957.75 + 98304.125) * 1024)},
}


def source_sha16(rel: str) -> str:
    import hashlib
    with open(os.path.join(ROOT, rel), "rb") as fh:
        return hashlib.sha256(fh.read()).hexdigest()[:16]


def counter(kernel: str, key: str):
    """A counter reading if it was taken at the kernel's current source, else None."""
    c = COUNTERS[kernel]
    if c.get(key) is None or c["sha16"] != source_sha16(c["source"]):
        return None
    return c[key]


def prefill_algorithmic(wl, T: int, B: int, N: int, init_state: bool):
    el = 2 if str(wl.dtype).endswith("bfloat16") else 4
    gel = 2 if str(wl.gate_dtype).endswith("bfloat16") else 4
    G = wl.Hv // wl.Hk
    per_tok_head = (2 * wl.dk * el) / G + wl.dv * el + 2 * gel + wl.dv * 4
    state = wl.dk * wl.dv * 4 * (2 if init_state else 1)
    nbytes = B * T * wl.Hv * per_tok_head + N * wl.Hv * state
    flops = B * T * wl.Hv * (6 * wl.dk * wl.dv + CHUNK * (3 * wl.dk + 2 * wl.dv))
    return nbytes, flops, per_tok_head


def decode_algorithmic(wl):
    el = 2
    gel = 4
    state = 2 * wl.B * wl.Hv * wl.dk * wl.dv * 4
    io = wl.B * (2 * wl.Hk * wl.dk * el + wl.Hv * wl.dv * el + 2 * wl.Hv * gel + wl.Hv * wl.dv * 4)
    return state, state + io


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=200)
    ap.add_argument("--decode-steps", type=int, default=128)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--prefill-only", action="store_true",
                    help="only the headline prefill and its two halves (for profiler runs)")
    ap.add_argument("--fused-norm-only", action="store_true",
                    help="only the prefill with the gated norm fused onto o, on the same inputs (profiler runs)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain 256 MiB device-to-device copy (HBM counter scaling)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported (the gated delta "
              "rule path here is a single-GPU build)", file=sys.stderr)
        return 2

    import numpy as np
    import ctypes

    import torch

    from gated_deltanet_delta_amd import _lib
    from gated_deltanet_delta_amd import (gdn_causal_conv1d, gdn_chunk_fwd, gdn_chunk_fwd_ex,
                                          gdn_chunk_bwd, gdn_chunk_bwd_ex, gdn_chunk_fwd_gating,
                                          gdn_chunk_fwd_gated_norm, gdn_gated_rmsnorm,
                                          gdn_recurrent_step, gdn_recurrent_step_gating, synth,
                                          workspace_size)

    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)

    if args.copy_calibration:
        nbytes = 256 << 20
        src = torch.ones(nbytes // 4, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        for _ in range(4):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes_read": nbytes, "copy_calibration_bytes_written": nbytes,
                          "launches": 4}), flush=True)
        return 0

    # ---------------- prefill -----------------------------------------------------------------
    # Four input sets (the workload's own draw and three more seeds), ~137 MB each with o: together
    # larger than the GPU's 256 MB last-level cache, so that calls cycling through them read their
    # inputs from HBM.  Repeating one set would leave most of it in that cache between calls.
    wl = synth.WORKLOADS["prefill"]
    B, T = wl.B, wl.T
    N = B
    NSETS = 4
    sets = []
    for i in range(NSETS):
        xi = synth.make(wl) if i == 0 else synth.make(wl, seed=wl.seed + 1000 + i)
        di = {key: (None if xi[key] is None else xi[key].to(dev).contiguous())
              for key in ("q", "k", "v", "g", "beta", "initial_state", "cu_seqlens")}
        raw_i = xi["raw"]
        di["a"] = torch.from_numpy(raw_i["a"]).to(wl.gate_dtype).to(dev)
        di["b"] = torch.from_numpy(raw_i["b"]).to(wl.gate_dtype).to(dev)
        di["A_log"] = torch.from_numpy(raw_i["A_log"]).to(dev)
        di["dt_bias"] = torch.from_numpy(raw_i["dt_bias"]).to(dev)
        di["o"] = torch.empty((B, T, wl.Hv, wl.dv), dtype=torch.float32, device=dev)
        di["fs"] = torch.empty((N, wl.Hv, wl.dk, wl.dv), dtype=torch.float32, device=dev)
        sets.append(di)
        if i == 0:
            x = xi
    d, o, fs = sets[0], sets[0]["o"], sets[0]["fs"]
    ga, gb, gA, gdt = d["a"], d["b"], d["A_log"], d["dt_bias"]
    ws_bytes = workspace_size(B, T, wl.Hk, wl.Hv, wl.dk, wl.dv, N, wl.dtype)
    ws = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device=dev)   # one workspace, shared

    def prefill_step(stage="all", i=0):
        s_ = sets[i % NSETS]
        gdn_chunk_fwd(s_["q"], s_["k"], s_["v"], s_["g"], s_["beta"], s_["initial_state"], None,
                      o=s_["o"], final_state=s_["fs"], workspace=ws, stage=stage)

    # Warm-up: at least --warmup calls and at least 0.3 s of them, whatever --warmup says (the
    # GPU's clocks take a few milliseconds of sustained work to settle; a cold stretch reads slow).
    warm0, warm_calls = time.perf_counter(), 0
    while warm_calls < args.warmup or time.perf_counter() - warm0 < 0.3:
        prefill_step(i=warm_calls)
        warm_calls += 1
        if warm_calls % 50 == 0:
            torch.cuda.synchronize()
    torch.cuda.synchronize()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    ev0.record()
    for i in range(args.steps):
        prefill_step(i=i)
    ev1.record()
    torch.cuda.synchronize()
    wall1 = time.perf_counter()
    ms_events = ev0.elapsed_time(ev1) / args.steps
    ms_wall = (wall1 - wall0) * 1e3 / args.steps
    tokens = B * T
    value = tokens / (ms_wall / 1e3)
    nbytes, flops, per_tok_head = prefill_algorithmic(wl, T, B, N, wl.init_state)
    gate_bytes = B * T * wl.Hv * 2 * (2 if str(wl.gate_dtype).endswith("bfloat16") else 4)
    scan_bytes = nbytes - gate_bytes

    def time_loop(fn):
        """ms per call over args.steps calls, fn(i) cycling through the input sets."""
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for i in range(args.steps):
            fn(i)
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / args.steps

    # for context: the same call repeated on one set of buffers (mostly last-level-cache resident)
    ms_same_buffers = time_loop(lambda i: prefill_step())

    # the two halves on their own, each timed with events on the stream the kernels run on
    # (torch's current stream, which the binding passes to the library)
    def time_stage(stage):
        prefill_step("prepare")     # scan reads what prepare left in the workspace
        return time_loop(lambda i: prefill_step(stage, i))

    ms_prepare = time_stage("prepare")
    ms_scan = time_stage("scan")
    if args.fused_norm_only:
        zr0 = np.random.default_rng(99).standard_normal((B, T, wl.Hv, wl.dv), dtype=np.float32)
        zs = [torch.from_numpy(zr0).to(torch.bfloat16).to(dev) for _ in range(NSETS)]
        ys = [torch.empty((B, T, wl.Hv, wl.dv), dtype=torch.bfloat16, device=dev) for _ in range(NSETS)]
        w1 = torch.ones(wl.dv, dtype=torch.float32, device=dev)
        fws_ = torch.empty(int(_lib.load().gdn_chunk_fwd_gated_norm_workspace_size(
            B, T, wl.Hk, wl.Hv, wl.dk, wl.dv, N, _lib.GDN_BF16)), dtype=torch.uint8, device=dev)

        def fused_only(i):
            s_ = sets[i % NSETS]
            gdn_chunk_fwd_gated_norm(s_["q"], s_["k"], s_["v"], s_["g"], s_["beta"], zs[i % NSETS], w1, 1e-6,
                                     initial_state=s_["initial_state"], y=ys[i % NSETS], final_state=s_["fs"],
                                     workspace=fws_)

        for i in range(max(args.warmup, 20)):
            fused_only(i)
        ms_f = time_loop(fused_only)
        print(json.dumps({"workload": "prefill B=1 T=4096 Hk=16 Hv=32 dk=dv=128 bf16 in, gated norm fused "
                                      "(bf16 z, y)", "ms_per_call_events": round(ms_f, 5),
                          "tokens_per_s": round(tokens / (ms_f / 1e3), 1)}), flush=True)
        return 0
    if args.prefill_only:
        print(json.dumps({"workload": "prefill B=1 T=4096 Hk=16 Hv=32 dk=dv=128 bf16 in",
                          "tokens_per_s": round(tokens / (ms_wall / 1e3), 1), "ms_per_call_wall": round(ms_wall, 5),
                          "ms_per_call_events": round(ms_events, 5), "ms_scan_events": round(ms_scan, 5),
                          "ms_prepare_events": round(ms_prepare, 5),
                          "scan_useful_mfma_frac": round(flops / (ms_scan / 1e3) / 1e12 / MI355X_BF16_TFLOPS, 4),
                          "scan_hbm_frac": round(scan_bytes / (ms_scan / 1e3) / 1e9 / MI355X_HBM_GBS, 4)}),
              flush=True)
        return 0

    # the same prefill with the gates formed in the kernels from the raw projections a, b
    def prefill_gating(i):
        s_ = sets[i % NSETS]
        gdn_chunk_fwd_gating(s_["q"], s_["k"], s_["v"], s_["a"], s_["b"], s_["A_log"], s_["dt_bias"],
                             s_["initial_state"], None, o=s_["o"], final_state=s_["fs"], workspace=ws)

    for i in range(args.warmup):
        prefill_gating(i)
    ms_gating = time_loop(prefill_gating)

    # and with q, k normalised to unit length in the kernels as well (every fused input step)
    def prefill_gating_l2(i):
        s_ = sets[i % NSETS]
        gdn_chunk_fwd_ex(s_["q"], s_["k"], s_["v"], s_["a"], s_["b"], A_log=s_["A_log"], dt_bias=s_["dt_bias"],
                         initial_state=s_["initial_state"], qk_l2norm=True, o=s_["o"], final_state=s_["fs"],
                         workspace=ws)

    for i in range(args.warmup):
        prefill_gating_l2(i)
    ms_gating_l2 = time_loop(prefill_gating_l2)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    achieved_gbs = scan_bytes / (ms_scan / 1e3) / 1e9
    useful_tflops = flops / (ms_events / 1e3) / 1e12
    scan_useful_tflops = flops / (ms_scan / 1e3) / 1e12
    scan_traffic = counter("scan", "traffic")
    scan_exec = counter("scan", "mfma_exec_flops")
    prep_traffic = counter("solve", "traffic")
    call_traffic = None if scan_traffic is None or prep_traffic is None else scan_traffic + prep_traffic

    # ---------------- ceilings measured on this GPU in the same run ----------------------------
    # bf16 GEMM through torch.matmul (the vendor library), 8192^3, and a plain 1 GiB device copy
    ga_ = torch.randn(8192, 8192, device=dev).to(torch.bfloat16)
    gb_ = torch.randn(8192, 8192, device=dev).to(torch.bfloat16)
    for _ in range(5):
        gc_ = torch.matmul(ga_, gb_)
    torch.cuda.synchronize()
    e0.record()
    for _ in range(20):
        gc_ = torch.matmul(ga_, gb_)
    e1.record()
    torch.cuda.synchronize()
    gemm_tflops = 2 * 8192 ** 3 / (e0.elapsed_time(e1) / 20 / 1e3) / 1e12
    del ga_, gb_, gc_
    csrc_ = torch.empty(1 << 28, dtype=torch.float32, device=dev).fill_(1.0)
    cdst_ = torch.empty_like(csrc_)
    for _ in range(3):
        cdst_.copy_(csrc_)
    torch.cuda.synchronize()
    e0.record()
    for _ in range(20):
        cdst_.copy_(csrc_)
    e1.record()
    torch.cuda.synchronize()
    copy_gbs = 2 * csrc_.numel() * 4 / (e0.elapsed_time(e1) / 20 / 1e3) / 1e9
    del csrc_, cdst_
    torch.cuda.empty_cache()
    ceilings = {"bf16_gemm_tflops": round(gemm_tflops, 1), "bf16_gemm": "torch.matmul 8192x8192x8192 bf16",
                "copy_gbs": round(copy_gbs, 1), "copy": "torch copy_ of 1 GiB (read + write counted)"}

    # ---------------- ablation: the same prefill through the token-serial (recurrent) kernel ----
    # gdn_recurrent_step with all 4096 tokens in one call: the state stays in registers and the tokens
    # are taken one after another, the pure-RNN mode the chunked form replaces
    st_r = torch.zeros((B, wl.Hv, wl.dk, wl.dv), dtype=torch.float32, device=dev)
    o_r = torch.empty_like(o)
    gdn_recurrent_step(d["q"], d["k"], d["v"], d["g"], d["beta"], st_r, o=o_r)
    torch.cuda.synchronize()
    e0.record()
    for _ in range(3):
        gdn_recurrent_step(d["q"], d["k"], d["v"], d["g"], d["beta"], st_r, o=o_r)
    e1.record()
    torch.cuda.synchronize()
    ms_recurrent = e0.elapsed_time(e1) / 3
    del st_r, o_r
    ablation = {"workload": "the prefill above", "recurrent_call": "gdn_recurrent_step, T=4096 in one call",
                "ms_recurrent": round(ms_recurrent, 4), "ms_chunked": round(ms_events, 5),
                "chunked_speedup": round(ms_recurrent / ms_events, 2),
                "pages_claim": "chunk mode 4-6x faster than a pure RNN in training (Qwen3-Next article, "
                               "jsqmd.com, section 2.2; hardware unstated)"}

    # ---------------- head size 64 with bf16 inputs --------------------------------------------
    w64 = synth.Workload(**{**wl.__dict__, "dk": 64, "dv": 64})
    x64 = synth.make(w64, seed=wl.seed + 64)
    d64 = {key: (None if x64[key] is None else x64[key].to(dev).contiguous())
           for key in ("q", "k", "v", "g", "beta")}
    del x64
    o64 = torch.empty((B, T, wl.Hv, 64), dtype=torch.float32, device=dev)
    f64_ = torch.empty((N, wl.Hv, 64, 64), dtype=torch.float32, device=dev)
    ws64 = torch.empty(max(workspace_size(B, T, wl.Hk, wl.Hv, 64, 64, N, wl.dtype), 1), dtype=torch.uint8,
                       device=dev)
    call64 = lambda: gdn_chunk_fwd(d64["q"], d64["k"], d64["v"], d64["g"], d64["beta"], None, None,  # noqa: E731
                                   o=o64, final_state=f64_, workspace=ws64)
    for _ in range(10):
        call64()
    torch.cuda.synchronize()
    e0.record()
    for _ in range(20):
        call64()
    e1.record()
    torch.cuda.synchronize()
    ms64 = e0.elapsed_time(e1) / 20
    nb64, fl64, _ = prefill_algorithmic(w64, T, B, N, False)
    dk64_res = {"workload": f"prefill B=1 T={T} Hk={wl.Hk} Hv={wl.Hv} dk=dv=64 bf16 in, fp32 state/out",
                "ms_per_call_events": round(ms64, 5), "tokens_per_s": round(tokens / (ms64 / 1e3), 1),
                "useful_tflops": round(fl64 / (ms64 / 1e3) / 1e12, 2),
                "achieved_gbs": round(nb64 / (ms64 / 1e3) / 1e9, 1)}
    del d64, o64, f64_, ws64

    clib = _lib.load()

    def time_c(fn, arg_sets):
        """ms per call of a C entry point over args.steps back-to-back calls (after the warm-up),
        cycling through the argument sets: three sets of buffers are larger than the GPU's 256 MB
        last-level cache, so every call reads and writes HBM rather than the previous call's lines."""
        for i in range(args.warmup):
            if fn(*arg_sets[i % len(arg_sets)]) != 0:
                raise RuntimeError(f"{fn.__name__} failed")
        torch.cuda.synchronize()
        e0.record()
        for i in range(args.steps):
            fn(*arg_sets[i % len(arg_sets)])
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / args.steps

    # ---------------- the gated output norm on the prefill's o ---------------------------------
    # (z drawn here with its own seed: the workloads do not define the z branch)
    zr = torch.from_numpy(np.random.default_rng(99).standard_normal(tuple(o.shape), dtype=np.float32))
    zn = zr.to(torch.bfloat16).to(dev)
    wn = torch.ones(wl.dv, dtype=torch.float32, device=dev)
    yn = torch.empty(tuple(o.shape), dtype=torch.bfloat16, device=dev)
    norm_sets = [(o, zn, yn)] + [(o.clone(), zn.clone(), torch.empty_like(yn)) for _ in range(2)]
    # One call through the binding checks the arguments; the timed calls go to the C entry point with
    # the arguments marshalled once, so that a kernel of a few tens of microseconds is not paced by
    # the binding's host-side work.
    gdn_gated_rmsnorm(o, zn, wn, 1e-6, out=yn)
    cstream = torch.cuda.current_stream().cuda_stream
    norm_args = [(ox.data_ptr(), zx.data_ptr(), wn.data_ptr(), ctypes.c_float(1e-6), o.numel() // wl.dv,
                  wl.dv, _lib.GDN_BF16, _lib.GDN_BF16, yx.data_ptr(), cstream) for ox, zx, yx in norm_sets]
    ms_norm = time_c(clib.gdn_gated_rmsnorm, norm_args)
    norm_bytes = o.numel() * (4 + 2 + 2) + wl.dv * 4

    # ---------------- the prefill with the gated norm fused onto o, against prefill then norm ----
    zsets = [zn] + [zn.clone() for _ in range(NSETS - 1)]
    ysets = [torch.empty_like(yn) for _ in range(NSETS)]
    fws = torch.empty(int(clib.gdn_chunk_fwd_gated_norm_workspace_size(B, T, wl.Hk, wl.Hv, wl.dk, wl.dv, N,
                                                                       _lib.GDN_BF16)),
                      dtype=torch.uint8, device=dev)

    def fused_norm_call(i):
        s_ = sets[i % NSETS]
        gdn_chunk_fwd_gated_norm(s_["q"], s_["k"], s_["v"], s_["g"], s_["beta"], zsets[i % NSETS], wn, 1e-6,
                                 initial_state=s_["initial_state"], y=ysets[i % NSETS], final_state=s_["fs"],
                                 workspace=fws)

    def prefill_then_norm(i):
        s_ = sets[i % NSETS]
        prefill_step(i=i)
        gdn_gated_rmsnorm(s_["o"], zsets[i % NSETS], wn, 1e-6, out=ysets[i % NSETS])

    for i in range(max(args.warmup, 20)):
        fused_norm_call(i)
        prefill_then_norm(i)
    ms_fused_norm = time_loop(fused_norm_call)
    ms_prefill_norm = time_loop(prefill_then_norm)
    del fws

    # ---------------- the causal conv1d of the QKV mixture (2 Hk dk + Hv dv channels) -----------
    # (inputs drawn here with their own seed: the workloads define q, k, v after the conv)
    Cc, Wc = 2 * wl.Hk * wl.dk + wl.Hv * wl.dv, 4
    crng = np.random.default_rng(98)
    xc = torch.from_numpy(crng.standard_normal((1, T, Cc), dtype=np.float32)).to(wl.dtype).to(dev)
    wc = torch.from_numpy((0.5 * crng.standard_normal((Cc, Wc))).astype(np.float32)).to(dev)
    sc = torch.zeros((1, Wc - 1, Cc), dtype=wl.dtype, device=dev)
    yc = torch.empty_like(xc)
    gdn_causal_conv1d(xc, wc, None, sc, silu=True, y=yc)
    conv_sets = [(xc, yc)] + [(xc.clone(), torch.empty_like(yc)) for _ in range(2)]
    conv_args = [(xx.data_ptr(), wc.data_ptr(), None, sc.data_ptr(), None, 0, None, 1, T, Cc, Wc, 1,
                  _lib.GDN_BF16, 1, yx.data_ptr(), cstream) for xx, yx in conv_sets]
    ms_conv = time_c(clib.gdn_causal_conv1d, conv_args)
    conv_bytes = 2 * xc.numel() * xc.element_size() + Cc * Wc * 4 + 2 * sc.numel() * sc.element_size()

    # ---------------- the backward pass of the prefill (training) -------------------------------
    # (the loss gradients d_o, d_final drawn here with their own seed)
    brng = np.random.default_rng(97)
    d_o = torch.from_numpy(brng.standard_normal(tuple(o.shape), dtype=np.float32)).to(dev)
    d_fin = torch.from_numpy(brng.standard_normal(tuple(fs.shape), dtype=np.float32)).to(dev)
    bws = torch.empty(int(clib.gdn_chunk_bwd_workspace_size(1, T, wl.Hk, wl.Hv, wl.dk, wl.dv, 1)),
                      dtype=torch.uint8, device=dev)
    bwd_calls = max(3, args.steps // 20)
    for _ in range(2):
        gdn_chunk_bwd(d["q"], d["k"], d["v"], d["g"], d["beta"], d_o, d["initial_state"], d_fin, workspace=bws)
    torch.cuda.synchronize()
    e0.record()
    for _ in range(bwd_calls):
        gdn_chunk_bwd(d["q"], d["k"], d["v"], d["g"], d["beta"], d_o, d["initial_state"], d_fin, workspace=bws)
    e1.record()
    torch.cuda.synchronize()
    ms_bwd = e0.elapsed_time(e1) / bwd_calls
    bwd_flops = BWD_FLOPS_PER_TOKEN_VHEAD * tokens * wl.Hv
    bwd_exec32 = counter("bwd", "mfma_exec_f32_flops")
    bwd_exec16 = counter("bwd", "mfma_exec_bf16_flops")
    del bws

    # the same through every input option (gates from a, b and q, k normalised, both differentiated)
    bws = torch.empty(int(clib.gdn_chunk_bwd_ex_workspace_size(1, T, wl.Hk, wl.Hv, wl.dk, wl.dv, 1, _lib.GDN_BF16,
                                                                1, 0, _lib.GDN_FLAG_QK_L2NORM)),
                      dtype=torch.uint8, device=dev)

    def bwd_every_option():
        gdn_chunk_bwd_ex(d["q"], d["k"], d["v"], ga, gb, d_o, A_log=gA, dt_bias=gdt,
                         initial_state=d["initial_state"], d_final=d_fin, qk_l2norm=True, workspace=bws)

    for _ in range(2):
        bwd_every_option()
    torch.cuda.synchronize()
    e0.record()
    for _ in range(bwd_calls):
        bwd_every_option()
    e1.record()
    torch.cuda.synchronize()
    ms_bwd_ex = e0.elapsed_time(e1) / bwd_calls
    del bws

    # ---------------- the long-context and packed variable-length prefills ---------------------
    # (the same call on the two larger prefill workloads, each with its own initial states; reported
    # beside the headline prefill, which the value and roofline describe)
    def time_workload(name, calls, warm):
        wx = synth.WORKLOADS[name]
        xx = synth.make(wx)
        dd = {key: (None if xx[key] is None else xx[key].to(dev).contiguous())
              for key in ("q", "k", "v", "g", "beta", "initial_state", "cu_seqlens")}
        del xx
        Tt = dd["q"].shape[1]
        Nn = wx.n_seqs if wx.n_seqs else wx.B
        oo = torch.empty((1, Tt, wx.Hv, wx.dv), dtype=torch.float32, device=dev)
        ff = torch.empty((Nn, wx.Hv, wx.dk, wx.dv), dtype=torch.float32, device=dev)
        wss = torch.empty(max(workspace_size(1, Tt, wx.Hk, wx.Hv, wx.dk, wx.dv, Nn, wx.dtype), 1),
                          dtype=torch.uint8, device=dev)

        def call():
            gdn_chunk_fwd(dd["q"], dd["k"], dd["v"], dd["g"], dd["beta"], dd["initial_state"], dd["cu_seqlens"],
                          o=oo, final_state=ff, workspace=wss)

        # about 0.1 s of calls first: building the inputs on the host leaves the GPU idle and its
        # clocks low
        for _ in range(warm):
            call()
        torch.cuda.synchronize()
        e0.record()
        for _ in range(calls):
            call()
        e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / calls
        nb, fl, _ = prefill_algorithmic(wx, Tt, 1, Nn, wx.init_state)
        shape = (f"{Nn} packed sequences of {wx.len_range[0]}..{wx.len_range[1]} tokens" if wx.n_seqs
                 else f"B=1 T={Tt}")
        res = {"workload": f"{name}: {shape}, Hk={wx.Hk} Hv={wx.Hv} dk=dv={wx.dk} bf16 in, fp32 initial "
                           f"state(s) and out", "tokens": Tt, "calls": calls,
               "ms_per_call_events": round(ms, 4), "tokens_per_s": round(Tt / (ms / 1e3), 1),
               "achieved_gbs": round(nb / (ms / 1e3) / 1e9, 1),
               "hbm_frac": round(nb / (ms / 1e3) / 1e9 / MI355X_HBM_GBS, 4),
               "useful_tflops": round(fl / (ms / 1e3) / 1e12, 2)}
        del dd, oo, ff, wss
        torch.cuda.empty_cache()
        return res

    long_res = time_workload("long", 10, 100)
    varlen_res = time_workload("varlen", 5, 12)

    # ---------------- decode ------------------------------------------------------------------
    wd = synth.WORKLOADS["decode"]
    x0 = synth.make(wd)
    A_log = x0["raw"]["A_log"]
    nd = args.decode_steps
    steps = [x0] + [synth.decode_step(wd, s, A_log) for s in range(1, nd)]
    dsteps = [{key: s[key].to(dev).contiguous() for key in ("q", "k", "v", "g", "beta")} for s in steps]
    state = x0["initial_state"].to(dev).contiguous()
    od = torch.empty((wd.B, 1, wd.Hv, wd.dv), dtype=torch.float32, device=dev)

    def decode_pass():
        for s in dsteps:
            gdn_recurrent_step(s["q"], s["k"], s["v"], s["g"], s["beta"], state, o=od)

    decode_pass()  # warm-up pass (advances the state; values stay bounded by the decay)
    torch.cuda.synchronize()
    ev0.record()
    decode_pass()
    ev1.record()
    torch.cuda.synchronize()
    ms_decode = ev0.elapsed_time(ev1) / nd

    # the decode steps with the gates formed in the kernel
    graw = [{key: torch.from_numpy(s["raw"][key]).to(dev) for key in ("a", "b")} for s in steps]
    dA = torch.from_numpy(x0["raw"]["A_log"]).to(dev)
    ddt = torch.from_numpy(x0["raw"]["dt_bias"]).to(dev)

    def decode_gating_pass():
        for s, r in zip(dsteps, graw):
            gdn_recurrent_step_gating(s["q"], s["k"], s["v"], r["a"], r["b"], dA, ddt, state, o=od)

    decode_gating_pass()
    torch.cuda.synchronize()
    ev0.record()
    decode_gating_pass()
    ev1.record()
    torch.cuda.synchronize()
    ms_decode_gating = ev0.elapsed_time(ev1) / nd
    state_bytes, total_bytes = decode_algorithmic(wd)
    state_gbs = state_bytes / (ms_decode / 1e3) / 1e9
    total_gbs = total_bytes / (ms_decode / 1e3) / 1e9

    # ---------------- CPU baseline: the oracle on the host cores --------------------------------
    cpu = None
    if not args.no_cpu_baseline:
        from oracle import oracle as O
        f = synth.to_f64
        arrs = [f(x[key]) for key in ("q", "k", "v", "g", "beta")]
        threads = O.default_threads()
        runs = []
        for _ in range(3):
            c0 = time.perf_counter()
            O.forward(*arrs, None, None, threads=threads)
            runs.append(time.perf_counter() - c0)
        sec = sorted(runs)[1]
        # one thread on 4 of the 32 v-heads, scaled to the whole workload
        mask = np.zeros((N, wl.Hv), dtype=bool)
        mask[:, :4] = True
        c0 = time.perf_counter()
        O.forward(*arrs, None, None, unit_mask=mask, threads=1)
        sec1 = (time.perf_counter() - c0) * wl.Hv / 4
        cpu_model = "unknown"
        try:
            with open("/proc/cpuinfo") as fh:
                for ln in fh:
                    if ln.startswith("model name"):
                        cpu_model = ln.split(":", 1)[1].strip()
                        break
        except OSError:
            pass
        cpu = {"value": round(tokens / sec, 1), "unit": "tokens/s", "cores": threads,
               "kind": "oracle",
               "sample": f"the whole prefill workload (T={T}, {wl.Hv} v-heads), fp64 token-by-token, "
                         f"median of 3 runs of {sec:.2f} s",
               "cpu_model": cpu_model,
               "threads_1": {"value": round(tokens / sec1, 1), "unit": "tokens/s",
                             "sample": "4 of the 32 v-heads on one thread, scaled to all 32"}}

    line = {
        "metric": METRIC,
        "value": round(value, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_wall, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": f"prefill B={B} T={T} Hk={wl.Hk} Hv={wl.Hv} dk=dv={wl.dk} bf16 in, fp32 "
                               f"state/out, zero initial state; calls cycle through {NSETS} input sets "
                               f"larger together than the last-level cache",
                   "global_batch": B, "seq_len": T, "parallelism": "none (1 GPU)"},
        "roofline": {"bound": "mfma", "achieved": round(scan_useful_tflops, 2), "peak": MI355X_BF16_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(scan_useful_tflops / MI355X_BF16_TFLOPS, 4),
                     "traffic": scan_traffic,
                     "kernel": "chunk_scan_kernel<128> (gdn_chunk_fwd_scan)",
                     "ms_per_launch_events": round(ms_scan, 5),
                     "flops_per_token_vhead": flops // (tokens * wl.Hv),
                     "algorithmic_flops_per_launch": int(flops),
                     "mfma_executed_flops_per_launch": scan_exec,
                     "mfma_executed_tflops": (None if scan_exec is None else
                                              round(scan_exec / (ms_scan / 1e3) / 1e12, 1)),
                     "mfma_frac_executed": (None if scan_exec is None else
                                            round(scan_exec / (ms_scan / 1e3) / 1e12 / MI355X_BF16_TFLOPS, 4)),
                     "hbm": {"achieved": round(achieved_gbs, 1), "peak": MI355X_HBM_GBS, "unit": "GB/s",
                             "frac": round(achieved_gbs / MI355X_HBM_GBS, 4),
                             "algorithmic_bytes_per_launch": int(scan_bytes),
                             "bytes_per_token_vhead": per_tok_head - 2 * (2 if str(wl.gate_dtype).endswith("bfloat16") else 4)},
                     "measured_ceilings": ceilings,
                     "frac_of_measured_gemm": round(scan_useful_tflops / ceilings["bf16_gemm_tflops"], 4),
                     "hbm_frac_of_measured_copy": round(achieved_gbs / ceilings["copy_gbs"], 4),
                     "prepare_ms_per_launch_events": round(ms_prepare, 5),
                     "prepare_traffic": prep_traffic,
                     "call_traffic": call_traffic,
                     "call_algorithmic_bytes": int(nbytes),
                     "call_traffic_vs_algorithmic": (None if call_traffic is None else
                                                     round(call_traffic / nbytes, 3)),
                     "call_ms_per_launch_events": round(ms_events, 5),
                     "call_ms_same_buffers_events": round(ms_same_buffers, 5),
                     "call_achieved_gbs": round(nbytes / (ms_events / 1e3) / 1e9, 1),
                     "call_useful_tflops": round(useful_tflops, 2),
                     "call_mfma_frac_useful": round(useful_tflops / MI355X_BF16_TFLOPS, 4)},
        "chunk_vs_recurrent": ablation,
        "prefill_dk64": dk64_res,
        "prefill_long": long_res,
        "prefill_varlen": varlen_res,
        "prefill_gating": {"call": "gdn_chunk_fwd_gating (gates formed in the kernels from a, b)",
                           "ms_per_call_events": round(ms_gating, 5),
                           "tokens_per_s": round(tokens / (ms_gating / 1e3), 1)},
        "prefill_gating_l2norm": {"call": "gdn_chunk_fwd_ex (gates from a, b and q, k L2-normalised, "
                                          "both in the kernels)",
                                  "ms_per_call_events": round(ms_gating_l2, 5),
                                  "tokens_per_s": round(tokens / (ms_gating_l2 / 1e3), 1)},
        "causal_conv1d": {"call": "gdn_causal_conv1d, QKV mixture of the prefill (bf16, W = 4, SiLU, cache)",
                          "tokens": T, "channels": Cc, "width": Wc,
                          "ms_per_call_events": round(ms_conv, 5),
                          "roofline": {"bound": "hbm", "achieved": round(conv_bytes / (ms_conv / 1e3) / 1e9, 1),
                                       "peak": MI355X_HBM_GBS, "unit": "GB/s",
                                       "frac": round(conv_bytes / (ms_conv / 1e3) / 1e9 / MI355X_HBM_GBS, 4),
                                       "traffic": counter("conv", "traffic"),
                                       "algorithmic_bytes_per_launch": int(conv_bytes)}},
        "prefill_fused_norm": {"call": "gdn_chunk_fwd_gated_norm (the prefill with the gated RMSNorm fused "
                                       "onto o: bf16 y out, o never stored; bf16 z)",
                               "ms_per_call_events": round(ms_fused_norm, 5),
                               "tokens_per_s": round(tokens / (ms_fused_norm / 1e3), 1),
                               "ms_prefill_then_norm_events": round(ms_prefill_norm, 5),
                               "traffic": (None if counter("scan_norm", "traffic") is None
                                           or counter("scan_norm", "prepare_traffic") is None else
                                           counter("scan_norm", "traffic") + counter("scan_norm", "prepare_traffic")),
                               "traffic_prefill_then_norm": (None if call_traffic is None or counter("norm", "traffic") is None
                                                             else call_traffic + counter("norm", "traffic")),
                               "speedup_vs_prefill_then_norm": round(ms_prefill_norm / ms_fused_norm, 3)},
        "gated_rmsnorm": {"call": "gdn_gated_rmsnorm on the prefill's o (fp32 in, bf16 z and out)",
                          "rows": o.numel() // wl.dv, "d": wl.dv,
                          "ms_per_call_events": round(ms_norm, 5),
                          "roofline": {"bound": "hbm", "achieved": round(norm_bytes / (ms_norm / 1e3) / 1e9, 1),
                                       "peak": MI355X_HBM_GBS, "unit": "GB/s",
                                       "frac": round(norm_bytes / (ms_norm / 1e3) / 1e9 / MI355X_HBM_GBS, 4),
                                       "traffic": counter("norm", "traffic"),
                                       "algorithmic_bytes_per_launch": int(norm_bytes)}},
        "backward": {"call": "gdn_chunk_bwd (dq, dk, dv, dg, dbeta, d_initial of the prefill; fp32-accurate "
                             "arithmetic: the slice kernel's products against K and Q on bf16 matrix cores with "
                             "three-piece operands, the others on fp32 matrix cores)",
                     "calls": bwd_calls, "ms_per_call_events": round(ms_bwd, 4),
                     "tokens_per_s": round(tokens / (ms_bwd / 1e3), 1),
                     "roofline": {"bound": "mfma", "achieved": round(bwd_flops / (ms_bwd / 1e3) / 1e12, 3),
                                  "peak": MI355X_F32_TFLOPS, "unit": "TFLOP/s",
                                  "frac": round(bwd_flops / (ms_bwd / 1e3) / 1e12 / MI355X_F32_TFLOPS, 4),
                                  "traffic": counter("bwd", "traffic"),
                                  "flops_per_token_vhead": BWD_FLOPS_PER_TOKEN_VHEAD,
                                  "algorithmic_flops_per_call": int(bwd_flops),
                                  "mfma_executed_f32_flops_per_call": bwd_exec32,
                                  "mfma_executed_bf16_flops_per_call": bwd_exec16,
                                  # the share of the call the matrix units would need at their peaks for
                                  # the work they executed (fp32 and bf16 parts each at its own peak)
                                  "mfma_time_frac_executed": (None if bwd_exec32 is None or bwd_exec16 is None else
                                                              round((bwd_exec32 / MI355X_F32_TFLOPS
                                                                     + bwd_exec16 / MI355X_BF16_TFLOPS)
                                                                    / 1e12 / (ms_bwd / 1e3), 4))},
                     "every_option": {"call": "gdn_chunk_bwd_ex (gates from a, b and q, k L2-normalised, "
                                              "both differentiated: da, db, dA_log, ddt_bias, raw dq, dk)",
                                      "ms_per_call_events": round(ms_bwd_ex, 4),
                                      "tokens_per_s": round(tokens / (ms_bwd_ex / 1e3), 1)}},
        "cpu_baseline": cpu,
        "pages_context": {
            "note": "layer- or model-level claims of the pages, hardware unstated: context, not targets",
            "vs_standard_attention_32k": "9.3x throughput, 1/8 memory (Qwen3-Next architecture write-up, "
                                         "intelliparadigm.com, section 2.2)",
            "vs_transformer_8192": "3.8x speed, 48G -> 12G memory (Gated DeltaNet deployment article, "
                                   "kwkr.cn, section 2.3)",
            "chunk_vs_rnn_training": "4-6x (Qwen3-Next Gated DeltaNet article, jsqmd.com, section 2.2)"},
        "decode": {"metric": "decode state GB/s", "value": round(state_gbs, 1), "unit": "GB/s",
                   "workload": f"decode B={wd.B} Hk={wd.Hk} Hv={wd.Hv} dk=dv={wd.dk}, {nd} one-token "
                               f"steps, fp32 state {wd.B * wd.Hv * wd.dk * wd.dv * 4 / 2**20:.0f} MiB",
                   "ms_per_step": round(ms_decode, 5),
                   "roofline": {"bound": "hbm", "achieved": round(total_gbs, 1), "peak": MI355X_HBM_GBS,
                                "unit": "GB/s", "frac": round(total_gbs / MI355X_HBM_GBS, 4),
                                "traffic": counter("decode", "traffic"), "kernel": "recurrent_kernel<128,128,bf16,f32>",
                                "algorithmic_bytes_per_launch": int(total_bytes),
                                "frac_of_measured_copy": round(total_gbs / ceilings["copy_gbs"], 4),
                                "state_frac_of_measured_copy": round(state_gbs / ceilings["copy_gbs"], 4)},
                   "gating": {"call": "gdn_recurrent_step_gating (gates formed in the kernel from a, b)",
                              "ms_per_step": round(ms_decode_gating, 5),
                              "state_gbs": round(state_bytes / (ms_decode_gating / 1e3) / 1e9, 1)}},
    }
    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
