"""Benchmark of the RQ LUT logits head on one MI355X.

One step = one pass of the serving hot path for one decode token on the
Gemma-2-2B-shaped tied head (256000 x 2304, M=384 subspaces of d=6, K=1024,
L=2, bf16 codebooks, fp32 table):
  rq_decode_rows (64 input token rows, bf16), and independently of it
  rq_build_lut (B=1)  ->  rq_lut_logits (lookup+sum, softcap 30, fp32 logits,
  argmax).
The row decode needs nothing the head computes, so it runs on a second stream
and the step's end waits for it (an event the main stream waits on): the
decode's few microseconds hide under the head's lookup+sum.
Inputs are synthetic (seeded), resident in HBM before timing; two copies of
the code stream are rotated so the 256 MB Infinity Cache cannot serve
repeated reads.

Prints ONE JSON line. value = vocab rows per second of the whole step.
Besides it: per-call times (HIP events on the stream the library launches
on), the roofline of the dominant kernel, the batched (B=16) head, one MLP
layer by LUT-matvec, the dense bf16 head on the same GPU, and the CPU oracle
timed on the host's cores.
"""
import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "LUT-logits vocab-rows/s at B=1/16 + achieved HBM GB/s vs peak (256000x2304 head)"
HBM_PEAK_GBS = 8000.0


def note(msg):
    """A progress line on stderr (stdout carries only the result line)."""
    print(f"bench: {msg}", file=sys.stderr, flush=True)


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=200)
    p.add_argument("--warmup", type=int, default=20)
    p.add_argument("--no-extras", action="store_true", help="only the headline step (used under profilers)")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--copy-calibration", action="store_true",
                   help="also run a plain 256 MiB device copy (counter calibration under rocprofv3 --pmc)")
    return p.parse_args()


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU; --gpus {args.gpus} is not supported: the library has no multi-GPU "
              "path (the head would shard over the vocabulary and merge the per-shard maxima with one small "
              "all-gather)", file=sys.stderr)
        sys.exit(2)

    import torch

    import lut_logits_amd as la
    from lut_logits_amd import formats, synth

    torch.cuda.set_device(0)
    dev = "cuda"
    cfg = synth.CONFIGS["gemma_b1"]
    V, D, M, K, L = cfg.V, cfg.D, cfg.M, cfg.K, cfg.L
    mat, h, ids = synth.make_head(cfg)
    # two resident copies of the matrix (rotation defeats the 256 MB Infinity Cache)
    Ws = [la.to_device(mat), la.to_device(mat)]
    ht = torch.from_numpy(h).to(dev)
    idt = torch.from_numpy(ids).to(dev)
    lut = la.build_lut(Ws[0], ht)
    logits = torch.empty((1, V), dtype=torch.float32, device=dev)
    rows_bf16 = torch.empty((len(ids), D), dtype=torch.int16, device=dev)
    ws = la.workspace(la.lut_logits_workspace(Ws[0], 1), dev)
    main_stream = torch.cuda.current_stream()
    side_stream = torch.cuda.Stream()   # default priority, like every stream here
    decoded = [torch.cuda.Event(), torch.cuda.Event()]
    torch.cuda.synchronize()

    def step(i):
        W = Ws[i & 1]
        with torch.cuda.stream(side_stream):
            la.decode_rows(W, idt, "bf16", out=rows_bf16)
        decoded[i & 1].record(side_stream)
        la.build_lut(W, ht, out=lut)
        r = la.lut_logits(W, lut, 1, softcap=cfg.softcap, out=logits, ws=ws)
        main_stream.wait_event(decoded[i & 1])   # the step ends when its rows are decoded too
        return r

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for i in range(args.steps):
        step(i)
    e1.record()
    torch.cuda.synchronize()
    ms_step = e0.elapsed_time(e1) / args.steps

    # Instrumented pass of the same steps (kept out of the headline timing: every event record
    # costs the stream a few microseconds): events between the calls and, through
    # rq_set_stage_events, the start and end of the lookup+sum kernel's own dispatch, all on the
    # stream the library launches on.
    n_calls = args.steps
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(n_calls)]
    gev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n_calls)]
    for i in range(n_calls):
        W = Ws[i & 1]
        ev[i][0].record()
        la.decode_rows(W, idt, "bf16")
        ev[i][1].record()
        la.build_lut(W, ht, out=lut)
        ev[i][2].record()
        la.set_stage_events(*gev[i])
        la.lut_logits(W, lut, 1, softcap=cfg.softcap, out=logits, ws=ws)
        ev[i][3].record()
    torch.cuda.synchronize()
    t_gather = float(np.mean([a.elapsed_time(b) for a, b in gev]))
    t_dec = float(np.mean([e[0].elapsed_time(e[1]) for e in ev]))
    t_build = float(np.mean([e[1].elapsed_time(e[2]) for e in ev]))
    t_logits = float(np.mean([e[2].elapsed_time(e[3]) for e in ev]))
    t_logits_med = float(np.median([e[2].elapsed_time(e[3]) for e in ev]))
    # spread of single steps in the instrumented pass (each step bracketed by events: a few
    # microseconds slower than the headline mean, which has none)
    step_inst = np.array([e[0].elapsed_time(e[3]) for e in ev])
    spread = {"p10": float(np.percentile(step_inst, 10)), "p50": float(np.percentile(step_inst, 50)),
              "p90": float(np.percentile(step_inst, 90)), "steps": len(step_inst)}

    code_bytes = formats.code_bytes(V, L, M)       # 1536 B per vocab row
    lut_b = formats.lut_bytes(1, L, M, K)
    algo_bytes = code_bytes + lut_b                # what the lookup+sum kernel must read once
    achieved = algo_bytes / (t_gather * 1e-3) / 1e9
    ceiling = stream_ceiling(la, torch, [W.codes for W in Ws])

    out = {
        "metric": METRIC,
        "value": V / (ms_step * 1e-3),
        "unit": "vocab-rows/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic (seeded; Gaussian codewords, uniform codes, N(0,1) hidden state)",
        "config": {"workload": "Gemma-2-2B tied head 256000x2304 RQ M=384 d=6 K=1024 L=2, bf16 codebooks, "
                               "fp32 table, B=1: decode 64 rows (second stream) + build table + lookup+sum + softcap 30 + "
                               "argmax",
                   "global_batch": 1, "rows": V, "D": D, "M": M, "K": K, "L": L, "codes_layout": "blocked"},
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBS, "traffic": measured_traffic(),
                     "kernel": "gather_kernel (lookup+sum of rq_lut_logits, B=1)",
                     "kernel_ms": t_gather, "algorithmic_bytes": algo_bytes,
                     "stream_ceiling_gbs": ceiling["gbs"], "frac_of_stream_ceiling": achieved / ceiling["gbs"],
                     "stream_ceiling": ceiling},
        "calls_ms": {"decode_rows_64": t_dec, "build_lut": t_build, "lut_logits": t_logits,
                     "lut_logits_median": t_logits_med, "lut_logits_gather_kernel": t_gather},
        "step_ms_instrumented": spread,
        "resident_bytes": {"lut_head": Ws[0].resident_bytes() + lut_b + ws.numel(),
                           "dense_bf16_head": formats.dense_bytes(V, D)},
    }

    if args.copy_calibration:
        src = torch.empty(256 << 20, dtype=torch.uint8, device=dev).fill_(1)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        out["copy_calibration_bytes"] = src.numel()

    note(f"headline step done: {ms_step * 1e3:.1f} us")
    if not args.no_extras:
        out.update(extras(args, la, synth, formats, torch, cfg, mat, Ws, ht, idt, dev, ms_step))
    del Ws, lut, ws
    torch.cuda.empty_cache()

    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(mat, h, cfg)
        note("cpu baseline done")
    print(json.dumps(out))


def measured_traffic():
    """HBM bytes per launch of the lookup+sum kernel from the committed rocprofv3 counter runs
    (FETCH_SIZE and WRITE_SIZE, each scaled by what the counter reads for a plain device copy),
    or None when the kernel sources changed since the counters were taken."""
    import hashlib
    path = os.path.join(ROOT, "profiles", "gather_kernel_gemma_head_b1_traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    h = hashlib.sha256()
    for src in rec["sources"]:
        with open(os.path.join(ROOT, src), "rb") as f:
            h.update(f.read())
    if h.hexdigest() != rec["sources_sha256"]:
        return None
    return rec["traffic_bytes_per_launch"]


def stream_ceiling(la, torch, bufs, reps=10):
    """The HBM stream-read ceiling on this GPU: rq_stream_read (one read of a buffer with 16-byte loads and
    nothing else) over the resident code arrays, alternating them so the Infinity Cache cannot serve repeats,
    in each grid configuration, each launch timed by its own dispatch (rq_set_stage_events, as the lookup+sum
    kernel is); the fastest configuration's mean, in GB/s (decimal)."""
    nbytes = bufs[0].numel() * bufs[0].element_size()
    best = None
    for config in range(la.stream_read_configs()):
        sink = la.stream_read(bufs[0], config)
        for i in range(2):
            la.stream_read(bufs[i & 1], config, sink)
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
        for i in range(reps):
            la.set_stage_events(*ev[i])
            la.stream_read(bufs[i & 1], config, sink)
        torch.cuda.synchronize()
        ms = sum(a.elapsed_time(b) for a, b in ev) / reps
        gbs = nbytes / (ms * 1e-3) / 1e9
        if best is None or gbs > best["gbs"]:
            best = {"gbs": gbs, "config": config, "workgroups": int(sink.numel()), "bytes": nbytes, "kernel_ms": ms}
    return best


def lds_roof(la, torch, reps=500, runs=5):
    """The LDS random-gather roof: rq_lds_gather (random entries of 128 KB of LDS, every CU) for entry widths of
    2, 4, 8 and 16 bytes, each launch timed by its own dispatch; mean TB/s (decimal) per width."""
    out = {}
    for width in (2, 4, 8, 16):
        sink = la.lds_gather(width, 1)
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(runs)]
        for i in range(runs):
            la.set_stage_events(*ev[i])
            la.lds_gather(width, reps, sink)
        torch.cuda.synchronize()
        ms = sum(a.elapsed_time(b) for a, b in ev) / runs
        lookups = la.lib().rq_lds_gather_sink_words() * 1024 * 8 * reps
        out[f"w{width}"] = {"tbs": lookups * width / (ms * 1e-3) / 1e12, "lookups_per_clk_per_cu": lookups / (ms * 1e-3) / 2.4e9 / 256,
                            "bytes_per_clk_per_cu": lookups * width / (ms * 1e-3) / 2.4e9 / 256}
    return out


def timed(fn, n, torch):
    """Mean milliseconds of fn() over n calls (HIP events on the current stream) after 3 warm-up calls."""
    for _ in range(3):
        fn()
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for i in range(n):
        fn(i)
    b.record()
    torch.cuda.synchronize()
    return a.elapsed_time(b) / n


def extras(args, la, synth, formats, torch, cfg, mat, Ws, ht, idt, dev, ms_step_b1):
    res = {}
    V = cfg.V
    roof = lds_roof(la, torch)
    res["lds_roof"] = roof
    note("lds_roof done")
    # the same B=1 step (row decode on a second stream, table build, lookup+sum, softcap, argmax) on the
    # 10-bit code stream: 1024 bytes per row instead of 1536
    P10 = [la.to_device(mat, layout="packed10"), la.to_device(mat, layout="packed10")]
    lut10 = la.build_lut(P10[0], ht)
    lg10 = torch.empty((1, V), dtype=torch.float32, device=dev)
    rows10 = torch.empty((idt.numel(), cfg.D), dtype=torch.int16, device=dev)
    ws10 = la.workspace(la.lut_logits_workspace(P10[0], 1), dev)
    main_stream, side_stream = torch.cuda.current_stream(), torch.cuda.Stream()
    decoded = [torch.cuda.Event(), torch.cuda.Event()]

    def step10(i=0):
        W = P10[i & 1]
        with torch.cuda.stream(side_stream):
            la.decode_rows(W, idt, "bf16", out=rows10)
        decoded[i & 1].record(side_stream)
        la.build_lut(W, ht, out=lut10)
        la.lut_logits(W, lut10, 1, softcap=cfg.softcap, out=lg10, ws=ws10)
        main_stream.wait_event(decoded[i & 1])

    t10 = timed(step10, 200, torch)
    gev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(50)]
    for i in range(50):
        la.set_stage_events(*gev[i])
        step10(i)
    torch.cuda.synchronize()
    tg10 = float(np.mean([a.elapsed_time(b) for a, b in gev]))
    cb10 = la.packed10_codes_bytes(V, cfg.L, cfg.M)
    res["b1_packed10"] = {"ms_per_step": t10, "vocab_rows_per_s": V / (t10 * 1e-3),
                          "gather_kernel_ms": tg10, "code_bytes": cb10,
                          "gather_gbs": (cb10 + formats.lut_bytes(1, cfg.L, cfg.M, cfg.K)) / (tg10 * 1e-3) / 1e9}
    note("b1_packed10 done")
    del P10, lut10, lg10, ws10, rows10

    # batched heads, B=16 and B=128 (same matrix): rq_logits, which puts B >= 8 on the matrix cores
    # (codebooks staged on chip, no per-vector table); logits [B][V] + argmax
    c16 = synth.CONFIGS["gemma_b16"]
    hb = torch.from_numpy(synth.gen_hidden(np.random.default_rng(c16.seed), 128, cfg.D)).to(dev)
    for B in (16, 128):
        hB = hb[:B].contiguous()
        lgB = torch.empty((B, V), dtype=torch.float32, device=dev)
        amB = torch.empty(B, dtype=torch.int32, device=dev)
        wsB = la.workspace(la.logits_workspace(Ws[0], B), dev)

        def headB(i=0):
            la.logits(Ws[i & 1], hB, softcap=30.0, out=lgB, argmax_out=amB, ws=wsB)

        tB = timed(headB, 20, torch)
        mm = la.logits_method(Ws[0], B) == la.RQ_METHOD_MATRIX_CORES
        # matrix-core work: per 16 rows x 16 vectors x 4 subspaces (k = 32 with d = 6 padded to 8), one
        # 16x16x32 bf16 MFMA per level and per bf16 part of h (3): dense-equivalent flops at 2.5 PFLOP/s
        n_mfma = (V // 16) * ((B + 15) // 16) * (cfg.L * cfg.M // 4) * 3
        mfma_tflops = n_mfma * 16 * 16 * 32 * 2 / (tB * 1e-3) / 1e12
        # LDS work of the matrix-core method: one 16-byte codeword read per (row, pair, 16-vector tile)
        lds_b = V * cfg.L * cfg.M * 16 * ((B + 63) // 64 if B > 32 else 1)
        res[f"b{B}"] = {"ms_per_call": tB, "vocab_rows_per_s": V / (tB * 1e-3), "token_rows_per_s": B * V / (tB * 1e-3),
                        "lds_bytes": lds_b, "lds_frac": lds_b / (tB * 1e-3) / (roof["w16"]["tbs"] * 1e12),
                        "method": "matrix_cores" if mm else "table",
                        "code_stream_gbs": formats.code_bytes(V, cfg.L, cfg.M) / (tB * 1e-3) / 1e9,
                        "mfma_tflops": mfma_tflops if mm else None,
                        "mfma_frac_of_bf16_peak": mfma_tflops / 2500.0 if mm else None}
        note(f"b{B} done")
        del lgB, amB, wsB
    # the two-call table form at B=16, for comparison
    h16 = hb[:16].contiguous()
    lut16 = la.build_lut(Ws[0], h16)
    lg16 = torch.empty((16, V), dtype=torch.float32, device=dev)
    ws16 = la.workspace(la.lut_logits_workspace(Ws[0], 16), dev)

    def head16(i=0):
        W = Ws[i & 1]
        la.build_lut(W, h16, out=lut16)
        la.lut_logits(W, lut16, 16, softcap=30.0, out=lg16, ws=ws16)

    t16 = timed(head16, 10, torch)
    # LDS work of the table method at 16 vectors: 4 lanes x 16 bytes per (row, pair)
    lds16 = V * cfg.L * cfg.M * 64
    res["b16_table"] = {"ms_per_call": t16, "vocab_rows_per_s": V / (t16 * 1e-3), "lds_bytes": lds16,
                        "lds_frac": lds16 / (t16 * 1e-3) / (roof["w16"]["tbs"] * 1e12)}
    note("b16_table done")
    del lut16, lg16, ws16, hb

    # dense bf16 head on the same GPU: E = bf16(decode(all rows)), built by rq_decode_rows. Two
    # comparators: this library's dense kernel (tiled E, with the softcap and argmax), and the
    # vendor GEMM behind torch's linear (hipBLASLt, row-major E, logits only, no epilogue); the
    # LUT is set against the faster of the two.
    E = la.decode_rows(Ws[0], torch.arange(V, dtype=torch.int32, device=dev), "bf16")
    Es = [la.pack_dense(E), la.pack_dense(E)]   # the tiled layout the dense kernel reads (same bytes: no padding)
    Eb = [E.view(torch.bfloat16), E.view(torch.bfloat16).clone()]
    del E
    lgd = torch.empty((128, V), dtype=torch.float32, device=dev)
    wsd = la.workspace(la.dense_logits_workspace(V, 128), dev)
    h128 = torch.from_numpy(synth.gen_hidden(np.random.default_rng(c16.seed), 128, cfg.D)).to(dev)
    dense = {"resident_bytes": formats.dense_bytes(V, cfg.D)}
    for B, hB, n in ((1, ht, 50), (16, h16, 20), (128, h128, 10)):
        tdB = timed(lambda i=0: la.dense_logits(Es[i & 1], hB, 30.0, ws=wsd, out=lgd[:B]), n, torch)
        hbf = hB.to(torch.bfloat16)
        tlib = timed(lambda i=0: torch.nn.functional.linear(hbf, Eb[i & 1]), n, torch)
        gbs = formats.dense_bytes(V, cfg.D) / (tdB * 1e-3) / 1e9
        dense[f"b{B}"] = {"ms": tdB, "gbs": gbs, "hbm_frac": gbs / HBM_PEAK_GBS,
                          "mfma_tflops": 2.0 * B * V * cfg.D / (tdB * 1e-3) / 1e12,
                          "library_gemm_ms": tlib,
                          "library_gemm_hbm_frac": formats.dense_bytes(V, cfg.D) / (tlib * 1e-3) / 1e9 / HBM_PEAK_GBS}
        lut_ms = res[f"b{B}"]["ms_per_call"] if B > 1 else ms_step_b1
        dense[f"b{B}"]["lut_over_dense_time"] = lut_ms / tdB
        dense[f"b{B}"]["lut_over_best_dense_time"] = lut_ms / min(tdB, tlib)
    res["dense_bf16"] = dense
    note("dense_bf16 done")
    del Es, Eb, lgd, wsd, h128

    # one Gemma-2-2B MLP layer: the fused block (rq_lut_mlp), and the three rq_lut_matvec calls
    # (gate, up, down with the gelu_tanh*up prologue) it replaces
    layers = [synth.make_mlp_layer(i) for i in range(2)]
    dl = [[la.to_device(m) for m in lay] for lay in layers]
    x = torch.from_numpy(synth.make_mlp_x()).to(dev)
    wsm = la.workspace(max(la.lut_matvec_workspace(w, 1) for lay in dl for w in lay), dev)
    wsf = la.workspace(la.lut_mlp_workspace(*dl[0], 1), dev)
    g = torch.empty((1, synth.MLP_INTER), device=dev)
    u = torch.empty_like(g)
    y = torch.empty((1, synth.MLP_HIDDEN), device=dev)

    def mlp(i=0):
        la.lut_mlp(*dl[i & 1], x, ws=wsf, out=y)

    def mlp3(i=0):
        Wg, Wu, Wd = dl[i & 1]
        la.lut_matvec(Wg, x, ws=wsm, out=g)
        la.lut_matvec(Wu, x, ws=wsm, out=u)
        la.lut_matvec(Wd, g, x2=u, prologue=la.RQ_PRO_GELU_TANH_MUL, ws=wsm, out=y)

    tm = timed(mlp, 20, torch)
    tm3 = timed(mlp3, 20, torch)
    code_b = sum(formats.code_bytes(m.rows, m.L, m.M) for m in layers[0])
    cb_b = sum(m.codebooks.nbytes for m in layers[0])
    gbs = (code_b + cb_b) / (tm * 1e-3) / 1e9
    res["mlp_layer"] = {"ms": tm, "method": "rq_lut_mlp (gate+up in one launch, down fed their partial sums)",
                        "ms_three_matvec_calls": tm3, "code_bytes": code_b, "codebook_bytes": cb_b,
                        "gbs_codes_plus_codebooks": gbs, "hbm_frac": gbs / HBM_PEAK_GBS,
                        "ms_26_layers_est": 26 * tm}
    note("mlp_layer done")
    del dl, wsm, wsf, g, u, y
    torch.cuda.empty_cache()

    # the same layer with its codes stored at 10 bits (the RQ_CODES_PACKED10 layout: 10 bits per code,
    # so 10 bits/param at d=2 and L=2)
    dp = [[la.to_device(m, "packed10") for m in lay] for lay in layers]
    wsp = la.workspace(la.lut_mlp_workspace(*dp[0], 1), dev)
    yp = torch.empty((1, synth.MLP_HIDDEN), device=dev)
    tp = timed(lambda i=0: la.lut_mlp(*dp[i & 1], x, ws=wsp, out=yp), 20, torch)
    code_p = sum(la.packed10_codes_bytes(m.rows, m.L, m.M) for m in layers[0])
    gbs_p = (code_p + cb_b) / (tp * 1e-3) / 1e9
    res["mlp_layer_packed10"] = {"ms": tp, "code_bytes": code_p, "codebook_bytes": cb_b,
                                 "gbs_codes_plus_codebooks": gbs_p, "hbm_frac": gbs_p / HBM_PEAK_GBS}
    note("mlp_layer_packed10 done")
    del dp, wsp, yp
    torch.cuda.empty_cache()

    # the MLP RQ page's second-attempt layer: d=8, K=1024 for gate/up (10-bit codes), K=256 for down
    # (8-bit codes), fp32 codebooks
    v2 = [synth.make_mlp_v2_layer(i) for i in range(2)]
    dv2 = [(la.to_device(a, "packed10"), la.to_device(b, "packed10"), la.to_device(c, "packed8")) for a, b, c in v2]
    wsv2 = la.workspace(la.lut_mlp_workspace(*dv2[0], 1), dev)

    def mlp_v2(i=0):
        la.lut_mlp(*dv2[i & 1], x, ws=wsv2, out=y2)

    y2 = torch.empty((1, synth.MLP_HIDDEN), device=dev)
    tv2 = timed(mlp_v2, 20, torch)
    code_v2 = sum(m.codes.numel() * m.codes.element_size() for m in dv2[0])
    cb_v2 = sum(m.codebooks.nbytes for m in v2[0])
    res["mlp_v2_layer"] = {
        "ms": tv2, "code_bytes": code_v2, "codebook_bytes": cb_v2,
        "gbs_codes_plus_codebooks": (code_v2 + cb_v2) / (tv2 * 1e-3) / 1e9,
        "bits_per_param": formats.mlp_average_bpp(synth.MLP_HIDDEN, synth.MLP_INTER, synth.MLP_V2_D_SUB,
                                                  synth.MLP_V2_K_GATE_UP, synth.MLP_V2_K_DOWN, synth.MLP_L),
        "what": "d=8; gate/up K=1024 (10-bit codes), down K=256 (8-bit codes); fp32 codebooks; rq_lut_mlp"}
    note("mlp_v2_layer done")
    del v2, dv2, wsv2, y2
    torch.cuda.empty_cache()

    # stress head: K=4096, L=4, B=64, softcap 30, top-50. rq_logits (one call: the matrix cores, one pair per
    # staged slot, fp32-level accuracy), and the two-call bf16-table form (build + logits) beside it
    cs = synth.CONFIGS["stress"]
    smat, sh, _ = synth.make_head(cs)
    SW = la.to_device(smat)
    shd = torch.from_numpy(sh).to(dev)
    slg = torch.empty((cs.B, cs.V), dtype=torch.float32, device=dev)
    sam = torch.empty(cs.B, dtype=torch.int32, device=dev)
    sws1 = la.workspace(la.logits_workspace(SW, cs.B, cs.topk), dev)

    def stress1(i=0):
        la.logits(SW, shd, softcap=cs.softcap, topk=cs.topk, out=slg, argmax_out=sam, ws=sws1)

    ts1 = timed(stress1, 5, torch)
    mm1 = la.logits_method(SW, cs.B) == la.RQ_METHOD_MATRIX_CORES
    # one 16x16x32 MFMA per 16 rows x 16 vectors x pair (h's three bf16 parts in its k-slots)
    n_mfma_s = (cs.V // 16) * ((cs.B + 15) // 16) * (cs.L * cs.M)
    tflops_s = n_mfma_s * 16 * 16 * 32 * 2 / (ts1 * 1e-3) / 1e12
    res["stress"] = {"ms_per_call": ts1, "vocab_rows_per_s": cs.V / (ts1 * 1e-3),
                     "method": "matrix_cores" if mm1 else "table",
                     "mfma_tflops": tflops_s if mm1 else None,
                     "mfma_frac_of_bf16_peak": tflops_s / 2500.0 if mm1 else None,
                     "code_stream_gbs": formats.code_bytes(cs.V, cs.L, cs.M) / (ts1 * 1e-3) / 1e9}
    note("stress done")
    del sws1
    slut = la.build_lut(SW, shd, lut_dtype="bf16")
    sws = la.workspace(la.lut_logits_workspace(SW, cs.B, cs.topk, "bf16"), dev)

    def stress(i=0):
        la.build_lut(SW, shd, lut_dtype="bf16", out=slut)
        la.lut_logits(SW, slut, cs.B, softcap=cs.softcap, lut_dtype="bf16", topk=cs.topk, out=slg, ws=sws)

    ts = timed(stress, 3, torch)
    # LDS work of the bf16 table in batch tiles of 4: one 8-byte read per (row, pair, tile)
    lds_s = cs.V * cs.L * cs.M * ((cs.B + 3) // 4) * 8
    res["stress_table"] = {"ms_per_call": ts, "vocab_rows_per_s": cs.V / (ts * 1e-3), "lds_bytes": lds_s,
                           "lds_frac": lds_s / (ts * 1e-3) / (roof["w8"]["tbs"] * 1e12),
                           "method": "bf16 table: build + lookup+sum in batch tiles from a batch-tiled copy"}
    note("stress_table done")
    del SW, slut, slg, sws, sam
    torch.cuda.empty_cache()

    # per-token composite: the token's embedding row, 26 distinct MLP layers chained (rq_lut_mlp) and the
    # head's argmax, fed back as the next token on the device; 80 tokens
    from lut_logits_amd.composite import DecodeLoop
    layers = []
    for i in range(synth.MLP_LAYERS):
        layers.append(tuple(la.to_device(m) for m in synth.make_mlp_layer(i)))
    loop = DecodeLoop(Ws[0], layers, softcap=cfg.softcap, max_tokens=80)
    loop.run(1, 8)
    torch.cuda.synchronize()
    ntok = 80
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    loop.run(1, ntok)
    e1.record()
    torch.cuda.synchronize()
    tt = e0.elapsed_time(e1) / ntok
    def cbb(m):
        return m.codebooks.numel() * m.codebooks.element_size()

    mlp_bytes = synth.MLP_LAYERS * sum(formats.code_bytes(m.rows, m.L, m.M) + cbb(m) for m in layers[0])
    head_bytes = formats.code_bytes(V, cfg.L, cfg.M) + cbb(Ws[0])
    res["per_token_composite"] = {
        "ms_per_token": tt, "tokens_per_s": 1e3 / tt, "tokens": ntok, "mlp_layers": synth.MLP_LAYERS,
        "bytes_per_token": mlp_bytes + head_bytes, "gbs": (mlp_bytes + head_bytes) / (tt * 1e-3) / 1e9,
        "resident_bytes": sum(m.resident_bytes() for lay in layers for m in lay) + Ws[0].resident_bytes(),
        "distinct_tokens": int(torch.unique(loop.ids[:ntok + 1]).numel()),
        "what": "embedding row (x sqrt(D)) -> 26 RQ MLP blocks chained -> RQ head softcap+argmax; no attention"}
    note("per_token_composite done")
    del loop, layers
    torch.cuda.empty_cache()
    return res


def cpu_baseline(mat, h, cfg):
    """The CPU oracle (decode + matmul in fp64) on the full head, repeated for >= 12 s of host time."""
    import oracle

    o = oracle.default()
    nt = o.max_threads()
    passes, t0 = 0, time.time()
    while passes < 200 and (passes == 0 or time.time() - t0 < 12.0):
        o.logits(mat.codes, mat.codebooks, mat.cb_is_bf16, h, cfg.softcap, nthreads=nt)
        passes += 1
    dt = time.time() - t0
    # the same oracle on one core, over the first 16,000 rows (about 4 s)
    rows1 = 16000
    codes1 = mat.codes[:rows1]
    p1, t1 = 0, time.time()
    while p1 < 50 and (p1 == 0 or time.time() - t1 < 4.0):
        o.logits(codes1, mat.codebooks, mat.cb_is_bf16, h, cfg.softcap, nthreads=1)
        p1 += 1
    dt1 = time.time() - t1
    return {"value": passes * cfg.V / dt, "unit": "vocab-rows/s", "cores": nt, "kind": "oracle",
            "sample": f"full 256000-row head at B=1 (decode+matmul+softcap in fp64), {passes} passes, {dt:.1f} s",
            "one_core": {"value": p1 * rows1 / dt1, "unit": "vocab-rows/s", "cores": 1,
                         "sample": f"first {rows1} rows of the same head, {p1} passes, {dt1:.1f} s"}}


if __name__ == "__main__":
    main()
