#!/usr/bin/env python3
"""Benchmark of the KDA hot path on one MI355X.

One step = one kda_chunk_fwd over the long-prefill workload (B=1, H=32, T=65536,
K=V=128, bf16 inputs, fp32 initial state 0.1*N(0,1)) followed by one kda_decode_step over
the decode workload (256 sequences x 32 heads, K=V=128, fp32 state 0.1*N(0,1), bf16 step
inputs). Inputs are synthetic, seeded and resident in HBM before timing starts.

Prints one JSON line. `value` is whole-step throughput (prefill tokens + decode tokens per
second); per-call figures, roofline fractions and the oracle's CPU rate are attached. After the
timed steps, the same line reports (each can be skipped by a flag): the input options on the
same shapes, one long sequence over two heads through the plain call and through the
chunk-parallel scan, the forward at 256 key channels and the training backward on the
long-prefill shape.
"""
import argparse
import csv
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "KDA chunk_fwd tokens/s (H=32,d=128) + decode_step GB/s, % of roofline"
PEAK_HBM = 8.0e12         # B/s, MI355X HBM3E
PEAK_BF16 = 2.5e15        # FLOP/s, dense bf16 MFMA
PEAK_FP32 = 157.3e12      # FLOP/s, fp32 (vector FMA; fp32 MFMA has the same peak)
CHUNK = 64


def chunk_alg_bytes(T, H, K, V, es, n_seqs, init, final, gate_dim=None):
    gd = K if gate_dim is None else gate_dim  # gate values per token and head (1: scalar gate)
    per_tok_head = es * (2 * K + gd + V + 1 + V)  # q, k, log_alpha, v, beta in; o out
    return T * H * per_tok_head + 4 * n_seqs * H * K * V * ((1 if init else 0) + (1 if final else 0))


def chunk_alg_flops(T, H, K, V, C=CHUNK):
    # state GEMMs W.S, Q.S, Kt^T.Delta (6KV), triangular A, P, W (C*K each) and U, P.Delta
    # (C*V each), triangular solve (C^2/3), per token-head
    return T * H * (6 * K * V + C * (3 * K + 2 * V) + C * C / 3.0)


def bwd_alg_flops(T, H, K, V, C=CHUNK):
    # per token-head, counting multiply-adds twice: the states' products (W.S, Kt^T.Delta in
    # the recomputation; P^T.dO, Kt.X, Qe^T.dO, W^T.dDelta in the reverse chain; dO.S^T,
    # dDelta.S^T, Delta.X^T per chunk: 8KV), the chunk's C x C x K products (A, P, W, T^T.dW,
    # dW.Ke^T and the four decay-weighted pairwise sums: 5CK), its C x C x V products (U,
    # P^T.dO, dO.Delta^T, T^T.dDelta, dDelta.V^T: 3CV) and the C x C x C ones (T, T^T.dT, .T^T)
    return T * H * (16 * K * V + 2 * C * (5 * K + 3 * V) + 7.0 * C * C / 3.0)


def chunk_dense_flops(T, H, K, V, C=CHUNK):
    return T * H * (6 * K * V + 2 * C * (3 * K + 2 * V))


def decode_alg_bytes(N, H, K, V, es, gate_dim=None):
    gd = K if gate_dim is None else gate_dim
    return N * H * (2 * 4 * K * V + es * (2 * K + gd + V + 1) + es * V)


# ---------------------------------------------------------------- measured HBM traffic
# The counters come from two `rocprofv3 --pmc` runs of this script (FETCH_SIZE, then
# WRITE_SIZE; KiB per dispatch). Each is scaled by what the same counter reads for a plain
# elementwise kernel of known size (torch.neg over COPY_MIB MiB of fp32: reads and writes
# exactly that many bytes), and the result is stored with a hash of the kernel sources; the
# JSON line carries it only while the sources are unchanged.
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "hbm_traffic_long_prefill_and_decode.json")
SOURCES = [os.path.join(ROOT, "gated_delta_rule_30_amd", "csrc", f)
           for f in ("kda_chunk.hip", "kda_decode.hip", "kda_device.h", "kda_internal.h",
                     "kda_record.h")]
CHUNK_KERNELS = ("table_kernel", "segment_kernel", "prep_kernel", "state_kernel", "state_split_kernel")
DECODE_KERNEL = "decode_step_kernel"
OTHER_PATHS = ("wide_", "bwd_", "scan_")  # kernels of other entry points with similar names
CALIB_KERNEL = "neg_kernel"


def source_hash():
    h = hashlib.sha256()
    for f in SOURCES:
        with open(f, "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def _per_kernel(csv_path, counter):
    rows = [r for r in csv.DictReader(open(csv_path)) if r["Counter_Name"] == counter]
    out = []
    for r in rows:
        out.append((r["Kernel_Name"], float(r["Counter_Value"])))
    return out


def summarize_pmc(fetch_csv, write_csv, copy_mib, command):
    """Per-call HBM bytes of kda_chunk_fwd and kda_decode_step from two counter runs."""
    res = {"source_sha256": source_hash(), "command": command, "copy_mib": copy_mib}
    for key, path, counter in (("fetch", fetch_csv, "FETCH_SIZE"), ("write", write_csv, "WRITE_SIZE")):
        rows = _per_kernel(path, counter)
        calib = [v for n, v in rows if CALIB_KERNEL in n]
        if not calib:
            raise SystemExit("no calibration kernel in " + path)
        factor = copy_mib * 1024.0 / calib[-1]  # true KiB / counted KiB
        calls = sum(1 for n, _ in rows if "table_kernel" in n)
        chunk_kib = sum(v for n, v in rows if any(k in n for k in CHUNK_KERNELS)
                        and not any(x in n for x in OTHER_PATHS))
        dec = [v for n, v in rows if DECODE_KERNEL in n]
        res[key] = {"factor": factor, "chunk_calls": calls,
                    "chunk_bytes_per_call": chunk_kib * 1024.0 * factor / max(calls, 1),
                    "decode_calls": len(dec),
                    "decode_bytes_per_call": sum(dec) * 1024.0 * factor / max(len(dec), 1)}
    res["chunk_bytes_per_call"] = res["fetch"]["chunk_bytes_per_call"] + res["write"]["chunk_bytes_per_call"]
    res["decode_bytes_per_call"] = res["fetch"]["decode_bytes_per_call"] + res["write"]["decode_bytes_per_call"]
    os.makedirs(os.path.dirname(TRAFFIC_FILE), exist_ok=True)
    with open(TRAFFIC_FILE, "w") as fh:
        json.dump(res, fh, indent=1)
    print(json.dumps(res))


# bf16 matrix-core work of one kda_chunk_fwd call from the SQ_INSTS_VALU_MFMA_MOPS_BF16 counter
# (one unit = 512 flops) of a `rocprofv3 --pmc` run of this script, stored with the source hash.
MFMA_FILE = os.path.join(ROOT, "profiles", "mfma_ops_long_prefill.json")
MOPS_FLOPS = 512


def summarize_mfma(csv_path, command):
    rows = _per_kernel(csv_path, "SQ_INSTS_VALU_MFMA_MOPS_BF16")
    busy = _per_kernel(csv_path, "SQ_VALU_MFMA_BUSY_CYCLES")
    calls = sum(1 for n, _ in _per_kernel(csv_path, "SQ_INSTS_VALU_MFMA_MOPS_BF16") if "table_kernel" in n)
    pick = lambda rs: sum(v for n, v in rs if any(k in n for k in CHUNK_KERNELS)
                          and not any(x in n for x in OTHER_PATHS))
    per_kernel = {}
    for n, v in rows:
        if any(k in n for k in CHUNK_KERNELS) and not any(x in n for x in OTHER_PATHS):
            short = n.split("(")[0].replace("void ", "")
            per_kernel[short] = per_kernel.get(short, 0.0) + v * MOPS_FLOPS / max(calls, 1)
    res = {"source_sha256": source_hash(), "command": command, "chunk_calls": calls,
           "bf16_flops_per_call": pick(rows) * MOPS_FLOPS / max(calls, 1),
           "mfma_busy_cycles_per_call": pick(busy) / max(calls, 1),
           "bf16_flops_per_call_by_kernel": per_kernel}
    with open(MFMA_FILE, "w") as fh:
        json.dump(res, fh, indent=1)
    print(json.dumps(res))


def measured_mfma_flops():
    try:
        with open(MFMA_FILE) as fh:
            t = json.load(fh)
    except (OSError, ValueError):
        return None
    return t.get("bf16_flops_per_call") if t.get("source_sha256") == source_hash() else None


def measured_traffic():
    try:
        with open(TRAFFIC_FILE) as fh:
            t = json.load(fh)
    except (OSError, ValueError):
        return None, None
    if t.get("source_sha256") != source_hash():
        return None, None
    return t.get("chunk_bytes_per_call"), t.get("decode_bytes_per_call")


def cpu_model():
    """The host CPU's model name (from /proc/cpuinfo), or the platform's processor string."""
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.lower().startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    import platform
    return platform.processor() or "unknown"


def stream_reference():
    """Bytes read + written per second by torch's elementwise kernels (neg out of place, add_ in
    place: the decode step's pattern, copy_) over fp32 buffers of 0.5, 1 and 4 GiB."""
    import torch
    dev = torch.device("cuda:0")

    def timed(fn, n=20):
        fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(n):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / n * 1e-3

    out = {}
    for mib in (512, 1024, 4096):
        n = mib * (1 << 18)
        x = torch.ones(n, device=dev)
        y = torch.empty_like(x)
        b = 2 * n * 4
        out[str(mib) + "MiB"] = {"neg_TBps": b / timed(lambda: torch.neg(x, out=y)) / 1e12,
                                 "add_inplace_TBps": b / timed(lambda: x.add_(1.0)) / 1e12,
                                 "copy_TBps": b / timed(lambda: y.copy_(x)) / 1e12}
        del x, y
    print(json.dumps({"stream_reference": out}), flush=True)


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--cpu-sample-tokens", type=int, default=65536,
                    help="tokens (all 32 heads) of the prefill workload the oracle is timed on")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-options-bench", action="store_true",
                    help="skip the timing of the input-option entry points (counter runs)")
    ap.add_argument("--no-scan-bench", action="store_true",
                    help="skip the few-head long-sequence comparison of kda_chunk_fwd and "
                         "kda_chunk_fwd_scan")
    ap.add_argument("--no-wide-bench", action="store_true",
                    help="skip kda_chunk_fwd at K = V = 256 (the wide-key path) on the long shape")
    ap.add_argument("--no-bwd-bench", action="store_true",
                    help="skip the training backward (kda_chunk_bwd) on the long-prefill shape")
    ap.add_argument("--no-varlen-bench", action="store_true",
                    help="skip the 16-sequence varlen prefill (129,148 tokens, H=32)")
    ap.add_argument("--no-prefill1m-bench", action="store_true",
                    help="skip the 1,048,576-token prefill (H=32)")
    ap.add_argument("--no-decode-loop-bench", action="store_true",
                    help="skip the 512-call decode loop (256 sequences x 32 heads)")
    ap.add_argument("--cpu-single-tokens", type=int, default=2048,
                    help="tokens (all 32 heads) of the prefill workload the oracle is timed on "
                         "with one thread")
    ap.add_argument("--copy-calibration-mib", type=int, default=0,
                    help="also run torch.neg over this many MiB of fp32 (counter calibration)")
    ap.add_argument("--summarize-pmc", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="write the per-call HBM traffic record from two counter runs and exit")
    ap.add_argument("--pmc-command", default="", help="command line recorded with --summarize-pmc")
    ap.add_argument("--summarize-mfma", metavar="CSV",
                    help="write the per-call bf16 matrix-core record from a counter run "
                         "(SQ_INSTS_VALU_MFMA_MOPS_BF16, SQ_VALU_MFMA_BUSY_CYCLES) and exit")
    ap.add_argument("--stream-reference", action="store_true",
                    help="time torch's elementwise kernels over 0.5-4 GiB of fp32 (bytes read + "
                         "written per second) as a practical HBM reference, and exit")
    args = ap.parse_args()
    if args.summarize_pmc:
        summarize_pmc(args.summarize_pmc[0], args.summarize_pmc[1], args.copy_calibration_mib,
                      args.pmc_command)
        return
    if args.summarize_mfma:
        summarize_mfma(args.summarize_mfma, args.pmc_command)
        return
    if args.stream_reference:
        stream_reference()
        return
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures a single GPU: every (sequence, head) chain of the operator is "
              "independent and no multi-GPU path is built; run with --gpus 1", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import gated_delta_rule_30_amd as kda
    import workloads

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    names = ("q", "k", "v", "log_alpha", "beta")

    # ---------------- inputs, resident in HBM
    wl = workloads.WORKLOADS["long"]
    T, H, K, V = wl["T"], wl["H"], wl["K"], wl["V"]
    inp = workloads.make_workload("long", device=dev)
    o = torch.empty((T, H, V), dtype=torch.bfloat16, device=dev)
    fin = torch.empty((1, H, K, V), dtype=torch.float32, device=dev)
    ws = torch.empty(kda.workspace_size(1, T, H, K, V, torch.bfloat16), dtype=torch.uint8, device=dev)

    wd = workloads.WORKLOADS["decode"]
    Nd, Hd = wd["num_seqs"], wd["H"]
    gen = torch.Generator(device=dev)
    gen.manual_seed(wd["seed"])
    state = wd["state_std"] * torch.randn((Nd, Hd, K, V), generator=gen, device=dev)
    dinp = workloads.gen_decode_inputs(Nd, Hd, K, V, dtype=torch.bfloat16, device=dev, gen=gen)
    od = torch.empty((Nd, Hd, V), dtype=torch.bfloat16, device=dev)

    def chunk_call():
        kda.chunk_fwd(*(inp[x] for x in names), init_state=inp["init_state"], o=o,
                      final_state=fin, workspace=ws)

    def decode_call():
        kda.decode_step(*(dinp[x] for x in names), state=state, o=od)

    for _ in range(args.warmup):
        chunk_call()
        decode_call()
    torch.cuda.synchronize()
    if args.copy_calibration_mib > 0:
        x = torch.ones(args.copy_calibration_mib * (1 << 18), dtype=torch.float32, device=dev)
        y = torch.empty_like(x)
        torch.neg(x, out=y)
        torch.cuda.synchronize()
        del x, y

    # ---------------- timed region
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for s in range(args.steps):
        ev[s][0].record()
        chunk_call()
        ev[s][1].record()
        decode_call()
        ev[s][2].record()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    chunk_ms = float(np.mean([e[0].elapsed_time(e[1]) for e in ev]))
    decode_ms = float(np.mean([e[1].elapsed_time(e[2]) for e in ev]))
    ms_per_step = (t1 - t0) * 1e3 / args.steps

    cb = chunk_alg_bytes(T, H, K, V, 2, 1, True, True)
    cf = chunk_alg_flops(T, H, K, V)
    cfd = chunk_dense_flops(T, H, K, V)
    db = decode_alg_bytes(Nd, Hd, K, V, 2)
    chunk_s = chunk_ms * 1e-3
    decode_s = decode_ms * 1e-3
    chunk = {
        "workload": "B=1 H=32 T=65536 K=V=128 bf16, init state 0.1*N(0,1)",
        "ms": chunk_ms,
        "tokens_per_s": T / chunk_s,
        "alg_bytes": cb,
        "hbm_GBps": cb / chunk_s / 1e9,
        "hbm_frac": cb / chunk_s / PEAK_HBM,
        "chunk_size": CHUNK,
        "mfma_frac_alg": cf / chunk_s / PEAK_BF16,
        "mfma_frac_dense": cfd / chunk_s / PEAK_BF16,
    }
    mf = measured_mfma_flops()
    if mf is not None:  # bf16 flops the matrix cores executed per call, by counter
        chunk["mfma_bf16_flops_counter"] = mf
        chunk["mfma_frac_counter"] = mf / chunk_s / PEAK_BF16
    decode = {
        "workload": "256 seqs x 32 heads, K=V=128, fp32 state, bf16 inputs",
        "ms": decode_ms,
        "GB_per_s": db / decode_s / 1e9,
        "hbm_frac": db / decode_s / PEAK_HBM,
        "tokens_per_s": Nd / decode_s,
        "alg_bytes": db,
    }
    # dominant work of the step: the chunkwise forward (HBM-bound at K=V=128, bf16 I/O); one
    # kda_chunk_fwd call is the launch unit (its kernels run back to back on one stream)
    traffic_chunk, traffic_decode = measured_traffic()
    roofline = {"bound": "hbm", "achieved": cb / chunk_s / 1e9, "peak": PEAK_HBM / 1e9,
                "unit": "GB/s", "frac": cb / chunk_s / PEAK_HBM, "traffic": traffic_chunk,
                "kernel": "kda_chunk_fwd call (table, segment, then prep + state kernel per segment)"}
    roofline_decode = {"bound": "hbm", "achieved": db / decode_s / 1e9, "peak": PEAK_HBM / 1e9,
                       "unit": "GB/s", "frac": db / decode_s / PEAK_HBM, "traffic": traffic_decode,
                       "kernel": "decode_step_kernel<128,128,bf16,false>"}
    value = (T + Nd) / (ms_per_step * 1e-3)

    # ---------------- the input options on the same shapes, timed after the headline steps:
    # the gated delta rule's scalar gate from logits, beta from logits, unit-norm q and k
    options = None
    if not args.no_options_bench:
        allo = kda.OPT_SCALAR_GATE | kda.OPT_GATE_LOGITS | kda.OPT_BETA_LOGITS | kda.OPT_L2NORM_QK
        raw = workloads.gen_raw(T, H, K, V, allo, dtype=torch.bfloat16, device=dev,
                                seed=wl["seed"], init_std=wl["init_std"])
        draw = workloads.gen_raw(Nd, Hd, K, V, allo, dtype=torch.bfloat16, device=dev,
                                 seed=wd["seed"] + 1)
        o2, fin2, od2 = torch.empty_like(o), torch.empty_like(fin), torch.empty_like(od)
        state2 = state.clone()

        def chunk_opt():
            kda.chunk_fwd(*(raw[x] for x in names), init_state=raw["init_state"], o=o2,
                          final_state=fin2, workspace=ws, options=allo)

        def decode_opt():
            kda.decode_step(*(draw[x] for x in names), state=state2, o=od2, options=allo)

        for _ in range(args.warmup):
            chunk_opt()
            decode_opt()
        evo = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
        for s in range(args.steps):
            evo[s][0].record()
            chunk_opt()
            evo[s][1].record()
            decode_opt()
            evo[s][2].record()
        torch.cuda.synchronize()
        cms = float(np.mean([e[0].elapsed_time(e[1]) for e in evo]))
        dms = float(np.mean([e[1].elapsed_time(e[2]) for e in evo]))
        cbo = chunk_alg_bytes(T, H, K, V, 2, 1, True, True, gate_dim=1)
        dbo = decode_alg_bytes(Nd, Hd, K, V, 2, gate_dim=1)
        options = {
            "options": "SCALAR_GATE|GATE_LOGITS|BETA_LOGITS|L2NORM_QK",
            "chunk_fwd": {"workload": "B=1 H=32 T=65536 K=V=128 bf16, gate [T,H] logits, beta "
                                      "logits, raw q/k", "ms": cms, "tokens_per_s": T / (cms * 1e-3),
                          "alg_bytes": cbo, "hbm_frac": cbo / (cms * 1e-3) / PEAK_HBM,
                          "mfma_frac_alg": cf / (cms * 1e-3) / PEAK_BF16},
            "decode_step": {"workload": "256 seqs x 32 heads, K=V=128, gate [N,H] logits",
                            "ms": dms, "GB_per_s": dbo / (dms * 1e-3) / 1e9,
                            "hbm_frac": dbo / (dms * 1e-3) / PEAK_HBM, "alg_bytes": dbo},
        }
        del raw, draw, o2, fin2, od2, state2

    # ---------------- one long sequence with few heads, where the chunk chains alone cannot fill
    # the device: the plain chunked call against the chunk-parallel scan over groups of chunks
    scan = None
    if not args.no_scan_bench:
        Hs, Gs = 2, 16
        sinp = workloads.gen_forward(T, Hs, K, V, dtype=torch.bfloat16, device=dev,
                                     seed=wl["seed"] + 7, init_std=wl["init_std"])
        os_p, os_s = (torch.empty((T, Hs, V), dtype=torch.bfloat16, device=dev) for _ in range(2))
        fs_p, fs_s = (torch.empty((1, Hs, K, V), dtype=torch.float32, device=dev) for _ in range(2))
        ws_p = torch.empty(kda.workspace_size(1, T, Hs, K, V, torch.bfloat16), dtype=torch.uint8,
                           device=dev)
        ws_s = torch.empty(int(kda.lib().kda_chunk_fwd_scan_workspace_size(1, T, Hs, K, V, 1, Gs)),
                           dtype=torch.uint8, device=dev)

        def plain_few():
            kda.chunk_fwd(*(sinp[x] for x in names), init_state=sinp["init_state"], o=os_p,
                          final_state=fs_p, workspace=ws_p)

        def scan_few():
            kda.chunk_fwd_scan(*(sinp[x] for x in names), init_state=sinp["init_state"],
                               num_groups=Gs, o=os_s, final_state=fs_s, workspace=ws_s)

        for _ in range(args.warmup):
            plain_few()
            scan_few()
        evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
        for s in range(args.steps):
            evs[s][0].record()
            plain_few()
            evs[s][1].record()
            scan_few()
            evs[s][2].record()
        torch.cuda.synchronize()
        pms = float(np.mean([e[0].elapsed_time(e[1]) for e in evs]))
        sms = float(np.mean([e[1].elapsed_time(e[2]) for e in evs]))
        rel = lambda a, b: float((a.float() - b.float()).abs().max() / b.float().abs().max())
        scan = {"workload": "B=1 H=%d T=%d K=V=%d bf16, init state 0.1*N(0,1)" % (Hs, T, K),
                "groups": Gs, "plain_ms": pms, "scan_ms": sms,
                "plain_tokens_per_s": T / (pms * 1e-3), "scan_tokens_per_s": T / (sms * 1e-3),
                "speedup": pms / sms,
                "o_max_rel_diff": rel(os_s, os_p), "final_state_max_rel_diff": rel(fs_s, fs_p)}
        del sinp, os_p, os_s, fs_p, fs_s, ws_p, ws_s

    # ---------------- 256 key channels (the wide-key path) on the long-prefill shape
    wide = None
    if not args.no_wide_bench:
        Kw = Vw = 256
        winp = workloads.gen_forward(T, H, Kw, Vw, dtype=torch.bfloat16, device=dev,
                                     seed=wl["seed"] + 13, init_std=wl["init_std"])
        ow = torch.empty((T, H, Vw), dtype=torch.bfloat16, device=dev)
        fw = torch.empty((1, H, Kw, Vw), dtype=torch.float32, device=dev)
        wsw = torch.empty(kda.workspace_size(1, T, H, Kw, Vw, torch.bfloat16), dtype=torch.uint8,
                          device=dev)

        def wide_call():
            kda.chunk_fwd(*(winp[x] for x in names), init_state=winp["init_state"], o=ow,
                          final_state=fw, workspace=wsw)

        wsteps = max(1, min(args.steps, 5))
        for _ in range(max(1, min(args.warmup, 2))):
            wide_call()
        torch.cuda.synchronize()
        ew0, ew1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        ew0.record()
        for _ in range(wsteps):
            wide_call()
        ew1.record()
        torch.cuda.synchronize()
        wms = ew0.elapsed_time(ew1) / wsteps
        # the same shape with every input option (applied inside the record kernel)
        wopts = (kda.OPT_SCALAR_GATE | kda.OPT_GATE_LOGITS | kda.OPT_BETA_LOGITS |
                 kda.OPT_L2NORM_QK)
        del winp
        winp = workloads.gen_raw(T, H, Kw, Vw, wopts, dtype=torch.bfloat16, device=dev,
                                 seed=wl["seed"] + 14, init_std=wl["init_std"])

        def wide_opt_call():
            kda.chunk_fwd(*(winp[x] for x in names), init_state=winp["init_state"], o=ow,
                          final_state=fw, workspace=wsw, options=wopts)

        for _ in range(max(1, min(args.warmup, 2))):
            wide_opt_call()
        torch.cuda.synchronize()
        ew0.record()
        for _ in range(wsteps):
            wide_opt_call()
        ew1.record()
        torch.cuda.synchronize()
        wms_opt = ew0.elapsed_time(ew1) / wsteps
        wfl = chunk_alg_flops(T, H, Kw, Vw)
        wb = chunk_alg_bytes(T, H, Kw, Vw, 2, 1, True, True)
        # bf16 inputs, no options: the fp32 record kernel and the bf16 matrix-core chain
        wide = {"workload": "B=1 H=32 T=65536 K=V=256 bf16, init state 0.1*N(0,1)",
                "path": "fp32 records (rec256_kernel), bf16 chain (state_split_kernel, 4 waves)",
                "ms": wms, "calls": wsteps, "tokens_per_s": T / (wms * 1e-3),
                "alg_bytes": wb, "hbm_frac": wb / (wms * 1e-3) / PEAK_HBM,
                "alg_flops": wfl, "mfma_frac_alg": wfl / (wms * 1e-3) / PEAK_BF16,
                "workspace_GB": wsw.numel() / 1e9,
                "with_options": {"options": "SCALAR_GATE|GATE_LOGITS|BETA_LOGITS|L2NORM_QK",
                                 "ms": wms_opt, "tokens_per_s": T / (wms_opt * 1e-3)}}
        del winp, ow, fw, wsw

    # ---------------- the other prefill workloads: 16 packed sequences of log-uniform lengths
    # (129,148 tokens, per-sequence initial states) and one 1,048,576-token sequence
    def time_calls(fn, calls, warm):
        for _ in range(warm):
            fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(calls):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / calls

    def prefill_entry(name, desc, calls):
        w = workloads.WORKLOADS[name]
        pin = workloads.make_workload(name, device=dev)
        Tt = int(pin["q"].shape[0])
        N = int(pin["num_seqs"])
        po = torch.empty((Tt, H, V), dtype=torch.bfloat16, device=dev)
        pf = torch.empty((N, H, K, V), dtype=torch.float32, device=dev)
        pws = torch.empty(kda.workspace_size(N, Tt, H, K, V, torch.bfloat16), dtype=torch.uint8,
                          device=dev)

        def call():
            kda.chunk_fwd(*(pin[x] for x in names), init_state=pin["init_state"],
                          cu_seqlens=pin["cu_seqlens"], num_seqs=N, o=po, final_state=pf,
                          workspace=pws)

        ms = time_calls(call, calls, 1)
        pb = chunk_alg_bytes(Tt, H, K, V, 2, N, pin["init_state"] is not None, True)
        pfl = chunk_alg_flops(Tt, H, K, V)
        res = {"workload": desc, "ms": ms, "calls": calls, "tokens": Tt,
               "tokens_per_s": Tt / (ms * 1e-3), "alg_bytes": pb,
               "hbm_frac": pb / (ms * 1e-3) / PEAK_HBM,
               "mfma_frac_alg": pfl / (ms * 1e-3) / PEAK_BF16}
        del pin, po, pf, pws
        torch.cuda.empty_cache()
        return res

    varlen = None
    if not args.no_varlen_bench:
        varlen = prefill_entry("varlen", "16 packed sequences, lengths log-uniform in [1024, "
                               "32768] (129,148 tokens), H=32, K=V=128 bf16, per-sequence init "
                               "states 0.1*N(0,1)", max(1, min(args.steps, 10)))
    prefill1m = None
    if not args.no_prefill1m_bench:
        prefill1m = prefill_entry("prefill1m", "B=1 H=32 T=1048576 K=V=128 bf16, zero init",
                                  max(1, min(args.steps, 3)))

    # ---------------- the serving loop: 512 sequential kda_decode_step calls over 256 sequences x
    # 32 heads, fresh bf16 inputs at every step (generated beforehand), timed back to back
    decode_loop = None
    if not args.no_decode_loop_bench:
        steps_d = wd["steps"]
        gl = torch.Generator(device=dev)
        gl.manual_seed(wd["seed"] + 3)
        st_l = wd["state_std"] * torch.randn((Nd, Hd, K, V), generator=gl, device=dev)
        step_inp = [workloads.gen_decode_inputs(Nd, Hd, K, V, dtype=torch.bfloat16, device=dev,
                                                gen=gl) for _ in range(steps_d)]
        od_l = torch.empty((Nd, Hd, V), dtype=torch.bfloat16, device=dev)

        def loop():
            for si in step_inp:
                kda.decode_step(*(si[x] for x in names), state=st_l, o=od_l)

        lms = time_calls(loop, 1, 1)
        decode_loop = {"workload": "256 seqs x 32 heads, K=V=128, fp32 state, %d sequential "
                                   "steps with fresh bf16 inputs" % steps_d,
                       "ms": lms, "steps": steps_d, "ms_per_step": lms / steps_d,
                       "tokens_per_s": Nd * steps_d / (lms * 1e-3),
                       "GB_per_s": db * steps_d / (lms * 1e-3) / 1e9,
                       "hbm_frac": db * steps_d / (lms * 1e-3) / PEAK_HBM}
        del step_inp, st_l, od_l

    # ---------------- the training backward on the long-prefill shape (gradients of
    # sum(dO * o) + sum(dS * S_final) for every input and the initial state, fp32)
    bwd = None
    if not args.no_bwd_bench:
        gen2 = torch.Generator(device=dev)
        gen2.manual_seed(wl["seed"] + 11)
        d_o = torch.randn((T, H, V), generator=gen2, device=dev).to(torch.bfloat16)
        d_fin = torch.randn((1, H, K, V), generator=gen2, device=dev)
        L = kda.lib()

        def time_bwd(wsbytes):
            wsb = torch.empty(int(wsbytes), dtype=torch.uint8, device=dev)

            def bwd_call():
                return kda.chunk_bwd(*(inp[x] for x in names), d_o, init_state=inp["init_state"],
                                     d_final_state=d_fin, workspace=wsb)

            bsteps = max(1, min(args.steps, 5))
            for _ in range(max(1, min(args.warmup, 2))):
                grads = bwd_call()
            torch.cuda.synchronize()
            eb0, eb1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            eb0.record()
            for _ in range(bsteps):
                grads = bwd_call()
            eb1.record()
            torch.cuda.synchronize()
            again = bwd_call()
            same = all(torch.equal(x, y) for x, y in zip(grads, again))
            return eb0.elapsed_time(eb1) / bsteps, bsteps, grads, same

        # the default workspace (segments of about 4 GiB, a second pass over the records for
        # the states at the segment boundaries), then one segment over every chunk
        ws_def = int(L.kda_chunk_bwd_workspace_size(1, T, H, K, V, 1))
        ws_one = int(L.kda_chunk_bwd_workspace_size_ex(1, T, H, K, V, 1, 0, 0))
        bms, bsteps, grads, same = time_bwd(ws_def)
        finite = bool(all(torch.isfinite(g).all().item() for g in grads))
        del grads
        bms1, _, grads1, same1 = time_bwd(ws_one)
        # with the forward's checkpoints: the forward that keeps them (timed), then the backward
        # from them with the default workspace (no boundary pass)
        ck = kda.ckpt_empty(1, T, H, K, V, dev)
        ock = torch.empty((T, H, V), dtype=torch.bfloat16, device=dev)
        fck = torch.empty((1, H, K, V), dtype=torch.float32, device=dev)
        wsf = torch.empty(kda.workspace_size(1, T, H, K, V, torch.bfloat16), dtype=torch.uint8,
                          device=dev)

        def fwd_ck():
            kda.chunk_fwd(*(inp[x] for x in names), init_state=inp["init_state"], o=ock,
                          final_state=fck, workspace=wsf, checkpoints=ck)

        def time_calls_(fn, calls, warm):
            for _ in range(warm):
                fn()
            torch.cuda.synchronize()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            for _ in range(calls):
                fn()
            e1.record()
            torch.cuda.synchronize()
            return e0.elapsed_time(e1) / calls

        fck_ms = time_calls_(fwd_ck, max(1, min(args.steps, 10)), max(1, min(args.warmup, 2)))
        wsd = torch.empty(int(ws_def), dtype=torch.uint8, device=dev)
        gck = [None]

        def bwd_ck():
            gck[0] = kda.chunk_bwd(*(inp[x] for x in names), d_o, init_state=inp["init_state"],
                                   d_final_state=d_fin, workspace=wsd, checkpoints=ck)

        bck_ms = time_calls_(bwd_ck, max(1, min(args.steps, 5)), max(1, min(args.warmup, 2)))
        ck_rel = max(float((a - b).abs().max() / b.abs().max().clamp_min(1e-30))
                     for a, b in zip(gck[0], grads1))
        del grads1, gck, ck, ock, fck, wsf, wsd
        bfl = bwd_alg_flops(T, H, K, V)
        bwd = {"workload": "B=1 H=32 T=65536 K=V=128 bf16 inputs, fp32 gradients of q, k, v, "
                           "log alpha, beta and the initial state",
               "ms": bms, "calls": bsteps, "tokens_per_s": T / (bms * 1e-3),
               "alg_flops": bfl, "fp32_TFLOPs": bfl / (bms * 1e-3) / 1e12,
               "fp32_frac": bfl / (bms * 1e-3) / PEAK_FP32,
               "workspace_GB": ws_def / 1e9,
               "segments": "of about 4 GiB of per-chunk arrays (default workspace)",
               "single_segment": {"ms": bms1, "workspace_GB": ws_one / 1e9,
                                  "tokens_per_s": T / (bms1 * 1e-3)},
               "bitwise_repeatable": bool(same and same1),
               "finite": finite,
               "with_checkpoints": {
                   "ms": bck_ms, "tokens_per_s": T / (bck_ms * 1e-3),
                   "workspace_GB": ws_def / 1e9,
                   "forward_with_checkpoints_ms": fck_ms,
                   "max_rel_diff_vs_single_segment": ck_rel,
                   "note": "segments start from the states the forward kept at its segment "
                           "boundaries (no boundary pass)"}}
        del d_o, d_fin

    # ---------------- parity spot check and CPU baseline (oracle on the same inputs)
    cpu = None
    parity = None
    if not args.no_cpu_baseline:
        import oracle
        S = min(args.cpu_sample_tokens, T)
        f = lambda t: t.float().cpu().numpy()
        sample = [f(inp[x][:S]) for x in names]
        init_np = inp["init_state"].double().cpu().numpy()
        ta = time.perf_counter()
        o_ref, _ = oracle.kda_fwd(*sample, init_state=init_np)
        tb = time.perf_counter()
        S1 = min(args.cpu_single_tokens, S)
        tc = time.perf_counter()
        oracle.kda_fwd(*(x[:S1] for x in sample), init_state=init_np, threads=1)
        td = time.perf_counter()
        cpu = {"value": S / (tb - ta), "unit": "tokens/s", "cores": oracle.max_threads(),
               "kind": "oracle", "cpu_model": cpu_model(),
               "sample": "first %d tokens x all %d heads of the prefill workload (fp64 token "
                         "recurrence, %.1f s wall)" % (S, H, tb - ta),
               "single_thread": {"value": S1 / (td - tc), "unit": "tokens/s",
                                 "sample": "first %d tokens x all %d heads, one thread "
                                           "(%.1f s wall)" % (S1, H, td - tc)}}
        got = o[:S].float().cpu().numpy().astype(np.float64)
        parity = float(np.abs(got - o_ref).max() / np.abs(o_ref).max())

    out = {
        "metric": METRIC,
        "value": value,
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
        "config": {"workload": "KDA long prefill B=1 H=32 T=65536 K=V=128 + decode step "
                               "256x32 heads", "global_batch": 1, "seq_len": T,
                   "parallelism": "single-gpu"},
        "roofline": roofline,
        "cpu_baseline": cpu,
        "chunk_fwd": chunk,
        "decode_step": decode,
        "roofline_decode": roofline_decode,
        "input_options": options,
        "few_head_scan": scan,
        "training_backward": bwd,
        "wide_key": wide,
        "varlen_prefill": varlen,
        "prefill_1m": prefill1m,
        "decode_loop": decode_loop,
        "parity_sample_max_rel_err": parity,
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
