"""Benchmark of the KDA hot path on one MI355X.

Prints one JSON line.  `value` is prefill throughput (tokens/s) of one
Kimi-Linear-width layer: B=1, H=32, T=32768, dk=dv=128, chunk 64, bf16 q/k/v,
fp32 gates, zero initial state.  The decode leg (reported under "decode") is
256 sequences x 32 heads x d=128 with an fp32 state cache initialised by a
4096-token prefill per sequence (untimed), then 512 timed decode steps with
fresh inputs per step.  All inputs are synthetic (seeded) and resident in HBM
before timing starts.

Usage: python bench.py [--gpus 1] [--steps 20] [--warmup 20]
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import torch

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, GB/s
MFMA_PEAK_TFLOPS = 2500.0      # dense fp16/bf16 matrix cores, TFLOP/s
PREFILL_BYTES_PER_TOKEN_HEAD = 3 * 128 * 2 + 128 * 4 + 4 + 128 * 4   # q,k,v bf16; g; beta; o fp32
DECODE_BYTES_PER_TOKEN_HEAD = 2 * 128 * 128 * 4 + 3 * 128 * 2 + 128 * 4 + 4 + 128 * 4
# general DPLR forward: q,k,v,a,b bf16, g in; o fp32 out
DPLR_BYTES_PER_TOKEN_HEAD = 5 * 128 * 2 + 128 * 4 + 128 * 4
# backward: q,k,v bf16, g, beta, grad_o in; grad q,k,v,g fp32 and grad beta out
BACKWARD_BYTES_PER_TOKEN_HEAD = 3 * 128 * 2 + 128 * 4 + 4 + 128 * 4 + 4 * 128 * 4 + 4


def prefill_flops_per_token_head(dk=128, dv=128, C=64):
    return 6 * dk * dv + (C + 1) * (3 * dk + 2 * dv) + C * C / 3.0


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--decode-steps", type=int, default=512)
    ap.add_argument("--no-decode", action="store_true")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-backward", action="store_true")
    ap.add_argument("--no-dplr", action="store_true")
    ap.add_argument("--no-packed", action="store_true")
    ap.add_argument("--profile-target",
                    choices=["prefill", "packed", "decode", "backward", "dplr", "copy"],
                    help="run only this workload a few times (target for rocprofv3) and exit")
    ap.add_argument("--traffic-from", metavar="DIR",
                    help="read rocprofv3 FETCH_SIZE/WRITE_SIZE runs of the three profile "
                         "targets from DIR/<target>_<counter>/ and write profiles/traffic.json")
    ap.add_argument("--stats-from", metavar="CSV",
                    help="print a rocprofv3 --stats kernel_stats.csv as a table and exit")
    ap.add_argument("--mfma-from", metavar="CSV",
                    help="print a rocprofv3 --pmc run of matrix-core counters "
                         "(counter_collection.csv) as a per-kernel table and exit")
    return ap.parse_args()


ROOT = os.path.dirname(os.path.abspath(__file__))
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")


def source_hash(names):
    import hashlib
    h = hashlib.sha256()
    for n in names:
        with open(os.path.join(ROOT, "linear_attention_sequence_chunkwise_amd", "csrc", n), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def measured_traffic(leg):
    """HBM bytes per call from the committed rocprofv3 FETCH_SIZE/WRITE_SIZE
    summary, or None when the kernel sources changed since it was taken."""
    try:
        rec = json.load(open(TRAFFIC_FILE))[leg]
    except (OSError, KeyError, ValueError):
        return None
    if rec.get("source_hash") != source_hash(rec["sources"]):
        return None
    return rec["bytes_per_call"]


LEG_SOURCES = {"prefill": ["kda_prefill.hip", "kda_chunk.h", "kda_common.h", "kda_internal.h"],
               "packed": ["kda_prefill.hip", "kda_chunk.h", "kda_common.h", "kda_internal.h"],
               "decode": ["kda_decode.hip", "kda_common.h", "kda_internal.h"],
               "backward": ["kda_prefill.hip", "kda_chunk.h", "kda_common.h", "kda_internal.h"],
               "dplr": ["kda_dplr.hip", "kda_chunk.h", "kda_common.h", "kda_internal.h"]}
LEG_KERNELS = {"prefill": ("kda_intra", "kda_seg_chain", "kda_seg_combine", "kda_inter"),
               "packed": ("kda_chunk_table", "kda_intra", "kda_seg_chain", "kda_inter"),
               "decode": ("decode_step_kernel",),
               "backward": ("kda_intra", "kda_state_chain", "kda_bwd_chain", "kda_bwd_vprod",
                            "kda_bwd_intra"),
               "dplr": ("kda_dplr_intra", "kda_dplr_inter")}
COPY_BYTES = 1 << 30   # the copy target reads and writes 1 GiB per dispatch


def _counter_means(path, counter):
    """Mean per-dispatch value of one counter, per kernel name, from a rocprofv3
    counter_collection.csv tree."""
    import csv
    import glob
    files = glob.glob(os.path.join(path, "**", "*counter_collection.csv"), recursive=True)
    if not files:
        raise SystemExit("no counter_collection.csv under %s" % path)
    acc = {}
    for fn in files:
        with open(fn, newline="") as f:
            for row in csv.DictReader(f):
                if row["Counter_Name"] != counter:
                    continue
                a = acc.setdefault(row["Kernel_Name"], [0.0, 0])
                a[0] += float(row["Counter_Value"])
                a[1] += 1
    return {k: v[0] / v[1] for k, v in acc.items()}


def traffic_from(d):
    """HBM bytes per call for each leg.  FETCH_SIZE and WRITE_SIZE come in KiB
    per dispatch; each is divided by what the same counter reads for a plain
    1 GiB elementwise copy (torch.mul(x, 1.0, out=y)), so that 1.0 means the
    bytes actually moved."""
    out = {"method": "rocprofv3 --pmc FETCH_SIZE and --pmc WRITE_SIZE in separate runs of "
                     "python bench.py --profile-target {copy,prefill,decode,backward,dplr}; per-dispatch "
                     "means, scaled by the copy kernel's reading of a 1 GiB read + 1 GiB write"}
    scale = {}
    for ctr in ("FETCH_SIZE", "WRITE_SIZE"):
        m = _counter_means(os.path.join(d, "copy_" + ctr), ctr)
        copy_k = [k for k in m if "mul" in k.lower() or "elementwise" in k.lower()]
        if not copy_k:
            raise SystemExit("copy kernel not found in %s counters" % ctr)
        scale[ctr] = max(m[k] for k in copy_k) * 1024.0 / COPY_BYTES
    out["scale"] = scale
    for leg, kern in LEG_KERNELS.items():
        per_kernel = {}
        for ctr in ("FETCH_SIZE", "WRITE_SIZE"):
            m = _counter_means(os.path.join(d, leg + "_" + ctr), ctr)
            for k, v in m.items():
                short = next((x for x in kern if x in k), None)
                if short is None:
                    continue
                if short == "kda_seg_chain" and leg == "packed":
                    short += " whole chains"
                elif short == "kda_seg_chain":   # pass 1 (state runs) and pass 3 (outputs)
                    short += " pass 3" if ("true>" in k or "Lb1E" in k) else " pass 1"
                per_kernel.setdefault(short, {})[ctr] = v * 1024.0 / scale[ctr]
        total = sum(v.get("FETCH_SIZE", 0.0) + v.get("WRITE_SIZE", 0.0)
                    for v in per_kernel.values())
        out[leg] = dict(bytes_per_call=total, per_kernel_bytes=per_kernel,
                        sources=LEG_SOURCES[leg], source_hash=source_hash(LEG_SOURCES[leg]))
    os.makedirs(os.path.dirname(TRAFFIC_FILE), exist_ok=True)
    with open(TRAFFIC_FILE, "w") as f:
        json.dump(out, f, indent=1)
    print(json.dumps(out, indent=1))


def kernel_label(name):
    """Readable label of a KDA kernel from its (mangled) name: base name,
    <dk,chunk>, record type and the variant flags."""
    import re
    m = re.search(r"(kda_[a-z_]+?|decode_step_kernel)(?:I|\(|<|$)", name)
    if m is None:
        return name[:60]
    base = m.group(1)
    targs = re.search(re.escape(base) + r"<([^>(]*)>", name)
    if targs:   # demangled: <128, 64, float, kda::bf16_t, false>
        args = [a.strip() for a in targs.group(1).split(",")]
        dims = [a for a in args if a.isdigit()][:2]
        ot = ("fp16 records" if "_Float16" in args else
              "fp32 records" if "float" in args and base not in ("kda_seg_combine",) else "")
        flags = ["1" if a == "true" else "0" for a in args if a in ("true", "false")]
    else:       # mangled: ILi128ELi64EDF16_...Lb1E
        dims = re.findall(r"Li(\d+)E", name)
        ot = "fp16 records" if "DF16_" in name else ("fp32 records" if "Eff" in name else "")
        flags = re.findall(r"Lb([01])E", name)
    extra = []
    if base == "kda_intra" and flags and flags[0] == "1":
        extra.append("with preparation")
    if base == "kda_seg_chain" and flags:
        extra.append("with outputs (pass 3)" if flags[0] == "1" else "state runs (pass 1)")
        if len(flags) > 1 and flags[1] == "1":
            extra.append("fused epilogue")
    parts = ", ".join([x for x in [ot] + extra if x])
    return "%s<%s>%s" % (base, ",".join(dims[:2]), " (" + parts + ")" if parts else "")


def stats_table(path):
    """Markdown table of a rocprofv3 kernel_stats.csv (KDA kernels first)."""
    import csv
    rows = list(csv.DictReader(open(path)))
    rows.sort(key=lambda r: -float(r["TotalDurationNs"]))
    print("| kernel | calls | avg us | min us | max us | % of GPU time |")
    print("|---|---|---|---|---|---|")
    for r in rows:
        kda_k = "kda" in r["Name"] or "decode_step" in r["Name"]
        name = kernel_label(r["Name"]) if kda_k else r["Name"][:50] + " (torch)"
        if not kda_k and float(r["Percentage"]) < 1.0:
            continue
        print("| %s | %s | %.1f | %.1f | %.1f | %.2f |" % (
            name, r["Calls"], float(r["AverageNs"]) / 1e3, float(r["MinNs"]) / 1e3,
            float(r["MaxNs"]) / 1e3, float(r["Percentage"])))


def mfma_table(path, xcds=8, simds=1024):
    """Per-kernel matrix-core table from a rocprofv3 --pmc counter_collection.csv
    with SQ_VALU_MFMA_BUSY_CYCLES, SQ_INSTS_VALU_MFMA_MOPS_F16/_F32,
    SQ_INSTS_MFMA, SQ_INSTS_VALU, SQ_WAVES, GRBM_GUI_ACTIVE.  MFMA busy % =
    SQ_VALU_MFMA_BUSY_CYCLES / (GRBM_GUI_ACTIVE / 8 XCDs x 1024 SIMDs) (the CSV's
    GRBM_GUI_ACTIVE sums the 8 XCDs' counters); TFLOP/s = 512 x MOPS / duration
    (dense-tile flops, masked tiles included); VALU/wave = SQ_INSTS_VALU / SQ_WAVES."""
    import collections
    import csv
    ctr = collections.defaultdict(lambda: collections.defaultdict(list))
    dur = collections.defaultdict(dict)
    for r in csv.DictReader(open(path)):
        if "kda" not in r["Kernel_Name"]:
            continue
        key = kernel_label(r["Kernel_Name"])
        ctr[key][r["Counter_Name"]].append(float(r["Counter_Value"]))
        dur[key][r["Dispatch_Id"]] = (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3
    print("| kernel | dispatches | avg us | MFMA busy % | f16 TFLOP/s | f32 TFLOP/s | "
          "MFMA instr | VALU/wave |")
    print("|---|---|---|---|---|---|---|---|")
    for key, c in ctr.items():
        avg = {k: sum(v) / len(v) for k, v in c.items()}
        us = sum(dur[key].values()) / len(dur[key])
        busy = 100 * avg["SQ_VALU_MFMA_BUSY_CYCLES"] / (avg["GRBM_GUI_ACTIVE"] / xcds * simds)
        f16 = 512 * avg["SQ_INSTS_VALU_MFMA_MOPS_F16"] / us / 1e6
        f32 = 512 * avg["SQ_INSTS_VALU_MFMA_MOPS_F32"] / us / 1e6
        vpw = avg["SQ_INSTS_VALU"] / max(avg["SQ_WAVES"], 1)
        print("| %s | %d | %.1f | %.1f | %.1f | %.1f | %.3g | %.0f |" % (
            key, len(dur[key]), us, busy, f16, f32, avg["SQ_INSTS_MFMA"], vpw))


def profile_target(kind):
    """Minimal workload for counter collection: 3 calls, nothing else timed."""
    import kda_inputs
    import linear_attention_sequence_chunkwise_amd as kda
    kda.load_library()
    if kind == "copy":
        x = torch.empty(256 << 20, dtype=torch.float32, device="cuda")   # 1 GiB
        y = torch.empty_like(x)
        for _ in range(3):
            torch.mul(x, 1.0, out=y)
    elif kind == "prefill":
        d = kda_inputs.config_inputs(2, "cuda")
        B, T, H, D = d["q"].shape
        ws = torch.empty(kda.kda_chunk_fwd_workspace_bytes(B, T, H, D, D, 64), dtype=torch.uint8,
                         device="cuda")
        o = torch.empty(B, T, H, D, device="cuda")
        S = torch.empty(B, H, D, D, device="cuda")
        for _ in range(3):
            kda.kda_chunk_fwd(d["q"], d["k"], d["v"], d["g"], d["beta"], chunk=64, o=o,
                              final_state=S, workspace=ws)
    elif kind == "packed":
        d = kda_inputs.config_inputs(3, "cuda")
        cu = d["cu_seqlens"]
        B, T, H, D = d["q"].shape
        N = cu.numel() - 1
        ws = torch.empty(kda.kda_chunk_fwd_workspace_bytes(B, T, H, D, D, 64, N),
                         dtype=torch.uint8, device="cuda")
        for _ in range(3):
            kda.kda_chunk_fwd(d["q"], d["k"], d["v"], d["g"], d["beta"], chunk=64, cu_seqlens=cu,
                              workspace=ws)
    elif kind == "dplr":
        c = kda_inputs.CONFIGS[2]
        B, T, H, D = c["B"], c["T"], c["H"], c["dk"]
        d = kda_inputs.dplr_inputs(kda_inputs.CFG_SEED[2] + 70, B, T, H, D, D, torch.bfloat16,
                                   "cuda")
        ws = torch.empty(kda.kda_dplr_chunk_fwd_workspace_bytes(B, T, H, D, D, 64),
                         dtype=torch.uint8, device="cuda")
        for _ in range(3):
            kda.kda_dplr_chunk_fwd(d["q"], d["k"], d["v"], d["a"], d["b"], d["g"], chunk=64,
                                   workspace=ws)
    elif kind == "backward":
        d = kda_inputs.config_inputs(2, "cuda")
        B, T, H, D = d["q"].shape
        ws = torch.empty(kda.kda_chunk_bwd_workspace_bytes(B, T, H, D, D, 64), dtype=torch.uint8,
                         device="cuda")
        do = torch.randn(B, T, H, D, device="cuda")
        for _ in range(3):
            kda.kda_chunk_bwd(d["q"], d["k"], d["v"], d["g"], d["beta"], do, chunk=64,
                              want_grad_initial_state=False, workspace=ws)
    else:
        c = kda_inputs.CONFIGS[4]
        N, H, D = c["N"], c["H"], c["dk"]
        gen = torch.Generator(device="cuda").manual_seed(3)
        cache = 0.1 * torch.randn(N, H, D, D, device="cuda", generator=gen)
        x = kda_inputs.decode_inputs(kda_inputs.CFG_SEED[4], 0, N, H, D, D, torch.bfloat16, "cuda")
        for _ in range(3):
            kda.kda_decode_step(x["q"], x["k"], x["v"], x["g"], x["beta"], cache)
    torch.cuda.synchronize()
    print("profile target %s done" % kind)


class StreamTimer:
    """HIP events recorded on the stream the kernels run on."""

    def __init__(self, stream):
        self.stream = stream
        self.t0 = torch.cuda.Event(enable_timing=True)
        self.t1 = torch.cuda.Event(enable_timing=True)

    def start(self):
        self.t0.record(self.stream)

    def stop(self):
        self.t1.record(self.stream)
        self.t1.synchronize()
        return self.t0.elapsed_time(self.t1)


def prefill_setup(kda, kda_inputs):
    """Inputs, outputs and workspace of the 32K-token layer, on the device."""
    c = kda_inputs.CONFIGS[2]
    B, T, H, D, C = c["B"], c["T"], c["H"], c["dk"], c["chunk"]
    d = kda_inputs.config_inputs(2, "cuda")
    o = torch.empty(B, T, H, D, device="cuda")
    S = torch.empty(B, H, D, D, device="cuda")
    ws = torch.empty(kda.kda_chunk_fwd_workspace_bytes(B, T, H, D, D, C), dtype=torch.uint8,
                     device="cuda")
    torch.cuda.synchronize()
    return d, o, S, ws


def bench_prefill(kda, kda_inputs, steps, warmup, stream, setup=None):
    c = kda_inputs.CONFIGS[2]
    B, T, H, D, C = c["B"], c["T"], c["H"], c["dk"], c["chunk"]
    d, o, S, ws = setup if setup is not None else prefill_setup(kda, kda_inputs)

    def call():
        kda.kda_chunk_fwd(d["q"], d["k"], d["v"], d["g"], d["beta"], chunk=C, o=o,
                          final_state=S, workspace=ws, stream=stream)

    for _ in range(warmup):
        call()
    torch.cuda.synchronize()
    tm = StreamTimer(stream)
    tm.start()
    for _ in range(steps):
        call()
    ms = tm.stop() / steps
    torch.cuda.synchronize()
    return dict(ms=ms, tokens=B * T, token_heads=B * T * H, inputs=d,
                segments=kda.kda_chunk_fwd_segments(B, T, H, D, D, C))


def bench_prefill_varlen(kda, kda_inputs, steps, warmup, stream):
    """The packed-sequence layer: 16 sequences of seeded lengths U[256, 8192],
    H=32, d=128, chunk 64, bf16, states reset at each boundary, per-sequence
    final states out."""
    d = kda_inputs.config_inputs(3, "cuda")
    cu = d["cu_seqlens"]
    B, T, H, D = d["q"].shape
    N = cu.numel() - 1
    ws = torch.empty(kda.kda_chunk_fwd_workspace_bytes(B, T, H, D, D, 64, N), dtype=torch.uint8,
                     device="cuda")
    o = torch.empty(B, T, H, D, device="cuda")
    S = torch.empty(N, H, D, D, device="cuda")
    torch.cuda.synchronize()

    def call():
        kda.kda_chunk_fwd(d["q"], d["k"], d["v"], d["g"], d["beta"], chunk=64, cu_seqlens=cu,
                          o=o, final_state=S, workspace=ws, stream=stream)

    for _ in range(warmup):
        call()
    torch.cuda.synchronize()
    tm = StreamTimer(stream)
    tm.start()
    for _ in range(steps):
        call()
    ms = tm.stop() / steps
    torch.cuda.synchronize()
    nbytes = PREFILL_BYTES_PER_TOKEN_HEAD * T * H + N * H * D * D * 4   # + final states
    return dict(ms_per_step=ms, value=T / (ms / 1e3), unit="tokens/s",
                hbm_frac=nbytes / (ms / 1e3) / 1e9 / HBM_PEAK_GBS, algorithmic_bytes=nbytes,
                chain_form=kda.kda_chunk_fwd_segments(B, T, H, D, D, 64, N),
                workload="packed prefill: %d sequences, %d tokens (lengths U[256, 8192], seeded), "
                         "H=32 dk=dv=128 chunk=64 bf16, per-sequence final states" % (N, T),
                inputs=d)


def bench_prefill_prep(kda, kda_inputs, steps, warmup, stream, with_epilogue=False):
    """The prefill layer on raw inputs with the in-kernel preparation (q/k L2
    normalisation, beta from logits, gate activation) and optionally the
    output epilogue (per-head RMSNorm, weight, sigmoid gate) --
    kda_chunk_fwd_ex."""
    c = kda_inputs.CONFIGS[2]
    B, T, H, D, C = c["B"], c["T"], c["H"], c["dk"], c["chunk"]
    d = kda_inputs.raw_layer_inputs(kda_inputs.CFG_SEED[2] + 50, B, T, H, D, D, torch.bfloat16,
                                    "cuda")
    prep = dict(normalize_qk=True, eps=1e-6, beta_logit=True, A_log=d["A_log"],
                dt_bias=d["dt_bias"])
    epi = None
    if with_epilogue:
        gen = torch.Generator(device="cuda").manual_seed(kda_inputs.CFG_SEED[2] + 51)
        epi = dict(eps=1e-6, weight=0.5 + torch.rand(D, device="cuda", generator=gen),
                   gate=torch.randn(B, T, H, D, device="cuda", generator=gen).to(torch.bfloat16))
    o = torch.empty(B, T, H, D, device="cuda")
    S = torch.empty(B, H, D, D, device="cuda")
    ws = torch.empty(kda.kda_chunk_fwd_workspace_bytes(B, T, H, D, D, C), dtype=torch.uint8,
                     device="cuda")

    def call():
        kda.kda_chunk_fwd(d["q"], d["k"], d["v"], d["g"], d["beta"], chunk=C, o=o,
                          final_state=S, workspace=ws, stream=stream, prep=prep, epilogue=epi)

    for _ in range(warmup):
        call()
    torch.cuda.synchronize()
    tm = StreamTimer(stream)
    tm.start()
    for _ in range(steps):
        call()
    ms = tm.stop() / steps
    torch.cuda.synchronize()
    return ms


def bench_backward(kda, kda_inputs, d, steps, warmup, stream):
    """Gradients of the same prefill layer (kda_chunk_bwd): random grad_o, no
    final-state gradient, zero initial state."""
    B, T, H, D = d["q"].shape
    C = kda_inputs.CONFIGS[2]["chunk"]
    gen = torch.Generator(device="cuda").manual_seed(kda_inputs.CFG_SEED[2] + 60)
    do = torch.randn(B, T, H, D, device="cuda", generator=gen)
    ws = torch.empty(kda.kda_chunk_bwd_workspace_bytes(B, T, H, D, D, C), dtype=torch.uint8,
                     device="cuda")

    def call():
        return kda.kda_chunk_bwd(d["q"], d["k"], d["v"], d["g"], d["beta"], do, chunk=C,
                                 want_grad_initial_state=False, workspace=ws, stream=stream)

    for _ in range(warmup):
        call()
    torch.cuda.synchronize()
    tm = StreamTimer(stream)
    keep = []
    tm.start()
    for _ in range(steps):
        keep.append(call())
        if len(keep) > 2:
            keep.pop(0)
    ms = tm.stop() / steps
    torch.cuda.synchronize()
    return dict(ms=ms, workspace_bytes=ws.numel())


def bench_dplr(kda, kda_inputs, kda_in, steps, warmup, stream):
    """The general-DPLR forward on the same layer shape, next to KDA: KDA's
    production path, and KDA with the register-staged chain kernel that the
    DPLR forward also uses (same machinery, like for like)."""
    c = kda_inputs.CONFIGS[2]
    B, T, H, D, C = c["B"], c["T"], c["H"], c["dk"], c["chunk"]
    d = kda_inputs.dplr_inputs(kda_inputs.CFG_SEED[2] + 70, B, T, H, D, D, torch.bfloat16, "cuda")
    o = torch.empty(B, T, H, D, device="cuda")
    S = torch.empty(B, H, D, D, device="cuda")
    ws = torch.empty(max(kda.kda_dplr_chunk_fwd_workspace_bytes(B, T, H, D, D, C),
                         kda.kda_chunk_fwd_workspace_bytes(B, T, H, D, D, C)),
                     dtype=torch.uint8, device="cuda")

    def timed(call):
        for _ in range(warmup):
            call()
        torch.cuda.synchronize()
        tm = StreamTimer(stream)
        tm.start()
        for _ in range(steps):
            call()
        ms = tm.stop() / steps
        torch.cuda.synchronize()
        return ms

    dplr_ms = timed(lambda: kda.kda_dplr_chunk_fwd(d["q"], d["k"], d["v"], d["a"], d["b"], d["g"],
                                                   chunk=C, o=o, final_state=S, workspace=ws,
                                                   stream=stream))
    kcall = lambda: kda.kda_chunk_fwd(kda_in["q"], kda_in["k"], kda_in["v"], kda_in["g"],
                                      kda_in["beta"], chunk=C, o=o, final_state=S, workspace=ws,
                                      stream=stream)
    kda_ms = timed(kcall)
    kda_reg_ms = timed(lambda: kda.kda_chunk_fwd(kda_in["q"], kda_in["k"], kda_in["v"], kda_in["g"],
                                                 kda_in["beta"], chunk=C, o=o, final_state=S,
                                                 workspace=ws, stream=stream, chain_form="reg16"))
    db = DPLR_BYTES_PER_TOKEN_HEAD * B * T * H
    roof = dict(bound="hbm", achieved=db / (dplr_ms / 1e3) / 1e9, peak=HBM_PEAK_GBS, unit="GB/s",
                algorithmic_bytes=db, traffic=measured_traffic("dplr"),
                kernel="kda_dplr_chunk_fwd call (kda_dplr_intra + kda_dplr_inter)")
    roof["frac"] = roof["achieved"] / HBM_PEAK_GBS
    return dict(ms_per_step=dplr_ms, value=B * T / (dplr_ms / 1e3), unit="tokens/s", roofline=roof,
                kda_ms_per_step=kda_ms, kda_register_staged_chain_ms_per_step=kda_reg_ms,
                kda_speedup=dplr_ms / kda_ms, kda_speedup_same_chain_kernel=dplr_ms / kda_reg_ms,
                workload="general-DPLR forward (kda_dplr_chunk_fwd), B=1 H=32 T=32768 "
                         "dk=dv=128 chunk=64 bf16 q/k/v/a/b, a and b independent "
                         "perturbations of the key direction; KDA on its own inputs of the "
                         "same shape")


def decode_setup(kda, kda_inputs, n_steps, stream):
    """The decode workload: a 256 x 32 x 128 x 128 fp32 state cache filled by a
    4096-token prefill per sequence (32 sequences per call), and the seeded
    inputs of n_steps decode steps, all on the device."""
    c = kda_inputs.CONFIGS[4]
    N, H, D, C, T0 = c["N"], c["H"], c["dk"], c["chunk"], c["init_T"]
    seed = kda_inputs.CFG_SEED[4]
    steps = [kda_inputs.decode_inputs(seed, s, N, H, D, D, torch.bfloat16, "cuda")
             for s in range(n_steps)]
    o = torch.empty(n_steps, N, H, D, device="cuda")
    cache = torch.empty(N, H, D, D, device="cuda")
    ws = torch.empty(kda.kda_chunk_fwd_workspace_bytes(DECODE_INIT_BATCH, T0, H, D, D, C),
                     dtype=torch.uint8, device="cuda")
    for b0 in range(0, N, DECODE_INIT_BATCH):
        d = decode_init_inputs(kda_inputs, b0, "cuda")
        kda.kda_chunk_fwd(d["q"], d["k"], d["v"], d["g"], d["beta"], chunk=C,
                          final_state=cache[b0:b0 + DECODE_INIT_BATCH], workspace=ws,
                          stream=stream)
        del d
    torch.cuda.synchronize()
    del ws
    return cache, steps, o


DECODE_INIT_BATCH = 32


def decode_init_inputs(kda_inputs, b0, device):
    """Prefill inputs that initialise sequences b0 .. b0+31 of the decode cache."""
    c = kda_inputs.CONFIGS[4]
    return kda_inputs.prefill_inputs(kda_inputs.CFG_SEED[4] * 1000 + b0, DECODE_INIT_BATCH,
                                     c["init_T"], c["H"], c["dk"], c["dv"], torch.bfloat16,
                                     device)


def decode_run(kda, cache, steps, o, stream):
    for s, x in enumerate(steps):
        kda.kda_decode_step(x["q"], x["k"], x["v"], x["g"], x["beta"], cache, o=o[s],
                            stream=stream)


def bench_decode_prep(kda, kda_inputs, cache, n_steps, stream):
    """Decode steps on raw inputs with the in-kernel preparation and the fused
    output epilogue, continuing from the benchmark's cache."""
    N, H, D = cache.shape[0], cache.shape[1], cache.shape[2]
    xs = [kda_inputs.raw_layer_inputs(kda_inputs.CFG_SEED[4] * 7 + s, 1, N, H, D, D,
                                      torch.bfloat16, "cuda") for s in range(16)]
    xs = [{k: (v[0].contiguous() if v.dim() >= 3 else v) for k, v in x.items()} for x in xs]
    o = torch.empty(N, H, D, device="cuda")
    gen = torch.Generator(device="cuda").manual_seed(kda_inputs.CFG_SEED[4] * 7 + 99)
    w = 0.5 + torch.rand(D, device="cuda", generator=gen)
    zs = [torch.randn(N, H, D, device="cuda", generator=gen).to(torch.bfloat16)
          for _ in range(16)]

    def step(x, z):
        kda.kda_decode_step(x["q"], x["k"], x["v"], x["g"], x["beta"], cache, o=o,
                            stream=stream, prep=dict(normalize_qk=True, eps=1e-6,
                                                     beta_logit=True, A_log=x["A_log"],
                                                     dt_bias=x["dt_bias"]),
                            epilogue=dict(eps=1e-6, weight=w, gate=z))

    for s in range(4):
        step(xs[s], zs[s])
    torch.cuda.synchronize()
    tm = StreamTimer(stream)
    tm.start()
    for s in range(n_steps):
        step(xs[s % 16], zs[s % 16])
    ms = tm.stop() / n_steps
    torch.cuda.synchronize()
    return ms


def bench_decode(kda, kda_inputs, n_steps, warmup, stream, setup=None):
    cache, steps, o = setup if setup is not None else decode_setup(kda, kda_inputs, n_steps,
                                                                    stream)
    # warm-up steps on the cache itself (its pages then are the ones in the
    # translation caches), then the cache restored to its initialised state
    saved = cache.clone()
    for s in range(warmup):
        x = steps[s % n_steps]
        kda.kda_decode_step(x["q"], x["k"], x["v"], x["g"], x["beta"], cache, o=o[0],
                            stream=stream)
    cache.copy_(saved)
    del saved
    torch.cuda.synchronize()
    tm = StreamTimer(stream)
    tm.start()
    decode_run(kda, cache, steps, o, stream)
    ms = tm.stop() / n_steps
    torch.cuda.synchronize()
    del steps, o
    ms_prep = bench_decode_prep(kda, kda_inputs, cache, 128, stream)
    return dict(ms=ms, ms_prep=ms_prep, N=cache.shape[0],
                token_heads=cache.shape[0] * cache.shape[1])


def cpu_baseline_prefill(d, target_s=10.0):
    """The fp64 oracle on a bounded sample of the prefill workload: all 32
    heads of the first T_s tokens (T_s grown until one run takes a quarter of
    the budget, or the whole layer), repeated until about target_s seconds
    have run.  Reported as tokens/s of the same layer."""
    import oracle
    T = d["q"].shape[1]
    Ts = 256
    while True:
        sl = lambda t: t[:, :Ts].float().cpu().numpy()
        q, k, v, g, b = (sl(d[n]) for n in ("q", "k", "v", "g", "beta"))
        t0 = time.perf_counter()
        oracle.kda_fwd(q, k, v, g, b, 128 ** -0.5)
        dt = time.perf_counter() - t0
        if dt >= target_s / 4 or Ts >= T:
            break
        Ts = min(T, Ts * 4)
    reps = 1
    while dt < target_s:
        t0 = time.perf_counter()
        oracle.kda_fwd(q, k, v, g, b, 128 ** -0.5)
        dt += time.perf_counter() - t0
        reps += 1
    return dict(value=Ts * reps / dt, unit="tokens/s", cores=oracle.num_threads(), kind="oracle",
                sample="prefill B1 H32 d128: all 32 heads of the first %d of %d tokens, %d run(s), "
                       "%.2f s" % (Ts, T, reps, dt))


def cpu_baseline_packed(d, target_s=5.0):
    """The fp64 oracle on the packed 16-sequence layer, whole (all sequences
    and heads), repeated until about target_s seconds have run."""
    import oracle
    cu = d["cu_seqlens"].cpu().numpy()
    q, k, v, g, b = (d[n].float().cpu().numpy() for n in ("q", "k", "v", "g", "beta"))
    T = q.shape[1]
    dt, reps = 0.0, 0
    while dt < target_s:
        t0 = time.perf_counter()
        oracle.kda_fwd(q, k, v, g, b, 128 ** -0.5, cu_seqlens=cu)
        dt += time.perf_counter() - t0
        reps += 1
    return dict(value=T * reps / dt, unit="tokens/s", cores=oracle.num_threads(), kind="oracle",
                sample="packed prefill, all %d sequences x 32 heads (%d tokens), %d run(s), %.2f s"
                       % (cu.shape[0] - 1, T, reps, dt))


def cpu_baseline_decode(kda_inputs, target_s=6.0):
    import numpy as np
    import oracle
    c = kda_inputs.CONFIGS[4]
    N, H, D = c["N"], c["H"], c["dk"]
    rng = np.random.default_rng(0)
    state = rng.standard_normal((N, H, D, D)) * 0.1
    xs = [kda_inputs.decode_inputs(kda_inputs.CFG_SEED[4], s, N, H, D, D, torch.bfloat16, "cpu")
          for s in range(8)]
    xs = [{k: v.float().numpy() for k, v in x.items()} for x in xs]
    t0 = time.perf_counter()
    n_steps = 0
    while time.perf_counter() - t0 < target_s:
        x = xs[n_steps % len(xs)]
        oracle.kda_decode_step(x["q"], x["k"], x["v"], x["g"], x["beta"], D ** -0.5, state)
        n_steps += 1
    dt = time.perf_counter() - t0
    return dict(value=N * n_steps / dt, unit="tokens/s", cores=oracle.num_threads(),
                kind="oracle", sample="decode N256 H32 d128: %d steps, %.2f s" % (n_steps, dt))


def main():
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU only: the KDA operator is benchmarked on a single "
              "MI355X (every (sequence, head) chain is independent, so more GPUs would shard "
              "sequences/heads with no exchange). Run with --gpus 1.", file=sys.stderr)
        sys.exit(2)
    if args.traffic_from:
        traffic_from(args.traffic_from)
        return
    if args.stats_from:
        stats_table(args.stats_from)
        return
    if args.mfma_from:
        mfma_table(args.mfma_from)
        return
    if args.profile_target:
        profile_target(args.profile_target)
        return
    import kda_inputs
    import linear_attention_sequence_chunkwise_amd as kda
    kda.load_library()
    torch.cuda.init()
    stream = torch.cuda.current_stream()

    # The prefill leg's inputs are made first, then the decode leg's state
    # cache is initialised (256 x 4096-token prefills, about 30 ms of GPU work,
    # untimed), and the prefill leg is timed right after it: the GPU's clocks,
    # which take some 20-30 ms of load to settle, are then already up.
    psetup = prefill_setup(kda, kda_inputs)
    dsetup = None
    if not args.no_decode:
        dsetup = decode_setup(kda, kda_inputs, args.decode_steps, stream)
        torch.cuda.synchronize()

    pf = bench_prefill(kda, kda_inputs, args.steps, args.warmup, stream, psetup)
    del psetup
    print("prefill %.4f ms/call" % pf["ms"], file=sys.stderr, flush=True)
    pf_prep_ms = bench_prefill_prep(kda, kda_inputs, args.steps, args.warmup, stream)
    print("prefill with preparation %.4f ms/call" % pf_prep_ms, file=sys.stderr, flush=True)
    pf_full_ms = bench_prefill_prep(kda, kda_inputs, args.steps, args.warmup, stream, True)
    print("prefill with preparation and epilogue %.4f ms/call" % pf_full_ms, file=sys.stderr,
          flush=True)
    pf_var = None
    if not args.no_packed:
        pf_var = bench_prefill_varlen(kda, kda_inputs, args.steps, args.warmup, stream)
        pf_var["traffic"] = measured_traffic("packed")
        print("packed prefill %.4f ms/call" % pf_var["ms_per_step"], file=sys.stderr, flush=True)
    th = pf["token_heads"]
    pf_bytes = PREFILL_BYTES_PER_TOKEN_HEAD * th
    pf_flops = prefill_flops_per_token_head() * th
    tok_s = pf["tokens"] / (pf["ms"] / 1e3)
    roof = dict(bound="hbm", achieved=pf_bytes / (pf["ms"] / 1e3) / 1e9, peak=HBM_PEAK_GBS,
                unit="GB/s", traffic=measured_traffic("prefill"),
                kernel="kda_chunk_fwd call (kda_intra, then the segment-parallel chain: "
                       "kda_seg_chain state runs, kda_seg_combine, kda_seg_chain with outputs)",
                chain_segments=pf["segments"],
                algorithmic_bytes=pf_bytes,
                mfma_tflops=pf_flops / (pf["ms"] / 1e3) / 1e12)
    roof["frac"] = roof["achieved"] / roof["peak"]
    roof["mfma_frac"] = roof["mfma_tflops"] / MFMA_PEAK_TFLOPS

    bwd = None
    if not args.no_backward:
        bw = bench_backward(kda, kda_inputs, pf["inputs"], args.steps, args.warmup, stream)
        print("backward %.4f ms/call" % bw["ms"], file=sys.stderr, flush=True)
        bb = BACKWARD_BYTES_PER_TOKEN_HEAD * th
        bwd = dict(ms_per_step=bw["ms"], value=pf["tokens"] / (bw["ms"] / 1e3), unit="tokens/s",
                   workload="gradients of the same layer (kda_chunk_bwd): grad_o random, no "
                            "final-state gradient, fp32 chunk records",
                   workspace_bytes=bw["workspace_bytes"],
                   roofline=dict(bound="hbm", achieved=bb / (bw["ms"] / 1e3) / 1e9,
                                 peak=HBM_PEAK_GBS, unit="GB/s", algorithmic_bytes=bb,
                                 traffic=measured_traffic("backward"),
                                 kernel="kda_chunk_bwd call (kda_intra, kda_state_chain, "
                                        "kda_bwd_chain, kda_bwd_vprod, kda_bwd_intra)"))
        bwd["roofline"]["frac"] = bwd["roofline"]["achieved"] / HBM_PEAK_GBS

    dplr = None
    if not args.no_dplr:
        dplr = bench_dplr(kda, kda_inputs, pf["inputs"], args.steps, args.warmup, stream)
        print("dplr %.4f ms/call (kda %.4f, kda register-staged chain %.4f)"
              % (dplr["ms_per_step"], dplr["kda_ms_per_step"],
                 dplr["kda_register_staged_chain_ms_per_step"]), file=sys.stderr, flush=True)

    dec = None
    if not args.no_decode:
        dc = bench_decode(kda, kda_inputs, args.decode_steps, args.warmup, stream, dsetup)
        dsetup = None
        print("decode %.4f ms/step" % dc["ms"], file=sys.stderr, flush=True)
        db = DECODE_BYTES_PER_TOKEN_HEAD * dc["token_heads"]
        dec = dict(metric="KDA decode tokens/s", value=dc["N"] / (dc["ms"] / 1e3),
                   unit="tokens/s", ms_per_step=dc["ms"], steps=args.decode_steps,
                   config=dict(workload="decode N256 H32 dk=dv=128 fp32 cache, 4096-token "
                               "prefill init, 512 steps, bf16 q/k/v"),
                   roofline=dict(bound="hbm", achieved=db / (dc["ms"] / 1e3) / 1e9,
                                 peak=HBM_PEAK_GBS, unit="GB/s",
                                 traffic=measured_traffic("decode"),
                                 kernel="decode_step_kernel<128, bf16, 1024 threads, streaming>",
                                 algorithmic_bytes=db))
        dec["roofline"]["frac"] = dec["roofline"]["achieved"] / HBM_PEAK_GBS
        dec["with_preparation"] = dict(
            ms_per_step=dc["ms_prep"], value=dc["N"] / (dc["ms_prep"] / 1e3), unit="tokens/s",
            steps=128, hbm_frac=db / (dc["ms_prep"] / 1e3) / 1e9 / HBM_PEAK_GBS,
            workload="same cache; raw q/k, beta logits and gate pre-activations prepared "
                     "in the kernel, output RMSNorm + sigmoid gate fused "
                     "(kda_decode_step_ex)")

    cpu = None
    packed_inputs = pf_var.pop("inputs") if pf_var is not None else None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline_prefill(pf["inputs"])
        if pf_var is not None:
            pf_var["cpu_baseline"] = cpu_baseline_packed(packed_inputs)
        if dec is not None:
            dec["cpu_baseline"] = cpu_baseline_decode(kda_inputs)
    del packed_inputs

    out = {
        "metric": "KDA prefill tokens/s (H=32, d=128)",
        "value": tok_s,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": pf["ms"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16/f32",
        "dtype_detail": "bf16 q/k/v in; fp16 matrix-core operands, fp32 accumulation, state, "
                        "gates and output",
        "data": "synthetic (seeded), resident in HBM",
        "config": {"workload": "prefill B=1 H=32 T=32768 dk=dv=128 chunk=64 bf16 q/k/v, fp32 "
                               "gates, zero initial state", "global_batch": 1, "seq_len": 32768,
                   "heads": 32, "head_dim": 128, "chunk": 64, "parallelism": "single GPU"},
        "roofline": roof,
        "prefill_with_preparation": dict(
            ms_per_step=pf_prep_ms, value=pf["tokens"] / (pf_prep_ms / 1e3), unit="tokens/s",
            overhead=pf_prep_ms / pf["ms"] - 1.0,
            hbm_frac=pf_bytes / (pf_prep_ms / 1e3) / 1e9 / HBM_PEAK_GBS,
            workload="same layer on raw inputs: q/k L2-normalised, beta from logits and the "
                     "gate activated inside the kernels (kda_chunk_fwd_ex)"),
        "prefill_with_preparation_and_epilogue": dict(
            ms_per_step=pf_full_ms, value=pf["tokens"] / (pf_full_ms / 1e3), unit="tokens/s",
            overhead=pf_full_ms / pf["ms"] - 1.0,
            workload="as above plus the output epilogue (per-head RMSNorm, weight, sigmoid "
                     "gate), fused into the chain's pass with outputs"),
        "prefill_packed": pf_var,
        "cpu_baseline": cpu,
        "backward": bwd,
        "general_dplr": dplr,
        "decode": dec,
    }
    print(json.dumps(out))


if __name__ == "__main__":
    main()
