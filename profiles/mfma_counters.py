"""Summarise a rocprofv3 --pmc run of MFMA / VALU counters per KDA kernel.

    python profiles/mfma_counters.py <run_counter_collection.csv>

Counters expected in the run: SQ_VALU_MFMA_BUSY_CYCLES, SQ_INSTS_VALU_MFMA_MOPS_F16,
SQ_INSTS_VALU_MFMA_MOPS_F32, SQ_INSTS_MFMA, SQ_INSTS_VALU, SQ_WAVES, GRBM_GUI_ACTIVE.

Per kernel (averaged over its dispatches):
  busy %   = SQ_VALU_MFMA_BUSY_CYCLES / (GRBM_GUI_ACTIVE / 8 * 1024 SIMDs): the CSV's
             GRBM_GUI_ACTIVE is the sum over the 8 XCDs' graphics-engine counters
             (8 x the dispatch's clock cycles), SQ_VALU_MFMA_BUSY_CYCLES the sum over
             all SIMDs;
  TFLOP/s  = 512 x SQ_INSTS_VALU_MFMA_MOPS_<type> / dispatch duration (dense-tile flops
             the matrix cores executed, masked tiles included);
  VALU/wave = SQ_INSTS_VALU / SQ_WAVES.
"""
import collections
import csv
import re
import sys

XCDS, SIMDS = 8, 1024


def label(name):
    """Readable kernel label from a (mangled) kernel name."""
    m = re.search(r"(kda_[a-z_]+?)(?:I|\(|<|$)", name)
    base = m.group(1) if m else name[:40]
    dims = re.findall(r"Li(\d+)E", name) or re.findall(r"<(\d+)", name)
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


def main(path):
    ctr = collections.defaultdict(lambda: collections.defaultdict(list))
    dur = collections.defaultdict(dict)
    for r in csv.DictReader(open(path)):
        name = r["Kernel_Name"]
        if "kda" not in name:
            continue
        key = label(name)
        ctr[key][r["Counter_Name"]].append(float(r["Counter_Value"]))
        dur[key][r["Dispatch_Id"]] = (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3
    print("| kernel | dispatches | avg us | MFMA busy % | f16 TFLOP/s | f32 TFLOP/s | "
          "MFMA instr | VALU/wave |")
    print("|---|---|---|---|---|---|---|---|")
    for key, c in ctr.items():
        avg = {k: sum(v) / len(v) for k, v in c.items()}
        us = sum(dur[key].values()) / len(dur[key])
        busy = 100 * avg["SQ_VALU_MFMA_BUSY_CYCLES"] / (avg["GRBM_GUI_ACTIVE"] / XCDS * SIMDS)
        f16 = 512 * avg["SQ_INSTS_VALU_MFMA_MOPS_F16"] / us / 1e6
        f32 = 512 * avg["SQ_INSTS_VALU_MFMA_MOPS_F32"] / us / 1e6
        vpw = avg["SQ_INSTS_VALU"] / max(avg["SQ_WAVES"], 1)
        print("| %s | %d | %.1f | %.1f | %.1f | %.1f | %.3g | %.0f |" % (
            key, len(dur[key]), us, busy, f16, f32, avg["SQ_INSTS_MFMA"], vpw))


if __name__ == "__main__":
    main(sys.argv[1])
