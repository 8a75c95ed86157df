"""Summaries of rocprofv3 runs for the measurement record.

  python -m block_sparse_full_ssa_amd.profile_summary stats DIR OUT.md TITLE
      kernel table from a `rocprofv3 --kernel-trace --stats --output-format
      csv` output directory;
  python -m block_sparse_full_ssa_amd.profile_summary traffic FETCH WRITE \\
          CAL_FETCH CAL_WRITE OUT.md OUT.json WORKLOAD TOP_K TITLE
      HBM bytes per launch from one `--pmc FETCH_SIZE` and one `--pmc
      WRITE_SIZE` pass (KiB per dispatch, averaged over the dispatches of a
      kernel), each scaled by what the same counter reads for the plain 1 GiB
      device copy of hbm_calibration.py; the JSON records, per matrix
      kernel, the bytes and the sha256 of the kernel's source so that a
      reader can tell when the figures no longer describe the code.

  python -m block_sparse_full_ssa_amd.profile_summary mfma PMC STATS OUT.md [OUT.json WORKLOAD TOP_K] TITLE
      matrix-core use per kernel from one `--pmc MfmaUtil
      SQ_INSTS_VALU_MFMA_MOPS_BF16 GRBM_GUI_ACTIVE` pass: MfmaUtil (the
      matrix pipes' busy cycles summed over the SIMDs over active cycles
      times the SIMD count), the bf16 matrix flops the kernel executed (MOPS
      x 512, the implemented work), and the clock the GPU ran at
      (GRBM_GUI_ACTIVE per XCD over the kernel's average duration in the
      stats run STATS); with OUT.json, those figures of the matrix kernels
      with the sha256 of each kernel's source, as for the traffic.

  python -m block_sparse_full_ssa_amd.profile_summary lds PMC OUT.md TITLE
      per mode of the LDS probe (lds_patterns.py launches modes 0 .. 9 once
      each, in order) from one `--pmc SQ_LDS_BANK_CONFLICT SQ_LDS_IDX_ACTIVE
      SQ_INSTS_LDS GRBM_GUI_ACTIVE` pass: LDS cycles per read instruction and
      the share of them lost to bank conflicts.

Commands are stated in the written summaries; this module only reads CSVs.
"""
from __future__ import annotations

import csv
import glob
import hashlib
import json
import os
import sys
from collections import defaultdict

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
COPY_BYTES = 1 << 30

# matrix kernels whose traffic the benchmark's roofline reports: name prefix -> (id, source)
KERNELS = [("k_bwd_mfma", "bwd_mfma", "bwd_mfma.hip"), ("k_fwd_mfma<0, false,", "fwd_mfma", "fwd_mfma.hip"),
           ("k_bwd_dq", "bwd_dq", "bwd_dq.hip"), ("k_bwd_sparse", "bwd_sparse", "sparse_bwd.hip")]


def short(name: str) -> str:
    n = name.replace("(anonymous namespace)::", "").split("(")[0]
    for pre in ("void ", "ssa::"):
        n = n.replace(pre, "")
    return n.strip()


def counters(d: str):
    """{kernel: {counter: mean value per dispatch}} over a --pmc output directory."""
    tot, cnt = defaultdict(lambda: defaultdict(float)), defaultdict(lambda: defaultdict(set))
    files = glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True)
    if not files:
        raise SystemExit(f"no counter CSV under {d}")
    for f in files:
        for r in csv.DictReader(open(f)):
            k = short(r["Kernel_Name"])
            tot[k][r["Counter_Name"]] += float(r["Counter_Value"])
            cnt[k][r["Counter_Name"]].add(r.get("Dispatch_Id") or r.get("Correlation_Id") or len(cnt[k][r["Counter_Name"]]))
    return {k: {c: v / max(1, len(cnt[k][c])) for c, v in cs.items()} for k, cs in tot.items()}


def copy_kib(d: str, counter: str) -> float:
    vals = [cs[counter] for k, cs in counters(d).items() if counter in cs and "copy" in k.lower()]
    if not vals:
        raise SystemExit(f"no copy kernel with {counter} under {d}")
    return max(vals)


def stats(d: str, out: str, title: str) -> None:
    files = glob.glob(os.path.join(d, "**", "*kernel_stats.csv"), recursive=True)
    if not files:
        raise SystemExit(f"no kernel_stats.csv under {d}")
    rows = list(csv.DictReader(open(files[0])))
    total = sum(float(r["TotalDurationNs"]) for r in rows)
    rows.sort(key=lambda r: -float(r["TotalDurationNs"]))
    lines = [f"| `{short(r['Name'])}` | {r['Calls']} | {float(r['AverageNs']) / 1e6:.3f} | "
             f"{float(r['MinNs']) / 1e6:.3f} | {float(r['MaxNs']) / 1e6:.3f} | "
             f"{100 * float(r['TotalDurationNs']) / total:.1f}% |" for r in rows if short(r["Name"]).startswith("k_")]
    with open(out, "w") as f:
        f.write(title.rstrip() + "\n\n| kernel | calls | avg ms | min ms | max ms | share |\n|---|---|---|---|---|---|\n")
        f.write("\n".join(lines) + "\n")


def traffic(fd, wd, cfd, cwd, out_md, out_json, workload, top_k, title) -> None:
    rf, wf = copy_kib(cfd, "FETCH_SIZE") * 1024 / COPY_BYTES, copy_kib(cwd, "WRITE_SIZE") * 1024 / COPY_BYTES
    fetch, write = counters(fd), counters(wd)
    names = sorted(set(fetch) | set(write), key=lambda k: -(fetch.get(k, {}).get("FETCH_SIZE", 0)
                                                           + write.get(k, {}).get("WRITE_SIZE", 0)))
    lines, table = [], {}
    for k in names:
        fk, wk = fetch.get(k, {}).get("FETCH_SIZE", 0.0), write.get(k, {}).get("WRITE_SIZE", 0.0)
        if not k.startswith("k_"):
            continue
        rb, wb = fk * 1024 / rf, wk * 1024 / wf
        lines.append(f"| `{k}` | {fk:.0f} | {wk:.0f} | {rb / 1e9:.3f} | {wb / 1e9:.3f} |")
        for pre, kid, src in KERNELS:
            if k.startswith(pre):
                sha = hashlib.sha256(open(os.path.join(CSRC, src), "rb").read()).hexdigest()
                table[f"{kid}/{workload}/top_k={top_k}"] = {
                    "bytes_per_launch": int(rb + wb), "read_bytes": int(rb), "write_bytes": int(wb),
                    "source": src, "source_sha256": sha, "from": os.path.relpath(out_md, os.path.dirname(HERE))}
    with open(out_md, "w") as f:
        f.write(title.rstrip() + f"\n\nCopy calibration: FETCH_SIZE reads {rf:.3f} KiB per KiB copied, "
                f"WRITE_SIZE {wf:.3f}; bytes = counter KiB * 1024 / factor.\n\n"
                "| kernel | FETCH_SIZE KiB | WRITE_SIZE KiB | read GB | write GB |\n|---|---|---|---|---|\n")
        f.write("\n".join(lines) + "\n")
    with open(out_json, "w") as f:
        json.dump(table, f, indent=1)
        f.write("\n")


def mfma(pd: str, sd: str, out: str, title: str, out_json: str = None, workload: str = None, top_k: int = None,
         n_xcd: int = 8) -> None:
    pmc = counters(pd)
    files = glob.glob(os.path.join(sd, "**", "*kernel_stats.csv"), recursive=True)
    if not files:
        raise SystemExit(f"no kernel_stats.csv under {sd}")
    avg_ns = {short(r["Name"]): float(r["AverageNs"]) for r in csv.DictReader(open(files[0]))}
    rows = [(k, cs) for k, cs in pmc.items() if k.startswith("k_") and cs.get("MfmaUtil", 0.0) > 0.0]
    rows.sort(key=lambda kc: -kc[1].get("SQ_INSTS_VALU_MFMA_MOPS_BF16", 0.0))
    lines, table = [], {}
    for k, cs in rows:
        flops = cs.get("SQ_INSTS_VALU_MFMA_MOPS_BF16", 0.0) * 512
        ns = avg_ns.get(k)
        clock = f"{cs.get('GRBM_GUI_ACTIVE', 0.0) / n_xcd / ns:.2f}" if ns else "-"
        rate = f"{flops / ns / 1e3:.0f}" if ns and flops else "-"
        lines.append(f"| `{k}` | {cs['MfmaUtil']:.1f} | {flops:.3g} | {rate} | {clock} |")
        for pre, kid, src in KERNELS:
            if out_json and k.startswith(pre):
                sha = hashlib.sha256(open(os.path.join(CSRC, src), "rb").read()).hexdigest()
                table[f"{kid}/{workload}/top_k={top_k}"] = {
                    "mfma_util_pct": round(cs["MfmaUtil"], 1), "executed_bf16_flops": flops,
                    "clock_ghz": round(cs.get("GRBM_GUI_ACTIVE", 0.0) / n_xcd / ns, 2) if ns else None,
                    "source": src, "source_sha256": sha, "from": os.path.relpath(out, os.path.dirname(HERE))}
    if out_json:
        with open(out_json, "w") as f:
            json.dump(table, f, indent=1)
            f.write("\n")
    with open(out, "w") as f:
        f.write(title.rstrip() + "\n\n| kernel | MfmaUtil % | bf16 matrix flops per launch | TFLOP/s (avg duration) "
                "| clock GHz |\n|---|---|---|---|---|\n")
        f.write("\n".join(lines) + "\n")


LDS_MODES = ["16-byte reads, lane l reads chunk l", "transposes, plain 128-byte rows",
             "transposes, 256-byte rows, c ^ (2 (r % 8) + (r / 8) % 2)",
             "transposes, 256-byte rows, c ^ (4 (r % 4) + (r / 4) % 4)",
             "transposes, 256-byte rows, c ^ (r % 16)",
             "row reads, 256-byte rows, c ^ (4 (r % 4) + (r / 4) % 4)",
             "row reads, 128-byte rows, c ^ (r % 8)",
             "row reads, 128-byte rows, c ^ (4 ((r / 2) % 2) + (r / 4) % 4)",
             "transposes, 128-byte rows, c ^ (r % 8)",
             "transposes, 128-byte rows, c ^ (4 ((r / 2) % 2) + (r / 4) % 4)"]


def lds(pd: str, out: str, title: str) -> None:
    files = glob.glob(os.path.join(pd, "**", "*counter_collection.csv"), recursive=True)
    if not files:
        raise SystemExit(f"no counter CSV under {pd}")
    by = defaultdict(lambda: defaultdict(float))
    for f in files:
        for r in csv.DictReader(open(f)):
            if "probe_lds" in r["Kernel_Name"]:
                by[int(r.get("Dispatch_Id") or r["Correlation_Id"])][r["Counter_Name"]] += float(r["Counter_Value"])
    ids = sorted(by)
    if len(ids) != len(LDS_MODES):
        raise SystemExit(f"expected {len(LDS_MODES)} probe dispatches, found {len(ids)}")
    lines = []
    for mode, d in enumerate(ids):
        c = by[d]
        cyc = c["SQ_LDS_IDX_ACTIVE"] / c["SQ_INSTS_LDS"]
        share = c["SQ_LDS_BANK_CONFLICT"] / max(c["SQ_LDS_IDX_ACTIVE"], 1.0)
        lines.append(f"| {mode} | {LDS_MODES[mode]} | {cyc:.2f} | {100 * share:.1f} |")
    with open(out, "w") as f:
        f.write(title.rstrip() + "\n\n| mode | pattern | LDS cycles per read instruction | conflict cycles % |\n"
                "|---|---|---|---|\n")
        f.write("\n".join(lines) + "\n")


if __name__ == "__main__":
    a = sys.argv[1:]
    if a and a[0] == "stats" and len(a) == 4:
        stats(a[1], a[2], a[3])
    elif a and a[0] == "traffic" and len(a) == 10:
        traffic(*a[1:8], int(a[8]), a[9])
    elif a and a[0] == "mfma" and len(a) == 5:
        mfma(a[1], a[2], a[3], a[4])
    elif a and a[0] == "mfma" and len(a) == 8:
        mfma(a[1], a[2], a[3], a[7], a[4], a[5], int(a[6]))
    elif a and a[0] == "lds" and len(a) == 4:
        lds(a[1], a[2], a[3])
    else:
        raise SystemExit(__doc__)
