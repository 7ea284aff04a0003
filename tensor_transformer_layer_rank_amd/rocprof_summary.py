"""Short text summaries of rocprofv3 CSV output (kernel traces and counter
passes), in the form kept under profiles/ and read back by bench.py.

    python -m tensor_transformer_layer_rank_amd.rocprof_summary stats --trace T.csv --out F --command "..."
    python -m tensor_transformer_layer_rank_amd.rocprof_summary traffic --fetch F.csv --write W.csv \\
        --kernel REGEX --grid N --calib-kernel REGEX --calib-bytes B --src gemm.hip --algo-bytes A \\
        --out F --command "..." --command "..."
    python -m tensor_transformer_layer_rank_amd.rocprof_summary sq --pass1 P1.csv --pass2 P2.csv \\
        --target "label=REGEX@GRID" ... --out F --command "..." --command "..."

Dispatches are told apart by kernel name and grid size (total work-items).
HBM traffic: FETCH_SIZE and WRITE_SIZE (KiB per dispatch) are scaled by what
the same counters read for a plain copy kernel of known size: the largest
dispatch of --calib-kernel moves --calib-bytes each way.
"""
from __future__ import annotations

import argparse
import collections
import csv
import hashlib
import os
import re

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "tensor_transformer_layer_rank_amd", "csrc")


def short_name(name: str) -> str:
    """Kernel name without namespaces and parameter lists (templates kept)."""
    n = re.sub(r"^void ", "", name)
    n = n.replace("tps::(anonymous namespace)::", "")
    depth, out = 0, []
    for ch in n:        # drop the argument list: the first '(' at template depth 0
        if ch == "<":
            depth += 1
        elif ch == ">":
            depth -= 1
        elif ch == "(" and depth == 0:
            break
        out.append(ch)
    return "".join(out).strip()


def read_trace(path):
    rows = []
    for r in csv.DictReader(open(path)):
        grid = int(r["Grid_Size_X"]) * int(r["Grid_Size_Y"]) * int(r["Grid_Size_Z"])
        rows.append((int(r["Dispatch_Id"]), short_name(r["Kernel_Name"]), grid,
                     (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3))
    return sorted(rows)


def read_counters(path):
    """{dispatch id: (short name, grid, {counter: value summed over the row's dims})}"""
    out = {}
    for r in csv.DictReader(open(path)):
        d = int(r["Dispatch_Id"])
        if d not in out:
            out[d] = (short_name(r["Kernel_Name"]), int(r["Grid_Size"]), collections.defaultdict(float))
        out[d][2][r["Counter_Name"]] += float(r["Counter_Value"])
    return out


def header(title, commands):
    lines = [f"# {title}"]
    for c in commands:
        lines.append(f"#   {c}")
    return lines


def cmd_stats(a):
    rows = read_trace(a.trace)
    groups = collections.OrderedDict()
    for _, name, grid, us in rows:
        groups.setdefault((name, grid), []).append(us)
    total = sum(us for _, _, _, us in rows)
    lines = header(a.title, a.command)
    lines.append("# kernel | grid (work-items) | calls | avg_us | min_us | max_us | pct_total")
    for (name, grid), v in sorted(groups.items(), key=lambda kv: -sum(kv[1])):
        lines.append(f"{name} | {grid} | {len(v)} | {sum(v) / len(v):.2f} | {min(v):.2f} | {max(v):.2f} | "
                     f"{100 * sum(v) / total:.2f}")
    open(a.out, "w").write("\n".join(lines) + "\n")


def _match(disp, regex, grid):
    rx = re.compile(regex)
    return [c for name, g, c in disp.values() if rx.search(name) and (grid is None or g == grid)]


def cmd_traffic(a):
    fe, wr = read_counters(a.fetch), read_counters(a.write)
    cal_f = max(c["FETCH_SIZE"] for c in _match(fe, a.calib_kernel, None))
    cal_w = max(c["WRITE_SIZE"] for c in _match(wr, a.calib_kernel, None))
    f_factor = a.calib_bytes / (cal_f * 1024.0)
    w_factor = a.calib_bytes / (cal_w * 1024.0)
    kf = [c["FETCH_SIZE"] for c in _match(fe, a.kernel, a.grid)]
    kw = [c["WRITE_SIZE"] for c in _match(wr, a.kernel, a.grid)]
    if not kf or not kw:
        raise SystemExit(f"no dispatch of {a.kernel} with grid {a.grid}")
    fkib, wkib = sum(kf) / len(kf), sum(kw) / len(kw)
    fetch_b, write_b = fkib * 1024 * f_factor, wkib * 1024 * w_factor
    sha = hashlib.sha256(open(os.path.join(CSRC, a.src), "rb").read()).hexdigest()[:16]
    lines = header(a.title, a.command)
    lines += [f"# Calibration: the largest dispatch of {a.calib_kernel} moves {a.calib_bytes} B each way and reads",
              f"#   FETCH_SIZE = {cal_f:.1f} KiB, WRITE_SIZE = {cal_w:.1f} KiB, so",
              f"#   fetch_factor = {f_factor:.4f}  (true bytes per counted KiB / 1024)",
              f"#   write_factor = {w_factor:.4f}",
              f"# kernel {a.kernel} at grid {a.grid}: {len(kf)} / {len(kw)} dispatches, mean FETCH_SIZE = "
              f"{fkib:.1f} KiB, WRITE_SIZE = {wkib:.1f} KiB",
              f"# algorithmic bytes per launch: {a.algo_bytes} ({a.algo_note})",
              f"# traffic / algorithmic = {(fetch_b + write_b) / a.algo_bytes:.3f}",
              f"kernel_src_sha = {sha}",
              f"fetch_bytes_per_launch = {fetch_b:.0f}",
              f"write_bytes_per_launch = {write_b:.0f}",
              f"traffic_bytes_per_launch = {fetch_b + write_b:.0f}"]
    open(a.out, "w").write("\n".join(lines) + "\n")


SQ_RATIOS = [
    ("wait", "SQ_WAIT_INST_ANY", "SQ_WAVE_CYCLES"),
    ("issue", "SQ_ACTIVE_INST_ANY", "SQ_WAVE_CYCLES"),
    ("lds_conflict", "SQ_LDS_BANK_CONFLICT", "SQ_LDS_IDX_ACTIVE"),
    ("valu_per_mfma", "SQ_INSTS_VALU", "SQ_INSTS_MFMA"),
    ("mfma_busy", "SQ_VALU_MFMA_BUSY_CYCLES", "SQ_BUSY_CYCLES"),
]


def cmd_sq(a):
    p1, p2 = read_counters(a.pass1), read_counters(a.pass2)
    lines = header(a.title, a.command)
    lines += ["# Mean per dispatch over the run's dispatches of each kernel (name and grid).  Ratios:",
              "#   wait = SQ_WAIT_INST_ANY / SQ_WAVE_CYCLES (share of wave lifetime in s_waitcnt)",
              "#   issue = SQ_ACTIVE_INST_ANY / SQ_WAVE_CYCLES (share of wave lifetime issuing)",
              "#   lds_conflict = SQ_LDS_BANK_CONFLICT / SQ_LDS_IDX_ACTIVE",
              "#   valu_per_mfma = SQ_INSTS_VALU / SQ_INSTS_MFMA",
              "#   mfma_busy = SQ_VALU_MFMA_BUSY_CYCLES / SQ_BUSY_CYCLES (per-SIMD MFMA busy summed over the",
              "#     chip's SIMDs, relative to the SQ busy cycles; compare kernels with it, not with 1.0)",
              "# label | kernel | grid | " + " | ".join(r[0] for r in SQ_RATIOS) + " | raw counters"]
    for t in a.target:
        label, rest = t.split("=", 1)
        regex, grid = rest.rsplit("@", 1)
        grid = int(grid)
        tot = collections.defaultdict(float)
        n1 = n2 = 0
        name = None
        for disp in (p1, p2):
            for nm, g, c in disp.values():
                if re.search(regex, nm) and g == grid:
                    name = nm
                    for k, v in c.items():
                        tot[k] += v
                    if disp is p1:
                        n1 += 1
                    else:
                        n2 += 1
        if not n1 or not n2:
            lines.append(f"{label} | {regex} | {grid} | (no dispatches)")
            continue
        mean = {k: v / (n1 if k in next(iter(p1.values()))[2] else n2) for k, v in tot.items()}
        ratios = []
        for _, num, den in SQ_RATIOS:
            ratios.append(f"{mean[num] / mean[den]:.3f}" if mean.get(den) else "-")
        raw = " ".join(f"{k}={mean[k]:.0f}" for k in sorted(mean))
        lines.append(f"{label} | {name} | {grid} | " + " | ".join(ratios) + f" | {raw}")
    open(a.out, "w").write("\n".join(lines) + "\n")


def main():
    ap = argparse.ArgumentParser()
    sp = ap.add_subparsers(dest="cmd", required=True)
    s = sp.add_parser("stats")
    s.add_argument("--trace", required=True)
    t = sp.add_parser("traffic")
    t.add_argument("--fetch", required=True)
    t.add_argument("--write", required=True)
    t.add_argument("--kernel", required=True)
    t.add_argument("--grid", type=int, required=True)
    t.add_argument("--calib-kernel", required=True)
    t.add_argument("--calib-bytes", type=int, required=True)
    t.add_argument("--src", required=True)
    t.add_argument("--algo-bytes", type=int, required=True)
    t.add_argument("--algo-note", default="")
    q = sp.add_parser("sq")
    q.add_argument("--pass1", required=True)
    q.add_argument("--pass2", required=True)
    q.add_argument("--target", action="append", required=True)
    for p in (s, t, q):
        p.add_argument("--out", required=True)
        p.add_argument("--title", required=True)
        p.add_argument("--command", action="append", default=[])
    a = ap.parse_args()
    {"stats": cmd_stats, "traffic": cmd_traffic, "sq": cmd_sq}[a.cmd](a)


if __name__ == "__main__":
    main()
