"""Text summaries of rocprofv3 runs (rocpd SQLite output) for profiles/.

    python -m sparse_mixture_experts_switch_amd.profsummary trace DB OUT --cmd "..."
        per-kernel dispatch count and average / min / max duration
    python -m sparse_mixture_experts_switch_amd.profsummary traffic FETCH_DB WRITE_DB OUT \
        --kernel NAME --cmd "..." --source FILE
        HBM bytes per launch of one kernel from FETCH_SIZE and WRITE_SIZE (KiB
        per dispatch), each scaled by what the same counter reads for a plain
        1 GiB device-to-device copy recorded in the same run
    python -m sparse_mixture_experts_switch_amd.profsummary mfma DB OUT --cmd "..." --simds N --xcds X --source FILE
        per kernel: MFMA busy fraction = SQ_VALU_MFMA_BUSY_CYCLES (summed over
        SIMDs) / (GRBM_GUI_ACTIVE / X x SIMDs) and bf16 MFMA flops per
        dispatch (SQ_INSTS_VALU_MFMA_MOPS_BF16 x 512)
    python -m sparse_mixture_experts_switch_amd.profsummary counters DB OUT --kernels a,b --cmd "..." --source FILE
        per listed kernel: the per-dispatch average of every counter the run
        collected, and, when present, LDS bank-conflict cycles per LDS-active
        cycle (SQ_LDS_BANK_CONFLICT / SQ_ACTIVE_INST_LDS) and the fraction of
        wave cycles spent waiting (SQ_WAIT_INST_ANY / SQ_WAVE_CYCLES)

Kernel names are the library's launch names: ffn_up / ffn_down are the
grouped-GEMM instantiations that gather token rows (ReLU epilogue) and that
scatter through the combine epilogue, reading tiled expert weights;
ffn_up_rows / ffn_down_rows the same on row-major weights.
"""

from __future__ import annotations

import argparse
import collections
import hashlib
import sqlite3

COPY_BYTES = 1 << 30
KERNEL_KEYS = {
    "ffn": ("ffn_fused_bf16_kernel", ""),
    # <MB, NBW, waves, gather, epilogue, tiled, ...>, mangled or demangled
    "ffn_up": ("ffn_gemm_bf16_kernel", ("Lb1ELi0ELb1E", "true, 0, true")),
    "ffn_down": ("ffn_gemm_bf16_kernel", ("Lb0ELi2ELb1E", "false, 2, true")),
    "ffn_up_rows": ("ffn_gemm_bf16_kernel", ("Lb1ELi0ELb0E", "true, 0, false")),
    "ffn_down_rows": ("ffn_gemm_bf16_kernel", ("Lb0ELi2ELb0E", "false, 2, false")),
    "router": ("router_fwd_bf16_kernel", ""),
    "router_planes": ("router_wplanes_kernel", ""),
    "assign": ("assign_one_kernel", ""),
    "assign_scan": ("assign_scan_kernel", ""),
    "assign_apply": ("assign_apply_layer_kernel", ""),
    "dispatch": ("dispatch_kernel", ""),
    "combine": ("combine_kernel", ""),
    "add_norm": ("add_norm_kernel", "Lb0E"),
    # the combine instantiation (its name has come back demangled without the bool value)
    "combine_add_norm": ("add_norm_kernel", ""),
    "route_fused": ("route_fused_bf16_kernel", ""),
    "route_clear": ("route_sync_clear_kernel", ""),
    "topk_sum": ("topk_sum_kernel", ""),
    "bwd_dz": ("bwd_gemm_bf16_kernel", "Lb0ELb1ELb0ELb1ELb0ELi0E"),
    "bwd_dx": ("bwd_gemm_bf16_kernel", "Lb0ELb0ELb0ELb1ELb0ELi1E"),
    # weight gradients: the resident-operand kernel (capacity <= 160; its name
    # comes back demangled or mangled), else the general tile kernel
    "bwd_dw_out": ("wgrad_res_bf16_kernel", ("<true, true>", "ILb1ELb1EE")),
    "bwd_dw_in": ("wgrad_res_bf16_kernel", ("<false, false>", "ILb0ELb0EE")),
    "bwd_dw_out_general": ("bwd_gemm_bf16_kernel", "Lb1ELb1ELb1ELb1ELb0ELi2E"),
    "bwd_dw_in_general": ("bwd_gemm_bf16_kernel", "Lb1ELb0ELb0ELb1ELb1ELi2E"),
    "bwd_router": ("router_bwd_bf16_kernel", ""),
    "bwd_router_dx": ("bwd_gemm_bf16_kernel", "Lb0ELb0ELb0ELb1ELb0ELi3E"),
    "bwd_router_planes": ("router_wr_planes_kernel", ""),
    "bwd_router_w": ("router_wgrad_bf16_kernel", ""),
    "bwd_router_w_sum": ("router_wgrad_sum_kernel", ""),
    "copy": ("__amd_rocclr_copyBuffer", ""),
}


def short_name(full: str) -> str:
    for short, (a, b) in KERNEL_KEYS.items():
        if a in full and any(x in full for x in (b if isinstance(b, tuple) else (b,))):
            return short
    return full[:60]


def _trace(db_path: str):
    db = sqlite3.connect(db_path)
    rows = db.execute("select name, start, end from kernels").fetchall()
    agg = collections.defaultdict(list)
    for name, s, e in rows:
        agg[name].append((e - s) / 1e3)
    return agg


def _counter(db_path: str, counter: str):
    db = sqlite3.connect(db_path)
    rows = db.execute("select kernel_name, value from counters_collection where counter_name = ?",
                      (counter,)).fetchall()
    agg = collections.defaultdict(list)
    for name, v in rows:
        agg[name].append(float(v))
    return agg


def trace_summary(db: str, cmd: str) -> str:
    agg = _trace(db)
    lines = [f"# rocprofv3 kernel trace summary", f"# command: {cmd}",
             "# kernel | dispatches | avg_us | min_us | max_us | full name"]
    for name, v in sorted(agg.items(), key=lambda kv: -sum(kv[1])):
        lines.append(f"{short_name(name)} | {len(v)} | {sum(v) / len(v):.2f} | {min(v):.2f} | {max(v):.2f} | {name[:160]}")
    return "\n".join(lines) + "\n"


def traffic_summary(fetch_db: str, write_db: str, kernel: str, cmd: str, source: str) -> str:
    fetch, write = _counter(fetch_db, "FETCH_SIZE"), _counter(write_db, "WRITE_SIZE")

    def pick(agg, short):
        vals = [v for name, vs in agg.items() if short_name(name) == short for v in vs]
        return vals

    kf, kw = pick(fetch, kernel), pick(write, kernel)
    cf, cw = pick(fetch, "copy"), pick(write, "copy")
    if not kf or not kw or not cf or not cw:
        raise SystemExit(f"missing dispatches: kernel fetch {len(kf)} write {len(kw)}, copy {len(cf)} {len(cw)}")
    fetch_factor = COPY_BYTES / (max(cf) * 1024.0)
    write_factor = COPY_BYTES / (max(cw) * 1024.0)
    f_kib, w_kib = sum(kf) / len(kf), sum(kw) / len(kw)
    hbm = f_kib * 1024.0 * fetch_factor + w_kib * 1024.0 * write_factor
    with open(source, "rb") as fh:
        digest = hashlib.sha256(fh.read()).hexdigest()[:16]
    return "\n".join([
        f"# HBM traffic of {kernel} (base workload), rocprofv3 --pmc",
        f"# command (FETCH_SIZE pass): {cmd.replace('COUNTER', 'FETCH_SIZE')}",
        f"# command (WRITE_SIZE pass): {cmd.replace('COUNTER', 'WRITE_SIZE')}",
        f"# calibration: a 1 GiB device-to-device copy in the same run reads {max(cf):.0f} KiB FETCH_SIZE",
        f"#   and {max(cw):.0f} KiB WRITE_SIZE; factors = true bytes / counter bytes",
        f"kernel = {kernel}",
        f"source_sha256 = {digest}",
        f"dispatches = {len(kf)}",
        f"fetch_kib_per_dispatch = {f_kib:.1f}",
        f"write_kib_per_dispatch = {w_kib:.1f}",
        f"fetch_factor = {fetch_factor:.4f}",
        f"write_factor = {write_factor:.4f}",
        f"hbm_bytes_per_launch = {hbm:.0f}",
    ]) + "\n"


def mfma_summary(db: str, cmd: str, simds: int, xcds: int, source: str) -> str:
    busy = _counter(db, "SQ_VALU_MFMA_BUSY_CYCLES")
    gui = _counter(db, "GRBM_GUI_ACTIVE")
    mops = _counter(db, "SQ_INSTS_VALU_MFMA_MOPS_BF16")
    with open(source, "rb") as fh:
        digest = hashlib.sha256(fh.read()).hexdigest()[:16]
    lines = [f"# MFMA use per kernel (base workload), rocprofv3 --pmc", f"# command: {cmd}",
             f"# mfma_busy = SQ_VALU_MFMA_BUSY_CYCLES (sum over SIMDs) / ((GRBM_GUI_ACTIVE / {xcds}) x {simds} SIMDs),",
             f"#   averaged over dispatches (GRBM_GUI_ACTIVE is stored summed over the {xcds} XCDs' GRBM instances)",
             f"# bf16_mfma_gflop = SQ_INSTS_VALU_MFMA_MOPS_BF16 x 512 / 1e9 per dispatch",
             f"source_sha256 = {digest}",
             "# kernel | dispatches | mfma_busy | bf16_mfma_gflop"]
    for name in sorted(busy, key=lambda n: -sum(busy[n])):
        short = short_name(name)
        if short not in KERNEL_KEYS or short == "copy" or name not in gui:
            continue
        b, g = busy[name], gui[name]
        frac = sum(bi / (gi / xcds * simds) for bi, gi in zip(b, g) if gi > 0) / len(b)
        gf = sum(mops.get(name, [0.0])) / max(len(mops.get(name, [])), 1) * 512 / 1e9
        lines.append(f"{short} | {len(b)} | {frac:.4f} | {gf:.2f}")
    return "\n".join(lines) + "\n"


def counters_summary(db: str, kernels: list, cmd: str, source: str) -> str:
    con = sqlite3.connect(db)
    names = [r[0] for r in con.execute("select distinct counter_name from counters_collection")]
    with open(source, "rb") as fh:
        digest = hashlib.sha256(fh.read()).hexdigest()[:16]
    lines = [f"# counters per dispatch (base workload), rocprofv3 --pmc", f"# command: {cmd}",
             f"source_sha256 = {digest}"]
    for short in kernels:
        vals = {}
        for cname in names:
            agg = _counter(db, cname)
            v = [x for name, xs in agg.items() if short_name(name) == short for x in xs]
            if v:
                vals[cname] = sum(v) / len(v)
        if not vals:
            lines.append(f"{short}: no dispatches")
            continue
        n = len([x for name, xs in _counter(db, names[0]).items() if short_name(name) == short for x in xs])
        lines.append(f"[{short}] dispatches = {n}")
        for cname in sorted(vals):
            lines.append(f"{short}.{cname} = {vals[cname]:.6g}")
        if vals.get("SQ_ACTIVE_INST_LDS") and "SQ_LDS_BANK_CONFLICT" in vals:
            lines.append(f"{short}.lds_bank_conflict_per_lds_active_cycle = "
                         f"{vals['SQ_LDS_BANK_CONFLICT'] / vals['SQ_ACTIVE_INST_LDS']:.4f}")
        if vals.get("SQ_WAVE_CYCLES") and "SQ_WAIT_INST_ANY" in vals:
            lines.append(f"{short}.wait_fraction_of_wave_cycles = {vals['SQ_WAIT_INST_ANY'] / vals['SQ_WAVE_CYCLES']:.4f}")
    return "\n".join(lines) + "\n"


def main():
    ap = argparse.ArgumentParser()
    sub = ap.add_subparsers(dest="mode", required=True)
    t = sub.add_parser("trace")
    t.add_argument("db")
    t.add_argument("out")
    t.add_argument("--cmd", required=True)
    c = sub.add_parser("traffic")
    c.add_argument("fetch_db")
    c.add_argument("write_db")
    c.add_argument("out")
    c.add_argument("--kernel", required=True)
    c.add_argument("--cmd", required=True)
    c.add_argument("--source", required=True)
    m = sub.add_parser("mfma")
    m.add_argument("db")
    m.add_argument("out")
    m.add_argument("--cmd", required=True)
    m.add_argument("--simds", type=int, required=True)
    m.add_argument("--xcds", type=int, required=True)
    m.add_argument("--source", required=True)
    k = sub.add_parser("counters")
    k.add_argument("db")
    k.add_argument("out")
    k.add_argument("--kernels", required=True)
    k.add_argument("--cmd", required=True)
    k.add_argument("--source", required=True)
    a = ap.parse_args()
    if a.mode == "trace":
        text = trace_summary(a.db, a.cmd)
    elif a.mode == "traffic":
        text = traffic_summary(a.fetch_db, a.write_db, a.kernel, a.cmd, a.source)
    elif a.mode == "counters":
        text = counters_summary(a.db, a.kernels.split(","), a.cmd, a.source)
    else:
        text = mfma_summary(a.db, a.cmd, a.simds, a.xcds, a.source)
    with open(a.out, "w") as fh:
        fh.write(text)
    print(text)


if __name__ == "__main__":
    main()
