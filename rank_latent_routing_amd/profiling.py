"""Summaries of rocprofv3 output for the committed profiles (host only).

Every markdown file under ``profiles/`` that reports counters or kernel times
is written by this module from the CSV files rocprofv3 leaves in its output
directories, through ``python bench.py --summarize NAME DIR [DIR ...]``.  Each
recipe below names the rocprofv3 commands that produce its inputs; the file
it writes repeats them.  Nothing here touches a GPU.

Counter conventions on gfx950 (rocprofv3's descriptions, checked against the
issue-rate probes of ``probes/issue.hip``, whose instruction mix is known):

* ``GRBM_GUI_ACTIVE`` is summed over the 8 XCDs: kernel cycles = value / 8.
* ``SQ_ACTIVE_INST_VALU`` counts VALU issue quad-cycles (4 cycles) summed over
  waves: one per VALU instruction or matrix-core issue, two per
  transcendental instruction.
* ``SQ_ACTIVE_INST_VALU2`` counts quad-cycles in which a SIMD issued two VALU
  instructions from two waves; while the matrix core is busy it stays near 0.
* ``SQ_VALU_MFMA_BUSY_CYCLES`` counts matrix-core busy cycles per SIMD (32 per
  v_mfma_f32_32x32x16_bf16).
* ``SQ_BUSY_CYCLES`` and ``SQ_CYCLES`` are per shader engine (32 of them):
  their ratio is the share of the kernel's time an engine held any wave.
"""
import collections
import csv
import glob
import os

XCDS = 8
SIMDS = 1024  # 256 compute units x 4

# VALU issue quads a 32 x 32 score block needs by the method: 4 matrix-core
# issues, 16 scale multiplies, 16 exponentials (2 quads each), 8 bf16 packs
# and 8 dot2 row sums.
BLOCK_FLOOR_QUADS = 4 + 16 + 32 + 8 + 8

BENCH_ARGS = "--steps 2 --warmup 1 --no-cpu --no-mix --no-bwd --no-sweep"
BENCH_STEP_LAUNCHES = (1, 3)  # the timed steps of BENCH_ARGS among each kernel's launches (after 1 warm-up)
PASSES = [
    "SQ_WAVE_CYCLES SQ_BUSY_CYCLES SQ_WAIT_ANY SQ_WAIT_INST_ANY SQ_ACTIVE_INST_ANY SQ_ACTIVE_INST_VALU "
    "SQ_ACTIVE_INST_VALU2 SQ_VALU_MFMA_BUSY_CYCLES GRBM_GUI_ACTIVE",
    "SQ_INSTS_VALU SQ_INSTS_MFMA SQ_INSTS_LDS SQ_INSTS_SALU SQ_INSTS_VALU_TRANS_F32 SQ_ACTIVE_INST_LDS "
    "SQ_WAIT_INST_LDS SQ_VALU_MFMA_COEXEC_CYCLES GRBM_GUI_ACTIVE",
    "SQ_INST_LEVEL_LDS SQ_LDS_IDX_ACTIVE SQ_LDS_BANK_CONFLICT SQ_ACTIVE_INST_SCA SQ_ACTIVE_INST_MISC "
    "SQ_INSTS_SMEM SQ_INSTS_BRANCH SQ_CYCLES GRBM_GUI_ACTIVE",
]
PROBE_MIXES = "mfma,mul,exp,cvt,dot2,mul+exp,mfma+8mul,mfma+16exp,block,block-dep,block-nomul,block-hilo"
PROBE_ITERS = 4000


def _pmc_commands(target, regex, outdir):
    return ["export TMPDIR=/tmp"] + [
        f"timeout -s KILL 90 rocprofv3 --pmc {p} --kernel-include-regex \"{regex}\" -f csv "
        f"-d gpurun_out/{outdir}{i + 1} -o run -- {target}" for i, p in enumerate(PASSES)]


BUDGET_CMDS = _pmc_commands(f"python3 -u bench.py {BENCH_ARGS}", "encode_bf16|decode_bf16|merge_kernel",
                            "pmc/bench")
PROBE_CMDS = _pmc_commands(
    f"python3 -u rank_latent_routing_amd/probes/run_probes.py --mixes {PROBE_MIXES} --wps 4 --no-split "
    f"--iters {PROBE_ITERS}", "probe_kernel", "pmc/probe")


def _csvs(dirs, pattern):
    out = []
    for d in dirs:
        out += sorted(glob.glob(os.path.join(d, "**", pattern), recursive=True))
    if not out:
        raise FileNotFoundError(f"no {pattern} under {dirs}")
    return out


def short_name(kernel):
    """'void flare::encode_bf16_kernel<32, 8>(flare::EncodeParams)' -> 'encode_bf16_kernel<32, 8>'."""
    k = kernel.replace("(anonymous namespace)::", "").split("(")[0]
    for pre in ("void ", "flare::"):
        k = k.replace(pre, "")
    return k.strip()


def dispatch_counters(dirs, select=None, by_pass=False):
    """{kernel: [ {counter: value} per dispatch ]} from every counter CSV under
    the given rocprofv3 output directories (the rows of a dispatch summed).
    With by_pass, {kernel: {csv path: [dispatches]}} instead."""
    per = collections.defaultdict(lambda: collections.defaultdict(lambda: collections.defaultdict(float)))
    for path in _csvs(dirs, "*counter_collection.csv"):
        for row in csv.DictReader(open(path)):
            k = short_name(row["Kernel_Name"])
            if select and not any(s in k for s in select):
                continue
            per[k][(path, row["Dispatch_Id"])][row["Counter_Name"]] += float(row["Counter_Value"])
    if by_pass:
        out = collections.defaultdict(lambda: collections.defaultdict(list))
        for k, d in per.items():
            for (path, _), v in d.items():
                out[k][path].append(v)
        return out
    return {k: list(d.values()) for k, d in per.items()}


def counter_means(dirs, select=None, launches=None):
    """{kernel: {counter: mean over the dispatches that read it}}; with
    `launches` = (lo, hi), over dispatches lo .. hi - 1 of each kernel in each
    run only."""
    out = {}
    if launches is not None:
        od = _ordered_dispatches(dirs, select)
        per = {k: [d for ds in byp.values() for d in ds[launches[0]:launches[1]]] for k, byp in od.items()}
    else:
        per = dispatch_counters(dirs, select)
    for k, ds in per.items():
        acc = collections.defaultdict(list)
        for d in ds:
            for c, v in d.items():
                acc[c].append(v)
        out[k] = {c: sum(v) / len(v) for c, v in acc.items()}
    return out


def cycle_budget(c, units, floor_quads):
    """Per-unit SIMD-cycle budget from counter means c (units: 32 x 32 score
    blocks per dispatch, or probe loop iterations of all waves)."""
    cycles = c["GRBM_GUI_ACTIVE"] / XCDS
    nan = float("nan")
    valu_q = c["SQ_ACTIVE_INST_VALU"] / units
    dual_q = c.get("SQ_ACTIVE_INST_VALU2", 0.0) / units
    issue = 4.0 * (valu_q - dual_q)
    simd = cycles * SIMDS / units
    return {
        "cycles": simd, "valu_quads": valu_q, "dual_quads": dual_q, "issue": issue,
        "floor": 4.0 * floor_quads, "extra": issue - 4.0 * floor_quads, "idle": simd - issue,
        "mfma_busy": c.get("SQ_VALU_MFMA_BUSY_CYCLES", nan) / units,
        "coexec": c.get("SQ_VALU_MFMA_COEXEC_CYCLES", nan) / units,
        "valu": c.get("SQ_INSTS_VALU", nan) / units, "trans": c.get("SQ_INSTS_VALU_TRANS_F32", nan) / units,
        "mfma": c.get("SQ_INSTS_MFMA", nan) / units, "lds": c.get("SQ_INSTS_LDS", nan) / units,
        "salu": c.get("SQ_INSTS_SALU", nan) / units,
        "se_busy": c["SQ_BUSY_CYCLES"] / c["SQ_CYCLES"] if "SQ_BUSY_CYCLES" in c and "SQ_CYCLES" in c else nan,
        "wait_inst": c["SQ_WAIT_INST_ANY"] / c["SQ_WAVE_CYCLES"] if "SQ_WAIT_INST_ANY" in c and "SQ_WAVE_CYCLES" in c
        else nan,
        "wait_any": c["SQ_WAIT_ANY"] / c["SQ_WAVE_CYCLES"] if "SQ_WAIT_ANY" in c and "SQ_WAVE_CYCLES" in c else nan,
    }


def _budget_rows(means, units, floor_quads):
    rows = ["| kernel | SIMD cycles per block | VALU issue | of which the method's floor | other VALU "
            "| no VALU issued | dual issue (quads) | MFMA busy | MFMA busy while VALU issues | VALU instr. "
            "| exp | MFMA | LDS instr. | SALU instr. | engines busy | waves waiting on operands | waves waiting (any) |",
            "|---|---|---|---|---|---|---|---|---|---|---|---|---|---|---|---|---|"]
    budgets = {}
    for k in sorted(means):
        b = cycle_budget(means[k], units, floor_quads)
        budgets[k] = b
        rows.append(f"| `{k}` | {b['cycles']:.0f} | {b['issue']:.0f} ({b['valu_quads']:.1f} quads) "
                    f"| {b['floor']:.0f} | {b['extra']:.0f} | {b['idle']:.0f} | {b['dual_quads']:.2f} "
                    f"| {b['mfma_busy']:.0f} | {b['coexec']:.0f} | {b['valu']:.1f} | {b['trans']:.1f} "
                    f"| {b['mfma']:.1f} | {b['lds']:.1f} | {b['salu']:.1f} | {100 * b['se_busy']:.0f}% "
                    f"| {100 * b['wait_inst']:.0f}% | {100 * b['wait_any']:.0f}% |")
    return rows, budgets


def write_units(out, dirs):
    """profiles/units.encdec_n1m.md: the per-block cycle budget of the bench's
    encode and decode kernels."""
    blocks = 8 * (1 << 20) * 256 // (32 * 32)
    means = counter_means(dirs, ["encode_bf16", "decode_bf16"], launches=BENCH_STEP_LAUNCHES)
    rows, b = _budget_rows(means, blocks, BLOCK_FLOOR_QUADS)
    text = ["# Cycle budget of the encode and decode kernels, bench workload (FLARE encode+decode, B=1, H=8, D=32, "
            "N=1048576, M=256, bf16)", "",
            "Commands (repo root, one MI355X; three counter passes, each a run of its own), then "
            "`python bench.py --summarize units gpurun_out/pmc/bench1 gpurun_out/pmc/bench2 gpurun_out/pmc/bench3`:",
            "", "```"] + BUDGET_CMDS + ["```", "",
            f"Values are means over the timed steps' launches of each kernel (launches "
            f"{BENCH_STEP_LAUNCHES[0]} .. {BENCH_STEP_LAUNCHES[1] - 1}, after the warm-up) in the three runs.  "
            "A block is 32 tokens x 32 "
            f"latents of one head ({blocks} per dispatch).  Cycles are SIMD cycles at the clock the kernel ran "
            "at: GRBM_GUI_ACTIVE / 8 XCDs x 1024 SIMDs, per block.  The counter readings are calibrated on "
            "probe kernels of known instruction mix in `issue_rates.gfx950.md`.", ""] + rows + ["",
            "How the columns add up, per block and SIMD:", "",
            "- *VALU issue* is 4 x (SQ_ACTIVE_INST_VALU - SQ_ACTIVE_INST_VALU2) per block: the cycles the SIMD's "
            "VALU port spends issuing. One quad per VALU instruction or matrix-core issue, two per exponential.",
            f"- *The method's floor* is {BLOCK_FLOOR_QUADS} quads: 4 matrix-core issues, 16 scale multiplies, "
            "16 exponentials, 8 bf16 packs and 8 dot2 row sums. *Other VALU* is the rest of the issue time "
            "(accumulator copies, address and range arithmetic, the epilogue, amortised per block).",
            "- *No VALU issued* is the kernel's cycles minus the issue time: cycles in which no wave of the SIMD "
            "had a VALU instruction ready (waiting on LDS, on the tile barrier, on the matrix core's result or "
            "its issue), plus the time a SIMD holds fewer waves (workgroup start-up and the tail; *engines busy* "
            "is SQ_BUSY_CYCLES / SQ_CYCLES).  The two waiting columns are SQ_WAIT_INST_ANY and SQ_WAIT_ANY over "
            "SQ_WAVE_CYCLES: the share of wave-cycles in which a wave waited for an instruction's operands "
            "(LDS, memory, the matrix core's result), and for anything (also barriers and counters).  With four "
            "(encoder) or three (decoder) waves per SIMD a wave may wait while another issues, so these shares "
            "are not cycles lost by the SIMD; *no VALU issued* is.",
            "- *MFMA busy* overlaps the VALU issue only in part (the co-execution column), and no dual issue "
            "happens while the matrix core is busy. A block's time answers to both: timed variants of the two "
            "kernels (not kept) that fold the scale into bf16 Q, 16 multiplies fewer (-64 issue cycles), took "
            "28 (encode) and 36 (decode) cycles less per block; variants that instead feed Q x scale as a bf16 "
            "high and low pair, no multiplies but 2 more products (+64 matrix-core cycles), took 70 and 38 "
            "cycles more.  HBM is not the limit (the traffic files: 1.03-1.04 x the algorithmic bytes at under "
            "30 % of the peak rate)."]
    open(out, "w").write("\n".join(text) + "\n")
    return b


PROBE_NAMES = {0: "mfma", 1: "mul", 2: "exp", 3: "cvt", 4: "dot2", 5: "mul+exp", 7: "mfma+8mul", 11: "mfma+16exp",
               12: "block", 13: "block-nomul", 15: "block-dep", 23: "block-hilo"}
# (VALU instructions, MFMA instructions, exponentials) per loop iteration of one wave
PROBE_MIX = {0: (8, 8, 0), 1: (32, 0, 0), 2: (32, 0, 32), 3: (16, 0, 0), 4: (16, 0, 0), 5: (32, 0, 16),
             7: (72, 8, 0), 11: (136, 8, 128), 12: (52, 4, 16), 13: (36, 4, 16), 15: (52, 4, 16), 23: (38, 6, 16)}


def write_issue_rates(out, dirs, timing_md):
    """profiles/issue_rates.gfx950.md: the probes' timing table (run_probes
    output) and their counter readings, which calibrate the counters."""
    passes = dispatch_counters(dirs, ["probe_kernel"], by_pass=True)
    per = {}
    for k, byp in passes.items():
        # each mix runs a short warm-up launch, then the measured one: take the
        # longer launch of every pass and merge the passes' counters
        merged = {}
        for ds in byp.values():
            merged.update(max(ds, key=lambda x: x.get("GRBM_GUI_ACTIVE", 0.0)))
        per[k] = [merged]
    waves = 256 * 16
    rows = ["| probe mix | waves/SIMD | SQ_INSTS_VALU per iteration (expected) | SQ_ACTIVE_INST_VALU quads "
            "(expected: 1 per instruction, 2 per exp) | dual-issue quads | MFMA busy cycles (expected 32 per "
            "product) | SIMD cycles per iteration |", "|---|---|---|---|---|---|---|"]
    for k in sorted(per, key=lambda s: int(s.split("<")[1].split(",")[0])):
        idx = int(k.split("<")[1].split(",")[0])
        d = max(per[k], key=lambda x: x.get("GRBM_GUI_ACTIVE", 0.0))  # the measured launch (not the warm-up)
        n = waves * PROBE_ITERS
        v, m, e = PROBE_MIX.get(idx, (0, 0, 0))
        vi = d.get("SQ_INSTS_VALU", float("nan")) / n
        q = d.get("SQ_ACTIVE_INST_VALU", float("nan")) / n
        dq = d.get("SQ_ACTIVE_INST_VALU2", float("nan")) / n
        mb = d.get("SQ_VALU_MFMA_BUSY_CYCLES", float("nan")) / n
        cyc = d["GRBM_GUI_ACTIVE"] / XCDS * SIMDS / n  # SIMD cycles per wave-iteration
        rows.append(f"| {PROBE_NAMES.get(idx, idx)} | 4 | {vi:.1f} ({v}) | {q:.1f} ({v + e}) | {dq:.2f} "
                    f"| {mb:.0f} ({32 * m}) | {cyc:.0f} |")
    text = ["# Issue rates of the inner-loop instructions on gfx950 (MI355X)", "",
            "Probe kernels (`rank_latent_routing_amd/probes/issue.hip`) loop over fixed instruction mixes on "
            "independent registers, one workgroup per compute unit.", "",
            "Timing (repo root, one MI355X): `python -m rank_latent_routing_amd.probes.run_probes`", "",
            open(timing_md).read().strip(), "",
            "## Counter calibration", "",
            "The same probes under the counter passes the kernels' cycle budget uses "
            "(`units.encdec_n1m.md`), then `python bench.py --summarize issue_rates gpurun_out/probes.md "
            "gpurun_out/pmc/probe1 gpurun_out/pmc/probe2 gpurun_out/pmc/probe3`:", "", "```"] + PROBE_CMDS + [
            "```", "", f"Per loop iteration of one wave ({waves} waves, {PROBE_ITERS} iterations):", ""] + rows + [
            "", "Reading:", "",
            "- SQ_ACTIVE_INST_VALU counts one quad-cycle per VALU instruction or matrix-core issue and two per "
            "v_exp_f32; the matrix core counts 32 busy cycles per 32x32x16 product.",
            "- Two waves can issue VALU in the same quad (the `mul` mix dual-issues), but not while an "
            "exponential is in flight or the matrix core is busy: the mixed streams issue one VALU "
            "instruction per 4 cycles.",
            "- A block's mix (4 products, 16 multiplies, 16 exponentials, 8 packs, 8 row-sum dot2) is 68 issue "
            "quads, 272 cycles; its 4 products (128 cycles) run under that issue time."]
    open(out, "w").write("\n".join(text) + "\n")


def write_kernel_stats(out, trace_dir, title, command, notes=()):
    """A kernel-time table from rocprofv3 --kernel-trace --stats output."""
    path = _csvs([trace_dir], "*kernel_stats.csv")[0]
    rows = list(csv.DictReader(open(path)))
    total = sum(float(r["TotalDurationNs"]) for r in rows)
    lines = [f"# {title}", "", "Command (repo root, one MI355X), then `python bench.py --summarize stats "
             f"{trace_dir} gpurun_out/prof_bench.log`:", "", "```", "export TMPDIR=/tmp", command, "```", "",
             "| kernel | calls | average (us) | min (us) | max (us) | share of GPU time |", "|---|---|---|---|---|---|"]
    for r in sorted(rows, key=lambda r: -float(r["TotalDurationNs"])):
        lines.append(f"| `{r['Name'][:90]}` | {r['Calls']} | {float(r['AverageNs']) / 1e3:.1f} "
                     f"| {float(r['MinNs']) / 1e3:.1f} | {float(r['MaxNs']) / 1e3:.1f} "
                     f"| {100 * float(r['TotalDurationNs']) / total:.1f}% |")
    lines += [""] + list(notes)
    open(out, "w").write("\n".join(lines) + "\n")


def trace_durations(trace_dir, select):
    """Durations (us) of each launch of the kernels matching `select`, in dispatch order."""
    path = _csvs([trace_dir], "*kernel_trace.csv")[0]
    out = collections.defaultdict(list)
    rows = sorted(csv.DictReader(open(path)), key=lambda r: int(r["Dispatch_Id"]))
    for r in rows:
        k = short_name(r["Kernel_Name"])
        if any(s in k for s in select):
            out[k].append((int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3)
    return dict(out)


GEMM_ARGS = "--steps 1 --warmup 0 --no-cpu --no-bwd --no-sweep"
GEMM_PASSES = [
    "SQ_WAVE_CYCLES SQ_BUSY_CYCLES SQ_WAIT_INST_ANY SQ_WAIT_ANY SQ_ACTIVE_INST_VALU SQ_ACTIVE_INST_LDS "
    "SQ_VALU_MFMA_BUSY_CYCLES SQ_WAIT_INST_LDS",
    "SQ_INSTS_VALU SQ_INSTS_MFMA SQ_INSTS_LDS SQ_LDS_BANK_CONFLICT SQ_INSTS_VMEM_WR SQ_INSTS_VMEM_RD GRBM_GUI_ACTIVE",
    "FETCH_SIZE",
    "WRITE_SIZE",
]


def _copy_factors(profiles_dir):
    """Read / write scale factors of FETCH_SIZE / WRITE_SIZE: bytes of a plain
    1 GiB device copy over what the counters read for it, from the committed
    traffic summary of the bench kernels."""
    import json
    d = json.load(open(os.path.join(profiles_dir, "traffic_encode_bf16_kernel.encdec_n1m.json")))
    return d["copy_factor_read"], d["copy_factor_write"]


def write_units_gemm(out, dirs, profiles_dir):
    """profiles/units_gemm.mix_n1m.md: counters of the projection GEMM in the
    first FLARE++ mixer call of the bench (four input projections, then W_O)."""
    fr, fw = _copy_factors(profiles_dir)
    firsts = {}
    for d in dirs:
        for path in _csvs([d], "*counter_collection.csv"):
            rows = [r for r in csv.DictReader(open(path)) if "gemm_bf16" in r["Kernel_Name"]]
            ids = sorted({int(r["Dispatch_Id"]) for r in rows})[:2]
            for r in rows:
                i = int(r["Dispatch_Id"])
                if i in ids:
                    key = ids.index(i)
                    firsts.setdefault(key, {"kernel": short_name(r["Kernel_Name"])})
                    firsts[key][r["Counter_Name"]] = firsts[key].get(r["Counter_Name"], 0.0) + float(r["Counter_Value"])
    R = 1 << 20
    alg_read = R * 256 * 2
    labels = {0: ("four input projections (X W_K, X W_V, X W_eK, X W_eV), head-major out", 4),
              1: ("output projection (Y W_O), row-major out", 1)}
    lines = ["# Projection GEMM counters, FLARE++ mixer (B=1, N=1048576, C=256, H=8, D=32, M=256, bf16, all "
             "projections)", "",
             "Commands (repo root, one MI355X; each counter group in a run of its own), then `python bench.py "
             "--summarize units_gemm gpurun_out/gpmc1 gpurun_out/gpmc2 gpurun_out/gpmc3 gpurun_out/gpmc4`:", "",
             "```", "export TMPDIR=/tmp"] + [
        f"timeout -s KILL 120 rocprofv3 --pmc {p} --kernel-include-regex gemm_bf16 -f csv -d gpurun_out/gpmc{i + 1} "
        f"-o run -- python3 -u bench.py {GEMM_ARGS}" for i, p in enumerate(GEMM_PASSES)] + ["```", "",
             "The first two GEMM dispatches of each run are the first FLARE++ mixer call: its four input "
             "projections, then its output projection.  The byte counters are scaled by the copy calibration of "
             f"`traffic.encdec_n1m.md` (read x{fr:.4f}, write x{fw:.4f}).  MFMA busy is SQ_VALU_MFMA_BUSY_CYCLES "
             "over SIMD cycles (GRBM_GUI_ACTIVE / 8 XCDs x 1024 SIMDs); each `v_mfma_f32_16x16x32_bf16` counts 16 "
             "busy cycles.", "",
             "| launch | kernel | MFMA instructions | MFMA busy | GB read (algorithmic) | GB written (algorithmic) "
             "| LDS bank conflicts |", "|---|---|---|---|---|---|---|"]
    for key in sorted(firsts):
        c = firsts[key]
        label, nout = labels.get(key, (str(key), 1))
        simd = c.get("GRBM_GUI_ACTIVE", float("nan")) / XCDS * SIMDS
        busy = c.get("SQ_VALU_MFMA_BUSY_CYCLES", float("nan")) / simd
        rd = c.get("FETCH_SIZE", float("nan")) * 1024 * fr / 1e9
        wr = c.get("WRITE_SIZE", float("nan")) * 1024 * fw / 1e9
        lines.append(f"| {label} | `{c['kernel']}` | {c.get('SQ_INSTS_MFMA', float('nan')):.4g} | {100 * busy:.0f}% "
                     f"| {rd:.3f} ({alg_read / 1e9:.3f}) | {wr:.3f} ({nout * alg_read / 1e9:.3f}) "
                     f"| {c.get('SQ_LDS_BANK_CONFLICT', float('nan')):.0f} |")
    lines += ["", "Reading:", "",
              "- X (0.537 GB) is read once; the rest of the read bytes are the weights and neighbouring blocks.",
              "- Every output is written exactly once. The row-major W_O output pairs its 32-column blocks "
              "(`PAIR`): both halves of each 128-byte line of a row are stored by one wave, back to back.",
              "- The matrix cores are busy for about 40 % of SIMD cycles in the four-output launch; the kernel sits "
              "between the matrix-core and HBM bounds."]
    open(out, "w").write("\n".join(lines) + "\n")


# ---------------------------------------------------------------- kernel time

STATS_CMD = ("timeout -k 10 900 rocprofv3 --kernel-trace --stats -f csv -d gpurun_out/prof_bench -o run "
             "-- python3 -u bench.py > gpurun_out/prof_bench.log")
STATS_NOTES = [
    "The run is the default bench: 5 warm-up and 20 timed encode+decode steps; the FLARE++ attention extra "
    "at the same sizes; the sharp-score extra (Q x 40: default and exact softmax); the backward leg (the "
    "one-call pair backward, the two-call chain, the one-call form with bf16 dK and dV); the shader-clock "
    "samples; the three mixer extras at N=1048576, C=256 with all projections; the small FLARE++ mixer "
    "(eager and graph replays); the sequence and block FLARE++ workloads; the sweep over the token count; "
    "and the oracle CPU sample.",
    "",
    "Each mixer call launches the projection GEMMs, the query synthesis (an encode) and one encode and decode "
    "of its own sizes, so the encode/decode rows average over every use; the bench line's roofline times the "
    "metric workload's launches alone, with HIP events on the launching stream."]


STATS_STEP_LAUNCHES = (5, 25)  # the default bench's 20 timed steps, after 5 warm-up steps


def write_stats(out, trace_dir, bench_log=None):
    """profiles/kernel_stats.encdec_n1m.md from a --kernel-trace --stats run of the default bench, with
    the metric step's own launches (the timed steps) beside the bench line's live timing of them."""
    import json
    per, _ = kernel_trace([trace_dir], ["encode_bf16_kernel<32, 8>", "merge_kernel", "decode_bf16_kernel<32>"])
    lo, hi = STATS_STEP_LAUNCHES
    steps = {k: v[lo:hi] for k, v in per.items()}
    live = {}
    if bench_log and os.path.exists(bench_log):
        for l in open(bench_log):
            if l.startswith("{"):
                e = json.loads(l)
                live = {"encode": e["extra"]["encode_ms"] * 1e3, "decode": e["extra"]["decode_ms"] * 1e3,
                        "kernel": e["roofline"]["kernel"]}
    notes = list(STATS_NOTES) + ["", f"The metric step's launches alone (dispatches {lo} .. {hi - 1} of each "
                                 "kernel: the 20 timed steps after 5 warm-up steps), from the same trace:", "",
                                 "| kernel | launches | average (us) | min (us) | max (us) |", "|---|---|---|---|---|"]
    for k in ("encode_bf16_kernel<32, 8>", "merge_kernel", "decode_bf16_kernel<32>"):
        v = steps.get(k, [])
        if v:
            notes.append(f"| `{k}` | {len(v)} | {sum(v) / len(v) / 1e3:.1f} | {min(v) / 1e3:.1f} | {max(v) / 1e3:.1f} |")
    if live and steps.get("decode_bf16_kernel<32>") and steps.get("encode_bf16_kernel<32, 8>"):
        enc = (sum(steps["encode_bf16_kernel<32, 8>"]) / len(steps["encode_bf16_kernel<32, 8>"])
               + sum(steps.get("merge_kernel", [0])) / max(1, len(steps.get("merge_kernel", [0])))) / 1e3
        dec = sum(steps["decode_bf16_kernel<32>"]) / len(steps["decode_bf16_kernel<32>"]) / 1e3
        notes += ["", f"The bench line of this traced run timed the encode call (encode + merge) at "
                  f"{live['encode']:.1f} us and the decode call at {live['decode']:.1f} us with HIP events on the "
                  f"launch stream, against {enc:.1f} and {dec:.1f} us of kernel time here; the events also take "
                  f"in the gap between launches.  Its roofline kernel: `{live['kernel']}`."]
    write_kernel_stats(out, trace_dir, "Kernel time, default bench run (metric workload: FLARE encode+decode, "
                       "B=1, H=8, D=32, N=1048576, M=256, bf16; plus every extra)", STATS_CMD, notes)


# ---------------------------------------------------------------- shader clock

CLOCK_STEP_LAUNCHES = (2, 7)  # the timed steps of the clock run among each kernel's launches
CLOCK_CMD = ("timeout -s KILL 120 rocprofv3 --pmc GRBM_GUI_ACTIVE --kernel-trace --kernel-include-regex "
             "\"encode_bf16|decode_bf16|merge_kernel\" -f csv -d gpurun_out/clk_bench -o run -- python3 -u "
             "bench.py --steps 5 --warmup 2 --no-cpu --no-mix --no-bwd --no-sweep")


def kernel_trace(dirs, select=None):
    """{kernel: [duration ns per dispatch]} and {(kernel, dispatch id): duration ns} from kernel traces."""
    per, by_id = collections.defaultdict(list), {}
    for path in _csvs(dirs, "*kernel_trace.csv"):
        rows = sorted(csv.DictReader(open(path)), key=lambda r: int(r["Dispatch_Id"]))
        for r in rows:
            k = short_name(r["Kernel_Name"])
            if select and not any(s in k for s in select):
                continue
            d = int(r["End_Timestamp"]) - int(r["Start_Timestamp"])
            per[k].append(d)
            by_id[(path, k, r["Dispatch_Id"])] = d
    return per, by_id


def write_clock(out, dirs):
    """profiles/clock.encdec_n1m.md: the shader clock under the bench's encode and decode kernels,
    from GRBM_GUI_ACTIVE (summed over the XCDs) over each dispatch's traced duration."""
    sel = ["encode_bf16", "decode_bf16", "merge_kernel"]
    per, _ = kernel_trace(dirs, sel)
    per = {k: v[CLOCK_STEP_LAUNCHES[0]:CLOCK_STEP_LAUNCHES[1]] for k, v in per.items()}
    od = _ordered_dispatches(dirs, sel)
    grbm = {k: [d["GRBM_GUI_ACTIVE"] for ds in byp.values() for d in ds[CLOCK_STEP_LAUNCHES[0]:CLOCK_STEP_LAUNCHES[1]]
                if "GRBM_GUI_ACTIVE" in d] for k, byp in od.items()}
    lines = ["# Shader clock under load, bench workload (FLARE encode+decode, B=1, H=8, D=32, N=1048576, M=256, "
             "bf16)", "", "Command (repo root, one MI355X), then `python bench.py --summarize clock "
             "gpurun_out/clk_bench`:", "", "```", "export TMPDIR=/tmp", CLOCK_CMD, "```", "",
             "GRBM_GUI_ACTIVE is summed over the 8 XCDs; clock = cycles / 8 / kernel duration (kernel trace of "
             "the same run).  bench.py also samples the clock live (a one-wave sampler kernel on a second "
             "stream reading the shader and the 100 MHz real-time counters while the kernel runs), and reports "
             "it with the roofline.", "",
             "| kernel | dispatches | mean duration (us) | GRBM_GUI_ACTIVE per dispatch | clock (GHz) |",
             "|---|---|---|---|---|"]
    for k in sorted(per):
        if not grbm.get(k):
            continue
        dur = sum(per[k]) / len(per[k])
        g = sum(grbm[k]) / len(grbm[k])
        lines.append(f"| `{k}` | {len(per[k])} | {dur / 1e3:.1f} | {g:.4g} | {g / XCDS / dur:.3f} |")
    lines += ["", "For a kernel of a few tens of microseconds (the merge) the counter window reaches past the "
              "kernel, so its figure is not a clock."]
    open(out, "w").write("\n".join(lines) + "\n")


# ------------------------------------------------------------- backward units

BWD_ARGS = "--steps 2 --warmup 1 --no-cpu --no-mix --no-sweep"
BWD_PASSES = [
    "SQ_WAVE_CYCLES SQ_BUSY_CYCLES SQ_WAIT_INST_ANY SQ_WAIT_ANY SQ_ACTIVE_INST_VALU SQ_ACTIVE_INST_VALU2 "
    "SQ_VALU_MFMA_BUSY_CYCLES GRBM_GUI_ACTIVE",
    "SQ_INSTS_VALU SQ_INSTS_MFMA SQ_INSTS_LDS SQ_VALU_MFMA_COEXEC_CYCLES SQ_INSTS_VALU_TRANS_F32 "
    "SQ_LDS_BANK_CONFLICT SQ_INSTS_SALU SQ_CYCLES GRBM_GUI_ACTIVE",
]
BWD_CMDS = ["export TMPDIR=/tmp"] + [
    f"timeout -s KILL 120 rocprofv3 --pmc {p} --kernel-include-regex \"tok_bwd|lat_bwd|tok_pair\" -f csv "
    f"-d gpurun_out/bpmc{i + 1} -o run -- python3 -u bench.py {BWD_ARGS}" for i, p in enumerate(BWD_PASSES)]
# The backward leg of `bench.py BWD_ARGS` runs three forms, 5 calls each (2 warm-up, 3 timed): the
# one-call pair backward with fp32 dK, dV; the two-call chain; the one-call form with bf16 dK, dV.
# Each kernel's dispatches, in order, split into the forms it runs in.
BWD_GROUPS = [
    ("tok_pair_kernel<32, false>", 0, 5, "token pass, both roles (`tok_pair_kernel<32, false>`, one-call backward, fp32 dK, dV)"),
    ("tok_pair_kernel<32, false>", 5, 10, "the same with bf16 dK, dV"),
    ("lat_bwd_kernel<32, false, 8, false>", 0, 5,
     "latent pass, decoder role, computing delta from Y (`lat_bwd_kernel<32, false, 8, false>`, one-call)"),
    ("lat_bwd_kernel<32, false, 8, false>", 5, 10, "latent pass, decoder role (`lat_bwd_kernel<32, false, 8, false>`, two-call chain)"),
    ("lat_bwd_kernel<32, false, 8, false>", 10, 15, "the one-call form's latent pass again, in the bf16 dK, dV calls"),
    ("lat_bwd_kernel<32, true, 4, false>", 0, 15, "latent pass, encoder role (`lat_bwd_kernel<32, true, 4, false>`, all forms)"),
    ("tok_bwd_kernel<32, false, false>", 0, 5, "token pass, decoder role (`tok_bwd_kernel<32, false, false>`, two-call chain)"),
    ("tok_bwd_kernel<32, true, false>", 0, 5, "token pass, encoder role (`tok_bwd_kernel<32, true, false>`, two-call chain)"),
]


def _ordered_dispatches(dirs, select):
    """{kernel: {csv path: [counters per dispatch, in dispatch order]}}."""
    per = collections.defaultdict(lambda: collections.defaultdict(lambda: collections.defaultdict(float)))
    for path in _csvs(dirs, "*counter_collection.csv"):
        for row in csv.DictReader(open(path)):
            k = short_name(row["Kernel_Name"])
            if select and not any(s in k for s in select):
                continue
            per[k][(path, int(row["Dispatch_Id"]))][row["Counter_Name"]] += float(row["Counter_Value"])
    out = collections.defaultdict(lambda: collections.defaultdict(list))
    for k, d in per.items():
        for (path, _), v in sorted(d.items(), key=lambda kv: (kv[0][0], kv[0][1])):
            out[k][path].append(v)
    return out


def write_units_bwd(out, dirs):
    """profiles/units_bwd.encdec_n1m.md: execution-unit counters of the backward kernels."""
    blocks = 8 * (1 << 20) * 256 // (32 * 32)
    od = _ordered_dispatches(dirs, ["tok_bwd", "lat_bwd", "tok_pair"])
    rows = ["| kernel | dispatches | cycles | SIMD-cycles per block | MFMA per block | MFMA busy | co-exec "
            "| VALU per block | VALU issue per block | transcendental per block | LDS instructions per block "
            "| LDS bank conflicts | waiting on operands | waiting (any) |",
            "|---|---|---|---|---|---|---|---|---|---|---|---|---|---|"]
    nan = float("nan")
    for kernel, lo, hi, label in BWD_GROUPS:
        if kernel not in od:
            continue
        acc = collections.defaultdict(list)
        n = 0
        for path, ds in od[kernel].items():
            part = ds[lo:hi]
            n = max(n, len(part))
            for d in part:
                for c, v in d.items():
                    acc[c].append(v)
        if not acc:
            continue
        c = {k: sum(v) / len(v) for k, v in acc.items()}
        cyc = c.get("GRBM_GUI_ACTIVE", nan) / XCDS
        simd = cyc * SIMDS / blocks
        busy = c.get("SQ_VALU_MFMA_BUSY_CYCLES", nan) / (cyc * SIMDS)
        coexec = c.get("SQ_VALU_MFMA_COEXEC_CYCLES", nan) / c.get("SQ_VALU_MFMA_BUSY_CYCLES", nan)
        issue = 4.0 * (c.get("SQ_ACTIVE_INST_VALU", nan) - c.get("SQ_ACTIVE_INST_VALU2", 0.0)) / blocks
        wait = c.get("SQ_WAIT_INST_ANY", nan) / c.get("SQ_WAVE_CYCLES", nan)
        wait_any = c.get("SQ_WAIT_ANY", nan) / c.get("SQ_WAVE_CYCLES", nan)
        rows.append(f"| {label} | {n} | {cyc:.4g} | {simd:.0f} | {c.get('SQ_INSTS_MFMA', nan) / blocks:.2f} "
                    f"| **{100 * busy:.1f}%** | {100 * coexec:.0f}% | {c.get('SQ_INSTS_VALU', nan) / blocks:.1f} "
                    f"| {issue:.0f} | {c.get('SQ_INSTS_VALU_TRANS_F32', nan) / blocks:.1f} "
                    f"| {c.get('SQ_INSTS_LDS', nan) / blocks:.1f} | {c.get('SQ_LDS_BANK_CONFLICT', nan):.0f} "
                    f"| {100 * wait:.0f}% | {100 * wait_any:.0f}% |")
    text = ["# Execution units, backward of the bench workload (FLARE encode+decode, B=1, H=8, D=32, N=1048576, "
            "M=256)", "", "Commands (repo root, one MI355X; two counter passes, each a run of its own), then "
            "`python bench.py --summarize units_bwd gpurun_out/bpmc1 gpurun_out/bpmc2`:", "", "```"] + BWD_CMDS + [
            "```", "",
            "The bench's backward leg runs the one-call pair backward (`flare_encdec_backward`) 5 times, then "
            "the two-call chain (`flare_decode_backward` + `flare_encode_backward`) 5 times, then the one-call "
            "form 5 times with bf16 dK and dV.  Values are means per dispatch over the dispatches of each group "
            f"and both passes.  A block is 32 tokens x 32 latents of one head: {blocks} blocks per call.  Cycles "
            "are GRBM_GUI_ACTIVE / 8 XCDs; SIMD-cycles that times 1024 SIMDs; MFMA busy is "
            "SQ_VALU_MFMA_BUSY_CYCLES over SIMD-cycles; co-exec is the share of those MFMA-busy cycles in which "
            "VALU instructions also executed; VALU issue is 4 x (SQ_ACTIVE_INST_VALU - SQ_ACTIVE_INST_VALU2) "
            "cycles; waiting on operands is SQ_WAIT_INST_ANY over SQ_WAVE_CYCLES (wave-cycles spent waiting for "
            "an instruction's operands: LDS, memory, or the matrix core's result); waiting (any) is SQ_WAIT_ANY "
            "over SQ_WAVE_CYCLES (also counting waits at barriers and on counters).", ""] + rows
    open(out, "w").write("\n".join(text) + "\n")


# ------------------------------------------------------------ X reuse probe

XREUSE_TIMING_CMD = "timeout -k 10 120 python3 -u rank_latent_routing_amd/probes/run_xreuse.py > gpurun_out/xreuse.md"
XREUSE_PMC_CMD = ("timeout -s KILL 120 rocprofv3 --pmc FETCH_SIZE --kernel-include-regex xreuse -f csv -d "
                  "gpurun_out/xreuse_pmc -o run -- python3 -u rank_latent_routing_amd/probes/run_xreuse.py --reps 3")


def write_xreuse(out, timing_md, pmc_dir, profiles_dir):
    """profiles/xreuse.block_c5.md: bytes fetched past L2 and time of the X-reuse probe per dispatch order."""
    from rank_latent_routing_amd.probes import run_xreuse as xr
    fr, _ = _copy_factors(profiles_dir)
    od = _ordered_dispatches([pmc_dir], ["xreuse"])
    per_order = collections.defaultdict(list)
    for k, d in od.items():
        order = int(k.split("<")[1].split(",")[0])
        for path, ds in d.items():
            per_order[order].append(ds)
    xbytes = xr.B * xr.N * xr.C * 2
    rows = ["| order | heads | dispatches | fetched past L2 per launch (GB) | per head, over X's bytes |",
            "|---|---|---|---|---|"]
    for label, heads, order in xr.RUNS:
        runs = per_order.get(order, [])
        vals = []
        for ds in runs:
            # order 0 serves two runs: first the one-head read, then the head-major one
            n = len(ds) // 2 if order == 0 else len(ds)
            part = ds[:n] if (order == 0 and heads == 1) else (ds[n:] if order == 0 else ds)
            vals += [c["FETCH_SIZE"] * 1024 * fr for c in part]
        if not vals:
            continue
        gb = sum(vals) / len(vals)
        rows.append(f"| {label} | {heads} | {len(vals)} | {gb / 1e9:.3f} | {gb / heads / xbytes:.2f} |")
    timing = open(timing_md).read().strip().splitlines()
    text = ["# X reuse across heads, FLARE++ block workload's projection input (X [B*N, C] bf16, B=4, N=262144, "
            "C=256, H=8)", "",
            "Would workgroups that each project one head's share of a token window (a fused projection-into-"
            "attention kernel reads all C input features of its tokens for every head) find X in L2?  The probe "
            "(`rank_latent_routing_amd/probes/xreuse.hip`) reads each 128-row block of X once per head in three "
            "dispatch orders.", "",
            "Commands (repo root, one MI355X), then `python bench.py --summarize xreuse gpurun_out/xreuse.md "
            "gpurun_out/xreuse_pmc`:", "", "```", "export TMPDIR=/tmp", XREUSE_TIMING_CMD, XREUSE_PMC_CMD, "```",
            "", "Timing:", ""] + timing + ["", "Bytes fetched past L2 (FETCH_SIZE, scaled by the copy calibration of "
            f"`traffic.encdec_n1m.md`, x{fr:.4f}):", ""] + rows
    open(out, "w").write("\n".join(text) + "\n")


# ------------------------------------------------------------- HBM traffic

TRAFFIC_ARGS = "--steps 3 --warmup 1 --no-cpu --no-mix --no-sweep"
TRAFFIC_RE = "encode_bf16|decode_bf16|merge_kernel|tok_bwd|lat_bwd|sum_splits|tok_pair"
TRAFFIC_CMDS = [
    "export TMPDIR=/tmp",
    f"timeout -s KILL 120 rocprofv3 --pmc FETCH_SIZE --kernel-include-regex \"{TRAFFIC_RE}\" -f csv -d "
    f"gpurun_out/pmc_fetch -o run -- python3 -u bench.py {TRAFFIC_ARGS}",
    f"timeout -s KILL 120 rocprofv3 --pmc WRITE_SIZE --kernel-include-regex \"{TRAFFIC_RE}\" -f csv -d "
    f"gpurun_out/pmc_write -o run -- python3 -u bench.py {TRAFFIC_ARGS}",
    "timeout -s KILL 120 rocprofv3 --pmc FETCH_SIZE -f csv -d gpurun_out/pmc_copy_fetch -o run -- "
    "python3 -u bench.py --copy-calibration",
    "timeout -s KILL 120 rocprofv3 --pmc WRITE_SIZE -f csv -d gpurun_out/pmc_copy_write -o run -- "
    "python3 -u bench.py --copy-calibration",
    "python bench.py --write-traffic gpurun_out/pmc_fetch/run_counter_collection.csv "
    "gpurun_out/pmc_write/run_counter_collection.csv gpurun_out/pmc_copy_fetch/run_counter_collection.csv "
    "gpurun_out/pmc_copy_write/run_counter_collection.csv",
]


def _csv_ordered(path, counter, select):
    """{kernel: [counter value per dispatch, in dispatch order]} from one counter CSV."""
    per = collections.defaultdict(dict)
    for row in csv.DictReader(open(path)):
        if row["Counter_Name"] != counter:
            continue
        k = short_name(row["Kernel_Name"])
        if select and not any(s in k for s in select):
            continue
        i = int(row["Dispatch_Id"])
        per[k][i] = per[k].get(i, 0.0) + float(row["Counter_Value"])
    return {k: [v for _, v in sorted(d.items())] for k, d in per.items()}


def write_traffic_md(out, fetch_csv, write_csv, f_read, f_write, copy_kib, step_launches):
    """profiles/traffic.encdec_n1m.md: bytes per launch of the forward and backward kernels of the bench
    workload against their algorithmic bytes."""
    B, H, N, D, M = 1, 8, 1 << 20, 32, 256
    S = min(max(1, (1024 + B * H - 1) // (B * H)), ((N + 127) // 128) // 2)  # encoder splits (plan)
    tok = B * H * N
    sel = TRAFFIC_RE.split("|")
    fe, wr = _csv_ordered(fetch_csv, "FETCH_SIZE", sel), _csv_ordered(write_csv, "WRITE_SIZE", sel)
    rows_fwd = [
        ("encode_bf16_kernel<32, 8>", None, 2 * tok * D * 2, "K and V read: 2 x 8 x 1048576 x 32 x 2 B"),
        ("merge_kernel", None, B * H * S * M * (D + 1) * 4,
         f"split partials: 8 x S x 256 x (32 + 1) x 4 B, S = {S}"),
        ("decode_bf16_kernel<32>", None, 2 * tok * D * 2, "K read, Y written: 8 x 1048576 x 32 x 2 B each"),
    ]
    rows_bwd = [
        ("lat_bwd_kernel<32, false, 8, false>", (0, 5), " (one call)", 3 * tok * D * 2 + 2 * tok * 4,
         "K, dY, Y read in bf16, lse read, delta written"),
        ("lat_bwd_kernel<32, false, 8, false>", (5, 10), " (two calls)", 2 * tok * D * 2 + 2 * tok * 4,
         "K, dY read in bf16, lse and delta read"),
        ("lat_bwd_kernel<32, true, 4, false>", None, "", 2 * tok * D * 2, "K, V read in bf16 once; each of the two 128-latent blocks of a split reads them"),
        ("tok_pair_kernel<32, false>", (0, 5), " (fp32 gradients)", 3 * tok * D * 2 + 2 * tok * 4 + 2 * tok * D * 4,
         "K, V, dY read in bf16, lse and delta read, dK and dV written in fp32"),
        ("tok_pair_kernel<32, false>", (5, 10), " (bf16 gradients)", 3 * tok * D * 2 + 2 * tok * 4 + 2 * tok * D * 2,
         "the same with dK and dV written in bf16"),
        ("tok_bwd_kernel<32, false, false>", None, "", 3 * tok * D * 2 + tok * D * 4 + 2 * tok * 4,
         "K, dY, Y read in bf16, dK written in fp32, lse read and delta written"),
        ("tok_bwd_kernel<32, true, false>", None, "", 2 * tok * D * 2 + 3 * tok * D * 4,
         "K, V read in bf16, dK read and written, dV written, all fp32"),
    ]

    def line(kernel, rng, label, alg, what, fwd=False):
        if kernel not in fe or kernel not in wr:
            return None
        f, w = fe[kernel], wr[kernel]
        if rng:
            f, w = f[rng[0]:rng[1]], w[rng[0]:rng[1]]
        if fwd:
            f, w = f[step_launches[0]:step_launches[1]], w[step_launches[0]:step_launches[1]]
        if not f or not w:
            return None
        fk, wk = sum(f) / len(f), sum(w) / len(w)
        rd, wb = fk * 1024 * f_read, wk * 1024 * f_write
        return (f"| `{kernel}`{label} | {fk:.0f} | {wk:.0f} | {rd / 1e9:.4f} | {wb / 1e9:.4f} | {alg / 1e9:.4f} "
                f"({what}) | {(rd + wb) / alg:.3f} |")

    head = ["| kernel | FETCH_SIZE (KiB) | WRITE_SIZE (KiB) | read (GB) | written (GB) | algorithmic bytes (GB) "
            "| ratio |", "|---|---|---|---|---|---|---|"]
    text = ["# HBM traffic per launch, bench workload (FLARE encode+decode, B=1, H=8, D=32, N=1048576, M=256, bf16)",
            "", "Commands (repo root, one MI355X; each counter in a run of its own):", "", "```"] + TRAFFIC_CMDS + [
            "```", "",
            f"Calibration: the 1 GiB device copy reads FETCH_SIZE = {copy_kib[0]:.0f} KiB and WRITE_SIZE = "
            f"{copy_kib[1]:.0f} KiB per launch, so read counts are scaled by {f_read:.4f} and write counts by "
            f"{f_write:.4f}.", "", "Forward (the bench step: means over each kernel's launches in the timed steps of the "
            "metric step loop, after its warm-up):", ""] + head
    text += [x for x in (line(k, r, "", a, w, True) for k, r, a, w in rows_fwd) if x]
    text += ["", "The encoder's write column is its split partials (read back by the merge); the decoder's write "
             "column is Y.", "",
             "Backward (the bench's backward leg, 5 calls of each form: the one-call pair gradient, then the two-"
             "call chain, then the one-call form with bf16 dK and dV; a kernel that runs in several forms is "
             "listed per form):", ""] + head
    text += [x for x in (line(k, r, lab, a, w) for k, r, lab, a, w in rows_bwd) if x]
    text += ["", "The latent passes' writes are their fp32 split partials.  The per-kernel JSON files beside this "
             "one hold the forward figures for bench.py (its `roofline.traffic`), keyed to the kernel sources "
             "they were taken on."]
    open(out, "w").write("\n".join(text) + "\n")
