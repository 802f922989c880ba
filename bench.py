#!/usr/bin/env python3
"""Throughput of the direct-convolution library on one MI355X.

Headline workload (one step): single-channel fp32 filtering of an 8192x8192
image, once with a 3x3, once with a 5x5 and once with a 7x7 filter (three
launches, each on its own input/output buffers so no launch finds the previous
one's data in cache). `value` is the step's algorithmic HBM bytes (x, y and w
once per launch) over its time, in GB/s.

Also reported, each timed on its own: the fp32 32->32 3x3 layer at 1280x720,
the 1280x720 upscaling chain fused and layer by layer (ms per frame) and the
fp16 NHWC 64->64 layer of 8x256x256, with GFLOP/s and fractions of peak.

Peaks: HBM 8.0 TB/s; fp32 FMA on the vector ALUs without packed-FP32
instructions 78.6 TFLOP/s (256 CUs x 4 SIMDs x 16 lanes x 2 FLOP x 2.4 GHz; the
kernels are built with packed FP32 off, which halves the 157.3 TFLOP/s figure
that counts packed FMAs); dense fp32 MFMA 157.3 TFLOP/s (the 32->32 fp32
layers run there); dense fp16 MFMA 2.5 PFLOP/s.

cpu_baseline: the fp64 CPU oracle on the host cores, full headline steps.
"""
import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)
sys.path.insert(1, os.path.join(ROOT, "tests"))   # tolerance.py: the parity tests' bounds

METRIC = "conv GFLOP/s and HBM GB/s as % of MI355X peak; ms per 1280x720 frame"
HBM_PEAK_GBS = 8000.0
FP32_VALU_PEAK_TFLOPS = 256 * 4 * 16 * 2 * 2.4e9 / 1e12     # 78.64, plain v_fma_f32
FP32_PACKED_PEAK_TFLOPS = 157.3
FP32_MFMA_PEAK_TFLOPS = 157.3    # dense fp32 matrix cores (v_mfma_f32_16x16x4_f32)
MFMA_F32_KERNELS = ("is_k5_mfma_f32",)
FP16_MFMA_PEAK_TFLOPS = 2500.0

# HBM traffic per launch from the FETCH_SIZE / WRITE_SIZE counters (two
# rocprofv3 --pmc runs of this script, summarised by --pmc-summary into
# TRAFFIC_FILE). Each figure is tied to a digest of the kernel's sources: once a
# source changes, the case reports traffic null until the counters are re-taken.
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "hbm_traffic_counters.md")
TRAFFIC_KERNELS = {   # bench case -> (kernel as the profiler names it, its source files)
    "8192x8192 3x3": ("is_k1_single<3, 3, true, false, false, 1>", ("k1_single.hip",)),
    "8192x8192 5x5": ("is_k1_single<5, 5, true, false, false, 1>", ("k1_single.hip",)),
    "8192x8192 7x7": ("is_k1_single<7, 7, true, false, false, 1>", ("k1_single.hip",)),
    "fp32 layer 1x32x720x1280 -> 32, 3x3": ("is_k5_mfma_f32", ("k5_mfma_f32.hip",)),
    "fp16 NHWC layer 8x256x256x64 -> 64, 3x3": ("is_k4_mfma<128, 64, 64, 0, 0, 0, false>", ("k4_mfma.hip",)),
    "upscaling chain 1280x720 (fused)": ("is_k3_chain", ("k3_chain.hip",)),
    "separable 7x7 filter, 8192x8192 fp32": ("is_k1_single<7, 7, true, false, true, 1>", ("k1_single.hip",)),
    "1 channel -> 8 filters 3x3, 4096x4096 fp32": ("is_k2_multi<3, 8, 1, false, false>", ("k2_multi.hip",)),
    "stencil pipeline 3x3 x3, 8192x8192 fp32 (auto)": ("is_k7_fused_stencil<3, 3, 3>", ("k7_fused_stencil.hip",)),
}
# The known-size dispatch: torch's elementwise negation of 256 MiB of fp32
# (run by _copy_reference), which reads 256 MiB and writes 256 MiB.
CALIB_KERNEL = "neg_kernel"
CALIB_BYTES = 256 << 20


def _source_digest(files):
    """Digest of the code of a kernel's sources: comments and whitespace are
    dropped first, so that an edit of the comments keeps the counters valid."""
    import hashlib
    import re
    h = hashlib.sha256()
    for f in tuple(files) + ("common.hpp",):
        with open(os.path.join(ROOT, "image_stencil_amd", "csrc", f)) as fh:
            text = fh.read()
        text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
        text = re.sub(r"//[^\n]*", " ", text)
        h.update(" ".join(text.split()).encode())
    return h.hexdigest()[:16]


def _short_kernel(name):
    import re
    if name.startswith("_ZN"):
        # Left mangled by the tracer (c++filt does not take the _Float16
        # mangling either): the innermost name and its integer template
        # arguments are enough here.
        i, parts = 3, []
        while i < len(name) and name[i].isdigit():
            j = i
            while name[j].isdigit():
                j += 1
            n = int(name[i:j])
            parts.append(name[j:j + n])
            i = j + n
        targs = re.findall(r"Li(-?\d+)E", name[i:name.find("EE", i) + 1]) if name[i:i + 1] == "I" else []
        if parts:
            return parts[-1] + ("<%s>" % ", ".join(targs) if targs else "")
    name = name.replace("void ", "").replace("is::(anonymous namespace)::", "").replace("(anonymous namespace)::", "")
    m = re.match(r"([^(<]+(<[^>]*>)?)", name)
    return m.group(1).strip() if m else name


def _counter_means(d, counter):
    """Mean per dispatch of one counter, by kernel, over every counter CSV under d.
    A kernel instance launched at several sizes (the 3x3 filter on the 8192x8192
    image and on the 256x256 one) keeps only its largest launches, which are the
    bench case the figure belongs to."""
    import csv
    import glob
    per = {}   # (kernel, file, dispatch) -> summed value
    grid = {}
    full = {}
    for f in sorted(glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True)):
        with open(f) as fh:
            for r in csv.DictReader(fh):
                if r["Counter_Name"] != counter:
                    continue
                k = _short_kernel(r["Kernel_Name"])
                full[k] = r["Kernel_Name"]
                key = (k, f, r["Dispatch_Id"])
                per[key] = per.get(key, 0.0) + float(r["Counter_Value"])
                grid[key] = int(r["Grid_Size"])
    acc = {}
    for key, v in per.items():
        acc.setdefault(key[0], []).append((grid[key], v))
    out = {}
    for k, gv in acc.items():
        top = max(g for g, _ in gv)
        vals = [v for g, v in gv if g == top]
        out[k] = (sum(vals) / len(vals), len(vals), full[k])
    return out


# Arguments of the bench runs under the profiler: the counter and trace runs of
# the bench workloads leave out the pages' net (its 64 -> 64 layer runs the same
# kernel instance as the fp16 layer workload and would mix into that row); the
# net has a kernel-trace run of its own.
PROFILE_ARGS = "--no-cpu-baseline --no-check --secondary fp32_layer,fp16_layer,upscale_chain,special_cases"
PMC_ARGS = "--steps 2 --warmup 1 --min-warm-s 0 " + PROFILE_ARGS
NET_PROFILE_ARGS = "--no-cpu-baseline --no-check --secondary pages_net"
NET_KERNELS = {
    "is_k4_mfma<128, 64, 64, 0, 60, 5, true>": "layers 1 + 2: the 1 -> 64 5x5 computed inside the 64 -> 64 3x3 (60-row units)",
    "is_k4_mfma<128, 64, 32, 0, 60, 0, true>": "layer 3: 64 -> 32, 3x3 (60-row units)",
    "is_k4_mfma<128, 32, 16, 3, 30, 0, false>": "layer 4: 32 -> 9 (as 16), 3x3, with the depth-to-space x3 in its stores (30-row units)",
    "is_k6_head_f16<5, 64>": "layer 1 alone: 1 -> 64, 5x5 (one-launch-per-layer run)",
    "is_k4_mfma<128, 64, 64, 0, 60, 0, true>": "layer 2 alone: 64 -> 64, 3x3 (one-launch-per-layer run)",
}


def pmc_summary(fetch_dir, write_dir):
    """Markdown summary of two counter runs: per-dispatch FETCH_SIZE and
    WRITE_SIZE of each bench case's kernel, scaled by the known-size dispatch."""
    fetch = _counter_means(fetch_dir, "FETCH_SIZE")
    write = _counter_means(write_dir, "WRITE_SIZE")

    def calib(tab):
        hits = [v for k, v in tab.items() if CALIB_KERNEL in v[2]]
        if len(hits) != 1:
            raise SystemExit("expected one calibration kernel (%s), found %d" % (CALIB_KERNEL, len(hits)))
        return hits[0]

    cf, cw = calib(fetch), calib(write)
    sf = CALIB_BYTES / (cf[0] * 1024.0)
    sw = CALIB_BYTES / (cw[0] * 1024.0)
    lines = ["# HBM traffic per launch from the FETCH_SIZE and WRITE_SIZE counters", "",
             "Commands (from the repository root, one MI355X; then the summary, on any machine):", "", "```",
             "rocprofv3 --pmc FETCH_SIZE --output-format csv -d %s -o run -- \\" % fetch_dir,
             "    python3 bench.py " + PMC_ARGS,
             "rocprofv3 --pmc WRITE_SIZE --output-format csv -d %s -o run -- \\" % write_dir,
             "    python3 bench.py " + PMC_ARGS,
             "python3 bench.py --pmc-summary %s %s > profiles/hbm_traffic_counters.md" % (fetch_dir, write_dir),
             "```", "",
             "Counters are in KiB per dispatch, averaged over the dispatches of each kernel. The scale",
             "factors make the known-size dispatch (torch's negation of 256 MiB of fp32: 256 MiB read,",
             "256 MiB written) read its true size: FETCH_SIZE x %.4f, WRITE_SIZE x %.4f." % (sf, sw), "",
             "| kernel | dispatches | FETCH_SIZE KiB | WRITE_SIZE KiB |", "|---|---|---|---|",
             "| `%s` (calibration) | %d | %.1f | %.1f |" % (_short_kernel(cf[2])[:60], cf[1], cf[0], cw[0]), "",
             "Machine-read by bench.py (traffic = scaled fetch + scaled write bytes per launch; the digest",
             "is that of the kernel's sources when the counters were taken):", "",
             "| case | kernel | dispatches | FETCH_SIZE KiB | WRITE_SIZE KiB | traffic bytes | source digest |",
             "|---|---|---|---|---|---|---|"]
    for case, (kern, files) in TRAFFIC_KERNELS.items():
        if kern not in fetch or kern not in write:
            continue
        f, n, _ = fetch[kern]
        w_, _, _ = write[kern]
        t = f * 1024.0 * sf + w_ * 1024.0 * sw
        lines.append("| %s | `%s` | %d | %.1f | %.1f | %.0f | %s |" % (case, kern, n, f, w_, t, _source_digest(files)))
    return "\n".join(lines) + "\n"


def stats_summary(trace_dir, net=False):
    """Markdown summary of a rocprofv3 --kernel-trace --stats run of this script:
    calls and durations per kernel, with the bench case each kernel times (net:
    the run of the pages' net, with the layer each kernel runs)."""
    import csv
    import glob
    files = sorted(glob.glob(os.path.join(trace_dir, "**", "*kernel_trace.csv"), recursive=True))
    if not files:
        raise SystemExit("no kernel_trace.csv under %s" % trace_dir)
    cases = dict(NET_KERNELS) if net else {k: c for c, (k, _) in TRAFFIC_KERNELS.items()}
    title = ("Kernel durations of the pages' fp16 net per 1280x720 frame" if net
             else "Kernel durations of the bench workloads")
    out_file = "pages_net_f16_kernels.md" if net else "kernel_durations_bench_workloads.md"
    # Dispatches grouped by kernel and launch size (workgroups x threads), so
    # that one instance run on two workloads gives two rows; the bench case is
    # named on the largest launch of its kernel.
    groups = {}
    with open(files[0]) as fh:
        for r in csv.DictReader(fh):
            k = _short_kernel(r["Kernel_Name"])
            g = int(r["Grid_Size_X"]) * int(r["Grid_Size_Y"]) * int(r["Grid_Size_Z"])
            ns = int(r["End_Timestamp"]) - int(r["Start_Timestamp"])
            groups.setdefault((k, g), []).append(ns)
    top = {}
    for (k, g) in groups:
        top[k] = max(top.get(k, 0), g)
    lines = ["# %s (rocprofv3 kernel trace)" % title, "",
             "Commands (from the repository root, one MI355X; then the summary, on any machine):", "", "```",
             "rocprofv3 --kernel-trace --stats --output-format csv -d %s -o run -- \\" % trace_dir,
             "    python3 bench.py " + (NET_PROFILE_ARGS if net else PROFILE_ARGS),
             "python3 bench.py --%s %s > profiles/%s" % ("net-stats-summary" if net else "stats-summary",
                                                        trace_dir, out_file),
             "```", "",
             "Durations in microseconds (end minus start of each dispatch in the kernel trace) over every",
             "dispatch of the run, warmup included, one row per kernel and launch size (grid threads). The",
             "bench's own per-launch event timings of the same run are printed in its JSON line.", "",
             "| kernel | grid threads | %s | calls | avg us | min us | max us |" % ("layer" if net else "bench case"),
             "|---|---|---|---|---|---|---|"]
    rows = sorted(groups.items(), key=lambda kv: -sum(kv[1]))
    for (k, g), ns in rows:
        case = cases.get(k, "") if g == top[k] else ""
        lines.append("| `%s` | %d | %s | %d | %.1f | %.1f | %.1f |" % (
            k[:70], g, case, len(ns), sum(ns) / len(ns) / 1e3, min(ns) / 1e3, max(ns) / 1e3))
    return "\n".join(lines) + "\n"


LDS_COUNTERS = ("SQ_LDS_BANK_CONFLICT", "SQ_LDS_IDX_ACTIVE", "SQ_INSTS_LDS", "SQ_WAIT_INST_LDS")


def lds_study(torch, isa, synth, stream, stream_obj, steps, warmup):
    """The LDS-staged kernels for a counter run of their bank conflicts: the fp16
    layer under each swizzle of its input tile (tuning variants of its plan; the
    kernel is instantiated per swizzle, so the profiler sees
    is_k4_mfma<0, 64, 64, 0, 0, 0, false>, <128, ...> and <256, ...>), the other LDS-staging kernels
    and the fp32 layer and the fused chain."""
    out = []
    x, w, b = synth.cnn_layer_f16_nhwc()
    xd, wd, bd = torch.from_numpy(x).cuda(), torch.from_numpy(w).cuda(), torch.from_numpy(b).cuda()
    yd = torch.empty((8, 256, 256, 64), dtype=torch.float16, device="cuda")
    desc = isa.make_desc(8, 64, 256, 256, 64, 3, 3, "f16", False)
    variants = isa.conv2d_list_variants(desc)
    for swz in (0, 128, 256):
        idx = [i for i, v in enumerate(variants) if v["kernel"] == "is_k4_mfma" and v["param"] == swz]
        plan = isa.Plan(desc, variant=idx[0])
        c = Case("fp16 layer, swizzle %d" % swz,
                 lambda plan=plan: isa.conv2d_forward(plan.handle, xd.data_ptr(), wd.data_ptr(), bd.data_ptr(),
                                                      yd.data_ptr(), stream),
                 0, 1, plan.info()["kernel"])
        _, per, _ = _time_cases(torch, [c], steps, warmup, stream_obj)
        out.append({"case": c.name, "swizzle_row_bytes": swz, "ms": round(per[0], 4)})
    x, w, b = synth.cnn_layer_f32()
    c = _layer_cases(torch, isa, stream, x, w, b, True, 1, "fp32 layer")[0]
    _, per, _ = _time_cases(torch, [c], steps, warmup, stream_obj)
    out.append({"case": c.name, "kernel": c.kernel, "ms": round(per[0], 4)})

    def variant_case(name, desc, kernel, param, xd, wd, bd, yd):
        """The plan variant of `desc` running `kernel` with tuning parameter `param`."""
        vs = isa.conv2d_list_variants(desc)
        idx = [i for i, v in enumerate(vs) if v["kernel"] == kernel and (param is None or v["param"] == param)]
        if not idx:
            raise SystemExit("no %s variant (param %s) for %s" % (kernel, param, name))
        plan = isa.Plan(desc, variant=idx[0])
        cc = Case(name, lambda: isa.conv2d_forward(plan.handle, xd.data_ptr(), wd.data_ptr(),
                                                     bd.data_ptr() if bd is not None else None, yd.data_ptr(),
                                                     stream), 0, 1, kernel)
        cc.keep = plan
        return cc

    # The register-blocked multi-channel kernel on the same fp32 layer (a
    # tuning variant: 32 output channels per workgroup), and on one channel
    # filtered by 8 3x3 filters (its default plan there).
    xd, wd, bd = torch.from_numpy(x).cuda(), torch.from_numpy(w).cuda(), torch.from_numpy(b).cuda()
    yd = torch.empty((1, 32, 720, 1280), device="cuda")
    more = [variant_case("multi-channel kernel, fp32 32->32 3x3 layer", isa.make_desc(1, 32, 720, 1280, 32, 3, 3,
                                                                                       "f32", True),
                         "is_k2_multi", 32, xd, wd, bd, yd)]
    x1 = torch.rand((1, 1, 4096, 4096), device="cuda")
    w8 = torch.randn((8, 1, 3, 3), device="cuda") / 3
    y8 = torch.empty((1, 8, 4096, 4096), device="cuda")
    more.append(variant_case("multi-channel kernel, 1 channel -> 8 filters 3x3", isa.make_desc(1, 1, 4096, 4096, 8,
                                                                                                3, 3),
                             "is_k2_multi", None, x1, w8, None, y8))
    # The pointwise kernel (1x1, 32 -> 32 on a 1280x720 frame).
    wp = torch.randn((32, 32, 1, 1), device="cuda") / 6
    more.append(variant_case("pointwise kernel, 1x1 32->32", isa.make_desc(1, 32, 720, 1280, 32, 1, 1), "is_k8_pointwise",
                             None, xd, wp, None, yd))
    # The fp16 first-layer kernel (1 -> 64, 5x5, the pages' net's first layer)
    # and the fp16 MFMA kernel's other instances (64 -> 32, 32 -> 16).
    xh = torch.rand((1, 720, 1280, 1), device="cuda").half()
    wh = (torch.randn((64, 1, 5, 5), device="cuda") / 5).half()
    bh = torch.zeros(64, device="cuda")
    yh = torch.empty((1, 720, 1280, 64), device="cuda", dtype=torch.float16)
    more.append(variant_case("fp16 first layer 1->64 5x5", isa.make_desc(1, 1, 720, 1280, 64, 5, 5, "f16", True),
                             "is_k6_head_f16", None, xh, wh, bh, yh))
    # The fp32 first-layer kernel (1 -> 32, 5x5, the upscaling chain's first layer).
    x1f = torch.rand((1, 1, 720, 1280), device="cuda")
    w1f = torch.randn((32, 1, 5, 5), device="cuda") / 5
    more.append(variant_case("fp32 first layer 1->32 5x5", isa.make_desc(1, 1, 720, 1280, 32, 5, 5, "f32", True),
                             "is_k9_head_f32", None, x1f, w1f, bd, yd))
    # The 4-filter matrix-core layer (32 -> 4 3x3, the upscaling chain's last layer).
    w4 = torch.randn((4, 32, 3, 3), device="cuda") / 17
    y4 = torch.empty((1, 4, 720, 1280), device="cuda")
    more.append(variant_case("4-filter matrix-core layer 32->4 3x3", isa.make_desc(1, 32, 720, 1280, 4, 3, 3, "f32"),
                             "is_k2_multi_mfma", None, xd, w4, bd[:4].contiguous(), y4))
    w32 = (torch.randn((32, 64, 3, 3), device="cuda") / 24).half()
    y32 = torch.empty((1, 720, 1280, 32), device="cuda", dtype=torch.float16)
    more.append(variant_case("fp16 layer 64->32", isa.make_desc(1, 64, 720, 1280, 32, 3, 3, "f16", True),
                             "is_k4_mfma", 128, yh, w32, bh[:32].contiguous(), y32))
    w16 = (torch.randn((16, 32, 3, 3), device="cuda") / 17).half()
    y16 = torch.empty((1, 720, 1280, 16), device="cuda", dtype=torch.float16)
    more.append(variant_case("fp16 layer 32->16", isa.make_desc(1, 32, 720, 1280, 16, 3, 3, "f16", True),
                             "is_k4_mfma", 128, y32, w16, bh[:16].contiguous(), y16))
    for cc in more:
        _, per, _ = _time_cases(torch, [cc], steps, warmup, stream_obj)
        out.append({"case": cc.name, "kernel": cc.kernel, "ms": round(per[0], 4)})
        cc.keep = None
    x, layers = synth.chain_f32()
    spec = [(w.shape[1], w.shape[0], w.shape[2], relu) for (w, b, relu) in layers]
    d = isa.make_chain_desc(1, 720, 1280, spec, 2, isa.IS_CHAIN_FUSED)
    xd = torch.from_numpy(x).cuda()
    wl = [(torch.from_numpy(w).cuda(), torch.from_numpy(b).cuda()) for (w, b, _) in layers]
    yc = torch.empty((1, 1, 1440, 2560), dtype=torch.float32, device="cuda")
    c = Case("fused chain", lambda: isa.conv_chain_forward(d, xd.data_ptr(), [w.data_ptr() for (w, _) in wl],
                                                           [b.data_ptr() for (_, b) in wl], yc.data_ptr(), None, 0,
                                                           stream), 0, 1, "is_k3_chain")
    _, per, _ = _time_cases(torch, [c], steps, warmup, stream_obj)
    out.append({"case": c.name, "kernel": c.kernel, "ms": round(per[0], 4)})
    # The pages' fp16 net (AUTO): the first layer computed inside the 64 -> 64
    # layer, then 64 -> 32 and 32 -> 9 with the x3 depth-to-space in its stores.
    x, layers = synth.chain_f16_nhwc()
    spec = [(w.shape[1], w.shape[0], w.shape[2], relu) for (w, b, relu) in layers]
    d = isa.make_chain_desc(1, 720, 1280, spec, 3, isa.IS_CHAIN_AUTO, "f16")
    ws_bytes = isa.conv_chain_workspace_size(d)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device="cuda")
    xd = torch.from_numpy(x).cuda()
    wl = [(torch.from_numpy(w).cuda(), torch.from_numpy(b).cuda()) for (w, b, _) in layers]
    yn = torch.empty((1, 2160, 3840, 1), dtype=torch.float16, device="cuda")
    c = Case("pages' net fp16", lambda: isa.conv_chain_forward(d, xd.data_ptr(), [w.data_ptr() for (w, _) in wl],
                                                               [b.data_ptr() for (_, b) in wl], yn.data_ptr(),
                                                               ws.data_ptr(), ws_bytes, stream),
             0, 1, isa.conv_chain_kernel_name(d))
    _, per, _ = _time_cases(torch, [c], steps, warmup, stream_obj)
    out.append({"case": c.name, "kernel": c.kernel, "ms": round(per[0], 4)})
    return out


def pmc_lds_summary(pmc_dir):
    """Markdown summary of a counter run of --lds-study: LDS counters per dispatch
    of each LDS-staged kernel."""
    tabs = {c: _counter_means(pmc_dir, c) for c in LDS_COUNTERS}
    kernels = [k for k in sorted(tabs[LDS_COUNTERS[0]]) if k.startswith("is_k")]
    lines = ["# LDS bank conflicts of the LDS-staged kernels", "",
             "Commands (from the repository root, one MI355X; then the summary, on any machine):", "", "```",
             "rocprofv3 --pmc %s --output-format csv -d %s -o run -- \\" % (" ".join(LDS_COUNTERS), pmc_dir),
             "    python3 bench.py --lds-study --steps 2 --warmup 1 --min-warm-s 0",
             "python3 bench.py --pmc-lds-summary %s > profiles/lds_bank_conflicts.md" % pmc_dir,
             "```", "",
             "Counter values per dispatch (cycles or instructions summed over the chip), averaged over the",
             "dispatches of each kernel. The fp16 layer runs once per swizzle of its input tile (row bytes",
             "0 = plain, 128, 256; the plan picks 128), and its 64 -> 32 and 32 -> 16 instances on a",
             "1280x720 frame; the register-blocked multi-channel kernel on the fp32 32 -> 32 layer (a tuning",
             "variant there) and on one channel with 8 3x3 filters (4096x4096); the pointwise kernel on a",
             "1x1 32 -> 32 layer; the fp16 first-layer kernel on 1 -> 64 5x5; the fp32 first-layer kernel",
             "on 1 -> 32 5x5; the 4-filter matrix-core form of the multi-channel kernel on the upscaling",
             "chain's last layer (32 -> 4 3x3, 1280x720); the pages' fp16 net on a 1280x720 frame (its first",
             "layer computed inside the 64 -> 64 layer, then 64 -> 32, then 32 -> 9 with the x3",
             "depth-to-space in its stores). conflict share =",
             "SQ_LDS_BANK_CONFLICT / SQ_LDS_IDX_ACTIVE.", "",
             "| kernel | dispatches | " + " | ".join(LDS_COUNTERS) + " | conflict share |",
             "|---|---|" + "---|" * len(LDS_COUNTERS) + "---|"]
    for k in kernels:
        vals = [tabs[c].get(k, (0.0, 0, ""))[0] for c in LDS_COUNTERS]
        share = vals[0] / vals[1] if vals[1] else 0.0
        lines.append("| `%s` | %d | %s | %.3f |" % (k, tabs[LDS_COUNTERS[0]][k][1],
                                                    " | ".join("%.0f" % v for v in vals), share))
    return "\n".join(lines) + "\n"


MFMA_COUNTERS = ("SQ_INSTS_VALU_MFMA_MOPS_F16", "SQ_INSTS_VALU_MFMA_MOPS_F32", "SQ_INSTS_VALU_FMA_F32",
                 "SQ_VALU_MFMA_BUSY_CYCLES", "SQ_BUSY_CYCLES", "GRBM_GUI_ACTIVE")


def _case_flops():
    """Algorithmic FLOPs of each counted bench case (2 per multiply-add of the
    definition; separable filters: R + S products per pixel)."""
    from image_stencil_amd import traffic
    chain = [(1, 32, 5), (32, 32, 3), (32, 32, 3), (32, 4, 3)]
    out = {"8192x8192 %dx%d" % (r, r): traffic.conv_flops(1, 1, 8192, 8192, 1, r, r) for r in (3, 5, 7)}
    out["fp32 layer 1x32x720x1280 -> 32, 3x3"] = traffic.conv_flops(1, 32, 720, 1280, 32, 3, 3)
    out["fp16 NHWC layer 8x256x256x64 -> 64, 3x3"] = traffic.conv_flops(8, 64, 256, 256, 64, 3, 3)
    out["upscaling chain 1280x720 (fused)"] = traffic.chain_flops(1, 720, 1280, chain)
    out["separable 7x7 filter, 8192x8192 fp32"] = 2.0 * 14 * 8192 * 8192
    out["1 channel -> 8 filters 3x3, 4096x4096 fp32"] = traffic.conv_flops(1, 1, 4096, 4096, 8, 3, 3)
    out["stencil pipeline 3x3 x3, 8192x8192 fp32 (auto)"] = 3 * traffic.conv_flops(1, 1, 8192, 8192, 1, 3, 3)
    return out


def pmc_mfma_summary(pmc_dir):
    """Markdown summary of a counter run of the arithmetic counters: the FLOPs
    the kernels' instructions perform (MFMA ops in units of 512 FLOPs, fp32
    vector FMAs at 128 FLOPs per wave instruction) against the algorithmic
    FLOPs, and the matrix cores' busy share."""
    tabs = {c: _counter_means(pmc_dir, c) for c in MFMA_COUNTERS}
    flops = _case_flops()
    lines = ["# Arithmetic counters of the bench workloads (rocprofv3 --pmc)", "",
             "Commands (from the repository root, one MI355X; then the summary, on any machine):", "", "```",
             "rocprofv3 --pmc %s --output-format csv -d %s -o run -- \\" % (" ".join(MFMA_COUNTERS), pmc_dir),
             "    python3 bench.py " + PMC_ARGS,
             "python3 bench.py --pmc-mfma-summary %s > profiles/arithmetic_counters.md" % pmc_dir,
             "```", "",
             "Per dispatch, averaged over the dispatches of each kernel. counted GFLOP = 512 x",
             "(SQ_INSTS_VALU_MFMA_MOPS_F16 + SQ_INSTS_VALU_MFMA_MOPS_F32) + 128 x SQ_INSTS_VALU_FMA_F32 (a",
             "wave's fp32 FMA: 64 lanes x 2 FLOPs; lanes masked off still count). The ratio to the",
             "algorithmic FLOPs shows work the kernel does beyond the definition (zero-padded MFMA operands,",
             "overlapped tiles, border taps of out-of-image rows) or FLOPs done elsewhere (bias, ReLU are not",
             "FMAs). MFMA busy share = SQ_VALU_MFMA_BUSY_CYCLES / (GRBM_GUI_ACTIVE / 8 x 256 CUs x 4",
             "SIMDs): GRBM_GUI_ACTIVE is read as the sum of the 8 XCDs' own counters (each XCD has its",
             "GRBM); so read, the shares of the fp16 and fp32 MFMA kernels equal their measured fractions",
             "of the MFMA peak.", "",
             "| case | kernel | dispatches | MFMA f16 GFLOP | MFMA f32 GFLOP | vector FMA GFLOP | "
             "counted / algorithmic | MFMA busy share |",
             "|---|---|---|---|---|---|---|---|"]
    for case, (kern, _) in TRAFFIC_KERNELS.items():
        if kern not in tabs[MFMA_COUNTERS[0]]:
            continue
        v = {c: tabs[c].get(kern, (0.0, 0, ""))[0] for c in MFMA_COUNTERS}
        f16 = 512.0 * v["SQ_INSTS_VALU_MFMA_MOPS_F16"] / 1e9
        f32 = 512.0 * v["SQ_INSTS_VALU_MFMA_MOPS_F32"] / 1e9
        fma = 128.0 * v["SQ_INSTS_VALU_FMA_F32"] / 1e9
        alg = flops.get(case, 0.0) / 1e9
        ratio = (f16 + f32 + fma) / alg if alg else 0.0
        gui = v["GRBM_GUI_ACTIVE"]
        busy = v["SQ_VALU_MFMA_BUSY_CYCLES"] / (gui / 8.0 * 256 * 4) if gui else 0.0
        lines.append("| %s | `%s` | %d | %.2f | %.2f | %.2f | %.3f | %.3f |" % (
            case, kern, tabs[MFMA_COUNTERS[0]][kern][1], f16, f32, fma, ratio, busy))
    return "\n".join(lines) + "\n"


def _traffic(case):
    """Counter-derived HBM bytes per launch of a bench case, or None when absent
    or taken with other kernel sources than the current ones."""
    if case not in TRAFFIC_KERNELS or not os.path.exists(TRAFFIC_FILE):
        return None
    with open(TRAFFIC_FILE) as fh:
        for line in fh:
            cols = [c.strip() for c in line.strip().strip("|").split("|")]
            if len(cols) == 7 and cols[0] == case:
                if cols[6] != _source_digest(TRAFFIC_KERNELS[case][1]):
                    return None
                return float(cols[5])
    return None


def _spread(cases):
    """Median and minimum launch time over every launch of a workload's buffer sets."""
    meds = sorted(c.median_ms for c in cases)
    return {"median_ms": round(meds[len(meds) // 2], 4), "min_ms": round(min(c.min_ms for c in cases), 4)}


def _oracle_check(y, ref, m, tau):
    """Outside the timed region: the largest |y - ref| / (tau * m) of one timed
    output against the oracle (at most 1 passes), with the element count."""
    import numpy as np
    y = np.asarray(y, dtype=np.float64)
    err = np.abs(y - ref)
    bound = tau * m
    with np.errstate(divide="ignore", invalid="ignore"):
        ratio = np.where(bound > 0, err / np.where(bound > 0, bound, 1.0), np.where(err > 0, np.inf, 0.0))
    worst = float(np.max(ratio)) if ratio.size else 0.0
    if not np.isfinite(y).all():
        worst = float("inf")
    return {"max_err_over_bound": float("%.3g" % worst), "tau": tau, "elements": int(y.size), "passed": worst <= 1.0}


def _host_info(oracle=None):
    """The host the CPU leg runs on: logical CPUs, those this process may use,
    the CPU model, and the oracle's OpenMP threads."""
    model = ""
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    info = {"nproc": os.cpu_count(), "cpus_allowed": len(os.sched_getaffinity(0)), "cpu_model": model}
    if oracle is not None:
        info["omp_threads"] = oracle.threads()
    return info


def _warm_ms(torch, case, steps, stream_obj):
    """Mean time per launch of one buffer set launched back to back (its data
    partly or wholly in the 256 MB last-level cache), beside the rotating-set
    (cold) figures."""
    for _ in range(3):
        case.launch()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream_obj)
    for _ in range(steps):
        case.launch()
    e1.record(stream_obj)
    torch.cuda.synchronize()
    return round(e0.elapsed_time(e1) / steps, 4)


class Case:
    """One kernel launch of a workload: callable, counted work, kernel name."""

    def __init__(self, name, launch, flops, nbytes, kernel, bound_peak=None):
        self.name, self.launch, self.flops, self.bytes, self.kernel = name, launch, flops, nbytes, kernel


def _single_large_cases(torch, isa, synth, stream):
    cases = []
    for R in (3, 5, 7):
        x, w = synth.large_image(R)
        xd = torch.from_numpy(x).cuda()
        wd = torch.from_numpy(w).cuda()
        yd = torch.empty_like(xd)
        plan = isa.Plan(isa.make_desc(1, 1, 8192, 8192, 1, R, R))
        info = plan.info()

        def launch(plan=plan, xd=xd, wd=wd, yd=yd):
            isa.conv2d_forward(plan.handle, xd.data_ptr(), wd.data_ptr(), None, yd.data_ptr(), stream)

        c = Case("8192x8192 %dx%d" % (R, R), launch, info["flops"], info["bytes"], info["kernel"])
        c.keep = (plan, xd, wd, yd)
        c.R = R
        cases.append(c)
    return cases


def _layer_cases(torch, isa, stream, x, w, b, relu, sets, label, variant=None):
    """One case per rotating buffer set (same values, distinct memory), so that
    consecutive launches do not find their inputs in the 256 MB last-level cache.
    variant: a tuning variant's index (None: the plan's choice)."""
    N, C, H, W = x.shape
    K, _, R, S = w.shape
    plan = isa.Plan(isa.make_desc(N, C, H, W, K, R, S, "f32", relu), variant=variant)
    info = plan.info()
    wd = torch.from_numpy(w).cuda()
    bd = torch.from_numpy(b).cuda() if b is not None else None
    cases = []
    for _ in range(sets):
        xd = torch.from_numpy(x).cuda()
        yd = torch.empty((N, K, H, W), dtype=torch.float32, device="cuda")

        def launch(xd=xd, yd=yd):
            isa.conv2d_forward(plan.handle, xd.data_ptr(), wd.data_ptr(), bd.data_ptr() if bd is not None else None,
                               yd.data_ptr(), stream)

        c = Case(label, launch, info["flops"], info["bytes"], info["kernel"])
        c.keep = (plan, xd, wd, bd, yd)
        cases.append(c)
    return cases


SECONDARY_GROUPS = ("fp32_layer", "fp16_layer", "upscale_chain", "pages_net", "special_cases")


def _secondary(torch, isa, synth, stream, stream_obj, steps, warmup, groups=SECONDARY_GROUPS, check=True):
    """Other workloads, each timed on its own (not part of the headline step); `groups` names
    which of SECONDARY_GROUPS to run. check: after timing, compare one timed
    output of each workload with the oracle (the full tensor)."""
    if check:
        import oracle
        from tolerance import TAU_F16, TAU_F32, tau_f16_chain
    out = {}
    if "fp32_layer" in groups:
        x, w, b = synth.cnn_layer_f32()
        cases = _layer_cases(torch, isa, stream, x, w, b, True, 4, "fp32 layer 1x32x720x1280 -> 32, 3x3")
        ms_step, per, _ = _time_cases(torch, cases, steps, warmup, stream_obj)
        ms = sum(per) / len(per)
        c = cases[0]
        out["cnn_layer_f32"] = {"workload": c.name + ", bias, ReLU", "kernel": c.kernel, "ms_per_frame": round(ms, 4),
                                **_spread(cases), "warm_ms": _warm_ms(torch, c, steps, stream_obj),
                                "gflops": round(c.flops / ms / 1e6, 1),
                                "frac_fp32_valu": round(c.flops / ms / 1e9 / FP32_VALU_PEAK_TFLOPS, 4),
                                "frac_fp32_packed_peak": round(c.flops / ms / 1e9 / FP32_PACKED_PEAK_TFLOPS, 4),
                                "roofline": _roofline(c, ms)}
        ref = m = None
        if check:
            y = c.keep[4].cpu().numpy()
            ref, m = oracle.conv2d(x, w, b, True)
            out["cnn_layer_f32"]["check"] = _oracle_check(y, ref, m, TAU_F32)
            del y
        for c in cases:
            c.keep = None
        # The same layer on the vector ALUs: every variant of the register-blocked
        # multi-channel kernel (output channels per workgroup), the fastest reported
        # against the fp32 vector peak.
        d = isa.make_desc(1, 32, 720, 1280, 32, 3, 3, "f32", True)
        per_variant = {}
        best = None
        for i, v in enumerate(isa.conv2d_list_variants(d)):
            if v["kernel"] != "is_k2_multi":
                continue
            vc = _layer_cases(torch, isa, stream, x, w, b, True, 4, "fp32 layer 1x32x720x1280 -> 32, 3x3", i)
            _, vper, _ = _time_cases(torch, vc, steps, warmup, stream_obj)
            vms = sum(vper) / len(vper)
            per_variant[v["param"]] = round(vms, 4)
            if best is None or vms < best[0]:
                if best is not None:
                    for oc in best[2]:
                        oc.keep = None
                best = (vms, v["param"], vc)
            else:
                for oc in vc:
                    oc.keep = None
        if best is not None:
            vms, param, vc = best
            c = vc[0]
            out["cnn_layer_f32_valu"] = {
                "workload": c.name + ", bias, ReLU, on the vector ALUs", "kernel": c.kernel,
                "channels_per_workgroup": param, "ms_per_frame": round(vms, 4), **_spread(vc),
                "gflops": round(c.flops / vms / 1e6, 1),
                "variants_ms": per_variant,
                "roofline": {"bound": "alu", "achieved": round(c.flops / vms / 1e9, 3),
                             "peak": round(FP32_VALU_PEAK_TFLOPS, 2), "unit": "TFLOP/s",
                             "frac": round(c.flops / vms / 1e9 / FP32_VALU_PEAK_TFLOPS, 4)}}
            if check:
                y = c.keep[4].cpu().numpy()
                out["cnn_layer_f32_valu"]["check"] = _oracle_check(y, ref, m, TAU_F32)
                del y
            for oc in vc:
                oc.keep = None
        del ref, m

    if "fp16_layer" in groups:
        # fp16 NHWC layer on the matrix cores.
        x, w, b = synth.cnn_layer_f16_nhwc()
        plan = isa.Plan(isa.make_desc(8, 64, 256, 256, 64, 3, 3, "f16", False))
        info = plan.info()
        wd, bd = torch.from_numpy(w).cuda(), torch.from_numpy(b).cuda()
        mcases = []
        for _ in range(4):
            xd = torch.from_numpy(x).cuda()
            yd = torch.empty((8, 256, 256, 64), dtype=torch.float16, device="cuda")

            def launch(xd=xd, yd=yd):
                isa.conv2d_forward(plan.handle, xd.data_ptr(), wd.data_ptr(), bd.data_ptr(), yd.data_ptr(), stream)

            c = Case("fp16 NHWC layer 8x256x256x64 -> 64, 3x3", launch, info["flops"], info["bytes"], info["kernel"])
            c.keep = (xd, yd)
            mcases.append(c)
        _, per, _ = _time_cases(torch, mcases, steps, warmup, stream_obj)
        ms = sum(per) / len(per)
        c = mcases[0]
        ach = c.flops / ms / 1e9
        out["mfma_layer_f16"] = {"workload": c.name + ", fp32 accumulate, fp16 out", "kernel": c.kernel,
                                 "ms": round(ms, 4), **_spread(mcases), "warm_ms": _warm_ms(torch, c, steps, stream_obj),
                                 "gflops": round(c.flops / ms / 1e6, 1),
                                 "gbs": round(c.bytes / ms / 1e6, 1),
                                 "roofline": {"bound": "mfma", "achieved": round(ach, 2), "peak": FP16_MFMA_PEAK_TFLOPS,
                                              "unit": "TFLOP/s", "frac": round(ach / FP16_MFMA_PEAK_TFLOPS, 4),
                                              "hbm_frac": round(c.bytes / ms / 1e6 / HBM_PEAK_GBS, 4),
                                              "traffic": _traffic(c.name)}}
        if check:
            y = c.keep[1].cpu().numpy()
            ref, m = oracle.conv2d(x, w, b, False, "NHWC")
            out["mfma_layer_f16"]["check"] = _oracle_check(y, ref, m, TAU_F16)
            del y, ref, m
        for c in mcases:
            c.keep = None
        del plan

    if "upscale_chain" in groups:
        # Upscaling chain on a 1280x720 frame: fused kernel and layer by layer.
        x, layers = synth.chain_f32()
        spec = [(w.shape[1], w.shape[0], w.shape[2], relu) for (w, b, relu) in layers]
        flops = sum(2.0 * 720 * 1280 * k * c * r * r for (c, k, r, _) in spec)
        nbytes = 4.0 * (720 * 1280 * 5) + sum(4.0 * (k * c * r * r + k) for (c, k, r, _) in spec)
        wl = [(torch.from_numpy(w).cuda(), torch.from_numpy(b).cuda()) for (w, b, _) in layers]
        chain_ref = oracle.chain(x, layers, d2s=2) if check else None
        for mode_name, mode in (("fused", isa.IS_CHAIN_FUSED), ("unfused", isa.IS_CHAIN_UNFUSED)):
            d = isa.make_chain_desc(1, 720, 1280, spec, 2, mode)
            kname = isa.conv_chain_kernel_name(d)
            ws_bytes = isa.conv_chain_workspace_size(d)
            ws = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device="cuda")
            ccases = []
            for _ in range(16):
                xd = torch.from_numpy(x).cuda()
                yd = torch.empty((1, 1, 1440, 2560), dtype=torch.float32, device="cuda")

                def launch(d=d, xd=xd, yd=yd, ws=ws, ws_bytes=ws_bytes):
                    isa.conv_chain_forward(d, xd.data_ptr(), [w.data_ptr() for (w, _) in wl],
                                           [b.data_ptr() for (_, b) in wl], yd.data_ptr(),
                                           ws.data_ptr() if ws_bytes else None, ws_bytes, stream)

                c = Case("upscaling chain 1280x720 (%s)" % mode_name, launch, flops, nbytes, kname)
                c.keep = (xd, yd)
                ccases.append(c)
            _, per, _ = _time_cases(torch, ccases, steps, warmup, stream_obj)
            ms = sum(per) / len(per)
            out["upscale_chain_" + mode_name] = {
                "workload": ccases[0].name + ": 5x5 1->32, 3x3 32->32 x2, 3x3 32->4, depth-to-space x2",
                "kernel": kname, "ms_per_frame": round(ms, 4), **_spread(ccases),
                "warm_ms": _warm_ms(torch, ccases[0], steps, stream_obj), "gflops": round(flops / ms / 1e6, 1),
                "frac_fp32_valu": round(flops / ms / 1e9 / FP32_VALU_PEAK_TFLOPS, 4),
                "frac_fp32_packed_peak": round(flops / ms / 1e9 / FP32_PACKED_PEAK_TFLOPS, 4),
                # both paths run the two 32 -> 32 layers (90% of the FLOPs) on the
                # fp32 matrix cores
                "roofline": _roofline(ccases[0], ms, mfma_f32=True)}
            if check:
                out["upscale_chain_" + mode_name]["check"] = _oracle_check(ccases[0].keep[1].cpu().numpy(),
                                                                           chain_ref[0], chain_ref[1], TAU_F32)
            for c in ccases:
                c.keep = None
            del ws
        del chain_ref

    if "pages_net" in groups:
        # The pages' own net in fp16 storage, layer by layer on the matrix cores.
        x, layers = synth.chain_f16_nhwc()
        spec = [(w.shape[1], w.shape[0], w.shape[2], relu) for (w, b, relu) in layers]
        flops = sum(2.0 * 720 * 1280 * k * c * r * r for (c, k, r, _) in spec)
        nbytes = 2.0 * 720 * 1280 * (1 + 9) + sum(2.0 * k * c * r * r + 4.0 * k for (c, k, r, _) in spec)
        wl = [(torch.from_numpy(w).cuda(), torch.from_numpy(b).cuda()) for (w, b, _) in layers]
        res = {}
        for mname, mode in (("auto", isa.IS_CHAIN_AUTO), ("unfused", isa.IS_CHAIN_UNFUSED)):
            d = isa.make_chain_desc(1, 720, 1280, spec, 3, mode, "f16")
            kname = isa.conv_chain_kernel_name(d)
            ws_bytes = isa.conv_chain_workspace_size(d)
            ws = torch.empty(ws_bytes, dtype=torch.uint8, device="cuda")
            ncases = []
            for _ in range(16):
                xd = torch.from_numpy(x).cuda()
                yd = torch.empty((1, 2160, 3840, 1), dtype=torch.float16, device="cuda")

                def launch(d=d, xd=xd, yd=yd, ws=ws, ws_bytes=ws_bytes):
                    isa.conv_chain_forward(d, xd.data_ptr(), [w.data_ptr() for (w, _) in wl],
                                           [b.data_ptr() for (_, b) in wl], yd.data_ptr(), ws.data_ptr(), ws_bytes,
                                           stream)

                c = Case("pages' net fp16 1280x720", launch, flops, nbytes, kname)
                c.keep = (xd, yd)
                ncases.append(c)
            _, per, _ = _time_cases(torch, ncases, steps, warmup, stream_obj)
            res[mname] = (sum(per) / len(per), ncases, kname, isa.conv_chain_groups(d), ws)
        ms, ncases, kname, groups, ws = res["auto"]
        ach = flops / ms / 1e9
        out["pages_net_f16"] = {
            "workload": ncases[0].name + ": 5x5 1->64, 3x3 64->64, 64->32, 32->9, depth-to-space x3, "
                        "fp16 storage, fp32 accumulate",
            "kernel": kname, "groups": groups, "ms_per_frame": round(ms, 4), **_spread(ncases),
            "warm_ms": _warm_ms(torch, ncases[0], steps, stream_obj),
            "ms_per_frame_one_launch_per_layer": round(res["unfused"][0], 4),
            "gflops": round(flops / ms / 1e6, 1),
            "roofline": {"bound": "mfma", "achieved": round(ach, 2), "peak": FP16_MFMA_PEAK_TFLOPS,
                         "unit": "TFLOP/s", "frac": round(ach / FP16_MFMA_PEAK_TFLOPS, 4), "traffic": None}}
        for c in res["unfused"][1]:
            c.keep = None
        if check:
            ref, m = oracle.chain_f16(x, layers, d2s=3)
            out["pages_net_f16"]["check"] = _oracle_check(ncases[0].keep[1].cpu().numpy(), ref, m,
                                                          tau_f16_chain(len(layers)))
            del ref, m
        for c in ncases:
            c.keep = None
        del ws

    if "special_cases" in groups:
        import numpy as np
        # The 256x256 3x3 image: its 0.52 MB move in well under a microsecond
        # at the HBM rate, so a launch is bound by launch latency and the
        # single wave per strip; reported as time per launch (back to back).
        x, w = synth.small_image_3x3()
        plan = isa.Plan(isa.make_desc(1, 1, 256, 256, 1, 3, 3))
        info = plan.info()
        wd = torch.from_numpy(w).cuda()
        tcases = []
        for _ in range(4):
            xd = torch.from_numpy(x).cuda()
            yd = torch.empty((1, 1, 256, 256), device="cuda")

            def launch(plan=plan, xd=xd, yd=yd):
                isa.conv2d_forward(plan.handle, xd.data_ptr(), wd.data_ptr(), None, yd.data_ptr(), stream)

            c = Case("256x256 3x3", launch, info["flops"], info["bytes"], info["kernel"])
            c.keep = (xd, yd)
            tcases.append(c)
        _, per, _ = _time_cases(torch, tcases, steps, warmup, stream_obj)
        ms = sum(per) / len(per)
        # At this size the event pair around each launch costs as much as the
        # launch; 400 launches back to back between two events give the rate a
        # caller issuing many small images sees.
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream_obj)
        for i in range(400):
            tcases[i % len(tcases)].launch()
        e1.record(stream_obj)
        torch.cuda.synchronize()
        b2b = e0.elapsed_time(e1) / 400
        out["small_image_3x3_256"] = {"workload": "single-channel fp32 256x256 3x3", "kernel": info["kernel"],
                                      "us": round(ms * 1e3, 2), "us_back_to_back": round(b2b * 1e3, 2),
                                      "gbs": round(info["bytes"] / ms / 1e6, 1),
                                      "frac_hbm": round(info["bytes"] / ms / 1e6 / HBM_PEAK_GBS, 4)}
        if check:
            ref, m = oracle.conv2d(x, w)
            out["small_image_3x3_256"]["check"] = _oracle_check(tcases[0].keep[1].cpu().numpy(), ref, m, TAU_F32)
        for c in tcases:
            c.keep = None
        del plan
        # The single-channel special case beyond one filter: a separable 7x7
        # filter (row pass + column pass) and 8 filters on one channel; both
        # are bound by HBM. A 1x1 filter (one multiply per pixel) on the same
        # kernel is the copy rate that its load and store streams reach with
        # no filter work: the practical ceiling of the 3x3/5x5 filters. Two
        # buffer sets each, so that no launch reads the previous one's data
        # from the last-level cache.
        specs = [("filter_1x1_8192", "1x1 filter (copy bound of the single-channel kernel), 8192x8192 fp32",
                  (1, 1, 8192, 8192, 1, 1, 1), False),
                 ("separable_7x7_8192", "separable 7x7 filter, 8192x8192 fp32", (1, 1, 8192, 8192, 1, 7, 7), True),
                 ("one_channel_8_filters_3x3_4096", "1 channel -> 8 filters 3x3, 4096x4096 fp32",
                  (1, 1, 4096, 4096, 8, 3, 3), False),
                 ("one_channel_4_filters_3x3_4096", "1 channel -> 4 filters 3x3, 4096x4096 fp32",
                  (1, 1, 4096, 4096, 4, 3, 3), False)]
        for key, name, (n_, c_, h_, w_, k_, r_, s_), sep in specs:
            plan = isa.Plan(isa.make_desc(n_, c_, h_, w_, k_, r_, s_, "f32", False, separable=sep))
            info = plan.info()
            rng = np.random.default_rng(0)
            wv = (rng.standard_normal(r_ + s_ if sep else k_ * c_ * r_ * s_) / r_).astype(np.float32)
            wd = torch.from_numpy(wv).cuda()
            scases = []
            for _ in range(2):
                xd = torch.rand((n_, c_, h_, w_), device="cuda")
                yd = torch.empty((n_, k_, h_, w_), device="cuda")

                def launch(plan=plan, xd=xd, yd=yd, wd=wd):
                    isa.conv2d_forward(plan.handle, xd.data_ptr(), wd.data_ptr(), None, yd.data_ptr(), stream)

                c = Case(name, launch, info["flops"], info["bytes"], info["kernel"])
                c.keep = (xd, yd)
                scases.append(c)
            _, per, _ = _time_cases(torch, scases, steps, warmup, stream_obj)
            ms = sum(per) / len(per)
            out[key] = {"workload": name, "kernel": info["kernel"], "ms": round(ms, 4),
                        "median_ms": round(sum(c.median_ms for c in scases) / len(scases), 4),
                        "gflops": round(info["flops"] / ms / 1e6, 1), "roofline": _roofline(scases[0], ms)}
            for c in scases:
                c.keep = None
            del plan

        # A stencil pipeline of three 3x3 filters (ReLU after each) on 8192^2:
        # the model's grouping (one fused launch) against one launch per filter.
        H = W = 8192
        rs = (3, 3, 3)
        flops = sum(2.0 * r * r * H * W for r in rs)
        nbytes = 8.0 * H * W + sum(4.0 * (r * r + 1) for r in rs)
        wl = [(torch.randn((1, 1, r, r), device="cuda") / r, torch.zeros(1, device="cuda")) for r in rs]
        res = {}
        for mode, mname in ((isa.IS_CHAIN_AUTO, "auto"), (isa.IS_CHAIN_UNFUSED, "unfused")):
            d = isa.make_chain_desc(1, H, W, [(1, 1, r, True) for r in rs], 1, mode)
            ws_bytes = isa.conv_chain_workspace_size(d)
            ws = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device="cuda")
            pcases = []
            for _ in range(2):
                xd = torch.rand((1, 1, H, W), device="cuda")
                yd = torch.empty((1, 1, H, W), device="cuda")

                def launch(d=d, xd=xd, yd=yd, ws=ws, ws_bytes=ws_bytes):
                    isa.conv_chain_forward(d, xd.data_ptr(), [w.data_ptr() for (w, _) in wl],
                                           [b.data_ptr() for (_, b) in wl], yd.data_ptr(),
                                           ws.data_ptr() if ws_bytes else None, ws_bytes, stream)

                c = Case("stencil pipeline 3x3 x3, 8192x8192 fp32 (%s)" % mname, launch, flops, nbytes,
                         isa.conv_chain_kernel_name(d))
                c.keep = (xd, yd)
                pcases.append(c)
            _, per, _ = _time_cases(torch, pcases, steps, warmup, stream_obj)
            res[mname] = (sum(per) / len(per), pcases[0], isa.conv_chain_groups(d))
            for c in pcases:
                c.keep = None
            del ws
        ms, c0, groups = res["auto"]
        out["stencil_pipeline_3x3x3_8192"] = {
            "workload": "three 3x3 filters with ReLU, 8192x8192 fp32", "kernel": c0.kernel,
            "groups": groups, "ms": round(ms, 4), "ms_one_launch_per_filter": round(res["unfused"][0], 4),
            "gflops": round(flops / ms / 1e6, 1), "roofline": _roofline(c0, ms)}
    return out


MIN_WARM_S = 0.3


def _time_cases(torch, cases, steps, warmup, stream_obj):
    """Warmup, then `steps` steps of all cases with an event pair around every
    launch, all on the stream the library launches on. The warmup runs at least
    `warmup` steps and at least MIN_WARM_S seconds: the ALU-bound launches
    measured up to 25% slower while the clock was still ramping after a short
    warmup."""
    t0w, n = time.perf_counter(), 0
    while n < warmup or time.perf_counter() - t0w < MIN_WARM_S:
        for c in cases:
            c.launch()
        n += 1
        if n % 16 == 0:
            torch.cuda.synchronize()
    torch.cuda.synchronize()
    ev = [[(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in cases]
          for _ in range(steps)]
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    t0.record(stream_obj)
    for s in range(steps):
        for i, c in enumerate(cases):
            ev[s][i][0].record(stream_obj)
            c.launch()
            ev[s][i][1].record(stream_obj)
    t1.record(stream_obj)
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    total_ms = t0.elapsed_time(t1)
    times = [[ev[s][i][0].elapsed_time(ev[s][i][1]) for s in range(steps)] for i in range(len(cases))]
    per = [sum(t) / steps for t in times]
    for c, t in zip(cases, times):   # median and minimum per launch, for the report
        st = sorted(t)
        c.median_ms = st[len(st) // 2] if len(st) % 2 else 0.5 * (st[len(st) // 2 - 1] + st[len(st) // 2])
        c.min_ms = st[0]
    return total_ms / steps, per, wall


def _roofline(c, ms, mfma_f32=False):
    """Roofline entry of one launch: bound by HBM, by the fp32 vector ALUs, or
    (mfma_f32: the dominant work runs on the fp32 matrix cores) by those."""
    sec = ms / 1e3
    ai = c.flops / c.bytes
    if mfma_f32 or c.kernel in MFMA_F32_KERNELS:
        ach = c.flops / sec / 1e12
        return {"bound": "mfma", "achieved": round(ach, 3), "peak": FP32_MFMA_PEAK_TFLOPS, "unit": "TFLOP/s",
                "frac": round(ach / FP32_MFMA_PEAK_TFLOPS, 4), "traffic": _traffic(c.name), "dtype": "f32"}
    ridge = FP32_VALU_PEAK_TFLOPS * 1e12 / (HBM_PEAK_GBS * 1e9)
    if ai > ridge:
        ach = c.flops / sec / 1e12
        return {"bound": "alu", "achieved": round(ach, 3), "peak": round(FP32_VALU_PEAK_TFLOPS, 2),
                "unit": "TFLOP/s", "frac": round(ach / FP32_VALU_PEAK_TFLOPS, 4), "traffic": _traffic(c.name),
                "peak_packed_fp32": FP32_PACKED_PEAK_TFLOPS}
    ach = c.bytes / sec / 1e9
    return {"bound": "hbm", "achieved": round(ach, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": round(ach / HBM_PEAK_GBS, 4), "traffic": _traffic(c.name)}


def _copy_reference(torch, stream_obj, mib=256, reps=5):
    """Two plain streaming references over `mib` MiB: a device-to-device copy
    (torch copy_, the runtime's copy kernel) and torch's elementwise negation
    (reads and writes each fp32 element once). The second has a kernel name of
    its own, which makes it the known-size dispatch that scales the FETCH_SIZE /
    WRITE_SIZE counters of a profiling run of this script."""
    n = mib * (1 << 20) // 4
    a = torch.ones(n, device="cuda")
    b = torch.empty_like(a)
    out = {"bytes_per_launch": 2 * n * 4}
    for name, fn in (("copy", lambda: b.copy_(a)), ("neg_kernel", lambda: torch.neg(a, out=b))):
        for _ in range(2):
            fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream_obj)
        for _ in range(reps):
            fn()
        e1.record(stream_obj)
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / reps
        out[name] = {"ms": round(ms, 4), "gbs": round(2 * n * 4 / ms / 1e6, 1)}
    return out


PROBES_LIB = os.path.join(ROOT, "image_stencil_amd", "libimgstencil_probes.so")


def _probes(ctypes_mod):
    if not os.path.exists(PROBES_LIB):
        raise SystemExit("%s is not built (run __graft_entry__.build())" % PROBES_LIB)
    lib = ctypes_mod.CDLL(PROBES_LIB)
    vp = ctypes_mod.c_void_p
    lib.isp_mfma_rate.argtypes = [ctypes_mod.c_int, ctypes_mod.c_int, ctypes_mod.c_int, vp, vp, vp]
    lib.isp_lds_probe.argtypes = [ctypes_mod.c_int, ctypes_mod.c_int, ctypes_mod.c_int, ctypes_mod.c_int, vp, vp]
    return lib


def _mfma_reference(torch, stream_obj, min_s=0.3):
    """The rate back-to-back matrix-core instructions sustain on this chip, the
    attainable ceiling beside the nominal peaks: 8 waves per CU (as the fp16
    layer) each issuing independent v_mfma_f32_16x16x32_f16 (or
    v_mfma_f32_16x16x4_f32) on varying random operands, with the shader clock
    over the loop from each wave's cycle counter against the 100 MHz real-time
    counter."""
    import ctypes
    lib = _probes(ctypes)
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    grid = 2 * cus
    waves = grid * 4
    out = {"cus": cus, "waves": waves}
    for kind, name, flop, iters, peak in ((0, "f16_16x16x32", 16384, 2048, FP16_MFMA_PEAK_TFLOPS),
                                          (1, "f32_16x16x4", 2048, 1024, FP32_MFMA_PEAK_TFLOPS)):
        stamps = torch.zeros(2 * waves, dtype=torch.int64, device="cuda")
        sink = torch.empty(grid * 256, dtype=torch.float32, device="cuda")
        stream = stream_obj.cuda_stream

        def launch():
            rc = lib.isp_mfma_rate(kind, grid, iters, stamps.data_ptr(), sink.data_ptr(), stream)
            if rc != 0:
                raise RuntimeError("isp_mfma_rate: hipError_t %d" % rc)

        t0 = time.perf_counter()
        while time.perf_counter() - t0 < min_s:   # the clock ramps up under load
            launch()
            torch.cuda.synchronize()
        reps = 5
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream_obj)
        for _ in range(reps):
            launch()
        e1.record(stream_obj)
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / reps
        st = stamps.cpu().view(-1, 2).double()
        clock_ghz = float(st[:, 0].sum() / st[:, 1].sum()) * 0.1   # ticks at 100 MHz
        tflops = waves * iters * 8 * flop / (ms / 1e3) / 1e12
        out[name] = {"ms": round(ms, 4), "tflops": round(tflops, 1), "peak": peak,
                     "frac_of_peak": round(tflops / peak, 4), "shader_clock_ghz": round(clock_ghz, 3)}
    return out


def mfma_chain_study(torch, stream_obj, min_s=0.1):
    """Sustained fp16 MFMA rate against the number of independent accumulators
    per wave (1 .. 8) and waves per SIMD (1 or 2): how far apart dependent
    matrix products must be to keep the matrix unit busy."""
    import ctypes
    lib = _probes(ctypes)
    lib.isp_mfma_chain_rate.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_void_p,
                                        ctypes.c_void_p, ctypes.c_void_p]
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    out = []
    for per_simd in (1, 2):
        grid = per_simd * cus
        waves = grid * 4
        stamps = torch.zeros(2 * waves, dtype=torch.int64, device="cuda")
        sink = torch.empty(grid * 256, dtype=torch.float32, device="cuda")
        for chains in (1, 2, 3, 4, 6, 8):
            iters = 2048 // per_simd

            def launch():
                rc = lib.isp_mfma_chain_rate(chains, grid, iters, stamps.data_ptr(), sink.data_ptr(),
                                             stream_obj.cuda_stream)
                if rc != 0:
                    raise RuntimeError("isp_mfma_chain_rate: hipError_t %d" % rc)

            t0 = time.perf_counter()
            while time.perf_counter() - t0 < min_s:
                launch()
                torch.cuda.synchronize()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream_obj)
            for _ in range(5):
                launch()
            e1.record(stream_obj)
            torch.cuda.synchronize()
            ms = e0.elapsed_time(e1) / 5
            st = stamps.cpu().view(-1, 2).double()
            clock = float(st[:, 0].sum() / st[:, 1].sum()) * 0.1
            mfmas = waves * iters * 8
            tflops = mfmas * 16384 / (ms / 1e3) / 1e12
            out.append({"waves_per_simd": per_simd, "chains": chains, "tflops": round(tflops, 1),
                        "clock_ghz": round(clock, 3),
                        "cycles_per_mfma_per_simd": round(clock * 1e9 * ms / 1e3 / (mfmas / (cus * 4)), 2)})
    return out


def lds_rate_study(torch, stream_obj, iters=4096):
    """LDS throughput per CU: conflict-free 16-byte reads, 16-byte writes and
    8-byte reads by 4, 8 and 16 waves per CU (one workgroup per CU), in bytes
    per shader clock from each wave's own cycle counter (the slowest wave of
    the launch) and in TB/s over the whole chip from the launch time."""
    import ctypes
    lib = _probes(ctypes)
    lib.isp_lds_rate.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_void_p,
                                 ctypes.c_void_p, ctypes.c_void_p]
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    out = []
    for op, name, width in ((0, "read 16 B", 16), (1, "write 16 B", 16), (2, "read 8 B", 8)):
        for waves in (4, 8, 16):
            stamps = torch.zeros(2 * cus * waves, dtype=torch.int64, device="cuda")
            sink = torch.empty(cus * waves * 64, dtype=torch.float32, device="cuda")

            def launch():
                rc = lib.isp_lds_rate(op, waves, cus, iters, stamps.data_ptr(), sink.data_ptr(),
                                      stream_obj.cuda_stream)
                if rc != 0:
                    raise RuntimeError("isp_lds_rate: hipError_t %d" % rc)

            for _ in range(3):
                launch()
            torch.cuda.synchronize()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream_obj)
            for _ in range(5):
                launch()
            e1.record(stream_obj)
            torch.cuda.synchronize()
            ms = e0.elapsed_time(e1) / 5
            st = stamps.cpu().view(-1, 2).double()
            per_cu = waves * iters * 8 * 64 * width
            clock = float(st[:, 0].sum() / st[:, 1].sum()) * 0.1
            out.append({"access": name, "waves_per_cu": waves,
                        "bytes_per_clock_per_cu": round(per_cu / float(st[:, 0].max()), 1),
                        "clock_ghz": round(clock, 3),
                        "chip_tb_s": round(per_cu * cus / (ms / 1e3) / 1e12, 2)})
    return out


MIX_PARTS = ((1, "lds_reads"), (2, "mfma"), (4, "row_writes"), (8, "barrier"), (16, "stores"), (32, "dma"),
             (64, "split_by_wave"))
MIX_CASES = (2, 3, 7, 15, 10, 11, 31, 47, 63, 5, 61, 127, 125)   # 64: the 8-wave flow only


def mix_study(torch, stream_obj, iters=512):
    """The fp16 layer's instruction mix taken apart (probes.hip isp_mix_rate):
    per combination of operand reads, MFMAs, finished-row writes, a barrier per
    4-row stage, global stores and global-to-LDS loads, the launch time and the
    matrix-core rate."""
    import ctypes
    lib = _probes(ctypes)
    lib.isp_mix_rate.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p,
                                 ctypes.c_void_p, ctypes.c_void_p]
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    gbuf = torch.zeros(cus * 65536, dtype=torch.uint8, device="cuda")
    stamps = torch.zeros(2 * cus * 8, dtype=torch.int64, device="cuda")
    sink = torch.empty(cus * 512, dtype=torch.float32, device="cuda")
    out = []
    for mix in MIX_CASES:
        def launch():
            rc = lib.isp_mix_rate(mix, cus, iters, stamps.data_ptr(), sink.data_ptr(), gbuf.data_ptr(),
                                  stream_obj.cuda_stream)
            if rc != 0:
                raise RuntimeError("isp_mix_rate: hipError_t %d" % rc)

        for _ in range(3):
            launch()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream_obj)
        for _ in range(5):
            launch()
        e1.record(stream_obj)
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / 5
        row = {"parts": "+".join(n for (b, n) in MIX_PARTS if mix & b), "ms": round(ms, 4)}
        if mix & 2:
            row["pflops"] = round(cus * 8 * iters * 72 * 16384 / (ms / 1e3) / 1e15, 3)
        # The same stage on the 4-wave data flow (isp_mix4_rate: a wave holds 64
        # output channels x half the k range; 12 products per operand read; the
        # k halves summed through LDS), the same products per CU and round.
        if mix & 64:
            out.append(row)
            continue
        lib.isp_mix4_rate.argtypes = lib.isp_mix_rate.argtypes
        rc = lib.isp_mix4_rate(mix, cus, iters, stamps.data_ptr(), sink.data_ptr(), gbuf.data_ptr(),
                               stream_obj.cuda_stream)
        if rc != 0:
            raise RuntimeError("isp_mix4_rate: hipError_t %d" % rc)
        torch.cuda.synchronize()
        e0.record(stream_obj)
        for _ in range(5):
            lib.isp_mix4_rate(mix, cus, iters, stamps.data_ptr(), sink.data_ptr(), gbuf.data_ptr(),
                              stream_obj.cuda_stream)
        e1.record(stream_obj)
        torch.cuda.synchronize()
        ms4 = e0.elapsed_time(e1) / 5
        row["ms_4wave"] = round(ms4, 4)
        if mix & 2:
            row["pflops_4wave"] = round(cus * 4 * iters * 144 * 16384 / (ms4 / 1e3) / 1e15, 3)
        out.append(row)
    return out


def lds_bank_probe(torch, stream_obj, iters=4096):
    """Launch every LDS probe (access width x address pattern) once, one wave
    per CU, for a counter run of their bank conflicts (see probes.hip)."""
    import ctypes
    lib = _probes(ctypes)
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    sink = torch.empty(cus * 64, dtype=torch.float32, device="cuda")
    for op in range(4):
        for pat in range(len(LDS_PROBE_PATS)):
            rc = lib.isp_lds_probe(op, pat, cus, iters, sink.data_ptr(), stream_obj.cuda_stream)
            if rc != 0:
                raise RuntimeError("isp_lds_probe: hipError_t %d" % rc)
            torch.cuda.synchronize()
    return {"probes": 4 * len(LDS_PROBE_PATS), "waves_per_probe": cus, "accesses_per_wave": iters}


CLOCK_COUNTERS = ("GRBM_GUI_ACTIVE", "GRBM_COUNT", "SQ_BUSY_CYCLES")


def clock_study(torch, isa, synth, stream, stream_obj, out_json):
    """The matrix-core kernels and the 8192^2 7x7 filter, 4 launches each, and
    the back-to-back MFMA probes (which measure their own shader clock from the
    cycle counter; written to out_json), for a counter run of the clock."""
    cases = []
    x, w, b = synth.cnn_layer_f16_nhwc()
    xd, wd, bd = torch.from_numpy(x).cuda(), torch.from_numpy(w).cuda(), torch.from_numpy(b).cuda()
    yd = torch.empty((8, 256, 256, 64), dtype=torch.float16, device="cuda")
    p16 = isa.Plan(isa.make_desc(8, 64, 256, 256, 64, 3, 3, "f16"))
    cases.append(lambda: p16.forward(xd, wd, bd, yd))
    x, w, b = synth.cnn_layer_f32()
    xf, wf, bf = torch.from_numpy(x).cuda(), torch.from_numpy(w).cuda(), torch.from_numpy(b).cuda()
    yf = torch.empty((1, 32, 720, 1280), device="cuda")
    p32 = isa.Plan(isa.make_desc(1, 32, 720, 1280, 32, 3, 3, "f32", True))
    cases.append(lambda: p32.forward(xf, wf, bf, yf))
    x, layers = synth.chain_f32()
    xc = torch.from_numpy(x).cuda()
    lc = [(torch.from_numpy(w).cuda(), torch.from_numpy(b).cuda(), r) for (w, b, r) in layers]
    cases.append(lambda: isa.conv_chain(xc, lc, depth_to_space=2, mode=isa.IS_CHAIN_FUSED))
    x, w = synth.large_image(7)
    xs, ws = torch.from_numpy(x).cuda(), torch.from_numpy(w).cuda()
    ys = torch.empty_like(xs)
    p7 = isa.Plan(isa.make_desc(1, 1, 8192, 8192, 1, 7, 7))
    cases.append(lambda: p7.forward(xs, ws, None, ys))
    for c in cases:
        for _ in range(4):
            c()
        torch.cuda.synchronize()
    ref = _mfma_reference(torch, stream_obj, min_s=0.1)
    with open(out_json, "w") as fh:
        json.dump(ref, fh)
    return ref


def pmc_clock_summary(pmc_dir):
    """Markdown summary of a counter run of --clock-study: the average shader
    clock of each dispatch, GRBM_GUI_ACTIVE (read per XCD: the counter sums
    the 8 XCDs) over the dispatch's duration, against the clock the MFMA probes
    measure themselves with the cycle counter."""
    import csv
    import glob
    per = {}
    for f in sorted(glob.glob(os.path.join(pmc_dir, "**", "*counter_collection.csv"), recursive=True)):
        with open(f) as fh:
            for r in csv.DictReader(fh):
                key = (_short_kernel(r["Kernel_Name"]), f, r["Dispatch_Id"])
                d = per.setdefault(key, {"ns": int(r["End_Timestamp"]) - int(r["Start_Timestamp"])})
                d[r["Counter_Name"]] = d.get(r["Counter_Name"], 0.0) + float(r["Counter_Value"])
    acc = {}
    for (k, _, _), d in per.items():
        if d["ns"] <= 0 or "GRBM_GUI_ACTIVE" not in d:
            continue
        a = acc.setdefault(k, [])
        a.append((d["ns"], d["GRBM_GUI_ACTIVE"], d.get("GRBM_COUNT", 0.0), d.get("SQ_BUSY_CYCLES", 0.0)))
    probe = {}
    pj = os.path.join(pmc_dir, "probe_clock.json")
    if os.path.exists(pj):
        with open(pj) as fh:
            probe = json.load(fh)
    lines = ["# Shader clock per dispatch (GRBM_GUI_ACTIVE over the dispatch time)", "",
             "Commands (from the repository root, one MI355X; then the summary, on any machine):", "", "```",
             "rocprofv3 --pmc %s --output-format csv -d %s -o run -- \\" % (" ".join(CLOCK_COUNTERS), pmc_dir),
             "    python3 bench.py --clock-study %s/probe_clock.json" % pmc_dir,
             "python3 bench.py --pmc-clock-summary %s > profiles/shader_clock.md" % pmc_dir,
             "```", "",
             "clock = GRBM_GUI_ACTIVE / 8 / dispatch time (the counter is read as the sum of the 8 XCDs'",
             "own). The MFMA probes measure their own clock over their loop from the cycle counter",
             "(s_memtime) against the 100 MHz real-time counter; their rows check the counter reading.", "",
             "| kernel | dispatches | avg us | GHz (GRBM_GUI_ACTIVE / 8) | GHz (GRBM_COUNT / 8) | GHz calibrated |",
             "|---|---|---|---|---|---|"]

    def ghz(k):
        a = acc[k]
        ns = sum(v[0] for v in a)
        return ns, sum(v[1] for v in a) / 8.0 / ns, sum(v[2] for v in a) / 8.0 / ns

    # Calibration: the probes' cycle-counter clocks over the counter reading of the same dispatches.
    ratios = []
    for name, key in (("isp_mfma_rate<true, 8>", "f16_16x16x32"), ("isp_mfma_rate<false, 8>", "f32_16x16x4")):
        own = probe.get(key, {}).get("shader_clock_ghz", 0.0)
        if name in acc and own > 0:
            ratios.append(own / ghz(name)[1])
    cal = sum(ratios) / len(ratios) if ratios else 1.0
    for k in sorted(acc, key=lambda kk: -sum(a[0] for a in acc[kk])):
        if not (k.startswith("is_k") or k.startswith("isp_mfma")):
            continue
        ns, gui, cnt = ghz(k)
        lines.append("| `%s` | %d | %.1f | %.3f | %.3f | %.3f |" % (k[:60], len(acc[k]), ns / len(acc[k]) / 1e3,
                                                                 gui, cnt, gui * cal))
    if probe:
        lines += ["", "The probes' own clocks over their loops (cycle counter): fp16 %.3f GHz, fp32 %.3f GHz; "
                      "calibrated = the counter reading x %.3f, their mean ratio." % (
                          probe.get("f16_16x16x32", {}).get("shader_clock_ghz", 0.0),
                          probe.get("f32_16x16x4", {}).get("shader_clock_ghz", 0.0), cal)]
    return "\n".join(lines) + "\n"


LDS_PAIR_OFFSETS = (1024, 4096)


def lds_pair_probe(torch, stream_obj, iters=1024):
    """For each access width, every lane-pair probe (lane 0 and one partner on
    the same bank position, at two row offsets), in a fixed order: width, then
    offset, then partner 1 .. 63 (see probes.hip)."""
    import ctypes
    lib = _probes(ctypes)
    lib.isp_lds_pair_probe.argtypes = [ctypes.c_int] * 5 + [ctypes.c_void_p, ctypes.c_void_p]
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    sink = torch.empty(cus * 64, dtype=torch.float32, device="cuda")
    n = 0
    for op in range(4):
        for off in LDS_PAIR_OFFSETS:
            for partner in range(1, 64):
                rc = lib.isp_lds_pair_probe(op, partner, off, cus, iters, sink.data_ptr(), stream_obj.cuda_stream)
                if rc != 0:
                    raise RuntimeError("isp_lds_pair_probe: hipError_t %d" % rc)
                n += 1
        torch.cuda.synchronize()
    return {"probes": n, "waves_per_probe": cus, "accesses_per_wave": iters}


LDS_STRIDE_GROUPS = (4, 8, 16)
LDS_STRIDES = (256, 512, 1024, 2048, 4096)
# Rows of 16 lanes at strides that are not multiples of 256 bytes, and
# shifted starts: (stride, offset) of the 16-lane groups, 16-byte reads.
LDS_ROW_CASES = [(st, off) for st in (256, 272, 288, 304, 320, 384, 512) for off in (0, 16, 128, 240)]


def _stride_cases():
    """(group, stride) pairs whose highest address fits the probe's 32 KB half."""
    return [(g, st) for g in LDS_STRIDE_GROUPS for st in LDS_STRIDES if (63 // g) * st + g * 16 <= 32768]


def lds_stride_probe(torch, stream_obj, iters=1024):
    """For each access width, group size and stride, one stride probe, in that
    order (see probes.hip)."""
    import ctypes
    lib = _probes(ctypes)
    lib.isp_lds_stride_probe.argtypes = [ctypes.c_int] * 6 + [ctypes.c_void_p, ctypes.c_void_p]
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    sink = torch.empty(cus * 64, dtype=torch.float32, device="cuda")
    n = 0

    def one(op, g, st, off):
        rc = lib.isp_lds_stride_probe(op, g, st, off, cus, iters, sink.data_ptr(), stream_obj.cuda_stream)
        if rc != 0:
            raise RuntimeError("isp_lds_stride_probe: hipError_t %d" % rc)

    for op in range(4):
        for g, st in _stride_cases():
            one(op, g, st, 0)
            n += 1
        torch.cuda.synchronize()
    for st, off in LDS_ROW_CASES:   # 16-byte reads of rows of 16 lanes, after the grid above
        one(0, 16, st, off)
        n += 1
    torch.cuda.synchronize()
    return {"probes": n, "waves_per_probe": cus, "accesses_per_wave": iters}


def pmc_lds_stride_summary(pmc_dir):
    """Markdown summary of a counter run of --lds-stride-probe: conflict cycles
    per instruction by access width, lane group and stride."""
    import csv
    import glob
    import re
    per = {}
    for f in sorted(glob.glob(os.path.join(pmc_dir, "**", "*counter_collection.csv"), recursive=True)):
        with open(f) as fh:
            for r in csv.DictReader(fh):
                m = re.search(r"isp_lds_stride_probe(?:ILi|<)(\d+)", r["Kernel_Name"])
                if not m:
                    continue
                d = per.setdefault((int(m.group(1)), int(r["Dispatch_Id"])), {})
                d[r["Counter_Name"]] = d.get(r["Counter_Name"], 0.0) + float(r["Counter_Value"])
    lines = ["# LDS bank conflicts against the distance between lane groups (gfx950, probe kernels)", "",
             "Commands (from the repository root, one MI355X; then the summary, on any machine):", "", "```",
             "rocprofv3 --pmc SQ_LDS_BANK_CONFLICT SQ_INSTS_LDS --output-format csv -d %s -o run -- \\" % pmc_dir,
             "    python3 bench.py --lds-stride-probe",
             "python3 bench.py --pmc-lds-stride-summary %s > profiles/lds_bank_strides.md" % pmc_dir,
             "```", "",
             "Lane l accesses (l mod G) x width + (l / G) x stride bytes: groups of G consecutive lanes",
             "cover contiguous bytes, the groups lie `stride` apart (`image_stencil_amd/probes/probes.hip`).",
             "Conflict cycles per wave instruction (SQ_LDS_BANK_CONFLICT / SQ_INSTS_LDS).", "",
             "| access | G | " + " | ".join("stride %d" % st for st in LDS_STRIDES) + " |",
             "|---|---|" + "---|" * len(LDS_STRIDES)]
    rows_disp = sorted(d for (o, d) in per if o == 0)[len(_stride_cases()):]
    for op in range(4):
        disp = sorted(d for (o, d) in per if o == op)[:len(_stride_cases())]
        order = _stride_cases()
        if len(disp) != len(order):
            lines.append("| `%s` | %d dispatches found, %d expected |" % (LDS_PROBE_OPS[op], len(disp), len(order)))
            continue
        vals = {}
        for d, key in zip(disp, order):
            v = per[(op, d)]
            vals[key] = v.get("SQ_LDS_BANK_CONFLICT", 0.0) / max(v.get("SQ_INSTS_LDS", 1.0), 1.0)
        for g in LDS_STRIDE_GROUPS:
            lines.append("| `%s` | %d | %s |" % (LDS_PROBE_OPS[op], g, " | ".join(
                "%.2f" % vals[(g, st)] if (g, st) in vals else "-" for st in LDS_STRIDES)))
    if len(rows_disp) == len(LDS_ROW_CASES):
        offs = sorted({o for _, o in LDS_ROW_CASES})
        lines += ["", "16-byte reads by rows of 16 lanes (G = 16) at strides that are not multiples of 256",
                  "bytes, all addresses moved up by an offset: conflict cycles per wave instruction.", "",
                  "| row stride (bytes) | " + " | ".join("offset %d" % o for o in offs) + " |",
                  "|---|" + "---|" * len(offs)]
        vals = {}
        for d, key in zip(rows_disp, LDS_ROW_CASES):
            v = per[(0, d)]
            vals[key] = v.get("SQ_LDS_BANK_CONFLICT", 0.0) / max(v.get("SQ_INSTS_LDS", 1.0), 1.0)
        for st in sorted({s_ for s_, _ in LDS_ROW_CASES}):
            lines.append("| %d | %s |" % (st, " | ".join("%.2f" % vals[(st, o)] for o in offs)))
    return "\n".join(lines) + "\n"


def pmc_lds_pair_summary(pmc_dir):
    """Markdown summary of a counter run of --lds-pair-probe: for each access
    width, the lanes served in the same LDS pass as lane 0."""
    import csv
    import glob
    import re
    per = {}   # (op, dispatch id) -> {counter: value}
    for f in sorted(glob.glob(os.path.join(pmc_dir, "**", "*counter_collection.csv"), recursive=True)):
        with open(f) as fh:
            for r in csv.DictReader(fh):
                name = r["Kernel_Name"]
                m = re.search(r"isp_lds_pair_probe(?:ILi|<)(\d+)", name)
                if not m:
                    continue
                key = (int(m.group(1)), int(r["Dispatch_Id"]))
                d = per.setdefault(key, {})
                d[r["Counter_Name"]] = d.get(r["Counter_Name"], 0.0) + float(r["Counter_Value"])
    lines = ["# Which lanes share an LDS pass with lane 0 (gfx950, probe kernels)", "",
             "Commands (from the repository root, one MI355X; then the summary, on any machine):", "", "```",
             "rocprofv3 --pmc SQ_LDS_BANK_CONFLICT SQ_INSTS_LDS --output-format csv -d %s -o run -- \\" % pmc_dir,
             "    python3 bench.py --lds-pair-probe",
             "python3 bench.py --pmc-lds-pair-summary %s > profiles/lds_lane_groups.md" % pmc_dir,
             "```", "",
             "Each probe: every lane of a wave accesses its own contiguous slot (lane x width, no",
             "conflict), except one partner lane, which accesses lane 0's bank position one row offset",
             "higher. The probe conflicts exactly when lane 0 and the partner are served in the same",
             "pass. Listed: the partners whose probe counted at least 0.5 conflict cycles per",
             "instruction (`image_stencil_amd/probes/probes.hip`).", "",
             "| access | row offset (bytes) | partners of lane 0 in its pass | conflict cycles / instr of those |",
             "|---|---|---|---|"]
    for op in range(4):
        disp = sorted(d for (o, d) in per if o == op)
        order = [(off, p) for off in LDS_PAIR_OFFSETS for p in range(1, 64)]
        if len(disp) != len(order):
            lines.append("| `%s` | | %d dispatches found, %d expected | |" % (LDS_PROBE_OPS[op], len(disp), len(order)))
            continue
        for off in LDS_PAIR_OFFSETS:
            hits = []
            for d, (o2, p) in zip(disp, order):
                if o2 != off:
                    continue
                v = per[(op, d)]
                c = v.get("SQ_LDS_BANK_CONFLICT", 0.0) / max(v.get("SQ_INSTS_LDS", 1.0), 1.0)
                if c >= 0.5:
                    hits.append((p, c))
            lines.append("| `%s` | %d | %s | %s |" % (LDS_PROBE_OPS[op], off, " ".join(str(p) for p, _ in hits) or "none",
                                                    " ".join("%.2f" % c for _, c in hits)))
    return "\n".join(lines) + "\n"


LDS_PROBE_OPS = {0: "ds_read_b128", 1: "ds_write_b128", 2: "ds_read_b64", 3: "ds_write_b64"}
LDS_PROBE_PATS = {0: "contiguous (lane x width)",
                  1: "all lanes in one 16-byte bank group, rows 128 B apart",
                  2: "8 consecutive lanes cover one 128-byte row; rows 256 B apart",
                  3: "16 consecutive lanes cover 256 bytes; lane pairs share a 16-byte group mod 128",
                  4: "fp16 layer operand pattern: 16 pixels x chunk, 128-byte XOR swizzle",
                  5: "every lane at one address (broadcast)",
                  6: "per 16 lanes: 15 on one address, 1 on another (rows 288 B apart)",
                  7: "per 16 lanes: 16 consecutive vectors (rows 288 B apart)"}


def pmc_lds_probe_summary(pmc_dir):
    """Markdown summary of a counter run of --lds-bank-probe: conflict and
    active LDS cycles per wave instruction of each access width and pattern."""
    import re
    tabs = {c: _counter_means(pmc_dir, c) for c in LDS_COUNTERS[:3]}
    rows = []
    for k, (v, n, full) in tabs["SQ_LDS_BANK_CONFLICT"].items():
        m = re.search(r"isp_lds_probe(?:ILi|<)(\d+)(?:ELi|, )(\d+)", full) or re.search(r"isp_lds_probe<(\d+), (\d+)>", k)
        if not m:
            continue
        op, pat = int(m.group(1)), int(m.group(2))
        insts = tabs["SQ_INSTS_LDS"].get(k, (0.0, 0, ""))[0]
        active = tabs["SQ_LDS_IDX_ACTIVE"].get(k, (0.0, 0, ""))[0]
        rows.append((op, pat, v / insts if insts else 0.0, active / insts if insts else 0.0, insts))
    lines = ["# LDS bank behaviour of gfx950, measured with probe kernels", "",
             "Commands (from the repository root, one MI355X; then the summary, on any machine):", "", "```",
             "rocprofv3 --pmc %s --output-format csv -d %s -o run -- \\" % (" ".join(LDS_COUNTERS[:3]), pmc_dir),
             "    python3 bench.py --lds-bank-probe",
             "python3 bench.py --pmc-lds-probe-summary %s > profiles/lds_bank_probe.md" % pmc_dir,
             "```", "",
             "One wave per CU repeats one LDS access 4096 times at a fixed address per lane",
             "(`image_stencil_amd/probes/probes.hip`). Per wave instruction, averaged over the chip:",
             "conflict = SQ_LDS_BANK_CONFLICT / SQ_INSTS_LDS, active = SQ_LDS_IDX_ACTIVE / SQ_INSTS_LDS",
             "(the LDS set-up writes and the final read are included in the counts, about 3% of the",
             "instructions).", "",
             "| access | address pattern | conflict cycles / instr | active cycles / instr |",
             "|---|---|---|---|"]
    for op, pat, c, a, _ in sorted(rows):
        lines.append("| `%s` | %s | %.2f | %.2f |" % (LDS_PROBE_OPS[op], LDS_PROBE_PATS[pat], c, a))
    return "\n".join(lines) + "\n"


def _cpu_baseline(synth, oracle, min_s=10.0, gpu_out=None, tau=None):
    """The oracle on full headline steps (3x3, 5x5 and 7x7 over 8192x8192),
    repeated until at least `min_s` seconds of oracle compute have run. With
    gpu_out ({R: the GPU's timed output}), the first step's oracle results
    also check those outputs (returned as the second value)."""
    import numpy as np
    data = []
    for R in (3, 5, 7):
        x, w = synth.large_image(R)
        data.append((R, x.astype(np.float64), w.astype(np.float64)))
        del x
    checks = {}
    total_bytes, secs, reps = 0.0, 0.0, 0
    while reps == 0 or secs < min_s:
        for R, xd, wd in data:
            t = time.perf_counter()
            ref, m = oracle.conv2d(xd, wd)
            secs += time.perf_counter() - t
            total_bytes += 4.0 * (2 * 8192 * 8192 + R * R)
            if reps == 0 and gpu_out is not None:
                checks["8192x8192 %dx%d" % (R, R)] = _oracle_check(gpu_out[R], ref, m, tau)
            del ref, m
        reps += 1
    base = {"value": round(total_bytes / secs / 1e9, 3), "unit": "GB/s", "cores": oracle.threads(),
            "kind": "oracle", "seconds": round(secs, 2), "steps": reps,
            "sample": "%d full steps: 8192x8192 fp32 image with 3x3, 5x5 and 7x7 filters, fp64 oracle "
                      "with error scale (compute only; input widening not timed)" % reps}
    base.update(_host_info(oracle))
    return base, checks


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--min-warm-s", type=float, default=0.3,
                    help="least warmup time per timed group, seconds (default %(default)s)")
    ap.add_argument("--no-cpu-baseline", action="store_true", help="skip the CPU oracle leg")
    ap.add_argument("--no-check", action="store_true",
                    help="skip the oracle check of the timed outputs (profiler runs)")
    ap.add_argument("--headline-only", action="store_true", help="skip the secondary workloads")
    ap.add_argument("--secondary", default=",".join(SECONDARY_GROUPS),
                    help="comma-separated secondary workloads to run (default: all of %(default)s); "
                         "the counter runs keep the pages' net apart, because its 64 -> 64 layer runs the "
                         "same kernel as the fp16 layer workload")
    ap.add_argument("--pmc-summary", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                    help="print the traffic summary of two rocprofv3 --pmc runs (FETCH_SIZE, WRITE_SIZE) "
                         "of this script and exit (no GPU needed)")
    ap.add_argument("--stats-summary", metavar="TRACE_DIR",
                    help="print the kernel-duration summary of a rocprofv3 --kernel-trace --stats run of "
                         "this script and exit (no GPU needed)")
    ap.add_argument("--pmc-mfma-summary", metavar="PMC_DIR",
                    help="print the arithmetic-counter summary of a rocprofv3 --pmc run and exit")
    ap.add_argument("--net-stats-summary", metavar="TRACE_DIR",
                    help="as --stats-summary, for a kernel-trace run of the pages' net alone")
    ap.add_argument("--lds-study", action="store_true",
                    help="time only the LDS-staged kernels (fp16 layer under each swizzle, fp32 layer, fused "
                         "chain), for a counter run of their bank conflicts")
    ap.add_argument("--pmc-lds-summary", metavar="PMC_DIR",
                    help="print the LDS counter summary of a rocprofv3 --pmc run of --lds-study and exit")
    ap.add_argument("--lds-bank-probe", action="store_true",
                    help="launch only the LDS bank probes (for a counter run) and exit")
    ap.add_argument("--pmc-lds-probe-summary", metavar="PMC_DIR",
                    help="print the summary of a rocprofv3 --pmc run of --lds-bank-probe and exit")
    ap.add_argument("--mix-study", action="store_true",
                    help="time the fp16 layer's instruction mix part by part and exit")
    ap.add_argument("--lds-rate-study", action="store_true",
                    help="time conflict-free LDS reads and writes per CU and exit")
    ap.add_argument("--mfma-chain-study", action="store_true",
                    help="time back-to-back fp16 MFMAs against accumulator chains per wave and exit")
    ap.add_argument("--clock-study", metavar="OUT_JSON",
                    help="launch only the clock study kernels (for a counter run) and exit")
    ap.add_argument("--pmc-clock-summary", metavar="PMC_DIR",
                    help="print the summary of a rocprofv3 --pmc run of --clock-study and exit")
    ap.add_argument("--lds-stride-probe", action="store_true",
                    help="launch only the LDS stride probes (for a counter run) and exit")
    ap.add_argument("--pmc-lds-stride-summary", metavar="PMC_DIR",
                    help="print the summary of a rocprofv3 --pmc run of --lds-stride-probe and exit")
    ap.add_argument("--lds-pair-probe", action="store_true",
                    help="launch only the LDS lane-pair probes (for a counter run) and exit")
    ap.add_argument("--pmc-lds-pair-summary", metavar="PMC_DIR",
                    help="print the summary of a rocprofv3 --pmc run of --lds-pair-probe and exit")
    args = ap.parse_args()
    globals()["MIN_WARM_S"] = args.min_warm_s
    if args.pmc_summary:
        sys.stdout.write(pmc_summary(*args.pmc_summary))
        return
    if args.stats_summary:
        sys.stdout.write(stats_summary(args.stats_summary))
        return
    if args.pmc_mfma_summary:
        sys.stdout.write(pmc_mfma_summary(args.pmc_mfma_summary))
        return
    if args.net_stats_summary:
        sys.stdout.write(stats_summary(args.net_stats_summary, net=True))
        return
    if args.pmc_lds_summary:
        sys.stdout.write(pmc_lds_summary(args.pmc_lds_summary))
        return
    if args.pmc_lds_probe_summary:
        sys.stdout.write(pmc_lds_probe_summary(args.pmc_lds_probe_summary))
        return
    if args.pmc_clock_summary:
        sys.stdout.write(pmc_clock_summary(args.pmc_clock_summary))
        return
    if args.pmc_lds_stride_summary:
        sys.stdout.write(pmc_lds_stride_summary(args.pmc_lds_stride_summary))
        return
    if args.pmc_lds_pair_summary:
        sys.stdout.write(pmc_lds_pair_summary(args.pmc_lds_pair_summary))
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path "
              "(run with --gpus 1)", file=sys.stderr)
        sys.exit(2)

    import torch
    import image_stencil_amd as isa
    import synth

    isa.load()
    torch.cuda.init()
    stream_obj = torch.cuda.current_stream()
    stream = stream_obj.cuda_stream

    if args.mix_study:
        print(json.dumps({"study": "mix", "results": mix_study(torch, stream_obj)}), flush=True)
        return
    if args.lds_rate_study:
        print(json.dumps({"study": "lds_rate", "results": lds_rate_study(torch, stream_obj)}), flush=True)
        return
    if args.mfma_chain_study:
        print(json.dumps({"study": "mfma_chains", "results": mfma_chain_study(torch, stream_obj)}), flush=True)
        return
    if args.clock_study:
        print(json.dumps({"study": "clock", **clock_study(torch, isa, synth, stream, stream_obj,
                                                           args.clock_study)}), flush=True)
        return
    if args.lds_stride_probe:
        print(json.dumps({"study": "lds_stride_probe", **lds_stride_probe(torch, stream_obj)}), flush=True)
        return
    if args.lds_pair_probe:
        print(json.dumps({"study": "lds_pair_probe", **lds_pair_probe(torch, stream_obj)}), flush=True)
        return
    if args.lds_bank_probe:
        print(json.dumps({"study": "lds_bank_probe", **lds_bank_probe(torch, stream_obj)}), flush=True)
        return
    if args.lds_study:
        print(json.dumps({"study": "lds", "results": lds_study(torch, isa, synth, stream, stream_obj, args.steps,
                                                                args.warmup)}), flush=True)
        return

    cases = _single_large_cases(torch, isa, synth, stream)
    ms_step, per, wall = _time_cases(torch, cases, args.steps, args.warmup, stream_obj)
    # After the timed region: one buffer set launched back to back (warm), and
    # the timed outputs copied to the host for the oracle check.
    warm = [_warm_ms(torch, c, args.steps, stream_obj) for c in cases]
    gpu_out = {c.R: c.keep[3].cpu().numpy() for c in cases} if not args.no_check else None
    step_bytes = sum(c.bytes for c in cases)
    step_flops = sum(c.flops for c in cases)
    value = step_bytes / (ms_step / 1e3) / 1e9
    kernels = []
    for c, ms, wms in zip(cases, per, warm):
        kernels.append({"case": c.name, "kernel": c.kernel, "ms": round(ms, 4),
                        "median_ms": round(c.median_ms, 4), "min_ms": round(c.min_ms, 4), "warm_ms": wms,
                        "gflops": round(c.flops / ms / 1e6, 1), "gbs": round(c.bytes / ms / 1e6, 1),
                        "roofline": _roofline(c, ms)})
    dom = max(range(len(cases)), key=lambda i: per[i])
    roof = dict(_roofline(cases[dom], per[dom]))
    roof["kernel"] = cases[dom].kernel + " (%s)" % cases[dom].name
    roof["launch_ms"] = round(per[dom], 4)

    out = {"metric": METRIC, "value": round(value, 1), "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
           "warmup": args.warmup, "ms_per_step": round(ms_step, 4), "higher_is_better": True,
           "scaling": "weak", "vs_baseline": None, "dtype": "f32", "data": "synthetic",
           "config": {"workload": "single-channel fp32 filtering, 8192x8192 image, 3x3 + 5x5 + 7x7 filters "
                                  "(one launch each per step)",
                      "image": [8192, 8192], "filters": [3, 5, 7], "parallelism": "none (1 GPU)"},
           "gflops": round(step_flops / ms_step / 1e6, 1), "hbm_frac": round(value / HBM_PEAK_GBS, 4),
           "roofline": roof, "kernels": kernels, "wall_s_timed": round(wall, 3)}
    for c in cases:
        c.keep = None
    torch.cuda.empty_cache()
    if not args.headline_only:
        groups = tuple(g for g in args.secondary.split(",") if g)
        for g in groups:
            if g not in SECONDARY_GROUPS:
                raise SystemExit("unknown secondary workload %r (choose from %s)" % (g, ", ".join(SECONDARY_GROUPS)))
        out["secondary"] = _secondary(torch, isa, synth, stream, stream_obj, args.steps, args.warmup, groups,
                                      check=not args.no_check)
        torch.cuda.empty_cache()

    out["copy_reference"] = _copy_reference(torch, stream_obj)
    out["mfma_reference"] = _mfma_reference(torch, stream_obj)
    if not args.no_cpu_baseline or not args.no_check:
        import oracle
        from tolerance import TAU_F32
        if not args.no_cpu_baseline:
            out["cpu_baseline"], checks = _cpu_baseline(synth, oracle, gpu_out=gpu_out, tau=TAU_F32)
        else:
            _, checks = _cpu_baseline(synth, oracle, min_s=0.0, gpu_out=gpu_out, tau=TAU_F32)
        if gpu_out is not None:
            for k in out["kernels"]:
                k["check"] = checks[k["case"]]
            out["check"] = _check_summary(out)
    print(json.dumps(out), flush=True)


def _check_summary(out):
    """Every oracle check of the run: the worst max err / bound and whether all passed."""
    found = [k["check"] for k in out.get("kernels", []) if "check" in k]
    for v in out.get("secondary", {}).values():
        if isinstance(v, dict) and "check" in v:
            found.append(v["check"])
    worst = max((c["max_err_over_bound"] for c in found), default=0.0)
    return {"outputs_checked": len(found), "worst_max_err_over_bound": worst,
            "all_passed": all(c["passed"] for c in found),
            "how": "after timing, one timed output of each workload is copied back and compared element by "
                   "element with the fp64 oracle: |y - y_oracle| <= tau * m"}


if __name__ == "__main__":
    main()
