"""Profiling driver and rocprofv3 result summarizer.

Run one kernel of the hot path a fixed number of times on a named synthetic
workload (for use under ``rocprofv3``)::

    python -m segment_autoregressive_dit_amd.profile_workload run --kernel attention --workload layer_bf16 --reps 5
    python -m segment_autoregressive_dit_amd.profile_workload run --kernel copy --bytes 1073741824
    python -m segment_autoregressive_dit_amd.profile_workload run --kernel qkv --workload layer_bf16

``--kernel copy`` runs a plain streaming kernel of known size (torch's elementwise
negation of a float32 buffer: reads N bytes, writes N bytes), the calibration for
the HBM byte counters FETCH_SIZE / WRITE_SIZE.

Summarize rocprofv3 SQLite results (``*_results.db``) into short text files::

    python -m segment_autoregressive_dit_amd.profile_workload trace DB --out FILE.md --command "..."
    python -m segment_autoregressive_dit_amd.profile_workload traffic --fetch DB --write DB \\
        --copy-fetch DB --copy-write DB --copy-bytes N --kernel attn_kernel --out FILE.json --command "..."
    python -m segment_autoregressive_dit_amd.profile_workload mfma DB --kernel attn_kernel \\
        --algorithmic-flop F --out FILE.json --command "..."

Counter figures are medians over the matching dispatches (a run's set-up
launches of the same kernel, such as an append workload's pre-fill, have other
sizes). ``calibration`` records the counters' scale for the plain copy and for
the global -> LDS stream (``run --kernel ldscopy``).

``traffic`` also reports the matched dispatches' median duration in the
counter runs and the HBM rate it implies (counter runs serialise kernels, so the
duration can read a little long). ``mfma`` reads a run of rocprofv3's derived
counters ``MfmaUtil`` (MFMA busy cycles over active cycles of all SIMDs, %) and
``MfmaFlopsBF16`` (bf16 MFMA operations x 512).
"""

import argparse
import collections
import hashlib
import json
import os
import re
import sqlite3
import statistics
import sys

HERE = os.path.dirname(os.path.abspath(__file__))


def source_digest(path):
    """sha256 of a source file's code with its comments and blank space taken out,
    so that a counter summary stays matched to a kernel whose comments alone
    changed (a change to the code itself changes the digest)."""
    text = open(path, encoding="utf-8").read()
    text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
    text = re.sub(r"//[^\n]*", " ", text)
    return hashlib.sha256(" ".join(text.split()).encode()).hexdigest()


def _dev(bits):
    import numpy as np
    import torch
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).cuda()


def cmd_run(a):
    import torch
    from segment_autoregressive_dit_amd import nomas, synth
    if a.kernel == "copy":
        src = torch.empty(a.bytes // 4, dtype=torch.float32, device="cuda").fill_(1.0)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        for _ in range(a.reps):
            torch.neg(src, out=dst)
        torch.cuda.synchronize()
        print(f"copy: {a.reps} x {a.bytes} bytes", file=sys.stderr)
        return
    if a.kernel == "ldscopy":
        src = torch.ones(a.bytes, dtype=torch.uint8, device="cuda")
        sink = nomas.nomas_calibrate_lds_stream(src)
        torch.cuda.synchronize()
        for _ in range(a.reps):
            nomas.nomas_calibrate_lds_stream(src, sink)
        torch.cuda.synchronize()
        print(f"ldscopy: {a.reps + 1} x {a.bytes} bytes", file=sys.stderr)
        return
    wl = synth.WORKLOADS[a.workload]
    H, D = wl.n_heads, wl.head_dim
    if a.kernel == "qkv":
        hidden = H * D
        x = _dev(synth.normal_bf16((wl.n_q, 1, hidden), 79, 0, 0, 0)[:, 0])
        w = _dev(synth.normal_bf16((3 * H * D, 1, hidden), 79, 0, 0, 1)[:, 0])
        table = nomas.nomas_rope3d_table(D, wl.t0, wl.seg_frames, wl.grid_h, wl.grid_w, wl.rope_split)
        y = torch.empty((wl.n_q, 3 * H * D), dtype=torch.bfloat16, device="cuda")
        torch.cuda.synchronize()
        for _ in range(a.reps):
            nomas.nomas_qkv_projection(x, w, H, D, n_video=wl.n_video, rope_table=table, qkv=y)
        torch.cuda.synchronize()
        print(f"qkv on {a.workload}: {a.reps} launches", file=sys.stderr)
        return
    cache = nomas.KVCache(H, D, wl.tpf, wl.capacity_frames, wl.kv_int8)
    kb, vb = synth.prefill_kv(wl)
    cache.nomas_kvcache_append(_dev(kb), _dev(vb), wl.cached_frames)
    q, k, v = (_dev(t) for t in synth.current_qkv(wl))
    out = torch.empty_like(q)
    ws = nomas.workspace_for(cache, wl.n_video, wl.n_text, a.splits)
    torch.cuda.synchronize()
    for _ in range(a.reps):
        if a.kernel == "attention":
            nomas.nomas_segment_attention(q, k, v, wl.n_video, wl.n_text, cache, out=out, n_splits=a.splits,
                                          workspace=ws)
        elif a.kernel == "rope":
            nomas.nomas_rope3d(q, k, wl.t0, wl.seg_frames, wl.grid_h, wl.grid_w, wl.rope_split, H, D)
        else:
            cache.nomas_kvcache_append(k, v, wl.seg_frames)
    torch.cuda.synchronize()
    print(f"{a.kernel} on {a.workload}: {a.reps} launches", file=sys.stderr)


def _kernel_rows(db):
    con = sqlite3.connect(db)
    cur = con.cursor()
    rows = cur.execute("select name, duration from kernels").fetchall()
    con.close()
    return rows


def cmd_trace(a):
    rows = _kernel_rows(a.db)
    agg = collections.OrderedDict()
    for name, dur in rows:
        s = agg.setdefault(name, [0, 0.0, float("inf"), 0.0])
        s[0] += 1
        s[1] += dur
        s[2] = min(s[2], dur)
        s[3] = max(s[3], dur)
    total = sum(s[1] for s in agg.values())
    lines = [f"# Kernel trace: {a.title}", "", "Command:", "", "```", a.command, "```", "",
             "| kernel | calls | total (us) | average (us) | min (us) | max (us) | % |",
             "|---|---|---|---|---|---|---|"]
    for name, (n, tot, mn, mx) in sorted(agg.items(), key=lambda kv: -kv[1][1]):
        short = name.split("(")[0].replace("void ", "")
        lines.append(f"| `{short}` | {n} | {tot / 1e3:.1f} | {tot / n / 1e3:.2f} | {mn / 1e3:.2f} | {mx / 1e3:.2f} | "
                     f"{100 * tot / total:.1f} |")
    text = "\n".join(lines) + "\n"
    with open(a.out, "w") as f:
        f.write(text)
    print(text)


def _per_dispatch(db, counter, kernel_substr):
    """{dispatch id: counter value summed over its instances} of the matching kernel."""
    con = sqlite3.connect(db)
    cur = con.cursor()
    rows = cur.execute("select kernel_name, dispatch_id, counter_name, value from counters_collection").fetchall()
    con.close()
    per = collections.defaultdict(float)
    for kn, did, cn, val in rows:
        if cn == counter and kernel_substr in kn:
            per[did] += val
    if not per:
        raise SystemExit(f"no {counter} values for a kernel matching {kernel_substr!r} in {db}")
    return per


def _counter_per_dispatch(db, counter, kernel_substr):
    """Median over the matching dispatches and their number. The median, not the
    mean: a run's set-up launches of the same kernel (the pre-fill append of an
    append workload, the fill that initialises the copy's source) have other
    sizes and would otherwise enter the figure."""
    vals = list(_per_dispatch(db, counter, kernel_substr).values())
    return statistics.median(vals), len(vals)


def _dispatch_duration_ns(db, counter, kernel_substr):
    con = sqlite3.connect(db)
    cur = con.cursor()
    rows = cur.execute("select dispatch_id, kernel_name, counter_name, duration from counters_collection").fetchall()
    con.close()
    per = {did: dur for did, kn, cn, dur in rows if cn == counter and kernel_substr in kn}
    return statistics.median(per.values()) if per else None


def cmd_traffic(a):
    fetch, nf = _counter_per_dispatch(a.fetch, "FETCH_SIZE", a.kernel)
    write, nw = _counter_per_dispatch(a.write, "WRITE_SIZE", a.kernel)
    cfetch, _ = _counter_per_dispatch(a.copy_fetch, "FETCH_SIZE", a.copy_kernel)
    cwrite, _ = _counter_per_dispatch(a.copy_write, "WRITE_SIZE", a.copy_kernel)
    # counters read KiB per dispatch; a plain copy of N bytes reads N and writes N,
    # so the calibration factors are (counter KiB * 1024) / N
    f_fac = cfetch * 1024 / a.copy_bytes
    w_fac = cwrite * 1024 / a.copy_bytes
    fetch_b = fetch * 1024 / f_fac
    write_b = write * 1024 / w_fac
    src = os.path.join(HERE, "csrc", a.source)
    out = {
        "kernel": a.kernel, "workload": a.workload,
        "fetch_kib_per_dispatch_raw": fetch, "write_kib_per_dispatch_raw": write,
        "dispatches": [nf, nw],
        "copy_bytes": a.copy_bytes, "copy_fetch_kib": cfetch, "copy_write_kib": cwrite,
        "fetch_calibration": f_fac, "write_calibration": w_fac,
        "hbm_read_bytes_per_launch": fetch_b, "hbm_write_bytes_per_launch": write_b,
        "hbm_bytes_per_launch": fetch_b + write_b,
        "source": a.source,
        "source_digest": source_digest(src),
        "command": a.command,
    }
    dur = _dispatch_duration_ns(a.fetch, "FETCH_SIZE", a.kernel)
    if dur:
        out["duration_us_in_counter_run"] = dur / 1e3
        out["hbm_gbps_counted"] = (fetch_b + write_b) / dur
        out["hbm_frac_of_8tbps_counted"] = (fetch_b + write_b) / dur / 8000.0
        if a.algorithmic_bytes:
            out["algorithmic_bytes_per_launch"] = a.algorithmic_bytes
            out["algorithmic_gbps"] = a.algorithmic_bytes / dur
    with open(a.out, "w") as f:
        json.dump(out, f, indent=1)
        f.write("\n")
    print(json.dumps(out, indent=1))


def cmd_mfma(a):
    util, nu = _counter_per_dispatch(a.db, "MfmaUtil", a.kernel)
    mflop, nf = _counter_per_dispatch(a.db, "MfmaFlopsBF16", a.kernel)
    dur = _dispatch_duration_ns(a.db, "MfmaUtil", a.kernel)
    src = os.path.join(HERE, "csrc", a.source)
    out = {
        "kernel": a.kernel, "workload": a.workload, "dispatches": [nu, nf],
        "mfma_util_pct": util,
        "mfma_bf16_flop_per_launch": mflop,
        "algorithmic_flop_per_launch": a.algorithmic_flop,
        "mfma_flop_over_algorithmic": mflop / a.algorithmic_flop if a.algorithmic_flop else None,
        "duration_us_in_counter_run": dur / 1e3 if dur else None,
        "algorithmic_tflops_in_counter_run": a.algorithmic_flop / dur / 1e3 if dur and a.algorithmic_flop else None,
        "source": a.source,
        "source_digest": source_digest(src),
        "command": a.command,
    }
    with open(a.out, "w") as f:
        json.dump(out, f, indent=1)
        f.write("\n")
    print(json.dumps(out, indent=1))


def cmd_calibration(a):
    """FETCH_SIZE / WRITE_SIZE scale for the two ways the library's kernels read
    memory: the plain copy (16-byte register loads and stores) and the
    global -> LDS stream (buffer_load ... lds, the attention and projection
    tiles), each over a known number of bytes."""
    out = {"bytes": a.bytes, "command": a.command, "patterns": {}}
    for name, db, counter, kern in (("copy_fetch", a.copy_fetch, "FETCH_SIZE", a.copy_kernel),
                                    ("copy_write", a.copy_write, "WRITE_SIZE", a.copy_kernel),
                                    ("lds_stream_fetch", a.lds_fetch, "FETCH_SIZE", "lds_stream")):
        per = _per_dispatch(db, counter, kern)
        out["patterns"][name] = {
            "kib_per_dispatch": [round(v, 3) for v in per.values()],
            "factor": statistics.median(per.values()) * 1024 / a.bytes,
        }
    with open(a.out, "w") as f:
        json.dump(out, f, indent=1)
        f.write("\n")
    print(json.dumps(out, indent=1))


def main(argv=None):
    p = argparse.ArgumentParser()
    sub = p.add_subparsers(dest="cmd", required=True)
    r = sub.add_parser("run")
    r.add_argument("--kernel", choices=["attention", "rope", "append", "qkv", "copy", "ldscopy"], required=True)
    r.add_argument("--workload", default="layer_bf16")
    r.add_argument("--reps", type=int, default=5)
    r.add_argument("--splits", type=int, default=0)
    r.add_argument("--bytes", type=int, default=1 << 30)
    t = sub.add_parser("trace")
    t.add_argument("db")
    t.add_argument("--out", required=True)
    t.add_argument("--title", default="")
    t.add_argument("--command", default="")
    f = sub.add_parser("traffic")
    for k in ("--fetch", "--write", "--copy-fetch", "--copy-write", "--out"):
        f.add_argument(k, required=True)
    f.add_argument("--copy-bytes", type=int, required=True)
    f.add_argument("--kernel", default="attn_kernel")
    f.add_argument("--copy-kernel", default="elementwise")
    f.add_argument("--workload", default="layer_bf16")
    f.add_argument("--source", default="attention.hip")
    f.add_argument("--command", default="")
    f.add_argument("--algorithmic-bytes", type=float, default=0.0)
    m = sub.add_parser("mfma")
    m.add_argument("db")
    m.add_argument("--out", required=True)
    m.add_argument("--kernel", default="attn_kernel")
    m.add_argument("--workload", default="layer_bf16")
    m.add_argument("--source", default="attention.hip")
    m.add_argument("--algorithmic-flop", type=float, default=0.0)
    m.add_argument("--command", default="")
    c = sub.add_parser("calibration")
    for k in ("--copy-fetch", "--copy-write", "--lds-fetch", "--out"):
        c.add_argument(k, required=True)
    c.add_argument("--bytes", type=int, required=True)
    c.add_argument("--copy-kernel", default="neg")
    c.add_argument("--command", default="")
    a = p.parse_args(argv)
    {"run": cmd_run, "trace": cmd_trace, "traffic": cmd_traffic, "mfma": cmd_mfma, "calibration": cmd_calibration}[a.cmd](a)


if __name__ == "__main__":
    main()
