"""Benchmark of the IceCache hot path on one MI355X.

Workload (default): a 36,000-token context for 32 layers x 8 KV heads (256
independent indexes), 4 query heads per KV head, d = 128, bf16 K/V, keys from
512-component Gaussian mixtures per head with a random rotation per head.
A timed step is one decode step of every layer: ``ice_decode`` (beam descent,
top-k pages, GQA union, page gather + sparse attention; one fused kernel) for
all 256 heads at a 256-token budget. The separate ``ice_select`` and
``ice_attend`` kernels, the index build (keys/s) and the insert of one token
per head are timed separately and reported beside it.

Prints ONE JSON line (see the fields below). ``--gpus N`` with N > 1 exits:
the library runs on one GPU and no multi-GPU figure is produced.
"""
from __future__ import annotations

import argparse
import csv
import glob
import hashlib
import json
import math
import os
import platform
import re
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "decode steps/s (select+gather+attend) & index keys/s at 36k ctx; % roofline"
HBM_PEAK_GBS = 8000.0
BF16_PEAK_TFLOPS = 2500.0

WORKLOADS = {
    # name: (layers*kv_heads, G, N, d, dtype, centres, rotate, description)
    "ctx36k": (256, 4, 36000, 128, "bf16", 512, True,
               "36k-token context, 32 layers x 8 KV heads x 4 query heads, d=128 bf16, 512-component "
               "Gaussian-mixture keys with per-head rotations"),
    "llama-layer": (8, 4, 32768, 128, "bf16", 512, False,
                    "one 32k-token layer, 8 KV heads x 4 query heads, d=128 bf16, 512-component mixtures"),
    "tiny": (1, 1, 2048, 64, "f32", 32, False, "1 head, 2048 tokens, d=64 fp32, 32-component mixture"),
}


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="ctx36k", choices=sorted(WORKLOADS))
    ap.add_argument("--budget", type=int, default=256)
    ap.add_argument("--budgets", default="", help="extra budgets to time beside --budget, e.g. 64,128")
    ap.add_argument("--builds", type=int, default=3)
    ap.add_argument("--cpu-heads", type=int, default=16, help="heads in the oracle's timed sample")
    ap.add_argument("--no-cpu", action="store_true", help="skip the oracle baseline")
    ap.add_argument("--no-host-pool", action="store_true", help="skip the host-pool mode measurement")
    ap.add_argument("--no-pipeline", action="store_true", help="skip the per-layer build pipeline measurement")
    ap.add_argument("--resident", type=int, default=68,
                    help="resident (sink + window) tokens per head for the resident-token leg; 0 skips it")
    ap.add_argument("--drift-steps", type=int, default=4096,
                    help="generated steps of the split-reading recall comparison (0 skips it)")
    ap.add_argument("--pdci-tokens", type=int, default=100000,
                    help="context of the P-DCI against exact-parent comparison (0 skips it)")
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--summarize", nargs="+", metavar="CSV",
                    help="print a markdown summary of rocprofv3 output instead of benchmarking: one "
                         "*_kernel_stats.csv, or a FETCH_SIZE and a WRITE_SIZE *_counter_collection.csv")
    ap.add_argument("--command", default="", help="the command that produced the CSVs (for --summarize)")
    ap.add_argument("--copy-mib", type=int, default=0,
                    help="also run one plain device copy of this many MiB (a known-size kernel that "
                         "calibrates hardware byte counters)")
    return ap.parse_args()


# ---- hardware byte counters ----------------------------------------------
# Sources each kernel is built from: a recorded counter reading is valid only
# while these are unchanged.
KERNEL_SOURCES = {
    "k_decode": ["k_select.hip", "attend_mfma.h", "ice_common.h", "ice_launch.h"],
    "k_select": ["k_select.hip", "attend_mfma.h", "ice_common.h", "ice_launch.h"],
    "k_attend": ["k_attend.hip", "attend_mfma.h", "ice_common.h", "ice_launch.h"],
}
CSRC = os.path.join(ROOT, "ann_retrieval_amd", "csrc")
PROFILES = os.path.join(ROOT, "profiles")


def source_hash(kernel):
    h = hashlib.sha256()
    for f in KERNEL_SOURCES[kernel]:
        with open(os.path.join(CSRC, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def recorded_traffic(kernel, workload):
    """HBM bytes per launch recorded under profiles/ for this kernel and
    workload, or None if none was recorded for the current sources."""
    want = source_hash(kernel)
    for path in sorted(glob.glob(os.path.join(PROFILES, "*.md"))):
        with open(path) as f:
            for line in f:
                m = re.match(r"traffic (\S+) workload=(\S+) bytes_per_launch=(\d+) source=(\w+)", line.strip())
                if m and m.group(1) == kernel and m.group(2) == workload and m.group(4) == want:
                    return int(m.group(3))
    return None


def short_name(name):
    name = name.replace("(anonymous namespace)::", "")
    m = re.search(r"(k_\w+)(<[^()]*>)?\(", name)
    if m and "ice::" in name:
        return m.group(1) + (m.group(2) or "")
    return name.split("(")[0][-70:]


def summarize(paths, command, copy_mib, workload):
    """Markdown summary of rocprofv3 CSV output (kernel stats, or counters)."""
    out = [f"Command: `{command}`", ""]
    if len(paths) == 1 and "counter_collection" in paths[0]:
        print("\n".join(out + summarize_mfma(paths[0])))
        return
    if len(paths) == 1:
        rows = list(csv.DictReader(open(paths[0])))
        out += ["| Kernel | Calls | Average (us) | Min (us) | Max (us) | Time share (%) |", "|---|---|---|---|---|---|"]
        # the 25 longest, then every other kernel of the library
        for r in rows[:25] + [r for r in rows[25:] if short_name(r["Name"]).startswith("k_")]:
            out.append(f"| `{short_name(r['Name'])}` | {r['Calls']} | {float(r['AverageNs'])/1e3:.2f} | "
                       f"{float(r['MinNs'])/1e3:.2f} | {float(r['MaxNs'])/1e3:.2f} | {float(r['Percentage']):.2f} |")
        print("\n".join(out))
        return
    per = {}
    factor = {}
    known = copy_mib * 1024.0           # KiB moved by each calibration copy
    for path in paths:
        cal = []
        for r in csv.DictReader(open(path)):
            c, v, k = r["Counter_Name"], float(r["Counter_Value"]), r["Kernel_Name"]
            if "copyBuffer" in k or "OnSelf_add" in k:    # the runtime copy and x + 0 of --copy-mib
                cal.append((v, k))
            per.setdefault((short_name(k), c), []).append(v)
        big = [v for v, _ in cal if v > 0.25 * known]
        factor[c] = known / (sum(big) / len(big))
        out.append(f"- {c}: calibration copies of {copy_mib} MiB read {', '.join(f'{v:.0f}' for v in big)} KiB "
                   f"-> factor {factor[c]:.3f}")
    out += ["", "| Kernel | Dispatches | FETCH_SIZE (KiB) | WRITE_SIZE (KiB) | HBM bytes / dispatch (scaled) |",
            "|---|---|---|---|---|"]
    names = sorted({k for k, _ in per if k.startswith("k_")})
    lines = []
    for k in names:
        f = per.get((k, "FETCH_SIZE"), [0.0])
        w = per.get((k, "WRITE_SIZE"), [0.0])
        fa, wa = sum(f) / len(f), sum(w) / len(w)
        tot = (fa * factor.get("FETCH_SIZE", 1.0) + wa * factor.get("WRITE_SIZE", 1.0)) * 1024.0
        out.append(f"| `{k}` | {len(f)} | {fa:.1f} | {wa:.1f} | {tot:.0f} |")
        base = k.split("<")[0]
        if base in KERNEL_SOURCES:
            lines.append(f"traffic {base} workload={workload} bytes_per_launch={tot:.0f} source={source_hash(base)}")
    out += ["", "Recorded for bench.py (the kernel's sources must still hash the same):", "", "```"] + lines + ["```"]
    print("\n".join(out))


def summarize_mfma(path):
    """Matrix-core use per dispatch of the library's MFMA kernels from one
    counter run of SQ_VALU_MFMA_BUSY_CYCLES, SQ_INSTS_MFMA, SQ_INSTS_VALU and
    GRBM_GUI_ACTIVE. GRBM_GUI_ACTIVE is summed over the 8 XCDs, so the
    dispatch's busy window is GRBM_GUI_ACTIVE / 8 GPU cycles; utilisation =
    MFMA busy cycles / (window x 1024 SIMDs)."""
    disp = {}
    for r in csv.DictReader(open(path)):
        k = short_name(r["Kernel_Name"])
        if not k.startswith("k_"):
            continue
        key = (k, r.get("Dispatch_Id", r.get("Correlation_Id", "")))
        disp.setdefault(key, {})[r["Counter_Name"]] = disp.setdefault(key, {}).get(r["Counter_Name"], 0.0) + \
            float(r["Counter_Value"])
    out = ["| Kernel | Dispatch | GPU cycles (window) | MFMA instructions | VALU instructions | VALU / MFMA | "
           "MFMA busy (% of 1024 SIMDs) |", "|---|---|---|---|---|---|---|"]
    for (k, d), c in sorted(disp.items(), key=lambda x: (x[0][0], int(x[0][1]) if str(x[0][1]).isdigit() else 0)):
        mf = c.get("SQ_INSTS_MFMA", 0.0)
        if mf <= 0:
            continue
        win = c.get("GRBM_GUI_ACTIVE", 0.0) / 8.0
        busy = c.get("SQ_VALU_MFMA_BUSY_CYCLES", 0.0)
        util = 100.0 * busy / (win * 1024) if win else float("nan")
        va = c.get("SQ_INSTS_VALU", 0.0)
        out.append(f"| `{k}` | {d} | {win:.0f} | {mf:.0f} | {va:.0f} | {va / mf:.1f} | {util:.1f} |")
    return out


def algorithmic_bytes(ix, trace, uni_n, n_uni, d, elt, G):
    """Bytes the method itself must move for one decode step, from the run's
    own selections. Per head: select reads the top-level keys, the keys of
    the unique level-1 candidates, the keys of the valid rows of the unique
    candidate pages and their list entries; attend reads the K and V rows of
    the union pages. The fused step reads every key once (the union pages'
    keys are among the candidates), then the union's V rows. Q in and O, lse
    out are counted where they move."""
    H = trace.shape[0]
    sel_b = kv_b = v_b = ent_b = 0
    for h in range(H):
        m = ix.meta[h]
        Lt = m["L_top"]
        rows_top = m["n_top"] if Lt >= 1 else 0
        c1_rows = blocks = pages = page_rows = 0
        if Lt == 2:
            kept2 = np.unique(trace[h, :, 0][trace[h, :, 0] >= 0])
            kept1 = np.unique(trace[h, :, 1][trace[h, :, 1] >= 0])
            c1_rows = int(m["kids1"][kept2].sum())
            blocks = int(m["blocks1"][kept2].sum())
        elif Lt == 1:
            kept1 = np.unique(trace[h, :, 0][trace[h, :, 0] >= 0])
        else:
            kept1 = None
        if kept1 is not None:
            pages = int(m["npages0"][kept1].sum())
            page_rows = int(m["rows0"][kept1].sum())
        else:
            pages, page_rows = m["P0"], m["n"]
        sel_b += (rows_top + c1_rows + page_rows) * d * elt + blocks * (16 * 4 + 8) + pages * 8
        u = uni_n[h][: n_uni[h]]
        rows = int(m["cnt0"][u].sum())
        kv_b += 2 * rows * d * elt
        v_b += rows * d * elt
        ent_b += len(u) * 8
    q = H * G * d * elt
    out = H * G * d * 4 + H * G * 4
    return dict(select=sel_b + q, attend=kv_b + ent_b + q + out, decode=sel_b + v_b + ent_b + q + out)


def head_meta(ix, H, cap):
    """Per-head owner -> (children, blocks, pages, rows) maps for the byte count."""
    from ann_retrieval_amd import _lib as L
    meta = []
    for h in range(H):
        st = ix.stats(h)
        m = dict(L_top=st["top_level"], n_top=st["n_top"], n=st["n_tokens"], P0=st["n_pages"][0])
        own0 = ix.export(h, L.ICE_EXP_PAGE_OWNER, 0)[: st["n_pages"][0]]
        cnt0 = ix.export(h, L.ICE_EXP_PAGE_CNT, 0)[: st["n_pages"][0]]
        m["cnt0"] = cnt0
        ok = own0 >= 0
        m["npages0"] = np.bincount(own0[ok], minlength=cap + 1)
        m["rows0"] = np.bincount(own0[ok], weights=cnt0[ok], minlength=cap + 1).astype(np.int64)
        if st["top_level"] >= 2:
            P1 = st["n_pages"][1]
            own1 = ix.export(h, L.ICE_EXP_PAGE_OWNER, 1)[:P1]
            cnt1 = ix.export(h, L.ICE_EXP_PAGE_CNT, 1)[:P1]
            m["kids1"] = np.bincount(own1, weights=cnt1, minlength=cap + 1).astype(np.int64)
            m["blocks1"] = np.bincount(own1, minlength=cap + 1)
        meta.append(m)
    ix.meta = meta


def time_pipeline(ix, w, a, H, N, heads_per_layer=8):
    """Prefill with the index built one layer at a time beside the model's
    work (the pages' pipeline of index construction and computation). The
    model's work per layer is stood in for by the three MLP GEMMs of a
    Llama-3.1-8B layer over the prompt (bf16, 4096 x 14336, N rows), about
    12.7 TFLOP at 36k tokens. Serial: every layer's GEMMs, then its build, on
    one stream. Pipelined: the build of layer i runs on a second stream once
    layer i's GEMMs are done, while layer i+1's GEMMs proceed. The index is
    the same either way (a build of head ranges equals a build of all heads)."""
    import torch
    n_layers = H // heads_per_layer
    dev = w.K.device
    gen = torch.Generator(device=dev)
    gen.manual_seed(a.seed + 7)
    dm, df = 4096, 14336
    X = (torch.randn(N, dm, device=dev, generator=gen) * 0.05).to(torch.bfloat16)
    Wg = (torch.randn(dm, df, device=dev, generator=gen) * 0.02).to(torch.bfloat16)
    Wu = (torch.randn(dm, df, device=dev, generator=gen) * 0.02).to(torch.bfloat16)
    Wd = (torch.randn(df, dm, device=dev, generator=gen) * 0.02).to(torch.bfloat16)

    def model_layer():
        h = torch.nn.functional.silu(X @ Wg) * (X @ Wu)
        return h @ Wd

    def build_layer(i, stream=None):
        h0 = i * heads_per_layer
        ix.ice_build_heads(w.K[h0:h0 + heads_per_layer], w.V[h0:h0 + heads_per_layer], h0, stream=stream)

    ev = lambda: torch.cuda.Event(enable_timing=True)
    model_layer()
    build_layer(0)
    torch.cuda.synchronize()
    e0, e1 = ev(), ev()
    e0.record()
    for i in range(n_layers):
        model_layer()
    e1.record()
    torch.cuda.synchronize()
    model_ms = e0.elapsed_time(e1)
    e0.record()
    for i in range(n_layers):
        build_layer(i)
    e1.record()
    torch.cuda.synchronize()
    build_ms = e0.elapsed_time(e1)
    e0.record()
    for i in range(n_layers):
        model_layer()
        build_layer(i)
    e1.record()
    torch.cuda.synchronize()
    serial_ms = e0.elapsed_time(e1)
    side = torch.cuda.Stream(device=dev)
    main = torch.cuda.current_stream(dev)
    e0.record()
    for i in range(n_layers):
        model_layer()
        done = ev()
        done.record(main)
        side.wait_event(done)
        build_layer(i, stream=side)
    end_side = ev()
    end_side.record(side)
    main.wait_event(end_side)
    e1.record()
    torch.cuda.synchronize()
    pipe_ms = e0.elapsed_time(e1)
    del X, Wg, Wu, Wd
    torch.cuda.empty_cache()
    hidden = (serial_ms - pipe_ms) / build_ms if build_ms > 0 else 0.0
    print(f"[bench] prefill pipeline, {n_layers} layers: model {model_ms:.1f} ms, per-layer builds {build_ms:.1f} ms, "
          f"serial {serial_ms:.1f} ms, pipelined {pipe_ms:.1f} ms ({hidden * 100:.0f}% of the build hidden)",
          file=sys.stderr, flush=True)
    return {"layers": n_layers, "heads_per_layer": heads_per_layer, "model_ms": model_ms,
            "per_layer_build_ms": build_ms, "serial_ms": serial_ms, "pipelined_ms": pipe_ms,
            "build_hidden_frac": hidden,
            "model_stand_in": "Llama-3.1-8B MLP GEMMs (bf16, 4096 x 14336) over the prompt, per layer"}


def time_reuse(ix, w, a, H, N, heads_per_layer=8):
    """Index build with inter-layer reuse: every odd layer takes the layout of
    the layer before it (its own rows and lift, no parent search), against
    building every layer. Median of 3 runs each."""
    import torch
    n_layers = H // heads_per_layer
    hp = heads_per_layer

    def run(reuse):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record()
        for i in range(n_layers):
            h0 = i * hp
            if reuse and i % 2 == 1:
                ix.ice_build_reuse(w.K[h0:h0 + hp], w.V[h0:h0 + hp], h0, h0 - hp)
            else:
                ix.ice_build_heads(w.K[h0:h0 + hp], w.V[h0:h0 + hp], h0)
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1)

    run(True)
    per_layer = sorted(run(False) for _ in range(3))[1]
    reuse = sorted(run(True) for _ in range(3))[1]
    print(f"[bench] per-layer builds {per_layer:.1f} ms; with every odd layer reusing the one before {reuse:.1f} ms",
          file=sys.stderr, flush=True)
    return {"layers": n_layers, "per_layer_build_ms": per_layer, "reuse_every_other_layer_ms": reuse,
            "index_keys_per_s_with_reuse": H * N / (reuse / 1000.0)}


def selection_recall(ix, Q, KT, budget):
    """Share of each query head's exact top-`budget` keys by q.k (Q [H, G, d],
    KT [H, d, n] fp32) that lie in the pages ice_select picks for it."""
    import torch
    from ann_retrieval_amd import _lib as L
    H, G = Q.shape[0], Q.shape[1]
    sel, _, _ = ix.ice_select(Q, budget, budget // 16)
    top = torch.topk(torch.bmm(Q.float(), KT), budget, dim=-1).indices
    hit = 0
    for h in range(H):
        tok = torch.from_numpy(ix.export(h, L.ICE_EXP_PAGE_TOK, 0).reshape(-1, 16)).to(Q.device)
        stok = tok[sel[h].long().clamp(min=0)].reshape(G, -1)
        stok = torch.where((sel[h] >= 0).repeat_interleave(16, dim=1), stok, -1)
        for g in range(G):
            hit += int(torch.isin(top[h, g], stok[g]).sum())
    return hit / (H * G * budget)


def pdci_leg(a):
    """Index build with P-DCI parents against the exact MFMA search at a
    100k-token context (8 KV heads x 4 query heads, d=128 bf16, 1024-centre
    mixture keys with rotations): build time, the share of level-0 parents
    equal to the exact ones, and the selection's token recall at a 64-token
    budget over 16 random decode queries per query head, per P-DCI setting
    (m composite indices of l simple indices, visits, candidates)."""
    import torch
    from ann_retrieval_amd import _lib as L
    from ann_retrieval_amd import synth
    from ann_retrieval_amd.api import IceIndex
    H, G, N, d, budget = 8, 4, a.pdci_tokens, 128, 64
    w, gen = synth.clustered_kv(H, N, d, 1024, "bf16", a.seed + 11, device="cpu", rotate=True)
    K, V = w.K.cuda(), w.V.cuda()
    KT = K.float().transpose(1, 2).contiguous()
    Qs = [synth.decode_queries(w, G, gen).cuda() for _ in range(16)]
    ix = IceIndex(H, G, d, "bf16", N, 3, 4, a.seed + 11, max_budget=budget)

    def timed(fn):
        ms = []
        for _ in range(3):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            torch.cuda.synchronize()
            e0.record()
            fn()
            e1.record()
            torch.cuda.synchronize()
            ms.append(e0.elapsed_time(e1))
        return sorted(ms)[1]

    def parents():
        return [ix.export(h, L.ICE_EXP_PARENT, 0)[:N].copy() for h in range(H)]

    exact_ms = timed(lambda: ix.ice_build(K, V))
    ref = parents()
    out = {"workload": f"{N}-token context, 8 KV heads x 4 query heads, d=128 bf16, 1024-centre mixtures",
           "exact": {"build_ms": exact_ms, "parent_agreement": 1.0,
                     "recall_at_64": float(np.mean([selection_recall(ix, Q, KT, budget) for Q in Qs]))}}
    print(f"[bench] exact parents: build {exact_ms:.2f} ms, recall@64 {out['exact']['recall_at_64']:.4f}",
          file=sys.stderr, flush=True)
    for m, l, visits, cands in [(2, 2, 64, 8), (4, 2, 256, 32), (4, 2, 1024, 64)]:
        dirs = synth.projection_dirs(m * l, d, a.seed + 12, device="cuda")
        ms = timed(lambda: ix.ice_build_pdci(K, V, dirs, m, l, visits, cands))
        got = parents()
        lev0 = [ix.export(h, L.ICE_EXP_LEVEL, np_dtype=np.int8)[:N] == 0 for h in range(H)]
        agree = float(np.mean(np.concatenate([(got[h] == ref[h])[lev0[h]] for h in range(H)])))
        rec = float(np.mean([selection_recall(ix, Q, KT, budget) for Q in Qs]))
        key = f"m{m}_l{l}_v{visits}_c{cands}"
        out[key] = {"build_ms": ms, "parent_agreement": agree, "recall_at_64": rec}
        print(f"[bench] P-DCI {key}: build {ms:.2f} ms, parents equal to the exact ones {agree:.4f}, "
              f"recall@64 {rec:.4f}", file=sys.stderr, flush=True)
    del ix
    return out


def split_drift(a):
    """Long generation under both split readings, on the same inputs: one
    Qwen3-32B-shaped layer (8 KV heads x 8 query heads, d=128 bf16, 512-centre
    mixture keys with per-head rotations), an 8192-token prompt, then
    ``a.drift_steps`` steps that each insert one key/value per head, queries
    walking between mixture centres. Every 256 steps, the selection's token
    recall at a 256-token budget: the share of each query head's exact
    top-256 keys by q.k that lie in its selected pages (mean over the 64 query
    heads). Also the mean time of one insert call (8 heads) per split reading."""
    import torch
    from ann_retrieval_amd import synth
    from ann_retrieval_amd.api import IceIndex
    H, G, N, d, budget, steps = 8, 8, 8192, 128, 256, a.drift_steps
    w, gen = synth.clustered_kv(H, N, d, 512, "bf16", a.seed + 7, device="cpu", rotate=True)
    walk = synth.QueryWalk(w, G, gen, seg=64)
    seq = [walk.step() for _ in range(steps)]
    Q = torch.stack([x[0] for x in seq]).cuda()
    Kn = torch.stack([x[1] for x in seq]).cuda()
    Vn = torch.stack([x[2] for x in seq]).cuda()
    # every key, transposed once: [H, d, N + steps] fp32
    KT = torch.cat([w.K.cuda(), Kn[:, :, 0].transpose(0, 1)], 1).float().transpose(1, 2).contiguous()
    marks = sorted(set(range(0, steps, 256)) | {steps - 1})
    out = {"workload": (f"one layer of 8 KV heads x 8 query heads, d=128 bf16, {N}-token prompt, {steps} steps "
                        f"inserting one token per head; recall at a {budget}-token budget every 256 steps")}
    for mode in ("append", "resort"):
        ix = IceIndex(H, G, d, "bf16", N + steps, 3, 4, a.seed + 7, max_budget=budget, resort=mode == "resort")
        ix.ice_build(w.K.cuda(), w.V.cuda())
        torch.cuda.synchronize()
        recall, ev = [], []
        # the inserts between two recall points are timed as one run, queued by
        # the host behind a short spin so that the figure is GPU time
        for a_, b_ in zip(marks, marks[1:] + [steps]):
            recall.append(selection_recall(ix, Q[a_], KT[:, :, :N + a_], budget))
            if b_ <= a_:
                continue
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            torch.cuda._sleep(int(5e7))
            e0.record()
            for s in range(a_, b_):
                ix.ice_insert(Kn[s], Vn[s])
            e1.record()
            ev.append((e0, e1))
        torch.cuda.synchronize()
        ins_us = 1000.0 * sum(x.elapsed_time(y) for x, y in ev) / steps
        splits = sum(ix.stats(h)["splits"] for h in range(H))
        out[mode] = {"recall": [round(r, 4) for r in recall], "recall_at_steps": marks, "insert_us": ins_us,
                     "splits": splits}
        print(f"[bench] {mode} split: recall {recall[0]:.4f} at step 0, {recall[-1]:.4f} at step {steps - 1}, "
              f"mean {np.mean(recall):.4f}; insert {ins_us:.1f} us/step; {splits} splits", file=sys.stderr, flush=True)
        del ix
    return out


def time_host_pool(w, Qs, a, H, G, N, d, dtype, budget, dev_attend_ms, n_ins):
    """Host-pool mode on the same workload: V pages in pinned host memory, each
    step gathers the union's V pages over the host link before attending.
    Bound by the link, not HBM, so it is reported beside the roofline, not in
    it. The gather's own time is estimated as the host-pool attend (gather +
    attention) minus the device-pool attend."""
    import torch
    from ann_retrieval_amd.api import IceIndex
    beam = budget // 16
    t0 = time.perf_counter()
    ix = IceIndex(H, G, d, dtype, N + n_ins, seed=a.seed, max_budget=budget, device=w.K.device, host_pool=True)
    alloc_s = time.perf_counter() - t0
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record()
    ix.ice_build(w.K, w.V)
    e1.record()
    torch.cuda.synchronize()
    build_ms = e0.elapsed_time(e1)
    for s in range(min(a.warmup, 3)):
        ix.ice_decode(Qs[s], budget, beam)
    torch.cuda.synchronize()
    steps = a.steps
    g0, g1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda._sleep(int(5e7))
    g0.record()
    for s in range(steps):
        ix.ice_decode(Qs[a.warmup + s], budget, beam)
    g1.record()
    torch.cuda.synchronize()
    ms_step = g0.elapsed_time(g1) / steps
    unis = [ix.ice_select(Qs[a.warmup + s], budget, beam)[1:] for s in range(steps)]
    torch.cuda.synchronize()
    pages = float(np.mean([float(n.sum()) for _, n in unis]))
    a0, a1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda._sleep(int(5e7))
    a0.record()
    for s in range(steps):
        ix.ice_attend(Qs[a.warmup + s], *unis[s])
    a1.record()
    torch.cuda.synchronize()
    att_ms = a0.elapsed_time(a1) / steps
    elt = 2 if dtype == "bf16" else 4
    gbytes = pages * 16 * d * elt
    gather_ms = max(att_ms - dev_attend_ms, 1e-6)
    out = dict(ms_per_step=round(ms_step, 6), steps_per_s=round(1000.0 / ms_step, 3),
               attend_with_gather_ms=round(att_ms, 6), gather_ms_est=round(gather_ms, 6),
               gather_bytes=gbytes, link_gbs_est=round(gbytes / gather_ms / 1e6, 3),
               build_ms=round(build_ms, 3), pool_bytes=ix.pool.nbytes, pool_alloc_s=round(alloc_s, 3))
    print(f"[bench] host pool T={budget}: {ms_step*1000:.1f} us/step; gather of {gbytes/1e6:.1f} MB about "
          f"{gather_ms*1000:.1f} us ({out['link_gbs_est']:.1f} GB/s); build {build_ms:.1f} ms",
          file=sys.stderr, flush=True)
    del ix
    return out


def cpu_baseline(w, Qs, budget, beam, heads, seed):
    """The fp64 oracle as it stands, on the host cores, on a bounded sample:
    its own index build of `heads` heads, then select + attend of those heads
    for every query of the first steps. Scaled to all heads of the workload."""
    import threadpoolctl
    from oracle import icecache as ic
    K = w.K[:len(heads)].float().cpu().double().numpy()
    V = w.V[:len(heads)].float().cpu().double().numpy()
    t0 = time.perf_counter()
    refs = [ic.build_head(K[i], V[i], h, seed) for i, h in enumerate(heads)]
    t_build = time.perf_counter() - t0
    n_steps = len(Qs)
    t0 = time.perf_counter()
    for s in range(n_steps):
        Q = Qs[s][:len(heads)].float().cpu().double().numpy()
        for i, ref in enumerate(refs):
            sels = [ic.select(ref, Q[i, g], budget, beam)["sel"] for g in range(Q.shape[1])]
            uni = ic.gqa_union(sels)
            for g in range(Q.shape[1]):
                ic.attend(ref, Q[i, g], uni, 1.0 / math.sqrt(Q.shape[2]))
    t_dec = (time.perf_counter() - t0) / n_steps
    info = threadpoolctl.threadpool_info()
    threads = max([i.get("num_threads", 1) for i in info] + [1])
    return t_build, t_dec, threads


def main():
    a = parse()
    if a.summarize:
        summarize(a.summarize, a.command, a.copy_mib or 1024, a.workload)
        return
    if a.gpus != 1:
        print(json.dumps({"error": "this library runs on one GPU; no multi-GPU figure is produced",
                          "n_gpus": a.gpus}))
        sys.exit(2)
    import torch
    from ann_retrieval_amd import synth
    from ann_retrieval_amd.api import IceIndex

    H, G, N, d, dtype, C, rotate, desc = WORKLOADS[a.workload]
    budgets = [int(b) for b in a.budgets.split(",") if b]
    if a.budget not in budgets:
        budgets.append(a.budget)
    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    print(f"[bench] workload={a.workload} H={H} G={G} N={N} d={d} {dtype}", file=sys.stderr, flush=True)
    w, gen = synth.clustered_kv(H, N, d, C, dtype, a.seed, device=dev, rotate=rotate)
    elt = 2 if dtype == "bf16" else 4
    n_ins = a.steps + a.warmup
    ix = IceIndex(H, G, d, dtype, N + n_ins, seed=a.seed, max_budget=max(budgets), device=dev,
                  resident=max(a.resident, 0))

    # ---- index build: median of a few full builds
    bt = []
    for i in range(a.builds + 1):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record()
        ix.ice_build(w.K, w.V)
        e1.record()
        torch.cuda.synchronize()
        if i:
            bt.append(e0.elapsed_time(e1))
    build_ms = float(np.median(bt))
    print(f"[bench] build {build_ms:.2f} ms", file=sys.stderr, flush=True)
    head_meta(ix, H, N + n_ins)

    if a.copy_mib:
        # two plain copies of a known size: the runtime's device-to-device copy
        # and an elementwise x + 0 (16-byte loads and stores per lane)
        src = torch.empty(a.copy_mib << 18, dtype=torch.float32, device=dev).fill_(1.0)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.add(src, 0.0, out=dst)
        torch.cuda.synchronize()
        del src, dst

    # ---- decode steps
    Qs = [synth.decode_queries(w, G, gen, device=dev) for _ in range(a.warmup + a.steps)]
    results = {}
    for budget in budgets:
        k = budget // 16
        beam = k
        for s in range(a.warmup):
            ix.ice_decode(Qs[s], budget, beam)
            _, uni, nuni = ix.ice_select(Qs[s], budget, beam)
            ix.ice_attend(Qs[s], uni, nuni)
        torch.cuda.synchronize()
        # whole steps: one ice_decode per step (the fused select + attend); a
        # short spin on the stream first lets the host queue the timed steps
        # ahead of the GPU, so the events bracket GPU work, not launch gaps
        t0 = time.perf_counter()
        g0, g1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda._sleep(int(5e7))
        g0.record()
        for s in range(a.steps):
            ix.ice_decode(Qs[a.warmup + s], budget, beam)
        g1.record()
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        ms_step = g0.elapsed_time(g1) / a.steps
        # the separate calls, each kernel on its own: the same launches back to
        # back between two events
        unis = []
        for s in range(a.steps):
            _, uni, nuni = ix.ice_select(Qs[a.warmup + s], budget, beam)
            unis.append((uni, nuni))
        e = [torch.cuda.Event(enable_timing=True) for _ in range(4)]
        torch.cuda._sleep(int(5e7))
        e[0].record()
        for s in range(a.steps):
            ix.ice_select(Qs[a.warmup + s], budget, beam)
        e[1].record()
        torch.cuda._sleep(int(5e7))
        e[2].record()
        for s in range(a.steps):
            ix.ice_attend(Qs[a.warmup + s], *unis[s])
        e[3].record()
        torch.cuda.synchronize()
        sel_ms = e[0].elapsed_time(e[1]) / a.steps
        att_ms = e[2].elapsed_time(e[3]) / a.steps
        # algorithmic bytes from the same selections (replayed with a trace)
        nb = min(a.steps, 4)
        byt = dict(select=0.0, attend=0.0, decode=0.0)
        for s in range(nb):
            q = Qs[a.warmup + s]
            _, uni, nuni, tr = ix.ice_select(q, budget, beam, trace=True)
            bb = algorithmic_bytes(ix, tr.cpu().numpy(), uni.cpu().numpy(), nuni.cpu().numpy(), d, elt, G)
            for k2 in byt:
                byt[k2] += bb[k2] / nb
        sb, ab, db = byt["select"], byt["attend"], byt["decode"]
        results[budget] = dict(ms_per_step=ms_step, steps_per_s=1000.0 / ms_step, wall_s=wall,
                               decode_bytes=db, decode_gbs=db / ms_step / 1e6,
                               select_ms=sel_ms, attend_ms=att_ms, select_bytes=sb, attend_bytes=ab,
                               select_gbs=sb / sel_ms / 1e6, attend_gbs=ab / att_ms / 1e6)
        print(f"[bench] T={budget}: {ms_step*1000:.1f} us/step fused ({db/ms_step/1e6:.0f} GB/s); separately "
              f"select {sel_ms*1000:.1f} us ({sb/sel_ms/1e6:.0f} GB/s) attend {att_ms*1000:.1f} us "
              f"({ab/att_ms/1e6:.0f} GB/s)", file=sys.stderr, flush=True)

    host_pool = None
    if not a.no_host_pool:
        host_pool = time_host_pool(w, Qs, a, H, G, N, d, dtype, a.budget, results[a.budget]["attend_ms"], n_ins)

    pipeline = reuse = None
    if not a.no_pipeline and H % 8 == 0 and H // 8 >= 2:
        pipeline = time_pipeline(ix, w, a, H, N)
        reuse = time_reuse(ix, w, a, H, N)
        ix.ice_build(w.K, w.V)       # the index as a whole build leaves it, for the legs below
        torch.cuda.synchronize()

    # ---- resident sink + window tokens beside the selected pages: the same
    # decode steps with a.resident extra tokens per head in every softmax
    resident = None
    if a.resident > 0:
        Kr, Vr = synth.resident_tokens(w, a.resident, gen, device=dev)
        r0, r1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        r0.record()
        ix.set_resident(Kr, Vr)
        r1.record()
        torch.cuda.synchronize()
        set_ms = r0.elapsed_time(r1)
        for s in range(min(a.warmup, 3)):
            ix.ice_decode(Qs[s], a.budget, a.budget // 16)
        torch.cuda.synchronize()
        torch.cuda._sleep(int(5e7))
        r0.record()
        for s in range(a.steps):
            ix.ice_decode(Qs[a.warmup + s], a.budget, a.budget // 16)
        r1.record()
        torch.cuda.synchronize()
        res_ms = r0.elapsed_time(r1) / a.steps
        ix.set_resident(None, None)
        torch.cuda.synchronize()
        resident = {"tokens_per_head": a.resident, "ms_per_step": res_ms, "set_resident_ms": set_ms,
                    "extra_bytes_per_step": 2 * H * a.resident * d * elt}
        print(f"[bench] resident {a.resident} tokens/head T={a.budget}: {res_ms*1000:.1f} us/step; "
              f"set_resident {set_ms*1000:.1f} us", file=sys.stderr, flush=True)

    # ---- insert: one token per head per step
    knew = [synth.new_tokens(w, gen, device=dev) for _ in range(n_ins)]
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    # the spin lets the host queue every insert before the first one starts
    torch.cuda._sleep(int(5e7))
    e0.record()
    for k_, v_ in knew:
        ix.ice_insert(k_, v_)
    e1.record()
    torch.cuda.synchronize()
    insert_ms = e0.elapsed_time(e1) / n_ins

    head = results[a.budget]
    # the step is one kernel (the fused decode); its launches run back to back
    # between the step events, so the step time is its average launch time
    dom_bytes = head["decode_bytes"]
    dom_ms = head["ms_per_step"]
    achieved = dom_bytes / dom_ms / 1e6
    out = {
        "metric": METRIC,
        "value": head["steps_per_s"],
        "unit": "decode steps/s",
        "n_gpus": 1,
        "steps": a.steps,
        "warmup": a.warmup,
        "ms_per_step": head["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": dtype,
        "data": "synthetic",
        "config": {"workload": desc, "heads": H, "group": G, "context": N, "d": d, "budget_tokens": a.budget,
                   "beam": a.budget // 16, "levels": 3, "promote": "1/16", "page": 16},
        "roofline": {"bound": "hbm", "kernel": "k_decode", "achieved": achieved, "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": achieved / HBM_PEAK_GBS,
                     "traffic": recorded_traffic("k_decode", a.workload) if a.budget == 256 else None,
                     "bytes_per_launch": dom_bytes, "launch_ms": dom_ms},
        "index_keys_per_s": H * N / (build_ms / 1000.0),
        "build_ms": build_ms,
        "insert_ms_per_step": insert_ms,
        "per_budget": {str(b): {k2: (round(v, 6) if isinstance(v, float) else v) for k2, v in r.items()}
                       for b, r in results.items()},
    }
    if host_pool is not None:
        out["host_pool"] = host_pool
    if resident is not None:
        out["resident"] = resident
    if pipeline is not None:
        out["prefill_pipeline"] = pipeline
    if reuse is not None:
        out["index_reuse"] = reuse
    if a.drift_steps > 0:
        out["split_drift"] = split_drift(a)
    if a.pdci_tokens > 0:
        out["pdci"] = pdci_leg(a)
    if not a.no_cpu:
        heads = list(range(min(a.cpu_heads, H)))
        n_cpu_steps = min(a.steps, 50)
        t_build, t_dec, threads = cpu_baseline(w, [Qs[a.warmup + s] for s in range(n_cpu_steps)], a.budget,
                                               a.budget // 16, heads, a.seed)
        per_head_step = t_dec / len(heads)
        out["cpu_baseline"] = {
            "value": 1.0 / (per_head_step * H), "unit": "decode steps/s", "cores": threads, "kind": "oracle",
            "sample": (f"fp64 oracle on {len(heads)} of {H} heads ({N} tokens each): its own index build, then "
                       f"select+attend for {G} query heads over {n_cpu_steps} steps at T={a.budget}; per-head time scaled to "
                       f"{H} heads"),
            "index_keys_per_s": len(heads) * N / t_build,
            "cpu": platform.processor() or platform.machine(),
        }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
