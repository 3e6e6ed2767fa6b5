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
    "qwen-gen": (512, 8, 8192, 128, "bf16", 512, False,
                 "8192-token prompt then generation, 64 layers x 8 KV heads x 8 query heads (Qwen3-32B shape), "
                 "d=128 bf16, 512-component mixtures, queries and new keys walking between centres"),
}


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="ctx36k", choices=sorted(WORKLOADS))
    ap.add_argument("--budget", type=int, default=256)
    ap.add_argument("--budgets", default="64,128", help="extra budgets to time beside --budget")
    ap.add_argument("--builds", type=int, default=3)
    ap.add_argument("--cpu-heads", type=int, default=16, help="heads in the oracle's timed sample")
    ap.add_argument("--no-cpu", action="store_true", help="skip the oracle baseline")
    ap.add_argument("--no-host-pool", action="store_true", help="skip the host-pool mode measurement")
    ap.add_argument("--no-pipeline", action="store_true", help="skip the per-layer build pipeline measurement")
    ap.add_argument("--resident", type=int, default=68,
                    help="resident (sink + window) tokens per head for the resident-token leg; 0 skips it")
    ap.add_argument("--drift-steps", type=int, default=0,
                    help="generated steps of the split-reading recall comparison (0 skips it; 4096 is the "
                         "Qwen3-32B-shaped generation)")
    ap.add_argument("--pdci-tokens", type=int, default=0,
                    help="context of the P-DCI against exact-parent comparison (0 skips it; 100000 is the needle "
                         "workload's context)")
    ap.add_argument("--no-configs", action="store_true",
                    help="skip the other workloads (Qwen3-32B-shaped generation, Llama layer, tiny, needle)")
    ap.add_argument("--no-recall", action="store_true", help="skip the selection-recall table")
    ap.add_argument("--recall-heads", type=int, default=64, help="heads in the selection-recall table")
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
    MFMA busy cycles / (window x 1024 SIMDs). SQ_INSTS_VALU counts the MFMA
    instructions too (they are vector-ALU instructions to the sequencer: a
    kernel of MFMAs and scalar loop control reads the same count in both), so
    the other vector instructions are SQ_INSTS_VALU - SQ_INSTS_MFMA."""
    disp = {}
    for r in csv.DictReader(open(path)):
        k = short_name(r["Kernel_Name"])
        if not k.startswith("k_"):
            continue
        key = (k, r.get("Dispatch_Id", r.get("Correlation_Id", "")))
        disp.setdefault(key, {})[r["Counter_Name"]] = disp.setdefault(key, {}).get(r["Counter_Name"], 0.0) + \
            float(r["Counter_Value"])
    out = ["| Kernel | Dispatch | GPU cycles (window) | MFMA instructions | other VALU instructions | "
           "other VALU / MFMA | MFMA busy (% of 1024 SIMDs) |", "|---|---|---|---|---|---|---|"]
    for (k, d), c in sorted(disp.items(), key=lambda x: (x[0][0], int(x[0][1]) if str(x[0][1]).isdigit() else 0)):
        mf = c.get("SQ_INSTS_MFMA", 0.0)
        if mf <= 0:
            continue
        win = c.get("GRBM_GUI_ACTIVE", 0.0) / 8.0
        busy = c.get("SQ_VALU_MFMA_BUSY_CYCLES", 0.0)
        util = 100.0 * busy / (win * 1024) if win else float("nan")
        va = c.get("SQ_INSTS_VALU", 0.0) - mf
        out.append(f"| `{k}` | {d} | {win:.0f} | {mf:.0f} | {va:.0f} | {va / mf:.2f} | {util:.1f} |")
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


def cpu_model():
    """The host CPU's model string (Linux), else the platform's name."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return platform.processor() or platform.machine()


def ev_pair():
    import torch
    return torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)


def decode_timing(ix, Qs, budget, steps, warmup, d, elt, G, separate=True):
    """Whole decode steps (one ice_decode each) between two events, queued by
    the host behind a short spin so the events bracket GPU work; then (if
    `separate`) the same steps as ice_select alone and ice_attend alone; and
    the algorithmic bytes of the run's own selections."""
    import torch
    beam = budget // 16
    for s in range(warmup):
        ix.ice_decode(Qs[s], budget, beam)
        if separate:
            _, uni, nuni = ix.ice_select(Qs[s], budget, beam)
            ix.ice_attend(Qs[s], uni, nuni)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    g0, g1 = ev_pair()
    torch.cuda._sleep(int(5e7))
    g0.record()
    for s in range(steps):
        ix.ice_decode(Qs[warmup + s], budget, beam)
    g1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_step = g0.elapsed_time(g1) / steps
    r = dict(ms_per_step=ms_step, steps_per_s=1000.0 / ms_step, wall_s=wall)
    nb = min(steps, 4)
    byt = dict(select=0.0, attend=0.0, decode=0.0)
    for s in range(nb):
        _, uni, nuni, tr = ix.ice_select(Qs[warmup + s], budget, beam, trace=True)
        bb = algorithmic_bytes(ix, tr.cpu().numpy(), uni.cpu().numpy(), nuni.cpu().numpy(), d, elt, G)
        for k2 in byt:
            byt[k2] += bb[k2] / nb
    r.update(decode_bytes=byt["decode"], decode_gbs=byt["decode"] / ms_step / 1e6)
    if separate:
        unis = []
        for s in range(steps):
            _, uni, nuni = ix.ice_select(Qs[warmup + s], budget, beam)
            unis.append((uni, nuni))
        e = [torch.cuda.Event(enable_timing=True) for _ in range(4)]
        torch.cuda._sleep(int(5e7))
        e[0].record()
        for s in range(steps):
            ix.ice_select(Qs[warmup + s], budget, beam)
        e[1].record()
        torch.cuda._sleep(int(5e7))
        e[2].record()
        for s in range(steps):
            ix.ice_attend(Qs[warmup + s], *unis[s])
        e[3].record()
        torch.cuda.synchronize()
        sel_ms = e[0].elapsed_time(e[1]) / steps
        att_ms = e[2].elapsed_time(e[3]) / steps
        r.update(select_ms=sel_ms, attend_ms=att_ms, select_bytes=byt["select"], attend_bytes=byt["attend"],
                 select_gbs=byt["select"] / sel_ms / 1e6, attend_gbs=byt["attend"] / att_ms / 1e6)
    return r


def build_timing(ix, w, builds):
    """After one untimed build: the median over `builds` builds of ice_build
    (events on the caller's stream around the call; a build of many heads
    runs as a two-stream pipeline that joins back into that stream), and the
    median over as many one-stream builds (ice_build_timed) of each phase and
    of their sum. Returns (build ms, phases ms, one-stream build ms, whether
    the two kinds of build left the index blob bit-identical)."""
    import torch
    ix.ice_build(w.K, w.V)
    torch.cuda.synchronize()
    tot = []
    for _ in range(builds):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        ix.ice_build(w.K, w.V)
        e1.record()
        e1.synchronize()
        tot.append(e0.elapsed_time(e1))
    # a copy in 128 MiB pieces: counter runs calibrate on whole 1 GiB copies
    # and must not mistake this one for them
    blob = torch.empty_like(ix.blob)
    piece = 128 << 20
    for i in range(0, ix.blob.numel(), piece):
        blob[i:i + piece].copy_(ix.blob[i:i + piece])
    runs = [ix.ice_build_timed(w.K, w.V) for _ in range(builds)]
    same = bool(torch.equal(blob, ix.blob))
    del blob
    ph = np.median(np.stack(runs), axis=0)
    return float(np.median(tot)), ph, float(np.median([x.sum() for x in runs])), same


def parent_flops(ix, H, level, d):
    """Algorithmic flops of the level-`level` parent search over all heads: two
    per multiply-add of a d-dimensional key product, for every point of the
    level that is not itself at the next level, against every point of the
    next level."""
    from ann_retrieval_amd import _lib as L
    tot = 0
    for h in range(H):
        n = ix.stats(h)["n_tokens"]
        lev = ix.export(h, L.ICE_EXP_LEVEL, np_dtype=np.int8)[:n]
        n_l, n_up = int((lev >= level).sum()), int((lev >= level + 1).sum())
        tot += 2 * (n_l - n_up) * n_up * d
    return tot


def recall_leg(ix, w, Qs, budgets, n_heads, G):
    """Selection quality at each budget T (k = T/16 pages per query head), over
    the first `n_heads` heads and a few decode queries: the share of each query
    head's exact top-T keys by q.k that lie in its selected pages, for beams
    k, 2k and 4k; for the best k semantic pages found by brute force (every
    page scored by its best key, the limit of an unbounded beam); and for the
    best k sequential 16-token pages (the layout the pages argue against)."""
    import torch
    from ann_retrieval_amd import _lib as L
    dev = w.K.device
    Kf = w.K[:n_heads].float()                                   # [h, N, d]
    N = Kf.shape[1]
    tok = [torch.from_numpy(ix.export(h, L.ICE_EXP_PAGE_TOK, 0).reshape(-1, 16)[:ix.stats(h)["n_pages"][0]]).to(dev)
           .long() for h in range(n_heads)]
    out = {}
    for T in budgets:
        k = T // 16
        hits = {f"beam_{m}k": 0 for m in (1, 2, 4)}
        hits.update(semantic_all_pages=0, sequential_pages=0)
        total = 0
        for Q in Qs:
            S = torch.bmm(Q[:n_heads].float(), Kf.transpose(1, 2))   # [h, G, N]
            top = torch.topk(S, T, dim=-1).indices                    # [h, G, T]
            sels = {m: ix.ice_select(Q, T, min(m * k, L.ICE_MAX_BEAM))[0][:n_heads].long() for m in (1, 2, 4)}
            seq_pad = torch.full((n_heads, G, (N + 15) // 16 * 16 - N), -float("inf"), device=dev)
            seq_best = torch.cat([S, seq_pad], -1).reshape(n_heads, G, -1, 16).amax(-1)
            seq_sel = torch.topk(seq_best, k, dim=-1).indices          # sequential page p = tokens 16p .. 16p+15
            for h in range(n_heads):
                tb = tok[h]
                sc = torch.where(tb[None] >= 0, S[h][:, tb.clamp(min=0)], torch.tensor(-float("inf"), device=dev))
                best = torch.topk(sc.amax(-1), min(k, tb.shape[0]), dim=-1).indices      # [G, k]
                for g in range(G):
                    want = top[h, g]
                    for m in (1, 2, 4):
                        pg = sels[m][h, g]
                        st = tb[pg[pg >= 0]].reshape(-1)
                        hits[f"beam_{m}k"] += int(torch.isin(want, st[st >= 0]).sum())
                    st = tb[best[g]].reshape(-1)
                    hits["semantic_all_pages"] += int(torch.isin(want, st[st >= 0]).sum())
                    sq = (seq_sel[h, g][:, None] * 16 + torch.arange(16, device=dev)[None]).reshape(-1)
                    hits["sequential_pages"] += int(torch.isin(want, sq[sq < N]).sum())
                    total += T
        out[str(T)] = {key: round(v / total, 4) for key, v in hits.items()}
        print(f"[bench] recall T={T}: " + ", ".join(f"{key} {v:.3f}" for key, v in out[str(T)].items()),
              file=sys.stderr, flush=True)
    return {"heads": n_heads, "queries": len(Qs) * n_heads * G,
            "definition": "share of each query head's exact top-T keys by q.k inside its k = T/16 pages", **out}


def needle_leg(a):
    """The needle workload (8 KV heads x 4 query heads, 100,000 tokens, d=128
    bf16, 1024-component background, a 16-token span with cosine 0.9 to query
    head 0's final query, budget 64) at five depths: for query head 0 of every
    KV head, the needle tokens inside its selected pages at beam 4 (= k) and at
    beam 64, the smallest beam whose pages hold a needle token, and the
    attention weight query head 0 gives the needle tokens in its head's union
    at beam 4."""
    import torch
    from ann_retrieval_amd import _lib as L
    from ann_retrieval_amd import synth
    from ann_retrieval_amd.api import IceIndex
    H, G, N, d, T = 8, 4, 100000, 128, 64
    out = {"workload": f"{N}-token context, {H} KV heads x {G} query heads, d=128 bf16, budget {T}", "depths": {}}
    for depth in (0.1, 0.3, 0.5, 0.7, 0.9):
        w, Q, start = synth.needle_workload(H, G, N, d, 1024, depth, seed=a.seed, device="cuda")
        ix = IceIndex(H, G, d, "bf16", N, seed=a.seed, max_budget=T)
        ix.ice_build(w.K, w.V)
        _, uni, nuni, O, lse = ix.ice_decode(Q, T, 4)
        sels = {b: ix.ice_select(Q, T, b)[0].cpu().numpy() for b in (4, 8, 16, 32, 64, 128, 256)}
        torch.cuda.synchronize()
        uni, nuni = uni.cpu().numpy(), nuni.cpu().numpy()
        rows = []
        for h in range(H):
            tb = ix.export(h, L.ICE_EXP_PAGE_TOK, 0).reshape(-1, 16)
            cov = {b: int(sum(1 for p in sels[b][h, 0] if p >= 0 for t in tb[p] if start <= t < start + 16))
                   for b in sels}
            first = next((b for b in sorted(sels) if cov[b] > 0), None)
            toks = np.array([t for p in uni[h, :nuni[h]] for t in tb[p] if t >= 0])
            lg = (w.K[h, toks].float() @ Q[h, 0].float()) / math.sqrt(d)
            wt = torch.softmax(lg, 0).cpu().numpy()
            mass = float(wt[(toks >= start) & (toks < start + 16)].sum())
            rows.append({"covered_beam4": cov[4], "covered_beam64": cov[64], "smallest_beam": first,
                         "attention_mass_beam4": round(mass, 4)})
        hits4 = sum(r["covered_beam4"] > 0 for r in rows)
        hits64 = sum(r["covered_beam64"] > 0 for r in rows)
        out["depths"][str(depth)] = {"heads_hit_beam4": hits4, "heads_hit_beam64": hits64, "per_head": rows}
        print(f"[bench] needle depth {depth}: query head 0 finds it in {hits4}/{H} heads at beam 4, {hits64}/{H} "
              f"at beam 64; smallest beams {[r['smallest_beam'] for r in rows]}", file=sys.stderr, flush=True)
        del ix, w
        torch.cuda.empty_cache()
    return out


def workload_leg(name, a, steps, warmup, with_inserts):
    """Build, decode steps (ice_decode at the workload's budgets) and one-token
    inserts of one workload; for the long-generation shape the queries and
    new keys walk between mixture centres (pages split)."""
    import torch
    from ann_retrieval_amd import synth
    from ann_retrieval_amd.api import IceIndex
    H, G, N, d, dtype, C, rotate, desc = WORKLOADS[name]
    budgets = BUDGETS[name]
    dev = torch.device("cuda", 0)
    w, gen = synth.clustered_kv(H, N, d, C, dtype, a.seed, device=dev, rotate=rotate)
    elt = 2 if dtype == "bf16" else 4
    n_ins = steps + warmup if with_inserts else 0
    ix = IceIndex(H, G, d, dtype, N + n_ins, seed=a.seed, max_budget=max(budgets), device=dev)
    build_ms, ph, _, _ = build_timing(ix, w, 3)
    head_meta(ix, H, N + n_ins)
    if name == "qwen-gen":
        walk = synth.QueryWalk(w, G, gen, device=dev)
        seq = [walk.step() for _ in range(warmup + steps)]
        Qs = [x[0] for x in seq]
        ins = [(x[1], x[2]) for x in seq]
    else:
        Qs = [synth.decode_queries(w, G, gen, device=dev) for _ in range(warmup + steps)]
        ins = [synth.new_tokens(w, gen, device=dev) for _ in range(n_ins)]
    res = {"workload": desc, "heads": H, "group": G, "context": N, "build_ms": build_ms,
           "index_keys_per_s": H * N / (build_ms / 1000.0), "per_budget": {}}
    for T in budgets:
        r = decode_timing(ix, Qs, T, steps, warmup, d, elt, G, separate=False)
        res["per_budget"][str(T)] = {k: round(v, 6) for k, v in r.items()}
        print(f"[bench] {name} T={T}: {r['ms_per_step'] * 1000:.1f} us/step ({r['decode_gbs']:.0f} GB/s)",
              file=sys.stderr, flush=True)
    if with_inserts:
        T = max(budgets)
        # inserts alone, then whole steps of decode + insert, both queued behind a spin
        e0, e1 = ev_pair()
        torch.cuda._sleep(int(5e7))
        e0.record()
        for k_, v_ in ins[:warmup]:
            ix.ice_insert(k_, v_)
        e1.record()
        torch.cuda.synchronize()
        ins_ms = e0.elapsed_time(e1) / max(warmup, 1)
        c0, c1 = ev_pair()
        torch.cuda._sleep(int(5e7))
        c0.record()
        for s in range(steps):
            ix.ice_decode(Qs[warmup + s], T, T // 16)
            ix.ice_insert(*ins[warmup + s])
        c1.record()
        torch.cuda.synchronize()
        comb_ms = c0.elapsed_time(c1) / steps
        splits = sum(ix.stats(h)["splits"] for h in range(H))
        res.update(insert_ms_per_step=ins_ms, decode_plus_insert_ms_per_step=comb_ms, splits=splits)
        print(f"[bench] {name}: insert {ins_ms * 1000:.1f} us/step; decode + insert {comb_ms * 1000:.1f} us/step; "
              f"{splits} page splits", file=sys.stderr, flush=True)
    del ix, w
    torch.cuda.empty_cache()
    return res


BUDGETS = {"qwen-gen": [256], "llama-layer": [64, 128, 256], "tiny": [64]}


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
    budgets = sorted({int(b) for b in a.budgets.split(",") if b} | {a.budget})
    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    print(f"[bench] workload={a.workload} H={H} G={G} N={N} d={d} {dtype}", file=sys.stderr, flush=True)
    w, gen = synth.clustered_kv(H, N, d, C, dtype, a.seed, device=dev, rotate=rotate)
    elt = 2 if dtype == "bf16" else 4
    n_ins = a.steps + a.warmup
    ix = IceIndex(H, G, d, dtype, N + n_ins, seed=a.seed, max_budget=max(budgets), device=dev,
                  resident=max(a.resident, 0))

    # ---- index build: median of a few builds; each phase from one-stream builds timed by events
    build_ms, phases, build_serial_ms, build_same = build_timing(ix, w, a.builds)
    if not build_same:
        raise RuntimeError("the pipelined build and the one-stream build left different index blobs")
    print(f"[bench] build {build_ms:.2f} ms (one stream {build_serial_ms:.2f} ms); phases (ms) "
          f"{np.round(phases, 3).tolist()}", file=sys.stderr, flush=True)
    head_meta(ix, H, N + n_ins)
    from ann_retrieval_amd import _lib as L
    gemm_ms = float(phases[L.ICE_PHASE_PARENT])
    gemm_flop = parent_flops(ix, H, 0, d)
    gemm_tflops = gemm_flop / (gemm_ms / 1000.0) / 1e12
    # the same keys with one level (no promotion, no parent search: the
    # virtual root owns every token in token order)
    ix1 = IceIndex(H, G, d, dtype, N + n_ins, levels=1, seed=a.seed, max_budget=max(budgets), device=dev)
    build1_ms, _, _, _ = build_timing(ix1, w, a.builds)
    del ix1
    torch.cuda.synchronize()
    print(f"[bench] build with one level {build1_ms:.2f} ms", file=sys.stderr, flush=True)

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

    # ---- decode steps at each budget
    Qs = [synth.decode_queries(w, G, gen, device=dev) for _ in range(a.warmup + a.steps)]
    results = {}
    for budget in budgets:
        r = decode_timing(ix, Qs, budget, a.steps, a.warmup, d, elt, G)
        results[budget] = r
        print(f"[bench] T={budget}: {r['ms_per_step']*1000:.1f} us/step fused ({r['decode_gbs']:.0f} GB/s); "
              f"separately select {r['select_ms']*1000:.1f} us ({r['select_gbs']:.0f} GB/s) attend "
              f"{r['attend_ms']*1000:.1f} us ({r['attend_gbs']:.0f} GB/s)", file=sys.stderr, flush=True)

    recall = None
    if not a.no_recall:
        recall = recall_leg(ix, w, Qs[a.warmup:a.warmup + 2], budgets, min(a.recall_heads, H), G)

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
        r0, r1 = ev_pair()
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
    e0, e1 = ev_pair()
    # the spin lets the host queue every insert before the first one starts
    torch.cuda._sleep(int(5e7))
    e0.record()
    for k_, v_ in knew:
        ix.ice_insert(k_, v_)
    e1.record()
    torch.cuda.synchronize()
    insert_ms = e0.elapsed_time(e1) / n_ins

    # ---- the oracle on the host cores, on a bounded sample of the same workload
    cpu = None
    if not a.no_cpu:
        heads = list(range(min(a.cpu_heads, H)))
        n_cpu_steps = min(a.steps, 50)
        t_build, t_dec, threads = cpu_baseline(w, [Qs[a.warmup + s] for s in range(n_cpu_steps)], a.budget,
                                               a.budget // 16, heads, a.seed)
        per_head_step = t_dec / len(heads)
        cpu = {
            "value": 1.0 / (per_head_step * H), "unit": "decode steps/s", "cores": threads, "kind": "oracle",
            "sample": (f"fp64 oracle on {len(heads)} of {H} heads ({N} tokens each): its own index build, then "
                       f"select+attend for {G} query heads over {n_cpu_steps} steps at T={a.budget}; per-head time "
                       f"scaled to {H} heads"),
            "index_keys_per_s": len(heads) * N / t_build,
            "cpu": cpu_model(),
        }
    del ix
    torch.cuda.empty_cache()

    # ---- the other workloads: Qwen3-32B-shaped long generation, one Llama
    # layer, the tiny case, the needle
    configs = needle = None
    if not a.no_configs:
        configs = {"qwen-gen": workload_leg("qwen-gen", a, a.steps, a.warmup, True),
                   "llama-layer": workload_leg("llama-layer", a, a.steps, a.warmup, True),
                   "tiny": workload_leg("tiny", a, a.steps, a.warmup, False)}
        q = configs["qwen-gen"]["per_budget"]["256"]
        q_ach = q["decode_bytes"] / q["ms_per_step"] / 1e6
        configs["qwen-gen"]["roofline"] = {"bound": "hbm", "kernel": "k_decode", "achieved": q_ach,
                                           "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": q_ach / HBM_PEAK_GBS,
                                           "traffic": recorded_traffic("k_decode", "qwen-gen"),
                                           "bytes_per_launch": q["decode_bytes"], "launch_ms": q["ms_per_step"]}
        needle = needle_leg(a)

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
        "roofline_build": {"bound": "mfma", "kernel": "k_parent_bf16", "level": 0, "achieved": gemm_tflops,
                           "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s", "frac": gemm_tflops / BF16_PEAK_TFLOPS,
                           "flop_per_launch": gemm_flop, "launch_ms": gemm_ms},
        "index_keys_per_s": H * N / (build_ms / 1000.0),
        "build_ms": build_ms,
        "build_one_stream_ms": build_serial_ms,
        "build_pipelined_equals_one_stream": build_same,
        "build_levels1_ms": build1_ms,
        "build_phases_ms": {"lift": float(phases[L.ICE_PHASE_LIFT]),
                            **{f"{nm}_l{lv}": float(phases[base + 4 * lv]) for lv in range(2)
                               for nm, base in (("operand", L.ICE_PHASE_OPERAND), ("parent", L.ICE_PHASE_PARENT),
                                                ("pack", L.ICE_PHASE_PACK), ("copy", L.ICE_PHASE_COPY))},
                            "top": float(phases[L.ICE_PHASE_TOP])},
        "insert_ms_per_step": insert_ms,
        "per_budget": {str(b): {k2: (round(v, 6) if isinstance(v, float) else v) for k2, v in r.items()}
                       for b, r in results.items()},
    }
    if recall is not None:
        out["recall"] = recall
    if configs is not None:
        out["configs"] = configs
    if needle is not None:
        out["needle"] = needle
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
    if cpu is not None:
        out["cpu_baseline"] = cpu
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
