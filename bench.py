"""Benchmark of one SparsePR call on one MI355X.

A step is one whole call (partition, route, attend, probe_fit, apply) on
synthetic inputs already resident in HBM. Prints ONE JSON line: executed-pair
TFLOP/s of the call (value), call ms, the build's dense attention ms and the
speedup, per-stage ms, the block-sparse kernel's roofline, and the fp64
oracle timed on a bounded sample on the host cores.

    python bench.py [--config hunyuan] [--steps 10] [--warmup 3] [--gpus 1]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "SparsePR call ms & speedup vs dense at 22% density; executed-pair TFLOP/s"
PEAK_BF16_TFLOPS = 2500.0
PEAK_HBM_GBS = 8000.0


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def source_hash(path):
    with open(path, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def load_traffic(workload):
    """HBM traffic of the block-sparse kernel from committed rocprofv3 PMC
    summaries, valid only while the kernel source is unchanged."""
    path = os.path.join(ROOT, "profiles", f"attend_traffic_{workload}.json")
    if not os.path.exists(path):
        return None
    rec = json.load(open(path))
    src = os.path.join(ROOT, "free_block_sparse_rcp_amd", "csrc", "attention.hip")
    if rec.get("attention_hip_sha256_16") != source_hash(src):
        return None
    return rec.get("bytes_per_launch")


SPARSE_KERNEL = "k_attn_mfma<128, 128, 0>"   # sparsepr_attend's kernel (d=128, B_q=128)
COPY_KERNEL = "neg_kernel"                    # the --calibration-copy-mib kernel
PMC_KERNELS = ("k_attn_mfma|k_group_mean|k_apply_mfma|k_rowvec_mfma|k_route_scores|"
               "k_metric|neg_kernel")              # the kernels the per-kernel traffic table covers


def pmc_summary(fetch_csv, write_csv, workload, copy_mib):
    """Per-launch HBM bytes of the block-sparse kernel from a FETCH_SIZE run and
    a WRITE_SIZE run (rocprofv3 --pmc ... --output-format csv), each scaled by
    what the same counter reports for the plain copy of copy_mib MiB (reads
    and writes copy_mib MiB exactly). Writes profiles/attend_traffic_<workload>.json."""
    import csv

    def per_dispatch(path, counter):
        vals = {"kernel": [], "copy": []}
        for r in csv.DictReader(open(path)):
            if r["Counter_Name"] != counter:
                continue
            if SPARSE_KERNEL in r["Kernel_Name"]:
                vals["kernel"].append(float(r["Counter_Value"]))
            elif COPY_KERNEL in r["Kernel_Name"]:
                vals["copy"].append(float(r["Counter_Value"]))
        if not vals["kernel"] or not vals["copy"]:
            raise SystemExit(f"{path}: no {counter} rows for the kernel and the copy")
        return sum(vals["kernel"]) / len(vals["kernel"]), sum(vals["copy"]) / len(vals["copy"]), \
            len(vals["kernel"])

    copy_kib = copy_mib * 1024.0
    f_k, f_c, nf = per_dispatch(fetch_csv, "FETCH_SIZE")
    w_k, w_c, nw = per_dispatch(write_csv, "WRITE_SIZE")
    f_scale, w_scale = copy_kib / f_c, copy_kib / w_c
    fetch_b = f_k * f_scale * 1024.0
    write_b = w_k * w_scale * 1024.0
    src = os.path.join(ROOT, "free_block_sparse_rcp_amd", "csrc", "attention.hip")
    rec = {"workload": workload, "kernel": SPARSE_KERNEL,
           "attention_hip_sha256_16": source_hash(src),
           "fetch_kib_per_dispatch_raw": f_k, "write_kib_per_dispatch_raw": w_k,
           "dispatches": {"fetch_run": nf, "write_run": nw},
           "copy_mib": copy_mib, "copy_fetch_kib_raw": f_c, "copy_write_kib_raw": w_c,
           "fetch_scale": f_scale, "write_scale": w_scale,
           "fetch_bytes_per_launch": fetch_b, "write_bytes_per_launch": write_b,
           "bytes_per_launch": fetch_b + write_b}
    out = os.path.join(ROOT, "profiles", f"attend_traffic_{workload}.json")
    with open(out, "w") as f:
        json.dump(rec, f, indent=1)
    print(json.dumps(rec))


def pmc_table(fetch_csv, write_csv, workload, copy_mib):
    """HBM bytes and achieved bandwidth of every kernel in a FETCH_SIZE run and a
    WRITE_SIZE run, each counter scaled by what it reports for the plain copy of
    copy_mib MiB; durations from the FETCH run's dispatch timestamps. Writes
    profiles/hbm_traffic_<workload>.md."""
    import csv
    from collections import defaultdict

    def short(name):
        name = name.replace("void ", "")
        return name.split("(")[0][:60]

    def per_kernel(path, counter):
        acc = defaultdict(list)
        dur = defaultdict(list)
        copy = []
        for r in csv.DictReader(open(path)):
            if r["Counter_Name"] != counter:
                continue
            v = float(r["Counter_Value"])
            if COPY_KERNEL in r["Kernel_Name"]:
                copy.append(v)
                continue
            k = short(r["Kernel_Name"])
            acc[k].append(v)
            dur[k].append((int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) * 1e-9)
        if not copy:
            raise SystemExit(f"{path}: no {counter} rows for the copy kernel")
        return acc, dur, sum(copy) / len(copy)

    copy_kib = copy_mib * 1024.0
    fk, fdur, fc = per_kernel(fetch_csv, "FETCH_SIZE")
    wk, _, wc = per_kernel(write_csv, "WRITE_SIZE")
    fs, ws = copy_kib / fc, copy_kib / wc
    rows = []
    for k in fk:
        if k not in wk:
            continue
        f_b = sum(fk[k]) / len(fk[k]) * fs * 1024.0
        w_b = sum(wk[k]) / len(wk[k]) * ws * 1024.0
        t = sum(fdur[k]) / len(fdur[k])
        rows.append((k, len(fk[k]), f_b, w_b, t))
    rows.sort(key=lambda r: -r[4] * r[1])
    lines = [f"| kernel | dispatches | fetch GB | write GB | avg ms | GB/s | % of 8 TB/s |",
             "|---|---:|---:|---:|---:|---:|---:|"]
    for k, n, f_b, w_b, t in rows:
        bw = (f_b + w_b) / t / 1e9 if t > 0 else 0.0
        lines.append(f"| `{k}` | {n} | {f_b / 1e9:.3f} | {w_b / 1e9:.3f} | {t * 1e3:.4f} | "
                     f"{bw:.0f} | {100 * bw / 8000:.1f} |")
    text = "\n".join(lines)
    out = os.path.join(ROOT, "profiles", f"hbm_traffic_{workload}.md")
    with open(out, "w") as f:
        # the commands as run: output directories are those of the two CSV files
        outdir = {c: os.path.dirname(path) for c, path in (("FETCH_SIZE", fetch_csv),
                                                           ("WRITE_SIZE", write_csv))}
        runs = "\n".join(
            f'timeout -s KILL 240 rocprofv3 --pmc {c} --kernel-include-regex "{PMC_KERNELS}" '
            f"--output-format csv -d {outdir[c]} -o run -- python3 bench.py --steps 1 --warmup 0 "
            f"--no-cpu-baseline --no-dense --no-comparator --calibration-copy-mib {copy_mib}"
            for c in ("FETCH_SIZE", "WRITE_SIZE"))
        f.write(f"# HBM traffic per kernel, {workload}\n\n"
                f"Scale factors from a {copy_mib} MiB copy: FETCH_SIZE x{fs:.3f}, WRITE_SIZE x{ws:.3f}. "
                "Durations are the dispatch timestamps of the FETCH_SIZE run (one call; counters "
                "serialise the dispatches). Commands (from the repository root, on one MI355X, each "
                "counter in a run of its own):\n\n```\ncd /tmp && export TMPDIR=/tmp && cd -\n"
                f"{runs}\npython3 bench.py --pmc-table {fetch_csv} {write_csv} "
                f"--calibration-copy-mib {copy_mib}\n```\n\n"
                + text + "\n")
    print(text)


SUPPORT_MASS = 0.9   # target mass of the support diagnostics


def support_summary(p, b, Q, K, scale, blocks):
    """Support and mass diagnostics of sampled blocks of head 0 for one
    partition's routing (sparsepr_support_stats), summarised."""
    import numpy as np
    from free_block_sparse_rcp_amd import binding

    st = binding.support_stats(p, 0, Q, K, scale, b, blocks, SUPPORT_MASS)
    v = st.valid
    s = st.support.astype(np.float64)
    mean_s = np.array([s[i][v[i]].mean() for i in range(len(blocks))])
    N = p.n_tokens
    return {"routed_mass_mean": float(st.routed_mass[v].mean()),
            "routed_mass_p10": float(np.quantile(st.routed_mass[v], 0.1)),
            "support_frac_mean": float(s[v].mean() / N),
            "support_on_route_mean": float((st.support_routed[v] / s[v]).mean()),
            "pooled_frac_mean": float(st.pooled.mean() / N),
            "pooled_over_mean_support": float((st.pooled / mean_s).mean()),
            "pooled_on_route_mean": float((st.pooled_routed / st.pooled).mean()),
            "route_frac": float(p.key_budget / N)}


def semantic_comparator(args, p, Q, K, V, scale, inp, ref, rn, mask, err_sparsepr):
    """Semantic block-sparse attention without residual correction at the same
    executed-pair density (no probes, so the whole budget goes to the sparse
    pass): its error on the rows SparsePR leaves unprobed, the error reduction
    1 - e(SparsePR) / e(semantic), and its call time. Runs after the timed
    region."""
    import dataclasses
    import numpy as np
    import torch
    from free_block_sparse_rcp_amd import binding

    ps = dataclasses.replace(p, partition_mode=binding.SEMANTIC, n_probes=0, rank=0)
    dev = Q.device
    cop = binding.SparsePR(ps, dev)
    cidx = cop.upload_indices(init_idx=inp.init_idx)
    log("[bench] semantic comparator")
    cop.run(Q, K, V, scale, cidx)
    torch.cuda.synchronize()
    n = max(1, min(args.steps, 3))
    evs = [dict() for _ in range(n)]
    for i in range(n):
        cop.run(Q, K, V, scale, cidx, events=evs[i])
    torch.cuda.synchronize()
    call_ms = float(np.mean([e["start"].elapsed_time(e["apply"]) for e in evs]))
    with torch.no_grad():
        ec = ((cop.buffers.O.float() - ref).norm(dim=2) / rn)[mask]
    E = int(cop.buffers.executed_pairs.sum().item())
    support = support_summary(ps, cop.buffers, Q, K, scale, support_blocks(p))
    out = {"rel_l2_mean_unprobed": float(ec.mean()),
           "error_reduction": 1.0 - err_sparsepr / float(ec.mean()),
           "realized_density": E / (p.heads * float(p.n_tokens) ** 2),
           "call_ms": call_ms,
           "definition": "k-means (same G, T, init rows) on raw key rows and on raw query rows, "
                         "queries in (cluster, token) order, same routing rule and kernels, "
                         "no probes or correction",
           "support": support}
    del cop
    return out


def support_blocks(p):
    """Eight query blocks spread over head 0, the first and the ragged last included."""
    import numpy as np
    return sorted(set(np.linspace(0, p.n_blocks - 1, 8).round().astype(int).tolist()))


def random_block_support(p, Q, K, V, scale, inp):
    """The random-block partition (no probes, same density) on the same inputs:
    its support diagnostics."""
    import dataclasses
    import torch
    from free_block_sparse_rcp_amd import binding

    pr = dataclasses.replace(p, partition_mode=binding.RANDOM_BLOCK, n_probes=0, rank=0)
    op = binding.SparsePR(pr, Q.device)
    idx = op.upload_indices(rand_key_perm=inp.rand_key_perm, rand_query_perm=inp.rand_query_perm)
    op.run(Q, K, V, scale, idx)
    torch.cuda.synchronize()
    out = support_summary(pr, op.buffers, Q, K, scale, support_blocks(p))
    del op
    return out


def unprobed_mask(p, b):
    """[H, N] token mask of the rows that are not probe rows of this call."""
    import torch
    H, N = p.heads, p.n_tokens
    mask = torch.ones(H, N, dtype=torch.bool, device=b.S.device)
    if p.n_probes:
        pos = torch.tensor([((2 * i + 1) * N) // (2 * p.n_probes) for i in range(p.n_probes)],
                           dtype=torch.long, device=b.S.device)
        mask.scatter_(1, b.query_perm.long().gather(1, pos[None].expand(H, -1)), False)
    return mask


def error_summary(p, b, ref, rn, mask):
    """Per-query relative L2 error against the dense output over all unprobed
    rows of every head (mean and 99th percentile, linear interpolation), for
    the corrected output and for the sparse output alone (hard drop)."""
    import numpy as np
    import torch
    D = p.head_dim
    with torch.no_grad():
        S_tok = torch.empty_like(b.S, dtype=torch.float32)
        S_tok.scatter_(1, b.query_perm.long()[:, :, None].expand(-1, -1, D), b.S.float())
        e = ((b.O.float() - ref).norm(dim=2) / rn)[mask].double().cpu().numpy()
        e0 = ((S_tok - ref).norm(dim=2) / rn)[mask].double().cpu().numpy()
    return {"rel_l2_mean_unprobed": float(e.mean()),
            "rel_l2_p99_unprobed": float(np.percentile(e, 99)),
            "hard_drop_rel_l2_mean": float(e0.mean()),
            "hard_drop_rel_l2_p99": float(np.percentile(e0, 99)),
            "correction_minus_hard_drop": float(e.mean() - e0.mean()),
            "rows": int(e.size)}


def residual_r2(p, b, ref, mask):
    """How affine-predictable the dense-minus-sparse residual is under one
    call's partition: R^2 of the fitted map r = U Theta^T [s; 1] on the rows the
    fit did not see (every unprobed row), against R = O_dense - S. Pooled over
    heads; each head's R is centred on its own mean over those rows."""
    import torch
    D = p.head_dim
    with torch.no_grad():
        S_tok = torch.empty_like(b.S, dtype=torch.float32)
        S_tok.scatter_(1, b.query_perm.long()[:, :, None].expand(-1, -1, D), b.S.float())
        num = den = 0.0
        for h in range(p.heads):
            m = mask[h]
            s = S_tok[h][m].double()
            R = ref[h][m].double() - s
            k = int(b.rank_eff[h].item())
            if k > 0:
                xa = torch.cat([s, torch.ones_like(s[:, :1])], dim=1)
                R_hat = (xa @ b.Theta[h][:, :k].double()) @ b.U[h][:, :k].double().T
            else:
                R_hat = torch.zeros_like(R)
            num += float(((R - R_hat) ** 2).sum())
            den += float(((R - R.mean(dim=0)) ** 2).sum())
    return 1.0 - num / den if den > 0 else float("nan")


def comparator_r2(p, mode, Q, K, V, scale, inp, ref):
    """Residual R^2 under another partition (random-block or semantic), with the
    same probe count, rank and ridge as the response-coupled call."""
    import dataclasses
    import torch
    from free_block_sparse_rcp_amd import binding

    pc = dataclasses.replace(p, partition_mode=mode)
    op = binding.SparsePR(pc, Q.device)
    if mode == binding.RANDOM_BLOCK:
        idx = op.upload_indices(rand_key_perm=inp.rand_key_perm, rand_query_perm=inp.rand_query_perm)
    else:
        idx = op.upload_indices(init_idx=inp.init_idx)
    op.run(Q, K, V, scale, idx)
    torch.cuda.synchronize()
    out = residual_r2(pc, op.buffers, ref, unprobed_mask(pc, op.buffers))
    del op
    return out


def cpu_baseline(wl, inp, block_stride):
    """The fp64 oracle, as it stands, on the heads held by `inp` (the bench
    passes heads 0, H/2 and H-1 of the same workload): every stage in the
    pages' order; the block-sparse attention step runs on every
    `block_stride`-th query block and its time is scaled by executed pairs.
    Throughput is executed-pair flops over the scaled time, summed over the
    timed heads."""
    import numpy as np
    from oracle import sparsepr_oracle as orc
    try:
        from threadpoolctl import threadpool_info
        cores = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        cores = os.cpu_count() or 1
    p = wl.params
    N = p.n_tokens
    t = {"partition": 0.0, "route": 0.0, "attend_sampled": 0.0, "attend_scaled": 0.0,
         "probe_fit_apply": 0.0}
    flops = 0.0
    n_sel = n_blocks = 0
    for i, h in enumerate(inp.heads):
        Q, K, V = (x[i].astype(np.float64) for x in (inp.Q, inp.K, inp.V))
        tau = float(inp.scale[i])
        t0 = time.perf_counter()
        if p.partition_mode == 0:
            R = orc.key_responses(Q, K, tau, inp.sample_idx)
            labels = orc.kmeans(R, inp.init_idx, p.kmeans_iters).labels
            del R
        else:
            labels = orc.random_block_labels(inp.rand_key_perm, p.n_groups)
        key_perm, group_off, sizes = orc.group_members(labels, p.n_groups)
        kbar, _ = orc.key_centroids(K, labels, p.n_groups)
        t["partition"] += time.perf_counter() - t0
        t0 = time.perf_counter()
        C = orc.query_coordinates(Q, kbar, tau)
        g1, v = orc.dominant_groups(C, sizes)
        qperm = orc.query_order(g1, v) if p.partition_mode == 0 else np.asarray(inp.rand_query_perm)
        blocks = orc.query_blocks(qperm, p.q_block)
        sigma = orc.block_scores(C, blocks)
        del C
        bptr, bgrp = orc.route(sigma, sizes, orc.key_budget(N, p.density, p.n_probes))
        ksets = orc.block_key_sets(bptr, bgrp, key_perm, group_off)
        t["route"] += time.perf_counter() - t0
        E = orc.executed_pairs(blocks, ksets, p.n_probes, N)
        flops += 4.0 * p.head_dim * E
        sp_all = E - p.n_probes * N
        sel = list(range(i % block_stride, len(blocks), block_stride))
        n_sel += len(sel)
        n_blocks += len(blocks)
        sp_sample = sum(len(blocks[b]) * len(ksets[b]) for b in sel)
        t0 = time.perf_counter()
        S, _ = orc.sparse_attention(Q, K, V, tau, [blocks[b] for b in sel], [ksets[b] for b in sel])
        dt = time.perf_counter() - t0
        t["attend_sampled"] += dt
        t["attend_scaled"] += dt * sp_all / max(sp_sample, 1)
        t0 = time.perf_counter()
        ptok = qperm[orc.probe_positions(N, p.n_probes)]
        Op, _ = orc.dense_attention(Q, K, V, tau, rows=ptok)
        _, U, _, Th = orc.fit_probe_map(S[ptok], Op, p.rank, p.ridge_lambda)
        O = S + orc.predicted_residual(S, U, Th)
        O[ptok] = Op
        t["probe_fit_apply"] += time.perf_counter() - t0
    total = t["partition"] + t["route"] + t["attend_scaled"] + t["probe_fit_apply"]
    spent = t["partition"] + t["route"] + t["attend_sampled"] + t["probe_fit_apply"]
    nh = len(inp.heads)
    return {"value": flops / total / 1e12, "unit": "TFLOP/s", "cores": int(cores), "kind": "oracle",
            "sample": f"heads {list(inp.heads)} of {p.heads}: every oracle stage in order; sparse "
                      f"attention on {n_sel} of {n_blocks} query blocks (every {block_stride}th "
                      f"per head), time scaled by executed pairs; {spent:.1f} s of CPU time",
            "stage_seconds": t, "call_ms_scaled_all_heads": total * 1e3 * p.heads / nh}


def run_sweep(args):
    """Sensitivity sweep on the sweep workload (32 heads, N = 65536: heads 0-15
    concentrated, 16-31 broad): probes per head x executed-pair density x
    partition (response-coupled or random-block), one JSON line per point.
    Each point: call ms (HIP events, mean of the timed calls), realized
    density, and against this build's dense output the per-query relative
    error of the corrected and of the uncorrected (hard-drop) output over all
    unprobed rows, overall and per head half, with the residual R^2 of the
    fitted map. The inputs and the dense output are made once."""
    import dataclasses
    import numpy as np
    import torch
    from free_block_sparse_rcp_amd import binding, configs

    binding.load()
    wl = configs.get(args.config)
    dev = torch.device("cuda:0")
    log(f"[sweep] generating {wl.name}")
    inp = wl.make_inputs()
    p0 = wl.params
    dt = binding.torch_dtype(p0)
    Q, K, V = (torch.from_numpy(x).to(dev, dt) for x in (inp.Q, inp.K, inp.V))
    scale = torch.from_numpy(inp.scale).to(dev)
    O_dense = torch.empty_like(Q)
    binding.dense_attention(p0, Q, K, V, scale, O_dense)
    torch.cuda.synchronize()
    ref = O_dense.float()
    rn = ref.norm(dim=2)
    del O_dense
    H = p0.heads
    halves = {"concentrated": [h for h in range(H) if inp.scale[h] > inp.scale.min()],
              "broad": [h for h in range(H) if inp.scale[h] == inp.scale.min()]}
    modes = ((0, "response_coupled"), (1, "random_block"))
    n_timed = max(1, args.steps)
    for mode, mode_name in modes:
        for rho in configs.SWEEP_DENSITIES:
            for m in configs.SWEEP_PROBES:
                p = dataclasses.replace(p0, density=rho, n_probes=m, partition_mode=mode)
                log(f"[sweep] {mode_name} rho={rho} m={m}")
                op = binding.SparsePR(p, dev)
                idx = op.upload_indices(inp.sample_idx, inp.init_idx, inp.rand_key_perm,
                                        inp.rand_query_perm)
                for _ in range(max(1, args.warmup)):
                    op.run(Q, K, V, scale, idx)
                evs = [dict() for _ in range(n_timed)]
                for e in evs:
                    op.run(Q, K, V, scale, idx, events=e)
                torch.cuda.synchronize()
                call_ms = float(np.mean([e["start"].elapsed_time(e["apply"]) for e in evs]))
                b = op.buffers
                E = int(b.executed_pairs.sum().item())
                mask = unprobed_mask(p, b)
                err = error_summary(p, b, ref, rn, mask)
                per_half = {}
                for name, hs in halves.items():
                    hm = torch.zeros_like(mask)
                    hm[hs] = mask[hs]
                    per_half[name] = {k: v for k, v in error_summary(p, b, ref, rn, hm).items()
                                      if k != "rows"}
                line = {"sweep_point": {"partition": mode_name, "density_target": rho,
                                        "n_probes": m, "rank": p.rank},
                        "workload": wl.name, "call_ms": call_ms, "timed_calls": n_timed,
                        "executed_pairs": E,
                        "realized_density": E / (H * float(p.n_tokens) ** 2),
                        "key_budget": p.key_budget, **err, "by_head_type": per_half,
                        "residual_r2": residual_r2(p, b, ref, mask),
                        "reference": "this build's dense kernel (bf16 output)"}
                print(json.dumps(line), flush=True)
                del op, b
                torch.cuda.empty_cache()


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--config", default=None,
                    help="workload (default hunyuan; the sweep runs on the sweep workload)")
    ap.add_argument("--sweep", action="store_true",
                    help="probes x density x partition sensitivity sweep on the sweep workload, "
                         "one JSON line per point")
    ap.add_argument("--cpu-block-stride", type=int, default=0,
                    help="oracle samples every n-th query block (0: chosen by workload size)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-dense", action="store_true")
    ap.add_argument("--no-comparator", action="store_true",
                    help="skip the semantic block-sparse comparator (error reduction)")
    ap.add_argument("--overlap", action="store_true",
                    help="attend the blocks holding probe rows first and run the probe fit on a "
                         "second stream while the other blocks are attended (default: the five "
                         "stages back to back on one stream)")
    ap.add_argument("--static-attention", action="store_true",
                    help="deal the attention's query blocks out statically, one workgroup each "
                         "(default: a persistent grid taking blocks from per-XCD work queues)")
    ap.add_argument("--calibration-copy-mib", type=int, default=0,
                    help="also run one plain device copy of this many MiB (a known-size "
                         "kernel for scaling the FETCH_SIZE / WRITE_SIZE counters)")
    ap.add_argument("--pmc-table", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="write a per-kernel HBM traffic table from two rocprofv3 --pmc runs "
                         "(FETCH_SIZE, WRITE_SIZE) that include the calibration copy")
    ap.add_argument("--pmc-summary", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="summarise two rocprofv3 PMC runs of this script (FETCH_SIZE, "
                         "WRITE_SIZE) into profiles/attend_traffic_<workload>.json and exit")
    args = ap.parse_args()
    args.config = args.config or ("sweep" if args.sweep else "hunyuan")
    if args.pmc_table:
        from free_block_sparse_rcp_amd import configs
        pmc_table(args.pmc_table[0], args.pmc_table[1], configs.get(args.config).name,
                  args.calibration_copy_mib or 1024)
        return
    if args.pmc_summary:
        from free_block_sparse_rcp_amd import configs
        pmc_summary(args.pmc_summary[0], args.pmc_summary[1], configs.get(args.config).name,
                    args.calibration_copy_mib or 1024)
        return
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only: the operator is per call and per head, and this "
              f"build has no multi-GPU path (asked for --gpus {args.gpus}).", file=sys.stderr)
        sys.exit(2)
    if args.sweep:
        run_sweep(args)
        return

    import numpy as np
    import torch
    from free_block_sparse_rcp_amd import binding, configs

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    binding.load()
    wl = configs.get(args.config)
    p = wl.params
    dev = torch.device("cuda:0")
    log(f"[bench] generating {wl.name}")
    t0 = time.perf_counter()
    inp = wl.make_inputs()
    log(f"[bench] inputs ready in {time.perf_counter() - t0:.1f} s")
    dt = binding.torch_dtype(p)
    Q, K, V = (torch.from_numpy(x).to(dev, dt) for x in (inp.Q, inp.K, inp.V))
    scale = torch.from_numpy(inp.scale).to(dev)
    use_queue = not args.static_attention
    op = binding.SparsePR(p, dev, use_queue=use_queue)
    idx = op.upload_indices(inp.sample_idx, inp.init_idx, inp.rand_key_perm, inp.rand_query_perm)
    b = op.buffers
    O_dense = torch.empty_like(Q)
    lse_dense = torch.empty(p.heads, p.n_tokens, dtype=torch.float32, device=dev)
    dense_queue = torch.empty(binding.QUEUE_BYTES, dtype=torch.uint8, device=dev)

    def dense_call():
        binding.dense_attention(p, Q, K, V, scale, O_dense, lse_dense, queue=dense_queue,
                                use_queue=use_queue)

    stages = ("partition", "route", "attend", "probe_fit", "apply")

    overlap = args.overlap

    def one_call(ev=None):
        op.run(Q, K, V, scale, idx, overlap=overlap, events=ev)

    if args.calibration_copy_mib:
        n = args.calibration_copy_mib * (1 << 20) // 4
        src = torch.ones(n, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        torch.neg(src, out=dst)   # reads and writes exactly n * 4 bytes
        torch.cuda.synchronize()
        del src, dst

    log(f"[bench] warmup {args.warmup}")
    for _ in range(args.warmup):
        one_call()
        if not args.no_dense:
            dense_call()
    torch.cuda.synchronize()

    # timed region: K whole calls, events between stages (on the library's streams)
    log(f"[bench] timing {args.steps} calls ({'overlapped' if overlap else 'serial'})")
    evs = [dict() for _ in range(args.steps)]
    torch.cuda.synchronize()
    w0 = time.perf_counter()
    for s in range(args.steps):
        one_call(evs[s])
    torch.cuda.synchronize()
    wall = time.perf_counter() - w0

    def span(e, a, b):
        return e[a].elapsed_time(e[b])

    if overlap:
        parts = {"partition": ("start", "partition"), "route": ("partition", "route"),
                 "attend_probe_blocks": ("route", "attend_probe_blocks"),
                 "attend_other_blocks": ("attend_probe_blocks", "attend"),
                 "probe_fit": ("probe_fit_start", "probe_fit"), "apply": ("join", "apply")}
    else:
        parts = {"partition": ("start", "partition"), "route": ("partition", "route"),
                 "attend": ("route", "attend"), "probe_fit": ("attend", "probe_fit"),
                 "apply": ("probe_fit", "apply")}
    stage_ms = {n: float(np.mean([span(e, a_, b_) for e in evs])) for n, (a_, b_) in parts.items()}
    if overlap:
        stage_ms["attend"] = stage_ms["attend_probe_blocks"] + stage_ms["attend_other_blocks"]
    attend_launches = 2 if overlap else 1
    call_ms = float(np.mean([span(e, "start", "apply") for e in evs]))

    dense_ms = None
    if not args.no_dense:
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record()
        for _ in range(args.steps):
            dense_call()
        e1.record()
        torch.cuda.synchronize()
        dense_ms = e0.elapsed_time(e1) / args.steps

    E = int(b.executed_pairs.sum().item())
    H, N, D = p.heads, p.n_tokens, p.head_dim
    sparse_pairs = E - H * p.n_probes * N
    call_tflops = 4.0 * D * E / (call_ms * 1e-3) / 1e12
    attend_tflops = 4.0 * D * sparse_pairs / (stage_ms["attend"] * 1e-3) / 1e12
    density = E / (H * float(N) ** 2)

    # quality on this synthetic call, against the build's own dense output
    quality = None
    if not args.no_dense:
        with torch.no_grad():
            ref = O_dense.float()
            mask = unprobed_mask(p, b)
            rn = ref.norm(dim=2)
        quality = {"reference": "this build's dense kernel (bf16 output)",
                   **error_summary(p, b, ref, rn, mask)}
        e_mean = quality["rel_l2_mean_unprobed"]
        if not args.no_comparator:
            quality["semantic"] = semantic_comparator(args, p, Q, K, V, scale, inp, ref, rn, mask,
                                                      e_mean)
            log("[bench] support diagnostics")
            quality["support"] = {
                "mass": SUPPORT_MASS, "head": 0, "blocks": support_blocks(p),
                "response_coupled": support_summary(p, b, Q, K, scale, support_blocks(p)),
                "semantic": quality["semantic"].pop("support"),
                "random_block": random_block_support(p, Q, K, V, scale, inp)}
            if p.n_probes and p.rank:
                log("[bench] residual R^2 per partition")
                quality["residual_r2"] = {
                    "response_coupled": residual_r2(p, b, ref, mask),
                    "random_block": comparator_r2(p, binding.RANDOM_BLOCK, Q, K, V, scale, inp, ref),
                    "semantic": comparator_r2(p, binding.SEMANTIC, Q, K, V, scale, inp, ref),
                    "definition": "1 - sum |R - U Theta^T [s;1]|^2 / sum |R - mean R|^2 over unprobed "
                                  "rows, R = dense - sparse output; same m, k, lambda per partition"}

    traffic = load_traffic(wl.name)
    roofline = {"bound": "mfma", "kernel": "k_attn_mfma (sparsepr_attend)",
                "achieved": attend_tflops, "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                "frac": attend_tflops / PEAK_BF16_TFLOPS, "traffic": traffic,
                "algorithmic_flops_per_launch": 4.0 * D * sparse_pairs / attend_launches,
                "launch_ms": stage_ms["attend"] / attend_launches,
                "launches_per_call": attend_launches}

    cpu = None
    if not args.no_cpu_baseline:
        stride = args.cpu_block_stride or max(1, int(round(8.0 * N / 118800)))
        heads = sorted({0, H // 2, H - 1})
        log(f"[bench] cpu baseline (oracle), heads {heads}, block stride {stride}")
        sub = inp if H == 1 else wl.make_inputs(heads)
        cpu = cpu_baseline(wl, sub, stride)

    out = {
        "metric": METRIC, "value": call_tflops, "unit": "TFLOP/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": call_ms,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": p.dtype,
        "data": "synthetic",
        "config": {"workload": wl.name, "heads": H, "n_tokens": N, "head_dim": D,
                   "density_target": p.density, "n_probes": p.n_probes, "n_groups": p.n_groups,
                   "n_samples": p.n_samples, "kmeans_iters": p.kmeans_iters,
                   "q_block": p.q_block, "rank": p.rank, "ridge_lambda": p.ridge_lambda},
        "call_ms": call_ms, "dense_ms": dense_ms,
        "speedup_vs_dense": (dense_ms / call_ms) if dense_ms else None,
        "attend_speedup_vs_dense": (dense_ms / stage_ms["attend"]) if dense_ms else None,
        "stage_ms": stage_ms, "wall_ms_per_step": wall * 1e3 / args.steps,
        "reconstruction_share": (stage_ms["probe_fit"] + stage_ms["apply"]) / call_ms,
        "pipeline": ("probe blocks attended first; probe fit on a second stream overlaps the "
                     "attention of the other blocks" if overlap else "stages back to back"),
        "attention_blocks": ("per-XCD work queues, persistent grid" if use_queue
                             else "static, one workgroup per block"),
        "executed_pairs": E, "realized_density": density,
        "dense_tflops": (4.0 * D * H * float(N) ** 2 / (dense_ms * 1e-3) / 1e12) if dense_ms else None,
        "quality": quality, "roofline": roofline, "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
