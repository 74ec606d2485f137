"""Throughput of the LLaTTE target-aware MLA forward on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--config c3]
    python bench.py --workload actions     (the action tokenization)
    python bench.py --workload summaries   (the LoRAMLP sequence summaries)
    python bench.py --workload backward    (the attention-core backward)
    python bench.py --workload ffn_backward (the FFN-sublayer backward)
    python bench.py --workload sublayer_backward (the attention-sublayer backward)
    python bench.py --workload compact     (the pyramid compaction, HBM-bound)
    python bench.py --workload vendor_gemm (hipBLASLt on the c3 layer-1 shapes, a reference)
    python bench.py --workload stack_backward (the whole-stack training backward)
    python bench.py --config c5            (the 12-layer stack with the token build)
    python bench.py --attn-phases          (adds the attention kernel's phase breakdown)
    python bench.py --gemm-phases          (adds the 128x128 GEMM tile's phase breakdown)

One step is one llatte_mla_forward over one batch of the workload (all
layers, the pyramid, the readout), inputs and weights already resident in
HBM. Prints ONE JSON line: user-sequences/s as `value`, TFLOP/s of the fixed
absorbed-form FLOP count (and its fraction of the bf16 MFMA peak), the
roofline of the dominant kernel (HIP events around each of its launches,
recorded by the library on the launch stream, over a second pass of the same
K steps), and the CPU oracle timed on a bounded sample of the same workload.
"""
import argparse
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
PEAK_F32_TFLOPS = 157.3     # MI355X fp32 (vector / MFMA dense)
PEAK_HBM_GBS = 8000.0

METRIC = ("user-sequences/sec + TFLOP/s (% MFMA bf16 peak), MLA stack at "
          "L=1600, 1 GPU")

WORKLOAD_TEXT = {
    "c1": "c1: 1 layer fp32, B=4, L=32, d=64, 2x32 heads, r=16, 4 candidates",
    "c2": "c2: online ranker, 3 layers bf16, B=256, L=400, d=256, 4x64, r=64, "
          "16 candidates, pyramid 400-200-100",
    "c3": "c3: upstream user model, 6 layers bf16, B=64, L=1600, d=512, 8x64 "
          "heads, r=128, pyramid 1600-800-400-200-100-50, 4-seed readout to 2048",
    "c4": "c4: jagged batch, 4 layers bf16, 128 users L~U[200,1600], d=256, "
          "4x64, r=64, 8 candidates, halving pyramid floor 64",
    "c5": "c5: 12 layers bf16, B=32, L=1600, d=1024, 16x64 heads, r=256, 16 candidates, "
          "geometric pyramid 1600->50, tokens built from a 1M x 1024 hashed-ID table + "
          "384-d semantic vectors (in the step)",
}


def layer_counts(cfg, lengths):
    """Per layer (incl. readout): (sum K, sum n, query rows M, allowed pairs)."""
    from target_aware_latent_amd import llatte as C
    from target_aware_latent_amd.model import make_desc
    keep = np.array(C.llatte_pyramid_counts_host(make_desc(cfg).pyramid, cfg.N,
                                                 list(lengths)), dtype=np.int64)
    out = []
    K = np.asarray(lengths, dtype=np.int64)
    for l in range(cfg.N + (1 if cfg.n_seeds else 0)):
        n = keep[l] if l < cfg.N else np.zeros_like(K)
        nq = cfg.n_q if l < cfg.N else cfg.n_seeds
        pairs = int(np.sum(n * (K - n) + n * (n + 1) // 2 + nq * K))
        out.append((int(K.sum()), int(n.sum()), int(n.sum()) + cfg.B * nq, pairs))
        K = n
    return out


def kernel_flops(cfg, lengths):
    """Algorithmic FLOPs per step by kernel label: 2mnk per product and
    4*r*h per allowed (query, key) pair (absorbed form)."""
    d, h, dk, r, dff = cfg.d, cfg.h, cfg.dk, cfg.r, 4 * cfg.d
    f = {}
    add = lambda k, v: f.__setitem__(k, f.get(k, 0) + v)
    for Ks, ns, M, pairs in layer_counts(cfg, lengths):
        add("gemm_down", 2 * Ks * d * r)
        if cfg.r_q:  # low-rank query path
            add("gemm_qdown", 2 * M * d * cfg.r_q)
            add("gemm_q", 2 * M * cfg.r_q * h * dk)
        else:
            add("gemm_q", 2 * M * d * h * dk)
        if cfg.dtype == "bf16":
            # the attention kernel also applies W_uk (prologue) and W_uv
            # (epilogue) of the absorbed form
            add("attention_mfma", 4 * r * h * pairs + 2 * (2 * M * h * dk * r))
        else:
            add("gemm_absorb_uk", 2 * M * h * dk * r)
            add("attention_f32", 4 * r * h * pairs)
            add("gemm_absorb_uv", 2 * M * h * r * dk)
        add("gemm_out", 2 * M * h * dk * d)
        add("gemm_ffn1", 2 * M * d * dff)
        add("gemm_ffn2", 2 * M * dff * d)
    if cfg.n_q:
        add("gemm_fusion", 2 * cfg.B * cfg.n_q * (d + cfg.d_c) * d)
    if cfg.n_seeds:
        add("gemm_readout", 2 * cfg.B * cfg.n_seeds * d * cfg.d_out)
    if cfg.semantic is not None:  # token build: semantic vector times W_s
        add("gemm_token_embed", 2 * (int(np.sum(lengths)) + cfg.B * cfg.n_q) * cfg.semantic.d_sem * d)
    return f


def family_bytes(cfg, lengths):
    """Algorithmic HBM bytes per step of the two kernel symbols (bf16 path):
    every operand read once, every result written once. GEMM family, per
    layer: W_dkv reads the KV rows (2d B) and writes the fp16 latent (2r B);
    W_uq reads the gathered rows (2d) and writes q (2 h dk); W_o reads o
    (2 h dk) and the fp32 residual (4d) and writes the fp32 result and its
    bf16 copy (4d + 2d); W1 reads that copy (2d) and writes the hidden layer
    (2 d_ff); W2 reads it (2 d_ff) and the fp32 residual (4d) and writes the
    fp32 result (4d), plus its bf16 copy (2d) except at the last layer; the
    weights once per layer; the readout's W_p product its rows, W_p and the
    embedding. Attention: q and o rows (2 h dk each), the fp16 latent rows
    (2r), W_uk and W_uv once per layer."""
    d, h, dk, r, dff = cfg.d, cfg.h, cfg.dk, cfg.r, 4 * cfg.d
    hd = h * dk
    g = a = 0
    layers = layer_counts(cfg, lengths)
    for l, (Ks, ns, M, pairs) in enumerate(layers):
        last = l == cfg.N - 1 or l >= cfg.N
        g += Ks * (2 * d + 2 * r) + M * (2 * d + 2 * hd)
        g += M * (2 * hd + 4 * d + 4 * d + 2 * d) + M * (2 * d + 2 * dff)
        g += M * (2 * dff + 4 * d + 4 * d + (0 if last else 2 * d))
        g += 2 * (d * r + d * hd + hd * d + 2 * d * dff)
        a += M * (2 * hd + 2 * hd) + Ks * 2 * r + 2 * (2 * r * hd)
    if cfg.n_seeds:
        g += cfg.B * cfg.n_seeds * d * 2 + cfg.n_seeds * d * cfg.d_out * 2 + cfg.B * cfg.d_out * 4
    return {"gemm_kernel": g, "attn_mfma_kernel": a}


def absorbed_flops(cfg, lengths):
    return sum(kernel_flops(cfg, lengths).values())


def non_absorbed_flops(cfg, lengths):
    d, h, dk, r, dff = cfg.d, cfg.h, cfg.dk, cfg.r, 4 * cfg.d
    t = 0
    for Ks, ns, M, pairs in layer_counts(cfg, lengths):
        qproj = (2 * M * d * cfg.r_q + 2 * M * cfg.r_q * h * dk) if cfg.r_q else 2 * M * d * h * dk
        t += 2 * Ks * d * r + qproj + 2 * (2 * Ks * r * h * dk)
        t += 4 * dk * h * pairs + 2 * M * h * dk * d + 2 * (2 * M * d * dff)
    if cfg.n_q:
        t += 2 * cfg.B * cfg.n_q * (d + cfg.d_c) * d
    if cfg.n_seeds:
        t += 2 * cfg.B * cfg.n_seeds * d * cfg.d_out
    if cfg.semantic is not None:
        t += 2 * (int(np.sum(lengths)) + cfg.B * cfg.n_q) * cfg.semantic.d_sem * d
    return t


def gemm_phases(cfg, lengths, step):
    """One forward with the phase stamps of the 128 x 128 GEMM tile: per
    instrumented product launch (W_dkv, W_uq, W_o, W1, W2 of the large
    layers, in launch order) the workgroups' summed wait for their first
    operands, K loop and epilogue, the launch span, and each phase's share
    of workgroup time. `*_us_est` spreads the span over the phases by those
    shares (two workgroups share a CU); `loop_tflops_est` divides the
    product's 2MNK by the loop's estimate."""
    import torch
    from target_aware_latent_amd import llatte as C
    d, hd, r, dff = cfg.d, cfg.h * cfg.dk, cfg.r, 4 * cfg.d
    # products by shape; W_uq and W_o share one when h d_k = d, and each
    # layer launches W_uq first, so equal shapes alternate in launch order
    names = {}
    for shape, name in (((r, d), "down"), ((hd, d), "q"), ((d, hd), "out"), ((dff, d), "ffn1"),
                        ((d, dff), "ffn2")):
        names.setdefault(shape, []).append(name)
    count = {}
    torch.cuda.synchronize()
    C.llatte_gemm_phases_enable(1 << 20)
    try:
        step()
        torch.cuda.synchronize()
        recs = C.llatte_gemm_phases_read()
    finally:
        C.llatte_gemm_phases_enable(0)
    seen, out = {}, []
    for rc in recs:
        shape = (int(rc["N"]), int(rc["K"]))
        cands = names.get(shape, ["other"])
        count[shape] = count.get(shape, 0) + 1
        name = cands[(count[shape] - 1) % len(cands)]
        seen[name] = seen.get(name, 0) + 1
        e = {k: round(v, 2) for k, v in rc.items()}
        e["product"], e["layer"] = name, seen[name]
        tot = rc["first_us"] + rc["loop_us"] + rc["epilogue_us"]
        if tot > 0:
            for ph in ("first", "loop", "epilogue"):
                share = rc[ph + "_us"] / tot
                e[ph + "_share"] = round(share, 4)
                e[ph + "_us_est"] = round(rc["span_us"] * share, 2)
            est = e["loop_us_est"]
            e["loop_tflops_est"] = round(2 * rc["M"] * rc["N"] * rc["K"] / (est * 1e-6) / 1e12, 1) \
                if est > 0 else None
        out.append(e)
    return out


def attention_phases(cfg, lengths, step):
    """One forward with the attention kernel's phase stamps: per launch (one
    per layer, then the readout) the workgroups' summed time in the W_uk
    prologue, the key loop and the W_uv epilogue, the launch span, and each
    phase's share of workgroup time. `*_us_est` spreads the span over the
    phases by those shares (two workgroups share a CU, so summed workgroup
    time exceeds the span); the rates divide each phase's algorithmic FLOPs
    by that estimate."""
    import torch
    from target_aware_latent_amd import llatte as C
    h, dk, r = cfg.h, cfg.dk, cfg.r
    torch.cuda.synchronize()
    C.llatte_attention_phases_enable(1 << 20)
    try:
        step()
        torch.cuda.synchronize()
        recs = C.llatte_attention_phases_read()
    finally:
        C.llatte_attention_phases_enable(0)
    lc = layer_counts(cfg, lengths)
    out = []
    for i, rc in enumerate(recs):
        e = {k: round(v, 2) for k, v in rc.items()}
        tot = rc["prologue_us"] + rc["loop_us"] + rc["epilogue_us"]
        if i < len(lc) and tot > 0:
            Ks, ns, M, pairs = lc[i]
            e["layer"] = i + 1 if i < cfg.N else "readout"
            e["query_rows"], e["allowed_pairs"] = M, pairs
            fl = {"prologue": 2 * M * h * dk * r, "loop": 4 * r * h * pairs,
                  "epilogue": 2 * M * h * dk * r}
            for ph, f in fl.items():
                share = rc[ph + "_us"] / tot
                est = rc["span_us"] * share
                e[ph + "_share"] = round(share, 4)
                e[ph + "_us_est"] = round(est, 2)
                e[ph + "_tflops_est"] = round(f / (est * 1e-6) / 1e12, 1) if est > 0 else None
        out.append(e)
    return out


def family_of(label):
    """Kernel symbol behind a timing label: the matrix products all run the
    GEMM kernel template; the attention labels the attention kernel."""
    if label.startswith("gemm_"):
        return "gemm_kernel"
    if label.startswith("attention_mfma"):
        return "attn_mfma_kernel"
    return label


def kernel_source(label):
    """Source file of the kernel behind a timing label or symbol."""
    name = ("attention.hip" if label.startswith(("attention", "attn")) else
            "plan.hip" if label == "pyramid_compact" else "gemm.hip")
    return os.path.join(ROOT, "target_aware_latent_amd", "csrc", name)


def read_traffic(path, label):
    """HBM bytes per launch of `label` from the RECORD line of a profile
    summary (`path`, or every profiles/c3_*_hbm_traffic.txt when None), or
    None when there is none or the kernel changed since it was taken."""
    import glob
    paths = [path] if path else sorted(glob.glob(os.path.join(ROOT, "profiles",
                                                              "c3_*_hbm_traffic.txt")))
    from target_aware_latent_amd.profsum import fingerprint
    for p in paths:
        if not os.path.exists(p):
            continue
        for line in open(p):
            if line.startswith("RECORD "):
                rec = json.loads(line[len("RECORD "):])
                if rec.get("kernel") == label and \
                        rec.get("fingerprint") == fingerprint(kernel_source(label)):
                    return rec.get("bytes")
    return None


def host_desc():
    """The host the CPU baseline ran on: CPU model and the BLAS numpy links."""
    model = blas = None
    try:
        with open("/proc/cpuinfo") as f:
            model = next((l.split(":", 1)[1].strip() for l in f if l.startswith("model name")), None)
    except OSError:
        pass
    try:
        b = np.show_config(mode="dicts")["Build Dependencies"]["blas"]
        blas = f"{b.get('name', '')} {b.get('version', '')}".strip() or None
    except Exception:
        pass
    return {"cpu_model": model, "blas": blas}


def emit(rec):
    """Prints the one JSON line; a CPU baseline gets the host description."""
    if isinstance(rec.get("cpu_baseline"), dict):
        rec["cpu_baseline"].update(host_desc())
    print(json.dumps(rec))


def _blas_threads():
    try:
        from threadpoolctl import threadpool_info
        return sum(p.get("num_threads", 0) for p in threadpool_info()
                   if p.get("user_api") == "blas") or None
    except Exception:
        return None


def cpu_baseline(prob, budget_s=36.0):
    """The oracle as it stands, in fp32 on the host cores: the median of
    three passes over the whole batch when three fit in about budget_s
    seconds, else the median of three passes over the first users whose pass
    takes about a third of it (at least one user)."""
    from oracle import llatte_oracle as O
    cfg, I, W = prob["cfg"], prob["inputs"], prob["weights"]
    threads = _blas_threads()

    def one_pass(users):
        t0 = time.perf_counter()
        O.forward(cfg, W, I["hist"], I["offsets"], I.get("cand"), I.get("ctx"),
                  users=users, dtype=np.float32)
        return time.perf_counter() - t0

    # a warm pass of the first user alone sizes the sample
    one_pass([0])
    t1 = one_pass([0])
    n = min(cfg.B, max(1, int(budget_s / 3 / max(t1, 1e-6))))
    users = list(range(n))
    times = sorted(one_pass(users) for _ in range(3))
    med = times[1]
    what = "the whole batch" if n == cfg.B else f"the first {n} of {cfg.B} users"
    return {"value": n / med, "unit": "user-seq/s",
            "cores": threads or len(os.sched_getaffinity(0)), "kind": "oracle",
            "affinity_cores": len(os.sched_getaffinity(0)), "blas_threads": threads,
            "sample": f"median of 3 passes over {what} of the same workload "
                      f"({', '.join(f'{t:.2f}' for t in times)} s), fp32 oracle "
                      f"(non-absorbed definition)"}


def cpu_baseline_tokens(prob, host_table, budget_s=12.0):
    """The same for a token-built workload: a user's table rows are gathered
    from the host copy of the table outside the timed region; the oracle's
    token build and forward of that user are timed."""
    from oracle import llatte_oracle as O
    import synth
    cfg, I, W = prob["cfg"], prob["inputs"], prob["weights"]
    off, nq = I["offsets"], cfg.n_q
    hist = np.zeros((int(off[-1]), cfg.d), np.float32)
    cand = np.zeros((cfg.B * nq, cfg.d), np.float32)
    Ws = W["W_s"].astype(np.float32)
    users, dt = 0, 0.0
    while users < cfg.B and dt < budget_s:
        u = users
        # the rows as the device holds them (bf16-rounded)
        hr = synth.round_bf16(host_table[I["hist_ids"][off[u]:off[u + 1]]])
        cr = synth.round_bf16(host_table[I["cand_ids"][u * nq:(u + 1) * nq]])
        t0 = time.perf_counter()
        hist[off[u]:off[u + 1]] = O.token_embed(hr, I["hist_sem"][off[u]:off[u + 1]].astype(np.float32), Ws)
        cand[u * nq:(u + 1) * nq] = O.token_embed(cr, I["cand_sem"][u * nq:(u + 1) * nq].astype(np.float32), Ws)
        O.forward(cfg, W, hist, off, cand, I.get("ctx"), users=[u], dtype=np.float32)
        dt += time.perf_counter() - t0
        users += 1
        print(f"  oracle user {users}: {dt:.1f} s", file=sys.stderr, flush=True)
    threads = _blas_threads()
    return {"value": users / dt, "unit": "user-seq/s",
            "cores": threads or len(os.sched_getaffinity(0)), "kind": "oracle",
            "affinity_cores": len(os.sched_getaffinity(0)), "blas_threads": threads,
            "sample": f"{users} of {cfg.B} users of the same workload, fp32 oracle (token build "
                      f"and non-absorbed forward; table-row gathering not timed), {dt:.1f} s"}


ACTIONS_METRIC = "actions/sec + TFLOP/s (% MFMA bf16 peak), action tokenization, 1 GPU"
ACTIONS_TEXT = ("a_c3: action tokenization, 64 users x 1600 actions, fields type 32 / item "
                "128 (1M-row Zipf table) / surface 32 / time 32 / meta 16->32, MLP_act "
                "256-1024-512, timestamp encoding on 64 dims")


def action_kernel_cost(cfg, n):
    """Per kernel label: (FLOPs, algorithmic HBM bytes) of one call."""
    es = 2 if cfg.dtype == "bf16" else 4
    tables = cfg.d_type + cfg.d_item + cfg.d_surf + cfg.d_time
    return {
        "action_concat": (2 * n * cfg.d_meta * cfg.d_meta_emb,
                          n * (5 * 4 + cfg.d_meta * es + tables * es + cfg.d_in * es + 4)),
        "gemm_act_a": (2 * n * cfg.d_in * cfg.d_hidden, None),
        "gemm_act_b": (2 * n * cfg.d_hidden * cfg.d, None),
    }


def bench_actions(args):
    import torch
    from oracle import actions as A
    from synth.actions import generate_actions, get_action_config
    from target_aware_latent_amd import llatte as C
    from target_aware_latent_amd.actions import DeviceActions

    assert torch.cuda.is_available(), "bench.py needs the GPU"
    cfg = get_action_config("a_c3")
    p = generate_actions(cfg, 0)
    W, I = p["weights"], p["inputs"]
    n = len(I["tau"])
    dev = DeviceActions(cfg, W)
    X = dev.inputs(I)
    out = torch.empty((n, cfg.d), dtype=torch.float32, device="cuda")
    stream = torch.cuda.current_stream()
    step = lambda: dev.tokenize(X, out=out, stream=stream)
    for _ in range(args.warmup):
        step()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    ev0.record(stream)
    for _ in range(args.steps):
        step()
    ev1.record(stream)
    torch.cuda.synchronize()
    ms_step = ev0.elapsed_time(ev1) / args.steps
    F = A.action_flops(n, cfg.d_meta, cfg.d_meta_emb, cfg.d_in, cfg.d_hidden, cfg.d)
    tflops = F / (ms_step / 1e3) / 1e12
    C.llatte_kernel_timing_reset()
    C.llatte_kernel_timing_enable(True)
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    kt = C.llatte_kernel_timing_read()
    C.llatte_kernel_timing_enable(False)
    cost = action_kernel_cost(cfg, n)
    kernels = {}
    for name, (cnt, tot) in kt.items():
        e = {"launches_per_step": cnt / args.steps, "ms_per_step": tot / args.steps}
        if name in cost:
            fl, by = cost[name]
            e["tflops"] = fl / (tot / cnt / 1e3) / 1e12
            if by:
                e["gb_per_s"] = by / (tot / cnt / 1e3) / 1e9
        kernels[name] = e
    dom = max((k for k in kt if k.startswith("gemm_act")), key=lambda k: kt[k][1])
    cnt, tot = kt[dom]
    achieved = cost[dom][0] / (tot / cnt / 1e3) / 1e12
    roofline = {"bound": "mfma", "kernel": dom, "achieved": round(achieved, 2),
                "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                "frac": round(achieved / PEAK_BF16_TFLOPS, 4), "traffic": None,
                "flops_per_launch": cost[dom][0], "avg_launch_ms": round(tot / cnt, 4)}
    cpu = None
    if not args.no_cpu_baseline:
        rows = np.arange(0, n, 4)           # every 4th action, all users
        t0 = time.perf_counter()
        A.action_tokens(W, I["t_req"], I["tau"], I["offsets"], I["type_id"], I["item_id"],
                        I["surf_id"], I["meta"], cfg.n_buckets, cfg.d_enc,
                        dtype=np.float32, rows=rows)
        dt = time.perf_counter() - t0
        cpu = {"value": round(len(rows) / dt, 1), "unit": "actions/s",
               "cores": len(os.sched_getaffinity(0)), "kind": "oracle",
               "sample": f"{len(rows)} of {n} actions (every 4th), fp32 oracle, {dt:.1f} s"}
    rec = {
        "metric": ACTIONS_METRIC, "value": round(n / (ms_step / 1e3), 1), "unit": "actions/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": cfg.dtype,
        "data": "synthetic (seeded ids, Zipf items, exponential action gaps, N(0,1) tables)",
        "config": {"workload": ACTIONS_TEXT, "global_batch": cfg.B, "seq_len": cfg.L,
                   "parallelism": "single GPU"},
        "tflops": round(tflops, 2), "pct_peak": round(100 * tflops / PEAK_BF16_TFLOPS, 2),
        "roofline": roofline, "cpu_baseline": cpu, "kernels": kernels,
    }
    emit(rec)


SUMMARIES_METRIC = "users/sec + TFLOP/s (% MFMA bf16 peak), sequence summaries, 1 GPU"
SUMMARIES_TEXT = ("s_c3: LoRAMLP sequence summaries of the upstream readout, 64 users, "
                  "Flatten(Z_raw) 2048 -> hidden 2048 -> 2048, 2 summaries, adapter rank 16")


def bench_summaries(args):
    import torch
    from oracle import llatte_oracle as O
    from synth.summaries import generate_summaries, get_summary_config
    from target_aware_latent_amd import llatte as C
    from target_aware_latent_amd.summaries import DeviceSummaries

    assert torch.cuda.is_available(), "bench.py needs the GPU"
    cfg = get_summary_config("s_c3")
    p = generate_summaries(cfg, 0)
    L, z = p["weights"], p["inputs"]["z"]
    ds = DeviceSummaries(cfg, L)
    zt = torch.from_numpy(np.ascontiguousarray(z, dtype=np.float32)).cuda()
    out = torch.empty((cfg.K, cfg.B, cfg.d_seq), dtype=torch.float32, device="cuda")
    stream = torch.cuda.current_stream()
    step = lambda: ds(zt, out=out, stream=stream)
    for _ in range(args.warmup):
        step()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    ev0.record(stream)
    for _ in range(args.steps):
        step()
    ev1.record(stream)
    torch.cuda.synchronize()
    ms_step = ev0.elapsed_time(ev1) / args.steps
    f1 = 2 * cfg.K * cfg.B * cfg.d_z * cfg.d_hidden
    f2 = 2 * cfg.K * cfg.B * cfg.d_hidden * cfg.d_seq
    F = f1 + f2
    C.llatte_kernel_timing_reset()
    C.llatte_kernel_timing_enable(True)
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    kt = C.llatte_kernel_timing_read()
    C.llatte_kernel_timing_enable(False)
    flops = {"gemm_summary_1": f1, "gemm_summary_2": f2}
    kernels = {}
    for name, (cnt, tot) in kt.items():
        e = {"launches_per_step": cnt / args.steps, "ms_per_step": tot / args.steps}
        if name in flops:
            e["tflops"] = flops[name] / (tot / cnt / 1e3) / 1e12
        kernels[name] = e
    dom = max(flops, key=lambda k: kt[k][1])
    cnt, tot = kt[dom]
    achieved = flops[dom] / (tot / cnt / 1e3) / 1e12
    roofline = {"bound": "mfma", "kernel": dom, "achieved": round(achieved, 2),
                "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                "frac": round(achieved / PEAK_BF16_TFLOPS, 4), "traffic": None,
                "flops_per_launch": flops[dom], "avg_launch_ms": round(tot / cnt, 4)}
    cpu = None
    if not args.no_cpu_baseline:
        t0 = time.perf_counter()
        reps = 0
        while time.perf_counter() - t0 < 5.0:
            O.lora_mlp_summaries(z, L, dtype=np.float32)
            reps += 1
        dt = time.perf_counter() - t0
        cpu = {"value": round(reps * cfg.B / dt, 1), "unit": "users/s",
               "cores": len(os.sched_getaffinity(0)), "kind": "oracle",
               "sample": f"{reps} full batches of {cfg.B} users, fp32 oracle "
                         f"(adapters merged per call), {dt:.1f} s"}
    rec = {
        "metric": SUMMARIES_METRIC, "value": round(cfg.B / (ms_step / 1e3), 1),
        "unit": "users/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": cfg.dtype,
        "data": "synthetic (N(0,1) readouts, N(0,1/fan_in) weights and adapters)",
        "config": {"workload": SUMMARIES_TEXT, "global_batch": cfg.B, "seq_len": None,
                   "parallelism": "single GPU"},
        "tflops": round(F / (ms_step / 1e3) / 1e12, 2),
        "pct_peak": round(100 * F / (ms_step / 1e3) / 1e12 / PEAK_BF16_TFLOPS, 2),
        "roofline": roofline, "cpu_baseline": cpu, "kernels": kernels,
    }
    emit(rec)


BACKWARD_METRIC = ("user-sequences/sec + TFLOP/s (% MFMA bf16 peak), attention-core backward "
                   "of the MLA stack at L=1600, 1 GPU")
BACKWARD_TEXT = ("c3 attention cores: d_q and d_C of the six causal layers (64 users, keys "
                 "1600-1600-800-400-200-100, query rows 1600-800-400-200-100-50) and the "
                 "4-seed readout over 50 keys, 8 heads, r=128, bf16")


def backward_layers(cfg):
    """(K per user, history query rows per user, candidate rows per user) of
    every attention core of the stack, all users of one length."""
    keep = [int(x) for x in cfg.pyramid.values]
    K = cfg.L
    out = []
    for n in keep:
        out.append((K, n, cfg.n_q))
        K = n
    if cfg.n_seeds:
        out.append((K, 0, cfg.n_seeds))
    return out


def bench_backward(args):
    import torch
    from oracle import llatte_oracle as O
    from target_aware_latent_amd import llatte as C
    import synth

    assert torch.cuda.is_available(), "bench.py needs the GPU"
    cfg = synth.get_config("c3")
    h, r, B = cfg.h, cfg.r, cfg.B
    scale = 1.0 / math.sqrt(cfg.dk)
    rng = np.random.default_rng(0)
    stream = torch.cuda.current_stream()
    layers = []
    flops = {"attn_bwd_dq": 0, "attn_bwd_dc": 0}
    for K, n, nc in backward_layers(cfg):
        kv = np.arange(B + 1, dtype=np.int32) * K
        hq = np.arange(B + 1, dtype=np.int32) * n
        Mtot, Ktot = B * (nc + n), B * K
        ad = C.llatte_attn_desc(h, r, nc, C.LLATTE_BF16, scale)
        q = torch.from_numpy(synth.round_bf16(rng.standard_normal((Mtot, h, r)) * 0.5)
                             .astype(np.float32)).cuda().to(torch.bfloat16)
        c = torch.from_numpy(synth.round_bf16(rng.standard_normal((Ktot, r)))
                             .astype(np.float32)).cuda().to(torch.bfloat16)
        g = torch.from_numpy(rng.standard_normal((Mtot, h, r)).astype(np.float32)).cuda()
        kvd, hqd = torch.from_numpy(kv).cuda(), torch.from_numpy(hq).cuda()
        out = torch.empty((Mtot, h, r), device="cuda")
        lse = torch.empty((Mtot, h), device="cuda")
        ws = torch.empty(C.llatte_mla_attention_workspace_size(ad, B, Mtot, Ktot),
                         dtype=torch.uint8, device="cuda")
        C.llatte_mla_attention(ad, q, c, kvd, hqd, B, Mtot, Ktot, out, lse, ws, stream=stream)
        dq = torch.empty((Mtot, h, r), device="cuda")
        dc = torch.empty((Ktot, r), device="cuda")
        bws = torch.empty(C.llatte_mla_attention_backward_workspace_size(ad, Mtot),
                          dtype=torch.uint8, device="cuda")
        layers.append((ad, q, c, kvd, hqd, Mtot, Ktot, K, out, lse, g, dq, dc, bws))
        # allowed (query row, key) pairs per user and head
        pairs = B * (n * (K - n) + n * (n + 1) // 2 + nc * K)
        flops["attn_bwd_dq"] += 6 * r * h * pairs   # S, dP = d_out C^T, d_q = dS C
        flops["attn_bwd_dc"] += 4 * r * h * pairs   # P^T d_out and dS^T q
    F = sum(flops.values())

    def step():
        for (ad, q, c, kvd, hqd, Mtot, Ktot, K, out, lse, g, dq, dc, bws) in layers:
            C.llatte_mla_attention_backward(ad, q, c, kvd, hqd, B, Mtot, Ktot, K, out, lse,
                                            g, dq, dc, bws, stream=stream)

    for _ in range(args.warmup):
        step()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    ev0.record(stream)
    for _ in range(args.steps):
        step()
    ev1.record(stream)
    torch.cuda.synchronize()
    ms_step = ev0.elapsed_time(ev1) / args.steps
    C.llatte_kernel_timing_reset()
    C.llatte_kernel_timing_enable(True)
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    kt = C.llatte_kernel_timing_read()
    C.llatte_kernel_timing_enable(False)
    kernels = {}
    for name, (cnt, tot) in kt.items():
        e = {"launches_per_step": cnt / args.steps, "ms_per_step": tot / args.steps}
        if name in flops:
            e["tflops"] = flops[name] / (tot / args.steps / 1e3) / 1e12
        kernels[name] = e
    dom = max(flops, key=lambda k: kt[k][1])
    cnt, tot = kt[dom]
    # the launches differ in size (one per layer): per launch = the step's
    # algorithmic FLOPs of the kernel over its launches, against the mean
    # launch duration
    per_launch = flops[dom] / (cnt / args.steps)
    achieved = per_launch / (tot / cnt / 1e3) / 1e12
    roofline = {"bound": "mfma", "kernel": dom, "achieved": round(achieved, 2),
                "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                "frac": round(achieved / PEAK_BF16_TFLOPS, 4), "traffic": None,
                "flops_per_launch": per_launch, "avg_launch_ms": round(tot / cnt, 4)}
    cpu = None
    if not args.no_cpu_baseline:
        # whole users through every attention core, fp64 oracle, until ~12 s
        # (the rows of the first users of each layer's synthetic inputs)
        qs, cs = [], []
        for (ad, q, c, kvd, hqd, Mtot, Ktot, K, out, lse, g, dq, dc, bws) in layers:
            nq = Mtot // B
            qs.append((q[:2 * nq].float().cpu().numpy().astype(np.float64),
                       g[:2 * nq].cpu().numpy().astype(np.float64)))
            cs.append(c[:2 * K].float().cpu().numpy().astype(np.float64))
        t0 = time.perf_counter()
        users = 0
        while time.perf_counter() - t0 < 12.0 and users < B:
            for li, (K, n, nc) in enumerate(backward_layers(cfg)):
                (qa, ga), ca = qs[li], cs[li]
                # one user: its candidate rows are the first nc, history after
                O.latent_attention_backward(qa[:nc + n], ca[:K], [0, K], [0, n], nc, scale,
                                            ga[:nc + n])
            users += 1
        dt = time.perf_counter() - t0
        cpu = {"value": round(users / dt, 3), "unit": "user-sequences/s",
               "cores": len(os.sched_getaffinity(0)), "kind": "oracle",
               "sample": f"{users} of {B} users through all {len(layers)} attention-core "
                         f"backwards, fp64 oracle, {dt:.1f} s"}
    rec = {
        "metric": BACKWARD_METRIC, "value": round(B / (ms_step / 1e3), 1),
        "unit": "user-sequences/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic (N(0,1/4) bf16 latent queries, N(0,1) bf16 latent, N(0,1) d_out)",
        "config": {"workload": BACKWARD_TEXT, "global_batch": B, "seq_len": cfg.L,
                   "parallelism": "single GPU"},
        "tflops": round(F / (ms_step / 1e3) / 1e12, 2),
        "pct_peak": round(100 * F / (ms_step / 1e3) / 1e12 / PEAK_BF16_TFLOPS, 2),
        "roofline": roofline, "cpu_baseline": cpu, "kernels": kernels,
    }
    emit(rec)


FFN_BWD_METRIC = ("user-sequences/sec + TFLOP/s (% MFMA bf16 peak), FFN-sublayer backward of "
                  "the MLA stack at L=1600, 1 GPU")
FFN_BWD_TEXT = ("c3 FFN sublayers: dR1, dg2, dW1, dW2 of the six layers' pre-norm FFN "
                "(64 users x 1600-800-400-200-100-50 rows, d=512, d_ff=2048), bf16 products")


def bench_ffn_backward(args):
    import torch
    from oracle import llatte_oracle as O
    from target_aware_latent_amd import llatte as C
    import synth

    assert torch.cuda.is_available(), "bench.py needs the GPU"
    cfg = synth.get_config("c3")
    d, F, B = cfg.d, cfg.d_ff, cfg.B
    rng = np.random.default_rng(0)
    f = C.llatte_ffn_desc(d, F, C.LLATTE_BF16, cfg.eps)
    rows = [B * int(n) for n in cfg.pyramid.values]
    ws = torch.empty(C.llatte_ffn_backward_workspace_size(f, max(rows)), dtype=torch.uint8,
                     device="cuda")
    layers = []
    for M in rows:
        r1 = torch.from_numpy(rng.standard_normal((M, d)).astype(np.float32)).cuda()
        g2 = torch.ones(d, device="cuda")
        w1 = torch.from_numpy((rng.standard_normal((d, F)) / np.sqrt(d)).astype(np.float32)).cuda()
        w2 = torch.from_numpy((rng.standard_normal((F, d)) / np.sqrt(F)).astype(np.float32)).cuda()
        do = torch.from_numpy(rng.standard_normal((M, d)).astype(np.float32)).cuda()
        outs = (torch.empty((M, d), device="cuda"), torch.empty(d, device="cuda"),
                torch.empty((d, F), device="cuda"), torch.empty((F, d), device="cuda"))
        layers.append((M, r1, g2, w1.to(torch.bfloat16), w2.to(torch.bfloat16), do, outs))
    stream = torch.cuda.current_stream()

    def step():
        for (M, r1, g2, w1, w2, do, (dr1, dg2, dw1, dw2)) in layers:
            C.llatte_ffn_backward(f, r1, g2, w1, w2, do, M, dr1, dg2, dw1, dw2, ws, stream=stream)

    for _ in range(args.warmup):
        step()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    ev0.record(stream)
    for _ in range(args.steps):
        step()
    ev1.record(stream)
    torch.cuda.synchronize()
    ms_step = ev0.elapsed_time(ev1) / args.steps
    # algorithmic FLOPs: the four gradient products (2 M d F each); the
    # recomputed pre-activation is not counted
    per = {k: sum(2 * M * d * F for M in rows) for k in
           ("gemm_bwd_dg", "gemm_bwd_dh", "gemm_bwd_dw1", "gemm_bwd_dw2")}
    Fl = sum(per.values())
    C.llatte_kernel_timing_reset()
    C.llatte_kernel_timing_enable(True)
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    kt = C.llatte_kernel_timing_read()
    C.llatte_kernel_timing_enable(False)
    kernels = {}
    for name, (cnt, tot) in kt.items():
        e = {"launches_per_step": cnt / args.steps, "ms_per_step": tot / args.steps}
        if name in per:
            e["tflops"] = per[name] / (tot / args.steps / 1e3) / 1e12
        kernels[name] = e
    dom = max(per, key=lambda k: kt[k][1])
    cnt, tot = kt[dom]
    per_launch = per[dom] / (cnt / args.steps)
    achieved = per_launch / (tot / cnt / 1e3) / 1e12
    roofline = {"bound": "mfma", "kernel": dom, "achieved": round(achieved, 2),
                "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                "frac": round(achieved / PEAK_BF16_TFLOPS, 4), "traffic": None,
                "flops_per_launch": per_launch, "avg_launch_ms": round(tot / cnt, 4)}
    cpu = None
    if not args.no_cpu_baseline:
        # whole users (1600 + 800 + ... + 50 rows) through the fp64 oracle
        W1 = layers[0][3].float().cpu().numpy().astype(np.float64)
        W2 = layers[0][4].float().cpu().numpy().astype(np.float64)
        g2 = np.ones(d)
        sample = [rng.standard_normal((int(n), d)) for n in cfg.pyramid.values]
        t0 = time.perf_counter()
        users = 0
        while time.perf_counter() - t0 < 12.0 and users < B:
            for x in sample:
                O.ffn_block_backward(x, g2, W1, W2, x)
            users += 1
        dt = time.perf_counter() - t0
        cpu = {"value": round(users / dt, 3), "unit": "user-sequences/s",
               "cores": len(os.sched_getaffinity(0)), "kind": "oracle",
               "sample": f"{users} of {B} users through all {len(rows)} FFN-sublayer "
                         f"backwards, fp64 oracle, {dt:.1f} s"}
    rec = {
        "metric": FFN_BWD_METRIC, "value": round(B / (ms_step / 1e3), 1),
        "unit": "user-sequences/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic (N(0,1) residual rows and d_out, N(0,1/fan_in) bf16 weights, gains 1)",
        "config": {"workload": FFN_BWD_TEXT, "global_batch": B, "seq_len": cfg.L,
                   "parallelism": "single GPU"},
        "tflops": round(Fl / (ms_step / 1e3) / 1e12, 2),
        "pct_peak": round(100 * Fl / (ms_step / 1e3) / 1e12 / PEAK_BF16_TFLOPS, 2),
        "roofline": roofline, "cpu_baseline": cpu, "kernels": kernels,
    }
    emit(rec)


SUB_BWD_METRIC = ("user-sequences/sec + TFLOP/s (% MFMA bf16 peak), attention-sublayer backward "
                  "of the MLA stack at L=1600, 1 GPU")
SUB_BWD_TEXT = ("c3 attention sublayers: gradients of the layer-input rows, g1, W_dkv, g_c, W_uq, "
                "W_uk, W_uv, W_o of the six causal layers (64 users, keys 1600-1600-800-400-200-100, "
                "query rows 1600-800-400-200-100-50; d=512, 8x64 heads, r=128), bf16 products")


def bench_sublayer_backward(args):
    import torch
    from oracle import llatte_oracle as O
    from target_aware_latent_amd import llatte as C
    import synth
    from types import SimpleNamespace

    assert torch.cuda.is_available(), "bench.py needs the GPU"
    cfg = synth.get_config("c3")
    d, h, dk, r, B = cfg.d, cfg.h, cfg.dk, cfg.r, cfg.B
    hd = h * dk
    rng = np.random.default_rng(0)
    desc = C.llatte_attn_sublayer_desc(d, h, dk, r, 0, C.LLATTE_BF16, 1, cfg.eps)
    dev = lambda a, dt=torch.float32: torch.from_numpy(np.ascontiguousarray(a, np.float32)).cuda().to(dt)
    W = {"g1": np.ones(d), "g_c": np.ones(r),
         "W_dkv": rng.standard_normal((d, r)) / np.sqrt(d),
         "W_uq": rng.standard_normal((d, hd)) / np.sqrt(d),
         "W_uk": rng.standard_normal((r, hd)) / np.sqrt(r),
         "W_uv": rng.standard_normal((r, hd)) / np.sqrt(r),
         "W_o": rng.standard_normal((hd, d)) / np.sqrt(hd)}
    wd = {"g1": dev(W["g1"]), "g_c": dev(W["g_c"]), "w_dkv": dev(W["W_dkv"], torch.bfloat16),
          "w_uq": dev(W["W_uq"], torch.bfloat16), "w_uk": dev(W["W_uk"], torch.bfloat16),
          "w_uv": dev(W["W_uv"], torch.bfloat16), "w_o": dev(W["W_o"], torch.bfloat16)}
    flops = {}
    add = lambda k, v: flops.__setitem__(k, flops.get(k, 0) + v)
    layers = []
    wsize = 0
    for K, n, _ in backward_layers(cfg)[:cfg.N]:
        kv = torch.from_numpy(np.arange(B + 1, dtype=np.int32) * K).cuda()
        hq = torch.from_numpy(np.arange(B + 1, dtype=np.int32) * n).cuda()
        Mtot, Ktot = B * n, B * K
        r_kv = dev(rng.standard_normal((Ktot, d)))
        dout = dev(rng.standard_normal((Mtot, d)))
        gd = {"g1": torch.empty(d, device="cuda"), "g_c": torch.empty(r, device="cuda"),
              "w_dkv": torch.empty((d, r), device="cuda"), "w_uq": torch.empty((d, hd), device="cuda"),
              "w_uk": torch.empty((r, hd), device="cuda"), "w_uv": torch.empty((r, hd), device="cuda"),
              "w_o": torch.empty((hd, d), device="cuda")}
        d_r_kv = torch.empty((Ktot, d), device="cuda")
        layers.append((kv, hq, Mtot, Ktot, K, r_kv, dout, d_r_kv, gd))
        wsize = max(wsize, C.llatte_attn_sublayer_backward_workspace_size(desc, B, Mtot, Ktot))
        pairs = B * (n * (K - n) + n * (n + 1) // 2)
        add("attn_bwd_dq", 6 * r * h * pairs)
        add("attn_bwd_dc", 4 * r * h * pairs)
        for lab in ("gemm_sub_dwo", "gemm_sub_do", "gemm_sub_dwuq", "gemm_sub_dhq"):
            add(lab, 2 * Mtot * d * hd)
        for lab in ("gemm_sub_dwuv", "gemm_sub_dolat", "gemm_sub_dq", "gemm_sub_dwuk"):
            add(lab, 2 * Mtot * r * hd)
        for lab in ("gemm_sub_dwdkv", "gemm_sub_dh"):
            add(lab, 2 * Ktot * d * r)
    ws = torch.empty(wsize, dtype=torch.uint8, device="cuda")
    stream = torch.cuda.current_stream()

    def step():
        for (kv, hq, Mtot, Ktot, K, r_kv, dout, d_r_kv, gd) in layers:
            C.llatte_attn_sublayer_backward(desc, wd, r_kv, None, kv, hq, B, Mtot, Ktot, K, dout,
                                            d_r_kv, None, gd, ws, stream=stream)

    for _ in range(args.warmup):
        step()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    ev0.record(stream)
    for _ in range(args.steps):
        step()
    ev1.record(stream)
    torch.cuda.synchronize()
    ms_step = ev0.elapsed_time(ev1) / args.steps
    Fl = sum(flops.values())
    C.llatte_kernel_timing_reset()
    C.llatte_kernel_timing_enable(True)
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    kt = C.llatte_kernel_timing_read()
    C.llatte_kernel_timing_enable(False)
    kernels = {}
    for name, (cnt, tot) in kt.items():
        e = {"launches_per_step": cnt / args.steps, "ms_per_step": tot / args.steps}
        if name in flops:
            e["tflops"] = flops[name] / (tot / args.steps / 1e3) / 1e12
        kernels[name] = e
    dom = max((k for k in flops if k in kt), key=lambda k: kt[k][1])
    cnt, tot = kt[dom]
    per_launch = flops[dom] / (cnt / args.steps)
    achieved = per_launch / (tot / cnt / 1e3) / 1e12
    roofline = {"bound": "mfma", "kernel": dom, "achieved": round(achieved, 2),
                "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                "frac": round(achieved / PEAK_BF16_TFLOPS, 4), "traffic": None,
                "flops_per_launch": per_launch, "avg_launch_ms": round(tot / cnt, 4)}
    cpu = None
    if not args.no_cpu_baseline:
        ocfg = SimpleNamespace(d=d, h=h, dk=dk, r=r, eps=cfg.eps, latent_norm=True, norm_mode="pre")
        sample = [(rng.standard_normal((K, d)), n, rng.standard_normal((n, d)))
                  for K, n, _ in backward_layers(cfg)[:cfg.N]]
        t0 = time.perf_counter()
        users = 0
        while time.perf_counter() - t0 < 12.0 and users < B:
            for Rh, n, dq in sample:
                O.attention_sublayer_backward(Rh, np.zeros((0, d)), n, W, ocfg, dq)
            users += 1
        dt = time.perf_counter() - t0
        cpu = {"value": round(users / dt, 3), "unit": "user-sequences/s",
               "cores": len(os.sched_getaffinity(0)), "kind": "oracle",
               "sample": f"{users} of {B} users through all {len(layers)} attention-sublayer "
                         f"backwards, fp64 oracle (non-absorbed), {dt:.1f} s"}
    rec = {
        "metric": SUB_BWD_METRIC, "value": round(B / (ms_step / 1e3), 1),
        "unit": "user-sequences/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic (N(0,1) layer-input rows and d_out, N(0,1/fan_in) bf16 weights, gains 1)",
        "config": {"workload": SUB_BWD_TEXT, "global_batch": B, "seq_len": cfg.L,
                   "parallelism": "single GPU"},
        "tflops": round(Fl / (ms_step / 1e3) / 1e12, 2),
        "pct_peak": round(100 * Fl / (ms_step / 1e3) / 1e12 / PEAK_BF16_TFLOPS, 2),
        "roofline": roofline, "cpu_baseline": cpu, "kernels": kernels,
    }
    emit(rec)


STACK_BWD_METRIC = ("user-sequences/sec + TFLOP/s (% MFMA bf16 peak), whole-stack training "
                    "backward (forward recomputed inside), 1 GPU")
STACK_BWD_TEXT = ("c3: llatte_mla_backward over 64 users x 1600 rows (6 layers, pyramid "
                  "1600-800-400-200-100-50, 4-seed readout to 2048): gradients of every weight, "
                  "the seeds and the history rows, from N(0,1) output gradients")


def stack_backward_flops(cfg, lengths):
    """Algorithmic FLOPs per kernel label of one llatte_mla_backward call: the
    forward it recomputes (absorbed count) and, per layer and the readout, the
    gradient products of the FFN and attention sublayers (as their own
    benches count them) and the readout's two projections."""
    fl = dict(kernel_flops(cfg, lengths))
    add = lambda k, v: fl.__setitem__(k, fl.get(k, 0) + v)
    d, h, dk, r, F, B = cfg.d, cfg.h, cfg.dk, cfg.r, cfg.d_ff, len(lengths)
    hd = h * dk
    for K, n, nc in backward_layers(cfg):
        M, Kt = B * (nc + n), B * K
        pairs = B * (n * (K - n) + n * (n + 1) // 2 + nc * K)
        add("attn_bwd_dq", 6 * r * h * pairs)
        add("attn_bwd_dc", 4 * r * h * pairs)
        for lab in ("gemm_sub_dwo", "gemm_sub_do", "gemm_sub_dwuq", "gemm_sub_dhq"):
            add(lab, 2 * M * d * hd)
        for lab in ("gemm_sub_dwuv", "gemm_sub_dolat", "gemm_sub_dq", "gemm_sub_dwuk"):
            add(lab, 2 * M * r * hd)
        for lab in ("gemm_sub_dwdkv", "gemm_sub_dh"):
            add(lab, 2 * Kt * d * r)
        for lab in ("gemm_bwd_dg", "gemm_bwd_dh", "gemm_bwd_dw1", "gemm_bwd_dw2"):
            add(lab, 2 * M * d * F)
    if cfg.n_seeds:
        for lab in ("gemm_bwd_readout", "wgrad_readout"):
            add(lab, 2 * B * cfg.d_out * cfg.n_seeds * d)
    return fl


def bench_stack_backward(args):
    import torch
    import synth
    from target_aware_latent_amd import llatte as C
    from target_aware_latent_amd.model import DeviceModel

    assert torch.cuda.is_available(), "bench.py needs the GPU"
    cfg = synth.get_config("c3")
    B = cfg.B
    lengths = [cfg.L] * B
    prob = synth.generate(cfg, seed=0, lengths=lengths)
    I = prob["inputs"]
    model = DeviceModel(cfg, prob["weights"])
    rng = np.random.default_rng(0)
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a, np.float32)).cuda()
    hist, offs = dev(I["hist"]), torch.from_numpy(I["offsets"].astype(np.int32)).cuda()
    n_out = B * int(cfg.pyramid.values[-1])
    d_hist = dev(rng.standard_normal((n_out, cfg.d)))
    d_emb = dev(rng.standard_normal((B, cfg.d_out)))
    grads = model.alloc_grads(lengths)
    stream = torch.cuda.current_stream()

    def step():
        model.backward(hist, offs, lengths, None, None, None, d_hist, d_emb, grads=grads,
                       stream=stream)

    for _ in range(args.warmup):
        step()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    ev0.record(stream)
    for _ in range(args.steps):
        step()
    ev1.record(stream)
    torch.cuda.synchronize()
    ms_step = ev0.elapsed_time(ev1) / args.steps
    per = stack_backward_flops(cfg, lengths)
    Fl = sum(per.values())
    C.llatte_kernel_timing_reset()
    C.llatte_kernel_timing_enable(True)
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    kt = C.llatte_kernel_timing_read()
    C.llatte_kernel_timing_enable(False)
    kernels = {}
    for name, (cnt, tot) in kt.items():
        e = {"launches_per_step": cnt / args.steps, "ms_per_step": tot / args.steps}
        if name in per:
            e["tflops"] = per[name] / (tot / args.steps / 1e3) / 1e12
        kernels[name] = e
    dom = max((k for k in per if k in kt), key=lambda k: kt[k][1])
    cnt, tot = kt[dom]
    per_launch = per[dom] / (cnt / args.steps)
    achieved = per_launch / (tot / cnt / 1e3) / 1e12
    roofline = {"bound": "mfma", "kernel": dom, "achieved": round(achieved, 2),
                "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                "frac": round(achieved / PEAK_BF16_TFLOPS, 4), "traffic": None,
                "flops_per_launch": per_launch, "avg_launch_ms": round(tot / cnt, 4)}
    rec = {
        "metric": STACK_BWD_METRIC, "value": round(B / (ms_step / 1e3), 1),
        "unit": "user-sequences/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic (the c3 workload's seeded inputs and weights, N(0,1) output gradients)",
        "config": {"workload": STACK_BWD_TEXT, "global_batch": B, "seq_len": cfg.L,
                   "parallelism": "single GPU"},
        "tflops": round(Fl / (ms_step / 1e3) / 1e12, 2),
        "pct_peak": round(100 * Fl / (ms_step / 1e3) / 1e12 / PEAK_BF16_TFLOPS, 2),
        "roofline": roofline, "cpu_baseline": None, "kernels": kernels,
    }
    emit(rec)


COMPACT_METRIC = "GB/s (algorithmic), pyramid compaction, 1 GPU"
COMPACT_TEXT = ("c3 layer-2 compaction: 64 users x 1600 fp32 rows of 512, the last 800 of each "
                "kept (values, offsets and source indices out)")


def bench_vendor_gemm(args):
    """A reference point, not the product path: the vendor GEMM (hipBLASLt,
    through torch.matmul on bf16 operands, fp32 accumulation, no epilogue)
    on the five product shapes of the c3 forward's first layer (M = 102,400
    rows: W_dkv, W_uq, W_o, W1, W2). `value` is the FLOP-weighted rate over
    the five; `products` gives each one's. The library's own rates for the
    same launches come from its per-launch table (profiles/)."""
    import torch
    assert torch.cuda.is_available(), "bench.py needs the GPU"
    M, d, r, hd, dff = 102400, 512, 128, 512, 2048
    shapes = [("down", r, d), ("q", hd, d), ("out", d, hd), ("ffn1", dff, d), ("ffn2", d, dff)]
    g = torch.Generator(device="cuda").manual_seed(0)
    prods, tot_f, tot_t = {}, 0.0, 0.0
    for name, N, K in shapes:
        A = torch.randn(M, K, device="cuda", generator=g).to(torch.bfloat16)
        Bt = (torch.randn(K, N, device="cuda", generator=g) / K ** 0.5).to(torch.bfloat16)
        C = torch.empty(M, N, device="cuda", dtype=torch.bfloat16)
        for _ in range(args.warmup):
            torch.matmul(A, Bt, out=C)
        ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        ev0.record()
        for _ in range(args.steps):
            torch.matmul(A, Bt, out=C)
        ev1.record()
        torch.cuda.synchronize()
        ms = ev0.elapsed_time(ev1) / args.steps
        f = 2.0 * M * N * K
        prods[name] = {"N": N, "K": K, "ms": round(ms, 4), "tflops": round(f / (ms / 1e3) / 1e12, 1)}
        tot_f += f
        tot_t += ms
        del A, Bt, C
    tf = tot_f / (tot_t / 1e3) / 1e12
    rec = {"metric": "vendor GEMM TFLOP/s (hipBLASLt via torch.matmul) on the c3 layer-1 product shapes",
           "value": round(tf, 1), "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
           "warmup": args.warmup, "ms_per_step": round(tot_t, 4), "higher_is_better": True,
           "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic (seeded N(0,1))",
           "config": {"workload": "c3 layer-1 product shapes, M=102400: W_dkv 512->128, W_uq 512->512, "
                                  "W_o 512->512, W1 512->2048, W2 2048->512; one step = the five products"},
           "roofline": {"bound": "mfma", "kernel": "vendor GEMM", "achieved": round(tf, 1),
                        "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                        "frac": round(tf / PEAK_BF16_TFLOPS, 4), "traffic": None},
           "cpu_baseline": None, "products": prods,
           "note": "reference measurement of the vendor library; the library does not use it"}
    print(json.dumps(rec))


def bench_compact(args):
    import torch
    from oracle import llatte_oracle as O
    from target_aware_latent_amd import llatte as C

    assert torch.cuda.is_available(), "bench.py needs the GPU"
    B, Lu, d, keep_n = 64, 1600, 512, 800
    rng = np.random.default_rng(0)
    vals = rng.standard_normal((B * Lu, d)).astype(np.float32)
    off_h = (np.arange(B + 1) * Lu).astype(np.int32)
    v = torch.from_numpy(vals).cuda()
    off = torch.from_numpy(off_h).cuda()
    keep = torch.full((B,), keep_n, dtype=torch.int32, device="cuda")
    out = torch.empty((B * keep_n, d), device="cuda")
    noff = torch.empty(B + 1, dtype=torch.int32, device="cuda")
    src = torch.empty(B * keep_n, dtype=torch.int32, device="cuda")
    stream = torch.cuda.current_stream()
    if args.calibrate_copy:
        cs = torch.empty(64 << 20, dtype=torch.float32, device="cuda").fill_(1.0)
        cd = torch.empty_like(cs)
        torch.cuda.synchronize()
        cd.copy_(cs)
        torch.cuda.synchronize()
        del cs, cd
    step = lambda: C.llatte_pyramid_compact(v, d, C.LLATTE_F32, off, B, B * Lu, keep, out, noff,
                                            src, stream=stream)
    for _ in range(args.warmup):
        step()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    ev0.record(stream)
    for _ in range(args.steps):
        step()
    ev1.record(stream)
    torch.cuda.synchronize()
    ms_step = ev0.elapsed_time(ev1) / args.steps
    # each kept row read once and written once, its source index written, the
    # offsets and keep counts read and the new offsets written
    nbytes = B * keep_n * (2 * 4 * d + 4) + (B + 1) * 4 * 2 + B * 4
    gbs = nbytes / (ms_step / 1e3) / 1e9
    C.llatte_kernel_timing_reset()
    C.llatte_kernel_timing_enable(True)
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    kt = C.llatte_kernel_timing_read()
    C.llatte_kernel_timing_enable(False)
    kernels = {n: {"launches_per_step": c / args.steps, "ms_per_step": t / args.steps}
               for n, (c, t) in kt.items()}
    dom = max(kt, key=lambda n: kt[n][1])
    cnt, tot = kt[dom]
    # measured HBM bytes of the row-copy kernel (the scan moves a few KB)
    cp_traffic = os.path.join(ROOT, "profiles", "compaction_hbm_traffic.txt")
    traffic = read_traffic(args.traffic if args.traffic and
                           args.traffic.endswith("compaction_hbm_traffic.txt") else cp_traffic, dom)
    roofline = {"bound": "hbm", "kernel": dom,
                "achieved": round(nbytes / (tot / cnt / 1e3) / 1e9, 1), "peak": PEAK_HBM_GBS,
                "unit": "GB/s", "frac": round(nbytes / (tot / cnt / 1e3) / 1e9 / PEAK_HBM_GBS, 4),
                "traffic": traffic, "bytes_per_launch": nbytes, "avg_launch_ms": round(tot / cnt, 4)}
    cpu = None
    if not args.no_cpu_baseline:
        t0 = time.perf_counter()
        reps = 0
        while time.perf_counter() - t0 < 5.0:
            O.compact(vals, off_h, np.full(B, keep_n))
            reps += 1
        dt = time.perf_counter() - t0
        cpu = {"value": round(reps * nbytes / dt / 1e9, 2), "unit": "GB/s",
               "cores": len(os.sched_getaffinity(0)), "kind": "oracle",
               "sample": f"{reps} full compactions, numpy oracle, {dt:.1f} s"}
    rec = {"metric": COMPACT_METRIC, "value": round(gbs, 1), "unit": "GB/s", "n_gpus": 1,
           "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_step, 4),
           "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f32",
           "data": "synthetic (N(0,1) rows)",
           "config": {"workload": COMPACT_TEXT, "global_batch": B, "seq_len": Lu,
                      "parallelism": "single GPU"},
           "roofline": roofline, "cpu_baseline": cpu, "kernels": kernels}
    emit(rec)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--config", default="c3")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-kernel-times", action="store_true")
    ap.add_argument("--gemm-phases", action="store_true",
                    help="after the timed steps, one more forward with the 128x128 GEMM tile's "
                         "phase stamps (first operands, K loop, epilogue) per launch; adds "
                         "gemm_phases to the line")
    ap.add_argument("--attn-phases", action="store_true",
                    help="after the timed steps, one more forward with the attention "
                         "kernel's phase stamps (W_uk prologue, key loop, W_uv "
                         "epilogue) per launch; adds attention_phases to the line")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="run one plain 256 MiB device-to-device copy first, "
                         "as the reference for HBM byte counters")
    ap.add_argument("--traffic", default=None,
                    help="profile summary whose RECORD line holds the measured "
                         "HBM bytes per launch of the dominant kernel (written "
                         "by target_aware_latent_amd.profsum traffic); by "
                         "default the c3 records under profiles/")
    ap.add_argument("--workload", default="stack", choices=["stack", "actions", "summaries", "backward", "ffn_backward",
                             "sublayer_backward", "stack_backward", "compact", "vendor_gemm"],
                    help="stack: the MLA forward (default); actions: the action "
                         "tokenization that builds the history tokens; summaries: the "
                         "LoRAMLP sequence summaries of the readout; backward: the attention-core "
                         "backward of every layer of the stack; ffn_backward: the FFN-sublayer "
                         "backward (GEMM gradients) of every layer; sublayer_backward: the "
                         "attention-sublayer backward of every layer; stack_backward: the "
                         "whole-stack training backward; compact: the pyramid compaction "
                         "(HBM-bound); vendor_gemm: hipBLASLt on the c3 layer-1 product "
                         "shapes, a reference point only")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU only: this build has no multi-GPU "
              "path (users shard across GPUs with no exchange; see the design "
              "notes). Run with --gpus 1.", file=sys.stderr)
        sys.exit(2)
    if args.workload == "actions":
        bench_actions(args)
        return
    if args.workload == "summaries":
        bench_summaries(args)
        return
    if args.workload == "backward":
        bench_backward(args)
        return
    if args.workload == "ffn_backward":
        bench_ffn_backward(args)
        return
    if args.workload == "sublayer_backward":
        bench_sublayer_backward(args)
        return
    if args.workload == "stack_backward":
        bench_stack_backward(args)
        return
    if args.workload == "compact":
        bench_compact(args)
        return
    if args.workload == "vendor_gemm":
        bench_vendor_gemm(args)
        return

    import torch
    import synth
    from target_aware_latent_amd import llatte as C
    from target_aware_latent_amd.model import DeviceModel

    assert torch.cuda.is_available(), "bench.py needs the GPU"
    cfg = synth.get_config(args.config)
    prob = synth.generate(cfg, seed=0)
    I = prob["inputs"]
    lengths = [int(x) for x in I["lengths"]]
    model = DeviceModel(cfg, prob["weights"])
    model.pack()
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()
    offs = dev(I["offsets"].astype(np.int32))
    ctx = dev(I["ctx"]) if (cfg.n_q and cfg.d_c) else None
    out = model.alloc_outputs(lengths)
    stream = torch.cuda.current_stream()
    build_tokens = None
    if cfg.semantic is not None:
        # token build (hashed-ID table row + semantic vector W_s) inside the
        # step: the 1M-row table and the ids / semantic vectors are resident
        sp = cfg.semantic
        table = torch.empty(sp.vocab, cfg.d, dtype=torch.bfloat16, device="cuda")
        host_table = None if args.no_cpu_baseline else np.empty((sp.vocab, cfg.d), np.float32)
        print(f"building the {sp.vocab} x {cfg.d} table", file=sys.stderr, flush=True)
        for nb, (row0, blk) in enumerate(synth.full_table(cfg, 0)):
            table[row0:row0 + blk.shape[0]] = torch.from_numpy(blk).to("cuda").to(torch.bfloat16)
            if host_table is not None:
                host_table[row0:row0 + blk.shape[0]] = blk
            if nb % 16 == 15:
                print(f"  table rows {row0 + blk.shape[0]}", file=sys.stderr, flush=True)
        print("table built", file=sys.stderr, flush=True)
        Ws = dev(prob["weights"]["W_s"].astype(np.float32)).to(torch.bfloat16)
        tws = torch.empty(C.llatte_token_embed_workspace_size(cfg.d, sp.d_sem, C.LLATTE_BF16),
                          dtype=torch.uint8, device="cuda")
        tok_in = [(dev(I[k + "_ids"].astype(np.int32)),
                   dev(I[k + "_sem"].astype(np.float32)).to(torch.bfloat16), I[k + "_ids"].size)
                  for k in ("hist", "cand")]
        hist = torch.empty((tok_in[0][2], cfg.d), device="cuda")
        cand = torch.empty((tok_in[1][2], cfg.d), device="cuda")

        def build_tokens():
            for (ids, sem, n), o in zip(tok_in, (hist, cand)):
                C.llatte_token_embed(table, sp.vocab, ids, sem, Ws, n, cfg.d, sp.d_sem,
                                     C.LLATTE_BF16, o, tws, stream=stream)
    else:
        hist = dev(I["hist"])
        cand = dev(I["cand"]) if cfg.n_q else None
    if args.calibrate_copy:
        src = torch.empty(64 << 20, dtype=torch.float32, device="cuda").fill_(1.0)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    def step():
        if build_tokens is not None:
            build_tokens()
        model.forward(hist, offs, lengths, cand, ctx, out=out, stream=stream)

    print("warm-up", file=sys.stderr, flush=True)
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    print("timed steps", file=sys.stderr, flush=True)
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    w0 = time.perf_counter()
    ev0.record(stream)
    for _ in range(args.steps):
        step()
    ev1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - w0
    ms = ev0.elapsed_time(ev1)
    ms_step = ms / args.steps
    value = cfg.B / (ms_step / 1e3)
    F = absorbed_flops(cfg, lengths)
    Fna = non_absorbed_flops(cfg, lengths)
    tflops = F / (ms_step / 1e3) / 1e12
    peak = PEAK_BF16_TFLOPS if cfg.dtype == "bf16" else PEAK_F32_TFLOPS

    roofline = None
    kernels = {}
    if not args.no_kernel_times:
        C.llatte_kernel_timing_reset()
        C.llatte_kernel_timing_enable(True)
        for _ in range(args.steps):
            step()
        torch.cuda.synchronize()
        kt = C.llatte_kernel_timing_read()
        C.llatte_kernel_timing_enable(False)
        kf = kernel_flops(cfg, lengths)
        for name, (cnt, tot) in kt.items():
            e = {"launches_per_step": cnt / args.steps, "ms_per_step": tot / args.steps}
            if name in kf:
                e["tflops"] = kf[name] / (tot / args.steps / 1e3) / 1e12
            kernels[name] = e
        # by kernel symbol: every matrix product label runs the one GEMM
        # kernel template (gemm_kernel, in several tile instances)
        fam = {}
        for name, (cnt, tot) in kt.items():
            if name not in kf:
                continue
            f = family_of(name)
            c0, t0, fl0 = fam.get(f, (0, 0.0, 0.0))
            fam[f] = (c0 + cnt, t0 + tot, fl0 + kf[name] * args.steps)
        families = {}
        fb = family_bytes(cfg, lengths) if cfg.dtype == "bf16" else {}
        for f, (cnt, tot, fl) in fam.items():
            tf = fl / (tot / 1e3) / 1e12
            families[f] = {"launches_per_step": cnt / args.steps,
                           "ms_per_step": round(tot / args.steps, 4),
                           "tflops": round(tf, 2), "frac": round(tf / peak, 4)}
            if f in fb:
                families[f]["algorithmic_bytes_per_launch"] = round(fb[f] * args.steps / cnt)
        dom = max(fam, key=lambda f: fam[f][1])
        cnt, tot, fl = fam[dom]
        per_launch_flops = fl / cnt
        avg_s = tot / cnt / 1e3
        achieved = per_launch_flops / avg_s / 1e12
        # the committed traffic records were measured on the c3 workload
        traffic = read_traffic(args.traffic, dom) if (args.traffic or cfg.name == "c3") else None
        roofline = {"bound": "mfma", "kernel": dom, "achieved": round(achieved, 2),
                    "peak": peak, "unit": "TFLOP/s",
                    "frac": round(achieved / peak, 4), "traffic": traffic,
                    "flops_per_launch": per_launch_flops,
                    "avg_launch_ms": round(tot / cnt, 4)}

    phases = attention_phases(cfg, lengths, step) if args.attn_phases and cfg.dtype == "bf16" else None
    gphases = gemm_phases(cfg, lengths, step) if args.gemm_phases and cfg.dtype == "bf16" else None

    token_build = None
    if build_tokens is not None and "gemm_token_embed" in kernels:
        # HBM-bound gather-add: per token the table row (2 d bytes), the
        # semantic vector (2 d_sem), the id (4) in, the fp32 token (4 d) out
        e = kernels["gemm_token_embed"]
        ntok = sum(t[2] for t in tok_in)
        nbytes = ntok * (2 * cfg.d + 2 * cfg.semantic.d_sem + 4 + 4 * cfg.d)
        token_build = {"ms_per_step": round(e["ms_per_step"], 4),
                       "algorithmic_bytes_per_step": nbytes,
                       "GB/s": round(nbytes / (e["ms_per_step"] / 1e3) / 1e9, 1),
                       "frac_of_hbm_peak": round(nbytes / (e["ms_per_step"] / 1e3) / 1e9 / PEAK_HBM_GBS, 4),
                       "tflops": round(e.get("tflops", 0.0), 2)}

    cpu = None
    if not args.no_cpu_baseline:
        print("timing the CPU oracle", file=sys.stderr, flush=True)
        cpu = cpu_baseline_tokens(prob, host_table) if cfg.semantic is not None else cpu_baseline(prob)

    rec = {
        "metric": METRIC, "value": round(value, 1), "unit": "user-seq/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": cfg.dtype,
        "data": "synthetic (seeded N(0,1) inputs, N(0,1/fan_in) weights)",
        "config": {"workload": WORKLOAD_TEXT.get(cfg.name, cfg.name),
                   "global_batch": cfg.B, "seq_len": cfg.L or cfg.len_range[1],
                   "parallelism": "single GPU"},
        "tflops": round(tflops, 2), "pct_peak": round(100 * tflops / peak, 2),
        "flops_per_step_absorbed": F, "flops_per_step_non_absorbed": Fna,
        "tflops_non_absorbed_count": round(Fna / (ms_step / 1e3) / 1e12, 2),
        "wall_s_timed": round(wall, 3),
        "roofline": roofline, "cpu_baseline": cpu, "kernels": kernels,
        "kernel_symbols": families if not args.no_kernel_times else None,
    }
    if token_build is not None:
        rec["token_build"] = token_build
    if phases is not None:
        rec["attention_phases"] = phases
    if gphases is not None:
        rec["gemm_phases"] = gphases
    emit(rec)


if __name__ == "__main__":
    main()
