"""Benchmark of the block-sparse attention path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--config 480p]

One step = one pass of the whole path over one synthetic layer resident in
HBM: sparse_attn_select (pool, score, top-p/top-k, CSR) -> kv_demand_pack
(demand union, packed gather) -> sparse_attn_forward (work queue, attention
over the selected blocks).  Every stage is timed with HIP events on the
stream the library launches on; L2 and the Infinity Cache are flushed
before each step, outside the events: a 512 MiB write evicts them, then a
512 MiB read of another buffer forces the write-back of those dirty lines, so
the first kernel of the step starts on cold, clean caches.

Prints ONE JSON line.  ``value`` is selected-block attention TFLOP/s of the
whole step, 4*B^2*d*nnz / step time; ``roofline`` is that of the dominant
kernel (the attention forward, bf16 MFMA).  ``cpu_baseline`` times the CPU
oracle on a bounded sample of the same workload on this host.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0      # MI355X dense bf16 MFMA
PEAK_F32_TFLOPS = 157.3        # MI355X fp32 vector
PEAK_HBM_GBS = 8000.0          # MI355X HBM3E
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "hbm_bytes_480p_32k.md")
# the attention forward's source: the kernel file and the headers it includes
ATTN_SOURCES = [os.path.join(ROOT, "block_sparse_attention_scores_amd", "csrc", f)
                for f in ("attn_fwd.hip", "attend_bf16.h", "mfma_bf16.h", "sa_common.h")]


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--config", default="480p",
                    help="tiny | 480p | 720p_rank | lowrank | hetero | hetero_scale1 | lowrank_max | lowrank_mass")
    ap.add_argument("--unpacked", action="store_true", help="attend straight from K/V (no pack)")
    ap.add_argument("--no-flush", action="store_true", help="keep caches warm between steps")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extras", action="store_true",
                    help="skip the untimed load-balance and dense-context measurements")
    ap.add_argument("--graph", action="store_true",
                    help="also time the step captured once in a HIP graph and replayed")
    ap.add_argument("--cpu-items", type=int, default=768,
                    help="(head, query block) items in the oracle's timed sample")
    ap.add_argument("--tiles", default=None, metavar="TT,TH,TW",
                    help="video-aware block organisation: Q, K, V are gathered into 3-D tile "
                         "order before select and O, LSE back to raster order after forward "
                         "(both inside the timed step)")
    ap.add_argument("--backward", action="store_true",
                    help="also time sparse_attn_backward after each step (reported apart from "
                         "the forward path's value)")
    ap.add_argument("--copy-probe", type=int, default=0, metavar="MIB",
                    help="before warmup, run one plain device copy of MIB MiB (untimed), the "
                         "known-size kernel that calibrates FETCH_SIZE / WRITE_SIZE counters")
    return ap.parse_args()


def source_digest(paths):
    h = hashlib.sha256()
    for path in paths:
        with open(path, "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def load_traffic(config_name, nnz):
    """HBM bytes per attention launch from the rocprofv3 FETCH_SIZE/WRITE_SIZE
    summary, only if it was taken on the current kernel source (the digest of
    ATTN_SOURCES) and workload."""
    try:
        with open(TRAFFIC_FILE) as f:
            line = next((l for l in f if l.startswith("traffic-record:")), None)
        rec = json.loads(line.split(":", 1)[1]) if line else {}
    except (OSError, ValueError):
        return None
    r = rec.get(config_name)
    if not r or r.get("source_sha256") != source_digest(ATTN_SOURCES) or r.get("nnz") != nnz:
        return None
    return r.get("bytes_per_launch")


def cpu_baseline(w, x, n_items, sa=None):
    """The oracle, as it stands, on a bounded sample: selection, CSR/demand/pack
    for every row (pro-rated by the item fraction) and dense masked attention
    for ``n_items`` randomly chosen (head, query block) items.  With the GPU
    path's buffers ``sa``, the oracle's results are also compared with the
    GPU's (after the timing): returned as a ``parity`` entry."""
    import numpy as np
    from threadpoolctl import threadpool_info
    from oracle import oracle as O

    rows = w.heads * w.n_qb
    # token-level scores cost a pass over every token pair of a row: score
    # and select the sampled rows only (CSR, demand and pack then cover
    # them), and sample fewer rows so the leg stays near 15 s
    token = w.score_mode in (2, 3)
    # an item's dense masked attention costs in proportion to the key count:
    # the default 768 items are sized for 32k keys
    n_items = max(64, n_items * 32768 // max(w.kv_rows, 32768))
    n_items = min(n_items // 4 if token else n_items, rows)
    pick = np.random.default_rng(0).choice(rows, size=n_items, replace=False)
    items = [(int(r) // w.n_qb, int(r) % w.n_qb) for r in sorted(pick)]
    t0 = time.perf_counter()
    if token:
        if w.score_mode == 2:
            s = O.block_scores_lowrank_max(x["q"], x["k"], w.q_valid, w.kv_valid, w.block,
                                           x["wq"], x["wk"], items=items)
        else:
            s = O.block_scores_lowrank_mass(x["q"], x["k"], w.q_valid, w.kv_valid, w.block,
                                            x["wq"], x["wk"], w.eff_score_scale, items=items)
        mask = np.zeros(s.shape, bool)
        recs = {}
        for h, i in items:
            rec = (O.select_row_top_p(s[h, i], w.top_p, w.top_k) if w.select_mode == 0
                   else O.select_row_top_k(s[h, i], w.top_k))
            mask[h, i, rec.order[:rec.m]] = True
            recs[(h, i)] = rec
    else:
        _, _, s = O.scores_for(x["q"], x["k"], w.q_valid, w.kv_valid, w.block, w.score_mode,
                               w.eff_score_scale, x.get("wq"), x.get("wk"))
        mask, rec_list = O.select(s, w.select_mode, w.top_p, w.top_k)
        recs = {(r // w.n_qb, r % w.n_qb): rec for r, rec in enumerate(rec_list)}
    rp, ci = O.csr(mask)
    dp, di, _, _ = O.demand(mask, rp, ci)
    O.pack(x["k"], dp, di, w.block)
    O.pack(x["v"], dp, di, w.block)
    t_sel = time.perf_counter() - t0
    sel_rows = n_items if token else rows
    t0 = time.perf_counter()
    o_ref, lse_ref = O.attention(x["q"], x["k"], x["v"], mask, w.q_valid, w.kv_valid, w.block,
                                 w.eff_sm_scale, items=items)
    t_att = time.perf_counter() - t0
    nnz_sample = int(sum(mask[h, i].sum() for h, i in items))
    t = t_att + t_sel * n_items / sel_rows
    flops = 4.0 * w.block * w.block * w.head_dim * nnz_sample
    threads = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    parity = (parity_report(w, x, sa, mask, recs, items, o_ref, lse_ref)
              if sa is not None else None)
    return parity, {"value": flops / t / 1e12, "unit": "TFLOP/s", "cores": threads, "kind": "oracle",
            "sample": (f"{n_items} of {rows} (head, query-block) items of {w.name}: dense fp32 "
                       f"masked attention for the sample ({t_att:.2f} s) + fp64 selection, CSR, "
                       f"demand and pack of " + ("the sampled rows" if token else "all rows") +
                       f" ({t_sel:.2f} s) pro-rated by {n_items}/{sel_rows}"),
            "seconds": round(t_att + t_sel, 3), "host_cpus": os.cpu_count(),
            "cpu_model": cpu_model()}


def cpu_model():
    """The host CPU's model name (first processor entry of /proc/cpuinfo)."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def parity_report(w, x, sa, mask_ref, recs, items, o_ref, lse_ref):
    """The GPU path's outputs of the timed run against the oracle's results of
    the cpu_baseline leg (untimed):
      - selection: every row the oracle selected (all rows, or the sampled
        rows of the token-level modes); a differing row is excused only by the
        oracle's near-tie rule at relative 1e-6 and counted, any other is
        counted as a mismatch;
      - CSR, demand set and slot map: bit-exact given the GPU's mask (every row);
      - attention: max-abs error of the output and the LSE on the sampled items
        (where a row was excused the oracle recomputes it on the GPU's mask);
      - structure: selected fraction per head (min / mean / max over heads) and
        the demand fraction (demanded blocks over H * nKB)."""
    import numpy as np
    from oracle import oracle as O
    H, nqb, nkb = w.heads, w.n_qb, w.n_kb
    gmask = O.bits_to_mask(sa.mask_bits.cpu().numpy().view(np.uint32), H, nqb, nkb)
    excused = mismatched = 0
    for (h, i), rec in recs.items():
        if not np.array_equal(mask_ref[h, i], gmask[h, i]):
            if O.row_mismatch_excused(rec, w.select_mode, w.top_p, w.top_k, gmask[h, i], rel=1e-6):
                excused += 1
            else:
                mismatched += 1
    grp, gci = sa.host_csr()
    orp, oci = O.csr(gmask)
    odp, odi, _, ocs = O.demand(gmask, orp, oci)
    total = int(odp[-1])
    csr_exact = bool(np.array_equal(grp, orp) and np.array_equal(gci, oci))
    demand_exact = bool(np.array_equal(sa.demand_ptr.cpu().numpy(), odp) and
                        np.array_equal(sa.demand_idx[:total].cpu().numpy(), odi) and
                        np.array_equal(sa.col_slot[:orp[-1]].cpu().numpy(), ocs))
    redo = [(h, i) for h, i in items if not np.array_equal(mask_ref[h, i], gmask[h, i])]
    if redo:
        o2, l2 = O.attention(x["q"], x["k"], x["v"], gmask, w.q_valid, w.kv_valid, w.block,
                             w.eff_sm_scale, items=redo)
        for h, i in redo:
            sl = slice(i * w.block, (i + 1) * w.block)
            o_ref[h, sl], lse_ref[h, sl] = o2[h, sl], l2[h, sl]
    go = sa.out.float().cpu().numpy()
    gl = sa.lse.cpu().numpy()
    err_o = err_l = 0.0
    for h, i in items:
        sl = slice(i * w.block, (i + 1) * w.block)
        err_o = max(err_o, float(np.max(np.abs(go[h, sl] - o_ref[h, sl]))))
        fin = np.isfinite(lse_ref[h, sl])
        if fin.any():
            err_l = max(err_l, float(np.max(np.abs(gl[h, sl][fin] - lse_ref[h, sl][fin]))))
    frac = gmask.mean(axis=(1, 2))
    return {"selection_rows_checked": len(recs), "near_tie_rows_excused": excused,
            "selection_rows_mismatched": mismatched, "near_tie_rel": 1e-6,
            "csr_bit_exact": csr_exact, "demand_and_slots_bit_exact": demand_exact,
            "attention_items_checked": len(items),
            "attention_max_abs_err": round(err_o, 6), "lse_max_abs_err": round(err_l, 6),
            "attention_tol": 2e-2 if w.dtype == "bf16" else 1e-5,
            "per_head_selected_fraction": {"min": round(float(frac.min()), 4),
                                           "mean": round(float(frac.mean()), 4),
                                           "max": round(float(frac.max()), 4)},
            "demand_fraction": round(total / (H * nkb), 4)}


def main():
    args = parse()
    if args.gpus != 1:
        print(json.dumps({"error": "this path runs on one GPU; --gpus above 1 is not supported",
                          "n_gpus": args.gpus}))
        sys.exit(2)
    import numpy as np
    import torch
    from block_sparse_attention_scores_amd import binding, inputs as I
    from block_sparse_attention_scores_amd.path import SparseAttention, VideoLayout, to_device

    binding.load()                       # fails loudly if the HIP library is missing
    if not torch.cuda.is_available():
        print(json.dumps({"error": "no GPU visible"}))
        sys.exit(1)
    w = I.named(args.config)
    x = I.generate(w)
    d = to_device(x, w)
    tiles = tuple(int(v) for v in args.tiles.split(",")) if args.tiles else None
    if tiles:
        lay = VideoLayout(w.latent, tiles, w.q_start, w.q_valid)
        qt, kt, vt = (torch.empty_like(d[n]) for n in ("q", "k", "v"))
        out_r = torch.empty_like(d["q"])
        lse_r = torch.empty(w.heads, w.q_rows, 1, dtype=torch.float32, device="cuda")
        sa = SparseAttention(w, qt, kt, vt, d.get("wq"), d.get("wk"))
    else:
        sa = SparseAttention(w, d["q"], d["k"], d["v"], d.get("wq"), d.get("wk"))
    packed = not args.unpacked
    if args.backward:
        g = torch.Generator(device="cuda").manual_seed(7)
        dout = torch.randn(d["q"].shape, generator=g, device="cuda").to(d["q"].dtype)
        dout[:, w.q_valid:] = 0
        grads = [torch.empty_like(t) for t in (sa.q, sa.k, sa.v)]
        bwd_ws_bytes = binding.sa_workspace_size(sa.prob, binding.SA_STAGE_BACKWARD)
        bwd_ws = torch.empty(max(bwd_ws_bytes, 1), dtype=torch.uint8, device="cuda")
    flush = None if args.no_flush else (
        torch.empty(512 << 20, dtype=torch.uint8, device="cuda"),
        torch.zeros(64 << 20, dtype=torch.int64, device="cuda"))

    def step(ev):
        ev[0].record()
        if tiles:
            lay.gather(d["q"], lay.q_order, w.q_rows, out=qt)
            lay.gather(d["k"], lay.kv_order, w.kv_rows, out=kt)
            lay.gather(d["v"], lay.kv_order, w.kv_rows, out=vt)
        ev[1].record()
        sa.select()
        ev[2].record()
        if packed:
            sa.pack()
        ev[3].record()
        sa.forward(packed=packed)
        ev[4].record()
        if tiles:
            lay.to_raster(sa.out, w.q_rows, out=out_r)
            lay.to_raster(sa.lse.unsqueeze(-1), w.q_rows, out=lse_r)
        ev[5].record()
        if args.backward:
            binding.sparse_attn_backward(sa.prob, sa.q, sa.k, sa.v, sa.out, dout, sa.lse,
                                         sa.row_ptr, sa.col_idx, *grads, bwd_ws, bwd_ws_bytes)
        ev[6].record()

    if args.copy_probe > 0:
        src = torch.ones(args.copy_probe << 20, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    mk = lambda: [torch.cuda.Event(enable_timing=True) for _ in range(7)]
    for _ in range(args.warmup):
        step(mk())
    torch.cuda.synchronize()

    evs = [mk() for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for k in range(args.steps):
        if flush is not None:
            flush[0].fill_(k & 0xff)
            flush[1].amax()
        step(evs[k])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0

    pin = np.array([e[0].elapsed_time(e[1]) for e in evs])
    sel = np.array([e[1].elapsed_time(e[2]) for e in evs])
    pck = np.array([e[2].elapsed_time(e[3]) for e in evs])
    fwd = np.array([e[3].elapsed_time(e[4]) for e in evs])
    pout = np.array([e[4].elapsed_time(e[5]) for e in evs])
    bwd = np.array([e[5].elapsed_time(e[6]) for e in evs])
    tot = pin + sel + pck + fwd + pout
    nnz = sa.nnz()
    dense_pairs = w.heads * w.n_qb * w.n_kb
    flops = 4.0 * w.block * w.block * w.head_dim * nnz
    ms_step = float(tot.mean())
    eb = 2 if w.dtype == "bf16" else 4
    demand = int(sa.demand_ptr[-1].item())
    sel_bytes = w.heads * (w.q_rows + w.kv_rows) * w.head_dim * eb
    pack_bytes = 2 * 2 * demand * w.block * w.head_dim * eb
    fwd_ms = float(fwd.mean())
    achieved = flops / (fwd_ms / 1e3) / 1e12
    peak = PEAK_BF16_TFLOPS if w.dtype == "bf16" else PEAK_F32_TFLOPS
    traffic = load_traffic(w.name, nnz)

    rec = {
        "metric": "block-sparse attn TFLOP/s (selected blocks) + ms/layer @32k tokens, 1 MI355X",
        "value": round(flops / (ms_step / 1e3) / 1e12, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16" if w.dtype == "bf16" else "f32",
        "data": "synthetic (seeded clustered video-latent Q/K, N(0,1) V)",
        "config": {"workload": w.name, "heads": w.heads, "head_dim": w.head_dim,
                   "block": w.block, "q_tokens": w.q_valid, "kv_tokens": w.kv_valid,
                   "latent_thw": list(w.latent), "top_p": w.top_p, "top_k": w.top_k,
                   "select_mode": "top_p" if w.select_mode == 0 else "top_k",
                   "score": ("pooled", f"lowrank{w.rank}", f"lowrank{w.rank}_tokenmax",
                             f"lowrank{w.rank}_tokenmass")[w.score_mode],
                   "packed_kv": packed, "cache": "warm" if flush is None else "flushed each step",
                   "layout": "tiles " + "x".join(map(str, tiles)) if tiles else "raster"},
        "ms_per_layer": round(ms_step, 4),
        "stages_ms": {"select": round(float(sel.mean()), 4), "pack": round(float(pck.mean()), 4),
                      "forward": round(fwd_ms, 4),
                      **({"permute_in": round(float(pin.mean()), 4),
                          "permute_out": round(float(pout.mean()), 4)} if tiles else {}),
                      "forward_p10_p90": [round(float(np.percentile(fwd, 10)), 4),
                                          round(float(np.percentile(fwd, 90)), 4)]},
        # median, p10 and p90 of every stage over the timed steps
        "stages_ms_dist": {name: {"median": round(float(np.median(a)), 4),
                                  "p10": round(float(np.percentile(a, 10)), 4),
                                  "p90": round(float(np.percentile(a, 90)), 4)}
                           for name, a in (("select", sel), ("pack", pck), ("forward", fwd),
                                           ("step", tot))},
        "selected_blocks": nnz, "dense_blocks": dense_pairs,
        "selected_fraction": round(nnz / dense_pairs, 4),
        "demanded_blocks": demand, "selected_tflop": round(flops / 1e12, 4),
        "stage_roofline": {
            "select_hbm_frac": round(sel_bytes / (float(sel.mean()) / 1e3) / 1e9 / PEAK_HBM_GBS, 4),
            "pack_hbm_frac": (round(pack_bytes / (float(pck.mean()) / 1e3) / 1e9 / PEAK_HBM_GBS, 4)
                              if packed else None),
            "select_bytes": sel_bytes, "pack_bytes": pack_bytes},
        "roofline": {"bound": "mfma", "achieved": round(achieved, 3), "peak": peak,
                     "unit": "TFLOP/s", "frac": round(achieved / peak, 4),
                     "traffic": traffic,
                     "kernel": "sparse_attn_forward (work-queue sort + attention)"},
        "wall_s_timed_region": round(wall, 3),
    }
    if args.backward:
        bflops = 10.0 * w.block * w.block * w.head_dim * nnz   # dS, dP, dV, dK, dQ GEMMs
        bms = float(bwd.mean())
        rec["backward"] = {
            "ms": round(bms, 4), "tflop": round(bflops / 1e12, 4),
            "tflops": round(bflops / (bms / 1e3) / 1e12, 3),
            "frac_of_peak": round(bflops / (bms / 1e3) / 1e12 / peak, 4),
            "flops_counted": "10*B^2*d per selected pair (five GEMMs; recomputed S and dP not counted)"}
    if args.graph:
        rec["graph"] = graph_step(sa, packed, flush, args.steps, ms_step)
    if w.dtype == "bf16" and not args.no_extras:
        rec["load_balance"] = load_balance(sa, packed, flush)
        rec["dense_context"] = dense_context(w, d, sa, flush, packed, flops)
        if w.score_mode in (0, 1) and not tiles:
            rec["fused"] = fused_leg(w, d, sa, flush, args.steps, ms_step, flops)
        if w.name == "hetero_40h_32k" and not tiles:
            rec["hetero_scale1"] = scale1_leg(w, d, sa, flush, packed)
        rec["machine"] = machine_context(flush)
    if not args.no_cpu_baseline:
        parity, rec["cpu_baseline"] = cpu_baseline(w, x, args.cpu_items, sa)
        rec["parity"] = parity
    print(json.dumps(rec), flush=True)


def _flush(flush, k=0):
    if flush is not None:
        flush[0].fill_(k & 0xff)
        flush[1].amax()


def _timed(fn, flush, reps):
    """Median ms of `reps` runs of fn, each after a cache flush."""
    import numpy as np
    import torch
    ts = []
    for r in range(reps):
        _flush(flush, r)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        fn()
        e1.record()
        torch.cuda.synchronize()
        ts.append(e0.elapsed_time(e1))
    return float(np.median(ts))


def machine_context(flush, reps=5):
    """Context for the roofline fractions, measured on this GPU: compute-unit
    count and architecture (device properties), the engine clock rocminfo
    lists, a 1 GiB device copy (flushed, median of `reps`; read + write bytes
    over time), a dense bf16 GEMM through torch.mm (the vendor BLAS,
    8192 x 8192 x 8192, median of `reps` after one untimed call) and a
    register-only MFMA loop (libsa_probe.so), the matrix rate the chip holds
    with nothing else running."""
    import subprocess
    import torch
    props = torch.cuda.get_device_properties(0)
    ctx = {"cu_count": props.multi_processor_count, "arch": props.gcnArchName.split(":")[0]}
    try:
        r = subprocess.run(["rocminfo"], capture_output=True, text=True, timeout=60)
        clock = None
        for agent in re.split(r"\n\*+\s*\n\s*Agent \d+", r.stdout)[1:]:
            name = re.search(r"^\s*Name:\s*(\S+)", agent, re.M)
            mhz = re.search(r"Max Clock Freq\. \(MHz\):\s*(\d+)", agent)
            if name and mhz and name.group(1).startswith("gfx"):
                clock = int(mhz.group(1))
                break
        ctx["rocminfo_max_clock_mhz"] = clock
    except (OSError, subprocess.SubprocessError):
        ctx["rocminfo_max_clock_mhz"] = None
    n = 1 << 30
    src = torch.ones(n, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    ms = _timed(lambda: dst.copy_(src), flush, reps)
    ctx["copy_1gib_gbs"] = round(2 * n / (ms / 1e3) / 1e9, 1)
    del src, dst
    m = 8192
    g = torch.Generator(device="cuda").manual_seed(11)
    a = torch.randn(m, m, generator=g, device="cuda").to(torch.bfloat16)
    b = torch.randn(m, m, generator=g, device="cuda").to(torch.bfloat16)
    c = torch.mm(a, b)
    torch.cuda.synchronize()
    ms = _timed(lambda: torch.mm(a, b, out=c), flush, reps)
    ctx["gemm_bf16_8192_tflops"] = round(2.0 * m ** 3 / (ms / 1e3) / 1e12, 1)
    del a, b, c
    # matrix pipes alone: 1024 workgroups (four waves per SIMD), each wave 8192
    # rounds of eight independent v_mfma_f32_32x32x16_bf16 on registers
    try:
        import ctypes
        probe = ctypes.CDLL(os.path.join(ROOT, "block_sparse_attention_scores_amd", "lib",
                                         "libsa_probe.so"))
        wgs, iters = 1024, 8192
        out = torch.empty(wgs * 256, dtype=torch.float32, device="cuda")
        stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)

        def run_probe():
            if probe.sa_probe_mfma_bf16(wgs, iters, ctypes.c_void_p(out.data_ptr()), stream) != 0:
                raise RuntimeError("sa_probe_mfma_bf16 failed")
        run_probe()
        torch.cuda.synchronize()
        ms = _timed(run_probe, None, reps)
        ctx["mfma_bf16_loop_tflops"] = round(wgs * 4 * iters * 8 * 32768 / (ms / 1e3) / 1e12, 1)
        del out
    except OSError:
        ctx["mfma_bf16_loop_tflops"] = None
    torch.cuda.synchronize()
    return ctx


def graph_step(sa, packed, flush, steps, eager_ms):
    """select -> pack -> forward captured once into a HIP graph (the library
    only enqueues kernels on the caller's stream), replayed `steps` times
    with the cache flush outside the graph; ms per replay."""
    import numpy as np
    import torch

    def run():
        sa.select()
        if packed:
            sa.pack()
        sa.forward(packed=packed)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        run()
    torch.cuda.current_stream().wait_stream(side)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        run()
    torch.cuda.synchronize()
    ts = []
    for k in range(steps):
        _flush(flush, k)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        g.replay()
        e1.record()
        torch.cuda.synchronize()
        ts.append(e0.elapsed_time(e1))
    ts = np.array(ts)
    return {"ms_per_step": round(float(ts.mean()), 4),
            "p10_p90": [round(float(np.percentile(ts, 10)), 4), round(float(np.percentile(ts, 90)), 4)],
            "eager_ms_per_step": round(eager_ms, 4), "replays": steps}


def load_balance(sa, packed, flush, reps=5):
    """Busy time of each persistent workgroup (device clock stamps at its
    start and when it finds no more work): max / mean over workgroups, the
    single-GPU reading of the load imbalance the Top-p abstract reports
    across ranks.  Beside it, the same forward launched one workgroup per
    work unit (hardware dispatch, no queue kernel reuse of workgroups)."""
    import numpy as np
    import torch
    from block_sparse_attention_scores_amd import binding
    n = sa.workgroups(binding.SA_SCHEDULE_PERSISTENT)
    clk = torch.zeros(2 * n, dtype=torch.int64, device="cuda")
    imb, span = [], []
    for r in range(reps):
        _flush(flush, r)
        sa.forward(packed=packed, wg_clock=clk)
        torch.cuda.synchronize()
        c = clk.view(n, 2).cpu().numpy().astype(np.float64)
        busy = c[:, 1] - c[:, 0]
        imb.append(busy.max() / busy.mean())
        span.append((c[:, 1].max() - c[:, 0].min()) / busy.mean())
    # the two schedules timed the same way (flush, then the forward alone),
    # alternating so that neither gains from running second
    pers, unit = [], []
    for r in range(reps):
        pers.append(_timed(lambda: sa.forward(packed=packed,
                                              schedule=binding.SA_SCHEDULE_PERSISTENT), flush, 1))
        unit.append(_timed(lambda: sa.forward(packed=packed,
                                              schedule=binding.SA_SCHEDULE_PER_UNIT), flush, 1))
    return {"workgroups": n, "busy_max_over_mean": round(float(np.median(imb)), 4),
            "span_over_mean_busy": round(float(np.median(span)), 4),
            "persistent_forward_ms": round(float(np.median(pers)), 4),
            "per_unit_workgroups": sa.workgroups(binding.SA_SCHEDULE_PER_UNIT),
            "per_unit_forward_ms": round(float(np.median(unit)), 4), "reps": reps,
            "default_schedule": "per_unit" if sa.w.select_mode == binding.SA_TOP_K else "persistent"}


def fused_leg(w, d, sa, flush, steps, three_call_ms, flops):
    """The fused single pass (sparse_attn_fused: pooling, then one kernel that
    scores, selects (top-p with the floor, or top-k) and attends per query
    block) timed like the step: a flush, then the call, ``steps`` times;
    against the three-call path's ms per layer of the timed steps.  Its kept
    sets are compared with the three-call path's mask row by row (in top-p the
    two sum the masses in different orders, so a row whose cut sits within
    rounding of p may differ by a block)."""
    import numpy as np
    import torch
    from block_sparse_attention_scores_amd import binding
    prob = sa.prob
    n = binding.sa_workspace_size(prob, binding.SA_STAGE_FUSED)
    ws = torch.empty(max(n, 256), dtype=torch.uint8, device="cuda")
    out = torch.empty_like(sa.out)
    lse = torch.empty_like(sa.lse)
    bits = torch.empty_like(sa.mask_bits)
    lowrank = w.score_mode == 1

    def run(mask=None):
        binding.sparse_attn_fused(prob, sa.q, sa.k, sa.v, d.get("wq") if lowrank else None,
                                  d.get("wk") if lowrank else None, out, lse, mask, ws, n)

    run(bits)
    torch.cuda.synchronize()
    same = bool(torch.equal(bits, sa.mask_bits))
    rows_differing = int((bits != sa.mask_bits).any(dim=1).sum())
    ts = []
    for r in range(steps):
        _flush(flush, r)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        run()
        e1.record()
        torch.cuda.synchronize()
        ts.append(e0.elapsed_time(e1))
    ts = np.array(ts)
    ms = float(np.median(ts))
    return {"ms_per_layer": round(ms, 4),
            "p10_p90": [round(float(np.percentile(ts, 10)), 4), round(float(np.percentile(ts, 90)), 4)],
            "tflops": round(flops / (ms / 1e3) / 1e12, 3),
            "three_call_ms_per_layer": round(three_call_ms, 4),
            "speedup_over_three_call": round(three_call_ms / ms, 3),
            "same_mask_as_three_call": same, "rows_differing": rows_differing,
            "steps": steps}


def scale1_leg(w, d, sa, flush, packed, reps=5):
    """The 40-head inputs selected at temperature 1 (score_scale 1): heads
    keep from about 2% to over 90% of their blocks, the per-head spread of
    the Top-p abstract's stragglers.  Reports that spread and both work
    schedules' forward (load_balance)."""
    import numpy as np
    from block_sparse_attention_scores_amd import inputs as I
    from block_sparse_attention_scores_amd.path import SparseAttention
    ws = I.named("hetero_scale1")
    s1 = SparseAttention(ws, sa.q, sa.k, sa.v, d.get("wq"), d.get("wk"))
    s1.select()
    if packed:
        s1.pack()
    rp = s1.row_ptr.cpu().numpy().astype(np.int64)
    per_head = (rp[ws.n_qb::ws.n_qb][:ws.heads] - rp[:-1:ws.n_qb][:ws.heads]) / (ws.n_qb * ws.n_kb)
    nnz = s1.nnz()
    flops = 4.0 * ws.block * ws.block * ws.head_dim * nnz
    lb = load_balance(s1, packed, flush, reps)
    out = {"workload": ws.name, "score_scale": ws.score_scale, "selected_blocks": int(nnz),
           "selected_fraction": round(nnz / (ws.heads * ws.n_qb * ws.n_kb), 4),
           "per_head_selected_fraction": {
               "min": round(float(per_head.min()), 4), "p25": round(float(np.percentile(per_head, 25)), 4),
               "median": round(float(np.median(per_head)), 4), "max": round(float(per_head.max()), 4)},
           "load_balance": lb,
           "persistent_tflops": round(flops / (lb["persistent_forward_ms"] / 1e3) / 1e12, 3),
           "per_unit_tflops": round(flops / (lb["per_unit_forward_ms"] / 1e3) / 1e12, 3)}
    del s1
    return out


def dense_context(w, d, sa, flush, packed, flops, reps=5):
    """The same attention kernel with every block selected (p = 1), attending
    straight from K/V: what the sparse forward is measured against.  Both are
    timed the same way (a flush, then the forward alone), alternating."""
    import numpy as np
    from block_sparse_attention_scores_amd.path import SparseAttention
    dn = SparseAttention(w.with_(top_p=1.0, select_mode=0), sa.q, sa.k, sa.v, d.get("wq"),
                         d.get("wk"), packed_cap=1)
    dn.select()
    dense_pairs = w.heads * w.n_qb * w.n_kb
    assert dn.nnz() == dense_pairs
    dense, sparse = [], []
    for r in range(reps):
        dense.append(_timed(lambda: dn.forward(packed=False), flush, 1))
        sparse.append(_timed(lambda: sa.forward(packed=packed), flush, 1))
    ms, sms = float(np.median(dense)), float(np.median(sparse))
    dflops = flops / sa.nnz() * dense_pairs
    del dn
    return {"forward_ms": round(ms, 4), "tflops": round(dflops / (ms / 1e3) / 1e12, 3),
            "sparse_forward_ms": round(sms, 4), "sparse_forward_speedup": round(ms / sms, 3),
            "reps": reps}


if __name__ == "__main__":
    main()
