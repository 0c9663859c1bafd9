"""Throughput of the vocabulary-sharded LM-head cross-entropy + masked embedding path
on one MI355X.

One step = the tied embedding + LM-head step over one batch:
    vemb_fwd (masked lookup of the input IDs)  ->  vce_fwd (fused logits GEMM +
    per-shard online max/sum-exp + cross-shard merge)  ->  vce_bwd (logit
    recompute into G = scale*(softmax - onehot), dh and dW GEMMs)  ->  vemb_bwd
    (scatter-add of dh into the same dW).
Default workload: T=16384 tokens, H=3072, V=201088 (GPT-OSS-20B's table), bf16,
8 contiguous vocabulary shards, Zipf(1.1) tokens, 1% out-of-range IDs, 2%
ignored targets; inputs are seeded, synthetic and already in HBM when the
timed region starts.

    python bench.py [--steps K] [--warmup W] [--workload c4|c3] [--no-cpu-baseline]

Prints one JSON line. Only one GPU is used; --gpus above 1 is refused.
"""

from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "fused LM-head CE fwd+bwd tokens/s (V=201088,H=3072,bf16); % MFMA peak"
PEAK_BF16 = 2.5e15      # MI355X dense bf16 MFMA, FLOP/s
PEAK_HBM = 8.0e12       # MI355X HBM3E, B/s
CSRC = os.path.join(ROOT, "vocab_embedding_softmax_amd", "csrc")
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_ce_gemms_c4.txt")


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="c4", choices=["c3", "c4"])
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-c3", action="store_true",
                    help="skip the CE-only field on the T=8192 workload")
    ap.add_argument("--no-sampled", action="store_true",
                    help="skip the sampled-softmax field (its own T=16384, H=1536 workload)")
    ap.add_argument("--cpu-tokens", type=int, default=4096,
                    help="tokens in the oracle's CPU-baseline sample")
    ap.add_argument("--sampled-only", action="store_true",
                    help="time only the sampled-softmax step (T=16384, H=1536, V=131072, "
                         "P=16384) and print its field; for its kernel summary")
    ap.add_argument("--emb-only", action="store_true",
                    help="time only the lookup and scatter-add of the tied workload (warm and "
                         "cold) and print their rooflines; for the traffic-counter runs")
    ap.add_argument("--copy-probe", action="store_true",
                    help="also run one elementwise pass over 1 GiB (read 1 GiB, write 1 GiB): "
                         "the reference kernel that calibrates FETCH_SIZE / WRITE_SIZE")
    return ap.parse_args()


# the sources the cross-entropy GEMM kernels are compiled from
GEMM_SOURCES = ("gemm_tn.hpp", "vce_ce.hip", "vce_device.hpp", "vce_internal.hpp")


def kernel_source_hash() -> str:
    """Hash of the GEMM kernels' code: comments (from // to the end of a line)
    and blank lines are left out, so that a comment edit keeps counters taken
    on the same compiled kernels valid."""
    h = hashlib.sha256()
    for name in GEMM_SOURCES:
        with open(os.path.join(CSRC, name), encoding="utf-8") as f:
            code = [line.split("//", 1)[0].rstrip() for line in f]
        h.update(name.encode())
        h.update("\n".join(line for line in code if line).encode())
    return h.hexdigest()[:16]


def measured_traffic(tag: str):
    """HBM bytes per launch of one CE GEMM kernel (tag: fwd, grad, dh, dw) from
    the committed rocprofv3 FETCH_SIZE / WRITE_SIZE summary, each counter
    scaled by its own reading for a copy of known size; None when absent or
    taken on other kernel sources."""
    try:
        vals = {}
        with open(TRAFFIC_FILE) as f:
            for line in f:
                if line.startswith("#") or not line.strip():
                    continue
                k, v = line.split(None, 1)
                vals[k] = v.strip()
        if vals.get("source_hash") != kernel_source_hash():
            return None
        copy_bytes = float(vals["copy_bytes"])
        f_scale = copy_bytes / (float(vals["copy_fetch_kib"]) * 1024.0)
        w_scale = copy_bytes / (float(vals["copy_write_kib"]) * 1024.0)
        return (float(vals[f"{tag}_fetch_kib"]) * 1024.0 * f_scale +
                float(vals[f"{tag}_write_kib"]) * 1024.0 * w_scale)
    except (OSError, KeyError, ValueError):
        return None


def cpu_baseline(inp, n_tok: int):
    """The float64 oracle as it stands (oracle.parallel: its definitions over
    token and vocabulary chunks on a pool of threads, one BLAS thread each),
    on the first n_tok tokens of the same workload, on this host's cores
    (at most 16, the host share of one GPU). Returns tokens/s of the oracle
    step on that sample."""
    import oracle
    workers = oracle.parallel.default_workers()
    W = oracle.decode(inp.W, inp.dtype)
    t0 = time.perf_counter()
    if inp.h is None:
        oracle.parallel.tied_step(inp.ids[:n_tok], inp.targets[:n_tok], W, inp.V_real, inp.V_pad,
                                  inp.num_shards, inp.ignore_index, workers=workers)
        what = "tied step (gather, CE fwd+bwd, scatter-add)"
    else:
        h = oracle.decode(inp.h[:n_tok], inp.dtype)
        oracle.parallel.cross_entropy(h, W, inp.targets[:n_tok], inp.V_real, inp.V_pad,
                                      inp.num_shards, inp.ignore_index, workers=workers)
        what = "CE fwd+bwd"
    dt = time.perf_counter() - t0
    del W
    return dict(value=n_tok / dt, unit="tokens/s", cores=int(workers), kind="oracle",
                cpu_model=oracle.parallel.cpu_model(), host_cpus=os.cpu_count(),
                sample=f"token sample: float64 oracle {what} on the first {n_tok} of the "
                       f"workload's {inp.T} tokens (full V={inp.V_real}, H={inp.H}), "
                       f"{workers} threads; {dt:.1f} s wall")


def sampled_field(V, dev, stream):
    """The sampled-softmax step on its own workload, timed back to back."""
    import numpy as np
    import torch
    from synth import config_inputs
    f32 = dict(dtype=torch.float32, device=dev)
    dt_code = V.VCE_BF16
    # Sampled-softmax step on its own workload (T=16384, H=1536, V=131072,
    # P=16384): candidates, gather of W[cand], CE fwd+bwd over the
    # candidates, scatter of dW[cand] back into the full table. The table
    # is kept from step to step (zeroed once): each step clears the
    # previous step's candidate rows and writes its own, which leaves the
    # same table as the whole-table fill (timed too, as ms_full_fill).
    # MFMA work = 8*T*H*n_cand.
    inp5 = config_inputs("c5")
    T5, H5, V5, P5 = inp5.T, inp5.H, inp5.V_real, inp5.P
    h5 = V.from_bits(inp5.h, inp5.dtype, dev)
    W5 = V.from_bits(inp5.W, inp5.dtype, dev)
    tg5 = torch.from_numpy(inp5.targets).to(dev)
    perm5 = torch.from_numpy(inp5.perm).to(dev)
    ws5 = V.Workspaces(dev, cand=V.vss_candidates_workspace_bytes(T5, V5),
                       fwd=V.vce_fwd_workspace_bytes(T5, H5, P5, P5, 1, dt_code),
                       bwd=V.vce_bwd_workspace_bytes(T5, H5, P5, P5, 1, dt_code))
    dW5 = torch.zeros(V5, H5, **f32)

    # the first call reads the candidate count from the device; the timed
    # calls of the same batch pass it (no synchronisation inside the step)
    r5 = V.sampled_step(h5, W5, tg5, perm5, P5, inp5.ignore_index, ws=ws5, dW=dW5,
                        prev_rows=torch.empty(0, dtype=torch.int32, device=dev))
    torch.cuda.synchronize()
    n_cand = int(r5.extra["n_cand"].item())
    kept = [r5.extra["rows"]]

    gl5 = torch.ones(1, **f32)

    def samp():
        r = V.sampled_step(h5, W5, tg5, perm5, P5, inp5.ignore_index, grad_loss=gl5, ws=ws5,
                           dW=dW5, prev_rows=kept[0], n_cand=n_cand, allow_bad=True)
        kept[0] = r.extra["rows"]

    def samp_full():
        V.sampled_step(h5, W5, tg5, perm5, P5, inp5.ignore_index, grad_loss=gl5, ws=ws5,
                       dW=dW5, n_cand=n_cand, allow_bad=True)

    def timed(fn, reps5=5):
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(reps5):
            fn()
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / reps5

    # untimed steps first (the clock ramps up over the first few after the
    # idle time of the input generation), then the two forms alternately
    for _ in range(5):
        samp()
    rounds = [(timed(samp), timed(samp_full)) for _ in range(2)]
    ms5 = float(np.mean([r[0] for r in rounds]))
    ms5_full = float(np.mean([r[1] for r in rounds]))
    out = {
        "workload": f"T={T5}, H={H5}, V={V5}, P={P5}, Zipf(1.1) targets",
        "n_cand": n_cand, "ms": ms5, "tokens_s": T5 / (ms5 * 1e-3),
        "mfma_frac": 8.0 * T5 * H5 * n_cand / (ms5 * 1e-3) / PEAK_BF16,
        "ms_full_fill": ms5_full}
    log(f"[bench] sampled-softmax step {ms5:.3f} ms")
    del h5, W5, ws5, dW5, r5
    torch.cuda.empty_cache()
    return out


def main():
    a = parse()
    if a.gpus != 1:
        print(json.dumps({"error": "this build runs on one GPU only; --gpus must be 1",
                          "n_gpus_requested": a.gpus}))
        sys.exit(2)
    import numpy as np
    import torch
    import vocab_embedding_softmax_amd as V
    from synth import config_inputs

    if not torch.cuda.is_available():
        raise SystemExit("bench.py needs a GPU")
    dev = torch.device("cuda:0")
    if a.sampled_only:
        stream = torch.cuda.current_stream(dev)
        print(json.dumps({"sampled_softmax": sampled_field(V, dev, stream)}), flush=True)
        return
    log(f"[bench] generating {a.workload} inputs")
    inp = config_inputs(a.workload)
    T, H, Vr, Vp, n = inp.T, inp.H, inp.V_real, inp.V_pad, inp.num_shards
    W = V.from_bits(inp.W, inp.dtype, dev)
    tg = torch.from_numpy(inp.targets).to(dev)
    tied = inp.h is None
    if tied:
        ids = torch.from_numpy(inp.ids).to(dev)
        h = torch.empty(T, H, dtype=torch.bfloat16, device=dev)
    else:
        h = V.from_bits(inp.h, inp.dtype, dev)
    dt_code = V.VCE_BF16
    ws = V.Workspaces(dev, fwd=V.vce_fwd_workspace_bytes(T, H, Vr, Vp, n, dt_code),
                      bwd=V.vce_bwd_workspace_bytes(T, H, Vr, Vp, n, dt_code),
                      emb=V.vemb_bwd_workspace_bytes(T, H, Vr, Vp))
    f32 = dict(dtype=torch.float32, device=dev)
    i32 = dict(dtype=torch.int32, device=dev)
    fo = V._lib.FwdOut(torch.empty(T, **f32), torch.empty(T, **f32), torch.empty(1, **f32),
                       torch.empty(1, **i32), torch.empty(1, **i32), None)
    dh = torch.empty(T, H, **f32)
    dW = torch.empty(Vp, H, **f32)
    nbad = torch.empty(1, **i32)
    gl = torch.ones(1, **f32)
    stream = torch.cuda.current_stream(dev)

    # events: 0 start | 1 after lookup | 2 after forward | backward: start, then per
    # vocabulary chunk (after G, after dh, after dW) | last: after the scatter
    n_bwd_ev = V._lib.vce_bwd_event_count(T, H, Vr, Vp, n, dt_code)
    n_chunks = (n_bwd_ev - 1) // 3
    n_ev = 3 + n_bwd_ev + 1

    def new_events():
        return [torch.cuda.Event(enable_timing=True) for _ in range(n_ev)]

    def step(ev=None):
        if ev is not None:
            ev[0].record(stream)
        if tied:
            V.vemb_fwd(ids, W, Vr, n, out=h, n_bad=nbad)
        if ev is not None:
            ev[1].record(stream)
        # bad targets are counted on the device and checked after the timed
        # steps (a check here would synchronise inside the step)
        V.vce_fwd(h, W, tg, Vr, n, inp.ignore_index, out=fo, ws=ws["fwd"], allow_bad=True)
        if ev is not None:
            ev[2].record(stream)
        V.vce_bwd(h, W, tg, fo.lse, gl, fo.n_valid, Vr, n, inp.ignore_index, V.REDUCE_MEAN,
                  dh=dh, dW=dW, accumulate_dW=False, ws=ws["bwd"],
                  events=None if ev is None else ev[3:3 + n_bwd_ev])
        if tied:
            V.vemb_bwd(ids, dh, Vr, Vp, n, dW=dW, accumulate=True, ws=ws["emb"])
        if ev is not None:
            ev[n_ev - 1].record(stream)

    # distinct valid IDs of the tied workload (the lookup's and the
    # scatter's algorithmic bytes count each touched row once)
    uniq = int(np.unique(inp.ids[(inp.ids >= 0) & (inp.ids < Vr)]).shape[0]) if tied else 0

    def per_call(fn, n_rep=20):
        """Mean time of one call, n_rep calls back to back after one untimed
        call (the in-step spans hold one short call each, so event overhead
        weighs on them)."""
        fn()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(n_rep):
            fn()
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / n_rep

    def emb_rooflines(ms_g_step, ms_s_step):
        """Lookup and scatter-add of the tied table, repeated back to back
        (warm) and after a cache-evicting read (cold), against 8 TB/s."""
        # algorithmic HBM bytes (unique rows read once, outputs written once)
        gather_bytes = uniq * H * 2 + T * H * 2 + 4 * T
        scatter_bytes = T * H * 4 + 8 * T + 2 * uniq * H * 4

        # Cold: a 512 MB read (twice the MALL) before every call evicts the
        # table rows and dout from the caches and leaves clean lines (a write
        # would leave dirty ones for the timed call to write back); it stays
        # queued ahead of the call, so the host's launch latency is not inside
        # the span.
        flush = torch.ones(128 << 20, dtype=torch.float32, device=dev)
        sink = torch.empty(1, dtype=torch.float32, device=dev)

        def cold_call(fn, n_rep=10):
            fn()
            ts = []
            for _ in range(n_rep):
                e0 = torch.cuda.Event(enable_timing=True)
                e1 = torch.cuda.Event(enable_timing=True)
                torch.amax(flush, dim=0, out=sink[0])
                e0.record(stream)
                fn()
                e1.record(stream)
                torch.cuda.synchronize()
                ts.append(e0.elapsed_time(e1))
            return float(np.median(ts))

        gather = lambda: V.vemb_fwd(ids, W, Vr, n, out=h, n_bad=nbad)
        scatter = lambda: V.vemb_bwd(ids, dh, Vr, Vp, n, dW=dW, accumulate=True, ws=ws["emb"])
        ms_g, ms_s = per_call(gather), per_call(scatter)
        ms_gc, ms_sc = cold_call(gather), cold_call(scatter)
        del flush, sink
        occ_bytes = 2 * T * H * 2 + 4 * T  # every token's row read and written

        def roof(nbytes, ms, ms_cold, ms_step_phase):
            return {"bytes": nbytes, "ms": ms, "ms_cold": ms_cold, "ms_in_step": ms_step_phase,
                    "GB_s": nbytes / (ms * 1e-3) / 1e9,
                    "frac": nbytes / (ms * 1e-3) / PEAK_HBM,
                    "frac_cold": nbytes / (ms_cold * 1e-3) / PEAK_HBM}

        return {
            "vemb_fwd": dict(roof(gather_bytes, ms_g, ms_gc, ms_g_step),
                             bytes_per_occurrence=occ_bytes,
                             frac_per_occurrence=occ_bytes / (ms_g * 1e-3) / PEAK_HBM),
            "vemb_bwd": roof(scatter_bytes, ms_s, ms_sc, ms_s_step),
        }

    def copy_probe():
        src = torch.ones(1 << 28, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        torch.neg(src, out=dst)
        torch.cuda.synchronize()
        del src, dst
        return (1 << 28) * 4

    def copy_reference():
        """Plain device copies of the lookup's output and the scatter's dout
        sizes, timed like the calls (warm: back to back; cold: after a 512 MB
        read), bytes counted in both directions."""
        flush = torch.ones(128 << 20, dtype=torch.float32, device=dev)
        sink = torch.empty(1, dtype=torch.float32, device=dev)
        out = {}
        for name, dt in (("bf16_TxH", torch.bfloat16), ("f32_TxH", torch.float32)):
            x = torch.ones(T, H, dtype=dt, device=dev)
            y = torch.empty_like(x)
            fn = lambda: y.copy_(x)
            fn()
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            for _ in range(20):
                fn()
            e1.record(stream)
            torch.cuda.synchronize()
            warm = e0.elapsed_time(e1) / 20
            ts = []
            for _ in range(10):
                torch.amax(flush, dim=0, out=sink[0])
                e0.record(stream)
                fn()
                e1.record(stream)
                torch.cuda.synchronize()
                ts.append(e0.elapsed_time(e1))
            cold = float(np.median(ts))
            nb = 2 * x.numel() * x.element_size()
            out[name] = {"bytes": nb, "ms": warm, "ms_cold": cold,
                         "frac": nb / (warm * 1e-3) / PEAK_HBM,
                         "frac_cold": nb / (cold * 1e-3) / PEAK_HBM}
            del x, y
        del flush, sink
        return out

    if a.emb_only:
        if not tied:
            raise SystemExit("--emb-only times the tied workload's lookup and scatter (c4)")
        gen = torch.Generator(device=dev)
        gen.manual_seed(5)
        dh.normal_(generator=gen)
        dW.zero_()
        res = {"workload": f"lookup and scatter-add of the tied step: T={T}, H={H}, "
                           f"V_real={Vr}, {n} shards, bf16 table, float32 dout",
               "hbm_rooflines": emb_rooflines(None, None),
               "copy_reference": copy_reference()}
        if a.copy_probe:
            res["copy_probe_bytes"] = copy_probe()
        print(json.dumps(res), flush=True)
        return

    log(f"[bench] warmup {a.warmup}")
    for _ in range(a.warmup):
        step(new_events())
    torch.cuda.synchronize()
    evs = [new_events() for _ in range(a.steps)]
    log(f"[bench] timing {a.steps} steps")
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for k in range(a.steps):
        step(evs[k])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_step = wall * 1e3 / a.steps
    if int(fo.n_bad.item()):
        raise SystemExit(f"{int(fo.n_bad.item())} bad targets in the workload")

    def span(i, j):
        return float(np.mean([e[i].elapsed_time(e[j]) for e in evs]))

    b0 = 3  # first backward event
    phase = {
        "vemb_fwd": span(0, 1),
        "vce_fwd": span(1, 2),
        "vce_bwd.recompute_G": sum(span(b0 + 3 * c, b0 + 3 * c + 1) for c in range(n_chunks)),
        "vce_bwd.dh": sum(span(b0 + 3 * c + 1, b0 + 3 * c + 2) for c in range(n_chunks)),
        "vce_bwd.dW": sum(span(b0 + 3 * c + 2, b0 + 3 * c + 3) for c in range(n_chunks)),
        "vemb_bwd": span(n_ev - 2, n_ev - 1),
    }
    log(f"[bench] {ms_step:.3f} ms/step, phases (ms) {json.dumps(phase)}")

    # Each of the four CE GEMMs does 2*T*H*V_real algorithmic flops per step.
    # The forward is one launch; each backward GEMM is one launch per
    # vocabulary chunk (2*T*H*(real rows of the chunk) flops), timed on the
    # stream it runs on; flops per launch / mean launch time equals the step
    # totals' ratio below.
    flop_gemm = 2.0 * T * H * Vr
    gemms = {
        "fwd": ("k_gemm_tn<bf16,EPI_FWD> (vce_fwd: logits GEMM + online max/sum-exp, 1 launch)",
                phase["vce_fwd"], 1),
        "grad": (f"k_gemm_tn<bf16,EPI_GRAD> (logit recompute + G = scale*(softmax-onehot), "
                 f"{n_chunks} launches, one per vocabulary chunk)", phase["vce_bwd.recompute_G"],
                 n_chunks),
        "dh": (f"k_gemm_tn<bf16,EPI_STORE,KC,KM> (dh += G_chunk W_chunk, {n_chunks} launches)",
               phase["vce_bwd.dh"], n_chunks),
        "dw": (f"k_gemm_tn<bf16,EPI_STORE,KM,KM> (dW_chunk = G_chunk^T h, {n_chunks} chunks: per "
               f"chunk the rows of the whole rounds of tiles in one launch, any rest in a K-split one)",
               phase["vce_bwd.dW"], n_chunks),
    }
    dom_tag = max(gemms, key=lambda k: gemms[k][1])
    dom, dom_ms, dom_launches = gemms[dom_tag]
    achieved = flop_gemm / (dom_ms * 1e-3) / 1e12
    traffic = measured_traffic(dom_tag) if a.workload == "c4" else None
    path_frac = 8.0 * T * H * Vr / (ms_step * 1e-3) / PEAK_BF16
    res = {
        "metric": METRIC,
        "value": T / (ms_step * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": a.steps,
        "warmup": a.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": ("tied embedding + LM-head step" if tied else "LM-head CE fwd+bwd")
                        + f": T={T}, H={H}, V_real={Vr}, V_pad={Vp}, {n} contiguous vocab shards, "
                          "bf16 inputs, fp32 accumulation, Zipf(1.1) tokens",
            "T": T, "H": H, "V_real": Vr, "V_pad": Vp, "num_shards": n,
        },
        "roofline": {
            "bound": "mfma",
            "kernel": dom,
            "launches_per_step": dom_launches,
            "achieved": achieved,
            "peak": PEAK_BF16 / 1e12,
            "unit": "TFLOP/s",
            "frac": achieved / (PEAK_BF16 / 1e12),
            "traffic": traffic,
        },
        "path_mfma_frac": path_frac,
        # the same over the stricter useful work 6*H*V_real per token (the
        # logit recompute of the backward not counted)
        "path_mfma_frac_useful": 0.75 * path_frac,
        "phases_ms": phase,
    }
    if tied:
        res["hbm_rooflines"] = emb_rooflines(phase["vemb_fwd"], phase["vemb_bwd"])
    # Greedy argmax over the same table and hidden rows (the decoding twin of
    # the forward: same logits GEMM, (max, lowest index) epilogue), timed on
    # its own after the step: flops per call = 2*T*H*V_real.
    ws_arg = torch.empty(V.vce_argmax_workspace_bytes(T, H, Vr, Vp, n, dt_code),
                         dtype=torch.uint8, device=dev)
    out_arg = V.vce_argmax(h, W, Vr, n, ws=ws_arg)
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    reps = 3
    e0.record(stream)
    for _ in range(reps):
        V.vce_argmax(h, W, Vr, n, out=out_arg, ws=ws_arg)
    e1.record(stream)
    torch.cuda.synchronize()
    ms_arg = e0.elapsed_time(e1) / reps
    res["argmax"] = {"kernel": "k_gemm_tn<bf16,EPI_ARGMAX> + k_argmax_merge (vce_argmax)",
                     "ms": ms_arg, "tokens_s": T / (ms_arg * 1e-3),
                     "achieved_TFLOP_s": flop_gemm / (ms_arg * 1e-3) / 1e12,
                     "frac": flop_gemm / (ms_arg * 1e-3) / PEAK_BF16}
    log(f"[bench] argmax {ms_arg:.3f} ms/call")
    # The forward under an explicit uneven layout of the same table (seeded:
    # one empty and one one-row shard among n, random cut points elsewhere),
    # timed beside the even layout on the same inputs.
    from synth import make_layout
    rows = [int(x) for x in make_layout(Vp, n, seed=8, n_empty=1, n_single=1)]
    ws_u = torch.empty(V.vce_fwd_workspace_bytes(T, H, Vr, Vp, n, dt_code, shard_rows=rows),
                       dtype=torch.uint8, device=dev)

    def time_fwd(**kw):
        V.vce_fwd(h, W, tg, Vr, n, inp.ignore_index, out=fo, **kw)
        e0.record(stream)
        for _ in range(reps):
            V.vce_fwd(h, W, tg, Vr, n, inp.ignore_index, out=fo, allow_bad=True, **kw)
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / reps

    ms_even = time_fwd(ws=ws["fwd"])
    ms_unev = time_fwd(ws=ws_u, shard_rows=rows)
    sizes = np.diff(np.asarray(rows))
    res["uneven_layout"] = {
        "call": "vce_fwd_ex", "shard_rows_min_max": [int(sizes.min()), int(sizes.max())],
        "ms": ms_unev, "ms_even_layout": ms_even,
        "achieved_TFLOP_s": flop_gemm / (ms_unev * 1e-3) / 1e12,
        "frac": flop_gemm / (ms_unev * 1e-3) / PEAK_BF16}
    log(f"[bench] forward, uneven layout {ms_unev:.3f} ms (even {ms_even:.3f} ms)")
    if tied:
        # OT-H step: the tied step plus a second, untied head two tokens ahead
        # at weight 0.1 (its own table of the same shape, drawn on the device:
        # only its timing is used here); flops = 8*H*V_real*(T + T - 1).
        g = torch.Generator(device=dev)
        g.manual_seed(7)
        W2 = (torch.randn(Vp, H, device=dev, generator=g) * 0.02).to(torch.bfloat16)
        tg2 = tg[1:].contiguous()
        ws2 = V.Workspaces(dev, fwd=V.vce_fwd_workspace_bytes(T - 1, H, Vr, Vp, n, dt_code),
                           bwd=V.vce_bwd_workspace_bytes(T - 1, H, Vr, Vp, n, dt_code))
        dW2 = torch.empty(Vp, H, **f32)

        def oth():
            V.ot_h_step(ids, tg, tg2, W, W2, Vr, n, inp.ignore_index, ws=ws, ws2=ws2, h=h,
                        dh=dh, dW=dW, dW2=dW2, allow_bad=True)

        oth()
        torch.cuda.synchronize()
        e0.record(stream)
        for _ in range(reps):
            oth()
        e1.record(stream)
        torch.cuda.synchronize()
        ms_oth = e0.elapsed_time(e1) / reps
        res["ot_h_step"] = {"ms": ms_oth, "tokens_s": T / (ms_oth * 1e-3),
                            "mfma_frac": 8.0 * H * Vr * (2 * T - 1) / (ms_oth * 1e-3) / PEAK_BF16}
        log(f"[bench] OT-H step {ms_oth:.3f} ms")
        del W2, ws2, dW2

        # Hashed n-gram input embedding (OT input side) over the same IDs, with
        # two 2^20-row n-gram tables (the pages' tables are billions of
        # parameters); table contents do not change the time of a gather, so
        # the n-gram tables are left uninitialised. Forward bytes: the distinct
        # rows of the three tables read once, the output written once.
        rows_ng = 1 << 20
        E2 = torch.empty(rows_ng, H, dtype=torch.bfloat16, device=dev)
        E3 = torch.empty(rows_ng, H, dtype=torch.bfloat16, device=dev)
        ng = V.vngram_fwd(ids, W, E2, E3, Vr, n)
        # distinct rows touched, counted from the rows the kernel reported
        i2 = ng.ids2.cpu().numpy()
        i3 = ng.ids3.cpu().numpy()
        u2 = int(np.unique(i2[i2 >= 0]).shape[0])
        u3 = int(np.unique(i3[i3 >= 0]).shape[0])
        ng_bytes = (uniq + u2 + u3) * H * 2 + T * H * 2 + 12 * T
        ms_ng = per_call(lambda: V.vngram_fwd(ids, W, E2, E3, Vr, n, out=ng))
        dE2 = torch.empty(rows_ng, H, **f32)
        dE3 = torch.empty(rows_ng, H, **f32)
        ws_ng = V.Workspaces(dev, emb=V.vemb_bwd_workspace_bytes(T, H, Vr, Vp),
                             emb2=V.vemb_bwd_workspace_bytes(T, H, rows_ng, rows_ng),
                             emb3=V.vemb_bwd_workspace_bytes(T, H, rows_ng, rows_ng))
        ms_ngb = per_call(lambda: V.ngram_bwd(ids, ng, dh, Vr, Vp, n, dE=dW, dE2=dE2, dE3=dE3,
                                              accumulate=True, ws=ws_ng))
        ngb_bytes = 3 * T * H * 4 + 24 * T + 2 * (uniq + u2 + u3) * H * 4
        res["ngram"] = {
            "tables_rows": [Vp, rows_ng, rows_ng], "distinct_rows": [uniq, u2, u3],
            "vngram_fwd": {"bytes": ng_bytes, "ms": ms_ng,
                           "GB_s": ng_bytes / (ms_ng * 1e-3) / 1e9,
                           "frac": ng_bytes / (ms_ng * 1e-3) / PEAK_HBM},
            "ngram_bwd": {"bytes": ngb_bytes, "ms": ms_ngb,
                          "GB_s": ngb_bytes / (ms_ngb * 1e-3) / 1e9,
                          "frac": ngb_bytes / (ms_ngb * 1e-3) / PEAK_HBM},
        }
        log(f"[bench] n-gram embedding fwd {ms_ng * 1e3:.1f} us, bwd {ms_ngb * 1e3:.1f} us")
        del E2, E3, dE2, dE3, ws_ng, ng
    if a.copy_probe:
        res["copy_probe_bytes"] = copy_probe()
    del ws, dh, dW, W, h, ws_arg, out_arg
    torch.cuda.empty_cache()
    if tied and not a.no_c3:
        # The LM-head cross-entropy alone (forward + backward, the metric's
        # own operation) on the T=8192, H=3072, V=201088 workload with
        # RMS-normalised hidden rows: tokens/s and MFMA fraction (8*T*H*V_real).
        inp3 = config_inputs("c3")
        T3, H3, V3, n3 = inp3.T, inp3.H, inp3.V_real, inp3.num_shards
        h3 = V.from_bits(inp3.h, inp3.dtype, dev)
        W3 = V.from_bits(inp3.W, inp3.dtype, dev)
        tg3 = torch.from_numpy(inp3.targets).to(dev)
        ws3 = V.Workspaces(dev, fwd=V.vce_fwd_workspace_bytes(T3, H3, V3, inp3.V_pad, n3, dt_code),
                           bwd=V.vce_bwd_workspace_bytes(T3, H3, V3, inp3.V_pad, n3, dt_code))
        dh3 = torch.empty(T3, H3, **f32)
        dW3 = torch.empty(inp3.V_pad, H3, **f32)

        def ce3():
            return V.ce_step(h3, W3, tg3, V3, n3, inp3.ignore_index, ws=ws3, dh=dh3, dW=dW3,
                             allow_bad=True)

        ce3()
        torch.cuda.synchronize()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        reps3 = 3
        e0.record(stream)
        for _ in range(reps3):
            ce3()
        e1.record(stream)
        torch.cuda.synchronize()
        ms3 = e0.elapsed_time(e1) / reps3
        res["ce_fwd_bwd_T8192"] = {
            "workload": f"T={T3}, H={H3}, V_real={V3}, {n3} shards, bf16, Zipf(1.1) targets",
            "ms": ms3, "tokens_s": T3 / (ms3 * 1e-3),
            "mfma_frac": 8.0 * T3 * H3 * V3 / (ms3 * 1e-3) / PEAK_BF16}
        log(f"[bench] CE fwd+bwd at T={T3}: {ms3:.3f} ms")

        def timed(fn, reps=3):
            fn()
            torch.cuda.synchronize()
            e0.record(stream)
            for _ in range(reps):
                fn()
            e1.record(stream)
            torch.cuda.synchronize()
            return e0.elapsed_time(e1) / reps

        # One rank's share of this workload if its 8 shards sat on 8 GPUs: the
        # same calls on shard 0's 25136 rows alone (targets folded into the
        # shard), the per-GPU kernel shape of the sharded design.
        S3 = inp3.V_pad // n3
        Wk = W3[:S3]
        tgk = torch.where(tg3 >= 0, tg3 % S3, tg3)
        wsk = V.Workspaces(dev, fwd=V.vce_fwd_workspace_bytes(T3, H3, S3, S3, 1, dt_code),
                           bwd=V.vce_bwd_workspace_bytes(T3, H3, S3, S3, 1, dt_code))
        dWk = torch.empty(S3, H3, **f32)
        msk = timed(lambda: V.ce_step(h3, Wk, tgk, S3, 1, inp3.ignore_index, ws=wsk, dh=dh3,
                                      dW=dWk, allow_bad=True))
        res["ce_fwd_bwd_T8192_one_shard"] = {
            "workload": f"T={T3}, H={H3}, V_real={S3} (one shard of {n3}), bf16",
            "ms": msk, "tokens_s": T3 / (msk * 1e-3),
            "mfma_frac": 8.0 * T3 * H3 * S3 / (msk * 1e-3) / PEAK_BF16}
        # Context only (never on the path): torch's bf16 GEMM (the vendor
        # library) on the forward's shapes, logits written out
        ms_tg = timed(lambda: torch.matmul(h3, W3.t()))
        ms_tgk = timed(lambda: torch.matmul(h3, Wk.t()))
        res["context_torch_gemm"] = {
            "what": "torch.matmul(h, W^T) in bf16 (hipBLASLt), the [T, V] logits written out",
            "full_V": {"ms": ms_tg, "TFLOP_s": 2.0 * T3 * H3 * inp3.V_pad / (ms_tg * 1e-3) / 1e12},
            "one_shard": {"ms": ms_tgk, "TFLOP_s": 2.0 * T3 * H3 * S3 / (ms_tgk * 1e-3) / 1e12}}
        log(f"[bench] one shard {msk:.3f} ms; torch GEMM {ms_tg:.3f} / {ms_tgk:.3f} ms")
        del h3, W3, ws3, dh3, dW3, Wk, wsk, dWk
        torch.cuda.empty_cache()
    if not a.no_sampled:
        res["sampled_softmax"] = sampled_field(V, dev, stream)
    if not a.no_cpu_baseline:
        log(f"[bench] CPU baseline: oracle on {a.cpu_tokens} tokens")
        res["cpu_baseline"] = cpu_baseline(inp, a.cpu_tokens)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
