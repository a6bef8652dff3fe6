#!/usr/bin/env python3
"""Benchmark of one rank's share of context-parallel diffusion attention on one GPU.

One step = one pass of the whole per-rank hot path for global rank 0 of the
chosen workload, with every input resident in HBM:

  1. cp_pack_qkv_dst_major   this rank's Q/K/V shard -> its staging buffer
  2. cp_sim_exchange         receive chunk 0 of every group member's staging buffer
                             (the other members' buffers are resident inputs,
                             packed before timing: they stand in for the peers)
  3. cp_unpack_head_sharded  -> head-sharded Q/K/V
  4. cp_attn_localq_globalkv the workload's local-Q/global-KV attention
  5. cp_output_reverse       send layout (B > 1 only; the identity for B == 1),
     cp_sim_exchange         exchange with the peers' resident send buffers,
     cp_output_reverse       merge of the W head groups

For the 2D workload (video_u2a2: Ulysses U=2 x AllGather-KV A=2) the steps chain:
step 3 writes K/V straight into region 0 of the gathered global K/V buffer
(region 1, the other AllGather rank's share, is resident), step 4 attends the
unpacked Q against it, and step 5 reverses its output.  For the AllGather-KV
workloads (tiny_w2, image_cp4, image_cp8, joint_cfg_cp4) the attention reads the
rank's local Q shard against the resident global K/V (standing in for the K/V
all-gather), and the output reverse runs on a resident head-sharded buffer of the
Ulysses layout.

`joint_segments` (masked workloads) times cp_attn_joint with image and text
K/V as separate segments, both layouts, against the concatenated call.
`chunked_kv` times the same share with its K/V arriving in W chunks
(cp_attn_partial per chunk, then cp_attn_merge).

`packed_varlen` (unmasked B = 1 AllGather-KV workloads) packs the sequence as
four documents and times, for every AllGather-KV rank, the remap of the packed
query boundaries plus cp_attn_varlen over the rank's rows.

For the 2D workload the JSON carries `ulysses_2d_fused`: the same step with the
unpack and the attention replaced by cp_attn_recv_to_send_2d.
For the workloads without an AllGather-KV stage the JSON also carries
`ulysses_fused`: the Ulysses-only rank step (attention of the rank's H/W heads
over the whole sequence, the same FLOPs) timed once with separate unpack and
send steps and once with cp_attn_recv_to_send, which reads Q/K/V from the
received buffer and writes the send layout directly.

Prints one JSON line.  The headline workload is video_u2a2 (the largest
one-GPU share: 16380 queries x 32760 keys, 6 heads).  `value` is attention
TFLOP/s over the whole step (algorithmic attention FLOPs / step time), with the
step captured once into a HIP graph and replayed (`--eager` launches it op by
op); the untimed warm-up (--warmup steps, then about a second of steps, JSON
`clock_warmup_s`) ends at the clock the GPU holds under this load, which the
first ~15 steps after idle do not run at.  Per-kernel durations come from HIP events on the launch stream around
HIP-graph replays of a burst of 100 back-to-back launches of each kernel on the
step's own buffers (three warm-up launches, one untimed replay, the median of
three timed ones), after about a second of step replays that brings the clock
to its loaded level; neither depends on --steps.  `per_config` repeats the
per-kernel measurement, the cold layout pass and the whole-output parity check
for the other workloads.  `cpu_baseline` times the fp64 oracle over the
headline's whole attention problem on the host cores, and `parity` compares
every element of the GPU output with that oracle result.
"""

from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "attn TFLOP/s + % bf16 MFMA peak (local-Q/global-KV); pack/unpack HBM GB/s"
PEAK_BF16_TFLOPS = 2500.0      # MI355X dense bf16 MFMA
PEAK_HBM_GBPS = 8000.0         # MI355X HBM3E
DEFAULT_WORKLOAD = "video_u2a2"
# Configurations measured beside the headline, each the same way (kernel bursts, cold
# layout, parity), reported under "per_config".
PER_CONFIG = ("image_cp4", "image_cp8", "joint_cfg_cp4", "tiny_w2")
KERNEL_BURST = 100             # launches per timed HIP-graph replay, whatever --steps is
CLOCK_WARMUP_S = 1.0           # replays of the step before the per-kernel bursts


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=100)
    p.add_argument("--warmup", type=int, default=10)
    p.add_argument("--workload", default=DEFAULT_WORKLOAD)
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--no-per-config", action="store_true",
                   help="measure the headline workload only (no per_config section)")
    p.add_argument("--no-cold", action="store_true", help="skip the cold-cache pack/unpack pass")
    p.add_argument("--eager", action="store_true",
                   help="launch the timed steps one by one instead of replaying a captured HIP graph")
    p.add_argument("--calib-copy", action="store_true",
                   help="run only a plain 256 MiB device copy (counter calibration for traffic)")
    p.add_argument("--summarize-traffic", nargs=3, metavar=("FETCH_DIR", "WRITE_DIR", "OUT_JSON"),
                   help="turn two rocprofv3 --pmc runs (FETCH_SIZE, WRITE_SIZE) of this bench and of "
                        "--calib-copy into a traffic summary; no GPU work")
    p.add_argument("--summarize-mfma", nargs=2, metavar=("PMC_DIR", "OUT_MD"),
                   help="turn one rocprofv3 --pmc run of this bench (SQ_VALU_MFMA_BUSY_CYCLES, "
                        "SQ_INSTS_VALU_MFMA_MOPS_BF16, SQ_BUSY_CU_CYCLES, GRBM_GUI_ACTIVE) into an MFMA "
                        "utilisation summary of the attention kernel; no GPU work")
    p.add_argument("--summarize-trace", nargs=3, metavar=("TRACE_DB", "OUT_MD", "COMMAND"),
                   help="turn a rocprofv3 --kernel-trace --stats database of a run of this bench into a "
                        "per-kernel summary (COMMAND: the profiled command line, quoted); no GPU work")
    p.add_argument("--no-extras", action="store_true",
                   help="skip the fused-chain, chunked-K/V and joint-segment sections (so a kernel "
                        "trace of the run holds only the headline step's launches)")
    p.add_argument("--uaa", action="store_true",
                   help="per-rank comparison of head padding (usp4+uaa) and the composed U2xA2 "
                        "layout at heads 14, D 128; prints its own JSON line")
    p.add_argument("--uaa-seqs", default="16384,32768,65536")
    p.add_argument("--only", default=None,
                   help="profile aid: run only this kernel's launches in the timed loop "
                        "(pack|unpack|attn|merge); the JSON line is then not the headline")
    return p.parse_args()


def to_dev(bits, dev):
    import torch
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(dev)


class RankPath:
    """Device buffers and launches of one rank's step."""

    def __init__(self, wl, dev):
        import torch

        import context_attention_diffusion_amd as cp
        import workloads

        self.cp, self.wl, self.dev = cp, wl, dev
        W, B, Sl, H, D, A = wl.W, wl.B, wl.S_local, wl.H, wl.D, wl.A
        Hl = H // W
        self.two_d = A > 1
        full = workloads.global_qkv(wl)
        # Ulysses group 0: ranks 0..W-1 with rows [r*S_l, (r+1)*S_l).
        shards = [[to_dev(np.ascontiguousarray(t[:, r * Sl:(r + 1) * Sl]), dev) for t in full]
                  for r in range(W)]
        self.q, self.k, self.v = shards[0]
        st_shape = (W, B * Sl, Hl, 3 * D)
        self.staging = [torch.empty(st_shape, dtype=torch.bfloat16, device=dev) for _ in range(W)]
        for r in range(1, W):      # peers' sends: resident inputs
            cp.cp_pack_qkv_dst_major(*shards[r], W, staging=self.staging[r])
        self.recv = torch.empty(st_shape, dtype=torch.bfloat16, device=dev)
        hs_shape = (B, W * Sl, Hl, D)
        self.q_hs = torch.empty(hs_shape, dtype=torch.bfloat16, device=dev)
        mask = workloads.key_mask(wl)
        self.mask = None if mask is None else torch.from_numpy(mask).to(dev)
        if self.two_d:
            assert B == 1
            # Gathered K/V of heads [0, H_l): region 0 comes from step 3, region 1 is resident.
            kg = np.ascontiguousarray(full[1][:, :, :Hl])
            vg = np.ascontiguousarray(full[2][:, :, :Hl])
            self.k_glob, self.v_glob = to_dev(kg, dev), to_dev(vg, dev)
            span = W * Sl
            self.k_hs = self.k_glob[:, :span]
            self.v_hs = self.v_glob[:, :span]
            self.attn_q, self.attn_k, self.attn_v = self.q_hs, self.k_glob, self.v_glob
            self.o_attn = torch.empty(hs_shape, dtype=torch.bfloat16, device=dev)
            self.o_hs = self.o_attn
        else:
            self.k_hs = torch.empty(hs_shape, dtype=torch.bfloat16, device=dev)
            self.v_hs = torch.empty(hs_shape, dtype=torch.bfloat16, device=dev)
            self.attn_q = self.q
            self.attn_k = to_dev(full[1][:, :, :wl.attn_heads], dev)
            self.attn_v = to_dev(full[2][:, :, :wl.attn_heads], dev)
            self.o_attn = torch.empty_like(self.attn_q)
            g = torch.Generator(device="cpu").manual_seed(wl.seed + 99)
            self.o_hs = torch.randn(hs_shape, generator=g).to(torch.bfloat16).to(dev)
        self.scale = 1.0 / math.sqrt(D)
        snd_shape = (W, B, Sl, Hl, D)
        self.snd = torch.empty(snd_shape, dtype=torch.bfloat16, device=dev)
        g = torch.Generator(device="cpu").manual_seed(wl.seed + 7)
        self.peer_snd = [None] + [torch.randn(snd_shape, generator=g).to(torch.bfloat16).to(dev)
                                  for _ in range(1, W)]
        self.rcv = torch.empty(snd_shape, dtype=torch.bfloat16, device=dev)
        self.out = torch.empty((B, Sl, H, D), dtype=torch.bfloat16, device=dev)
        self.full = full
        self.mask_np = mask
        # Fill every intermediate buffer with real data once, so that a run that
        # times only some of the kernels still feeds them the workload's values.
        self.pack()
        self.exchange_in()
        self.unpack()
        torch.cuda.synchronize()

    # -- the launches of one step
    def pack(self):
        self.cp.cp_pack_qkv_dst_major(self.q, self.k, self.v, self.wl.W, staging=self.staging[0])

    def exchange_in(self):
        self.cp.cp_sim_exchange(self.staging, 0, recv=self.recv)

    def unpack(self):
        self.cp.cp_unpack_head_sharded(self.recv, self.wl.B, self.wl.W,
                                       out=(self.q_hs, self.k_hs, self.v_hs))

    def attn(self):
        self.cp.cp_attn_localq_globalkv(self.attn_q, self.attn_k, self.attn_v, self.mask,
                                        scale=self.scale, out=self.o_attn)

    def send(self):
        W, B = self.wl.W, self.wl.B
        if B == 1:
            return self.o_hs.view(self.snd.shape)     # identity layout
        return self.cp.cp_output_reverse(0, self.o_hs, W, B, out=self.snd)

    def exchange_out(self, snd):
        self.cp.cp_sim_exchange([snd] + self.peer_snd[1:], 0, recv=self.rcv)

    def merge(self):
        self.cp.cp_output_reverse(1, self.rcv, self.wl.W, self.wl.B, out=self.out)


def attn_flops(wl, mask):
    """Algorithmic attention FLOPs: 4*B*H*Sq*D*(valid keys per batch)."""
    if mask is None:
        return wl.attn_flops_dense()
    valid = mask.astype(np.int64).sum(axis=1)
    return int(4 * wl.attn_heads * wl.attn_rows * wl.D * valid.sum())


def run_steps(path, n, events=None, only=None):
    import torch
    names = ["pack", "exchange_in", "unpack", "attn", "send", "exchange_out", "merge"]
    for _ in range(n):
        rec = {} if events is not None else None

        def timed(name, fn):
            if rec is None:
                return fn()
            s = torch.cuda.Event(enable_timing=True)
            e = torch.cuda.Event(enable_timing=True)
            s.record()
            r = fn()
            e.record()
            rec[name] = (s, e)
            return r

        if only is None or only == "pack":
            timed("pack", path.pack)
        if only is None:
            timed("exchange_in", path.exchange_in)
        if only is None or only == "unpack":
            timed("unpack", path.unpack)
        if only is None or only == "attn":
            timed("attn", path.attn)
        if only is None:
            snd = timed("send", path.send)
            timed("exchange_out", lambda: path.exchange_out(snd))
        if only is None or only == "merge":
            timed("merge", path.merge)
        if rec is not None:
            events.append(rec)
    return names


def cold_layout_gbps(wl, dev, rounds=4):
    """Pack and unpack with rotating buffer sets whose READ footprint alone exceeds 600 MB,
    so each launch's loads miss the 256 MB Infinity Cache whatever the stores leave resident
    there (nontemporal stores do not evict the read sets).  Returns (pack GB/s, unpack GB/s,
    GB/s of torch's device copy of the same bytes, as three tensor copies, for reference)."""
    import torch

    import context_attention_diffusion_amd as cp

    W, B, Sl, H, D = wl.W, wl.B, wl.S_local, wl.H, wl.D
    read_per_set = wl.pack_bytes() // 2          # pack reads Q/K/V, unpack reads the staging
    nsets = max(3, int(math.ceil(600e6 / read_per_set)))
    sets = []
    for i in range(nsets):
        x = [torch.empty((B, Sl, H, D), dtype=torch.bfloat16, device=dev).normal_() for _ in range(3)]
        st = torch.empty((W, B * Sl, H // W, 3 * D), dtype=torch.bfloat16, device=dev)
        outs = tuple(torch.empty((B, W * Sl, H // W, D), dtype=torch.bfloat16, device=dev)
                     for _ in range(3))
        sets.append((x, st, outs))
    copy_dst = {id(st): torch.empty_like(st) for _, st, _ in sets}
    res = []
    for which in ("pack", "unpack", "copy"):
        def launch(sset):
            x, st, outs = sset
            if which == "pack":
                cp.cp_pack_qkv_dst_major(*x, W, staging=st)
            elif which == "unpack":
                cp.cp_unpack_head_sharded(st, B, W, out=outs)
            else:   # reference: one device copy of the same bytes (staging -> a buffer of its size)
                copy_dst[id(st)].copy_(st)
        for sset in sets:
            launch(sset)
        torch.cuda.synchronize()
        order = [sets[i % len(sets)] for i in range(rounds * len(sets))]
        it = iter(order * 2)
        ms = time_burst(lambda: launch(next(it)), len(order))
        res.append(wl.pack_bytes() / (ms * 1e-3) / 1e9)
    del sets, copy_dst
    torch.cuda.empty_cache()
    return res


def blas_threads():
    threads = os.cpu_count()
    try:
        from threadpoolctl import threadpool_info
        info = [x for x in threadpool_info() if x.get("user_api") == "blas"]
        if info:
            threads = max(int(x.get("num_threads", 1)) for x in info)
    except Exception:
        pass
    return threads


def oracle_attention(wl, full, mask):
    """The fp64 oracle over the rank's whole attention problem (query rows [0, attn_rows),
    heads [0, attn_heads), every key); returns (output, seconds)."""
    from oracle import attention as OA
    from oracle import bf16

    q = bf16.bits_to_f64(np.ascontiguousarray(full[0][:, :wl.attn_rows, :wl.attn_heads]))
    k = bf16.bits_to_f64(np.ascontiguousarray(full[1][:, :, :wl.attn_heads]))
    v = bf16.bits_to_f64(np.ascontiguousarray(full[2][:, :, :wl.attn_heads]))
    t = time.perf_counter()
    ref = OA.attention(q, k, v, mask, 1.0 / math.sqrt(wl.D))
    return ref, time.perf_counter() - t


def layout_ramp(dev, seqs=(256, 1088, 4352, 17408, 69632), H=24, D=128, W=4):
    """Pack kernel and a plain device copy of the same bytes, cold, over a range of
    sizes (one rank of an H=24, D=128, W=4 layout with S_local rows): the time of one
    launch against its algorithmic bytes, and the least-squares fit
    t = t0 + bytes / bw_sustained over the sizes, i.e. the fixed per-launch cost and
    the streaming bandwidth.  Read sets smaller than 600 MB rotate over enough buffer
    sets to miss the 256 MB Infinity Cache."""
    import torch

    import context_attention_diffusion_amd as cp

    rows = []
    for Sl in seqs:
        nbytes = 2 * 3 * Sl * H * D * 2
        read = nbytes // 2
        nsets = max(1, int(math.ceil(600e6 / read))) if read < 600e6 else 1
        nsets = max(nsets, 2)
        sets = []
        for _ in range(nsets):
            x = [torch.empty((1, Sl, H, D), dtype=torch.bfloat16, device=dev).normal_() for _ in range(3)]
            st = torch.empty((W, Sl, H // W, 3 * D), dtype=torch.bfloat16, device=dev)
            sets.append((x, st, torch.empty_like(st)))
        rec = {"S_local": Sl, "bytes": nbytes}
        for which in ("pack", "copy"):
            def launch(sset):
                x, st, cpy = sset
                if which == "pack":
                    cp.cp_pack_qkv_dst_major(*x, W, staging=st)
                else:
                    cpy.copy_(st)
            for sset in sets:
                launch(sset)
            torch.cuda.synchronize()
            rounds = max(1, int(40 // nsets))
            order = [sets[i % nsets] for i in range(rounds * nsets)]
            it = iter(order * 2)
            ms = time_burst(lambda: launch(next(it)), len(order))
            rec[f"{which}_us"] = ms * 1e3
            rec[f"{which}_GBps"] = nbytes / (ms * 1e-3) / 1e9
        rows.append(rec)
        del sets
        torch.cuda.empty_cache()
    res = {"H": H, "D": D, "W": W, "sizes": rows}
    for which in ("pack", "copy"):
        x = np.array([r["bytes"] for r in rows], dtype=np.float64)
        y = np.array([r[f"{which}_us"] for r in rows], dtype=np.float64) * 1e-6
        A = np.stack([np.ones_like(x), x], axis=1)
        (t0, inv_bw), *_ = np.linalg.lstsq(A, y, rcond=None)
        res[f"{which}_fixed_us"] = float(t0 * 1e6)
        res[f"{which}_sustained_GBps"] = float(1.0 / inv_bw / 1e9)
    res["note"] = ("t = fixed + bytes / sustained fitted over the sizes; at a workload's pack bytes the "
                   "attainable GB/s of a single launch is bytes / (fixed + bytes / sustained)")
    return res


def cpu_baseline(wl, flops, seconds):
    return {
        "value": flops / seconds / 1e12, "unit": "TFLOP/s", "cores": blas_threads(), "kind": "oracle",
        "sample": f"fp64 oracle attention over the whole rank problem: query rows [0,{wl.attn_rows}), "
                  f"{wl.attn_heads} heads, all {wl.S} keys, B={wl.B}; one pass of {seconds:.2f} s; "
                  f"host cpu_count={os.cpu_count()}",
    }


def parity_whole(path, wl, ref):
    """Every element of the step's attention output against the oracle result, and the
    unpacked Q against its closed form (head slice 0 of the group's sequence)."""
    import torch

    # the step's unpack and attention once more, so that the buffers compared are
    # the step's own results whatever the sections before them wrote
    path.pack()
    path.exchange_in()
    path.unpack()
    path.attn()
    torch.cuda.synchronize()
    Hl = wl.H // wl.W
    span = wl.W * wl.S_local
    got = path.q_hs.view(torch.int16).cpu().numpy().view(np.uint16)
    o = path.o_attn.float().cpu().numpy().astype(np.float64)
    err = np.abs(o - ref)
    return {"unpack_q_bit_exact": bool(np.array_equal(got, path.full[0][:, :span, :Hl])),
            "attn_elements_compared": int(err.size),
            "attn_max_abs_err": float(err.max()), "attn_mean_abs_err": float(err.mean()),
            "attn_within_tolerance": bool(err.max() <= 2e-2 and err.mean() <= 2e-3)}


def warm_clock(fn, seconds=CLOCK_WARMUP_S):
    """Run fn back to back for about `seconds` so that the timed bursts after it see the
    clock the GPU settles at under load, not the idle clock of the first launches."""
    import torch
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    n = 0
    while True:
        fn()
        n += 1
        if n % 8 == 0:
            torch.cuda.synchronize()
            if time.perf_counter() - t0 >= seconds:
                break
    torch.cuda.synchronize()


def time_burst(fn, burst, repeats=3):
    """Duration (ms) of one launch of `fn`: three warm-up launches, then `burst` back-to-back
    launches captured once into a HIP graph, replayed once untimed and `repeats` times
    timed with HIP events on the launch stream; the median replay over `burst`.  Host
    launch overhead does not enter the figure."""
    import torch
    for _ in range(3):
        fn()
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        for _ in range(burst):
            fn()
    graph.replay()
    torch.cuda.synchronize()
    times = []
    for _ in range(repeats):
        s = torch.cuda.Event(enable_timing=True)
        e = torch.cuda.Event(enable_timing=True)
        s.record()
        graph.replay()
        e.record()
        torch.cuda.synchronize()
        times.append(s.elapsed_time(e) / burst)
    return float(np.median(times))


def time_together(fns, burst, rounds=7, warm_s=0.5):
    """Duration (ms) of one launch of each function in `fns` (name -> callable), measured
    side by side: each is captured once into a HIP graph of `burst` back-to-back launches,
    the graphs are replayed in turn for about warm_s seconds, then in each of `rounds`
    rounds every graph is replayed once and timed with HIP events, in an order that
    rotates from round to round; the median over the rounds, divided by `burst`.
    Functions compared in one call see the same clock whatever their order, which
    timing them one after another does not give."""
    import torch
    graphs = {}
    for name, fn in fns.items():
        for _ in range(3):
            fn()
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            for _ in range(burst):
                fn()
        graphs[name] = graph
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < warm_s:
        for graph in graphs.values():
            graph.replay()
        torch.cuda.synchronize()
    names = list(graphs)
    times = {n: [] for n in names}
    for r in range(rounds):
        k = r % len(names)
        for n in names[k:] + names[:k]:
            s = torch.cuda.Event(enable_timing=True)
            e = torch.cuda.Event(enable_timing=True)
            s.record()
            graphs[n].replay()
            e.record()
            torch.cuda.synchronize()
            times[n].append(s.elapsed_time(e) / burst)
    return {n: float(np.median(t)) for n, t in times.items()}


def kernel_bursts(path, only=None, burst=KERNEL_BURST):
    """Average duration (ms) of each kernel of the step over `burst` back-to-back launches."""
    snd = path.send()
    launches = {
        "pack": path.pack, "exchange_in": path.exchange_in, "unpack": path.unpack,
        "attn": path.attn, "exchange_out": lambda: path.exchange_out(snd), "merge": path.merge,
    }
    if path.wl.B > 1:
        launches["send"] = path.send
    res = {}
    for name, fn in launches.items():
        if only is not None and name != only:
            continue
        res[name] = time_burst(fn, burst)
    return res


def ulysses_chain(path, burst=10):
    """Ulysses-only rank step (no AllGather-KV), unfused and fused, on the step's buffers.

    unfused: pack -> exchange -> unpack -> attention of the rank's H/W heads over the
             whole sequence -> send layout -> exchange -> merge
    fused:   pack -> exchange -> cp_attn_recv_to_send -> exchange -> merge
    Both attentions do the same FLOPs as the workload's local-Q/global-KV share.
    Returns step and attention durations (us, graph-replayed bursts) and whether the
    two chains' send buffers are bit-identical."""
    import torch
    cp, wl = path.cp, path.wl
    W, B = wl.W, wl.B
    o_u = torch.empty_like(path.q_hs)
    snd_u = torch.empty_like(path.snd)
    snd_f = torch.empty_like(path.snd)

    def attn_unfused():
        cp.cp_attn_localq_globalkv(path.q_hs, path.k_hs, path.v_hs, path.mask, scale=path.scale, out=o_u)

    def send_unfused():
        if B == 1:
            return o_u.view(snd_u.shape)
        return cp.cp_output_reverse(0, o_u, W, B, out=snd_u)

    def attn_fused():
        cp.cp_attn_recv_to_send(path.recv, B, W, path.mask, scale=path.scale, out=snd_f)

    def step_unfused():
        path.pack()
        path.exchange_in()
        path.unpack()
        attn_unfused()
        path.exchange_out(send_unfused())
        path.merge()

    def step_fused():
        path.pack()
        path.exchange_in()
        attn_fused()
        path.exchange_out(snd_f)
        path.merge()

    step_unfused()
    step_fused()
    torch.cuda.synchronize()
    same = bool(torch.equal(send_unfused(), snd_f))
    t = time_together({"unfused_step": step_unfused, "fused_step": step_fused,
                       "unfused_attn": attn_unfused, "fused_attn": attn_fused}, burst)
    res = {f"{n}_us": ms * 1e3 for n, ms in t.items()}
    res["fused_send_equals_unfused"] = same
    res["step_speedup"] = res["unfused_step_us"] / res["fused_step_us"]
    return res


def ulysses_2d_chain(path, burst=5):
    """2D-layout rank step (Ulysses x AllGather-KV), unfused and fused, on the step's buffers.

    unfused: pack -> exchange -> unpack (K/V into region 0 of the gathered buffer) ->
             attention over the gathered K/V -> send layout -> exchange -> merge
    fused:   pack -> exchange -> cp_attn_recv_to_send_2d (Q and the own region's K/V
             from the received buffer, the other region from the gathered buffer)
             -> exchange -> merge
    Returns step and attention durations (us, graph-replayed bursts) and the largest
    difference between the two send buffers: the fused call attends the two regions
    as two key segments, whose tiles start at each region's first key, so its
    summation order differs from the gathered call's where a region's length is not
    a multiple of the 64-key tile."""
    import torch
    cp, wl = path.cp, path.wl
    W, B = wl.W, wl.B
    span = W * wl.S_local
    k_oth, v_oth = path.k_glob[:, span:], path.v_glob[:, span:]   # contiguous: B == 1
    snd_f = torch.empty_like(path.snd)

    def attn_fused():
        cp.cp_attn_recv_to_send_2d(path.recv, k_oth, v_oth, B, W, False, None, None, scale=path.scale, out=snd_f)

    def step_unfused():
        path.pack()
        path.exchange_in()
        path.unpack()
        path.attn()
        path.exchange_out(path.send())
        path.merge()

    def step_fused():
        path.pack()
        path.exchange_in()
        attn_fused()
        path.exchange_out(snd_f)
        path.merge()

    step_unfused()
    step_fused()
    torch.cuda.synchronize()
    diff = float((path.send().float() - snd_f.float()).abs().max())
    t = time_together({"unfused_step": step_unfused, "fused_step": step_fused,
                       "unfused_attn": path.attn, "fused_attn": attn_fused}, burst)
    res = {f"{n}_us": ms * 1e3 for n, ms in t.items()}
    res["max_abs_diff_fused_vs_unfused"] = diff
    res["step_speedup"] = res["unfused_step_us"] / res["fused_step_us"]
    return res


def chunked_kv(path, burst=10):
    """The local-Q/global-KV share with K/V arriving in W chunks (one per AllGather
    rank): W cp_attn_partial calls and one cp_attn_merge; or cp_attn_partial on the
    first chunk and cp_attn_partial_accum on the others (the last one writing the
    output); against the dense call.  last_chunk_accumulate_us is what remains after
    the last chunk arrives."""
    import torch
    cp, wl = path.cp, path.wl
    W, Sl = wl.W, wl.S_local
    q, k, v = path.attn_q, path.attn_k, path.attn_v
    B, Sq, H, D = q.shape
    ks = [k[:, r * Sl:(r + 1) * Sl].contiguous() for r in range(W)]
    vs = [v[:, r * Sl:(r + 1) * Sl].contiguous() for r in range(W)]
    ms = [None if path.mask is None else path.mask[:, r * Sl:(r + 1) * Sl].contiguous() for r in range(W)]
    o_parts = torch.empty((W, B, Sq, H, D), dtype=torch.float32, device=q.device)
    lses = torch.empty((W, B, H, Sq), dtype=torch.float32, device=q.device)
    out = torch.empty_like(q)

    def partials():
        for r in range(W):
            cp.cp_attn_partial(q, ks[r], vs[r], ms[r], scale=path.scale, out=o_parts[r], lse=lses[r])

    def merge():
        cp.cp_attn_merge(o_parts, lses, out=out)

    st_o = torch.empty((B, Sq, H, D), dtype=torch.float32, device=q.device)
    st_l = torch.empty((B, H, Sq), dtype=torch.float32, device=q.device)
    out_acc = torch.empty_like(q)

    def accumulate():
        cp.cp_attn_partial(q, ks[0], vs[0], ms[0], scale=path.scale, out=st_o, lse=st_l)
        for r in range(1, W):
            cp.cp_attn_partial_accum(q, ks[r], vs[r], st_o, st_l, ms[r], scale=path.scale,
                                     final=r == W - 1, out=out_acc)

    def last_accumulate():
        cp.cp_attn_partial_accum(q, ks[W - 1], vs[W - 1], st_o, st_l, ms[W - 1], scale=path.scale,
                                 final=True, out=out_acc)

    out_dense = torch.empty_like(q)

    def dense_call():
        cp.cp_attn_localq_globalkv(q, k, v, path.mask, scale=path.scale, out=out_dense)

    # the results, compared with a dense call into a tensor of their own
    partials()
    merge()
    accumulate()
    dense = cp.cp_attn_localq_globalkv(q, k, v, path.mask, scale=path.scale)
    torch.cuda.synchronize()
    diff = (out.float() - dense.float()).abs()
    diff_acc = (out_acc.float() - dense.float()).abs()
    t = time_together({"partials": partials, "merge": merge, "accumulate": accumulate,
                       "last_chunk_accumulate": last_accumulate, "dense": dense_call}, burst)
    res = {"chunks": W, "partials_us": t["partials"] * 1e3, "merge_us": t["merge"] * 1e3,
           "merge_bytes": int(o_parts.numel() * 4 + lses.numel() * 4 + out.numel() * 2),
           "max_abs_diff_vs_dense": float(diff.max()),
           "elements_differing_from_dense": int((diff > 0).sum()),
           "accumulate_us": t["accumulate"] * 1e3,
           "last_chunk_accumulate_us": t["last_chunk_accumulate"] * 1e3,
           "accumulate_max_abs_diff_vs_dense": float(diff_acc.max()),
           "dense_us": t["dense"] * 1e3}
    res["merge_GBps"] = res["merge_bytes"] / (res["merge_us"] * 1e-6) / 1e9
    res["total_us"] = res["partials_us"] + res["merge_us"]
    res["total_over_dense"] = res["total_us"] / res["dense_us"]
    res["accumulate_over_dense"] = res["accumulate_us"] / res["dense_us"]
    return res


def joint_segments(path, burst=10):
    """The joint workload's attention with image and text K/V as two segments (the text
    keys re-attached behind or in front of the image keys, text padding mask on the
    text segment only), against the concatenated masked call."""
    import torch
    cp, wl = path.cp, path.wl
    S_img = wl.S - wl.text_tokens
    k, v, m = path.attn_k, path.attn_v, path.mask
    ki, vi = k[:, :S_img].contiguous(), v[:, :S_img].contiguous()
    kj, vj, jm = k[:, S_img:].contiguous(), v[:, S_img:].contiguous(), m[:, S_img:].contiguous()
    out = torch.empty_like(path.attn_q)
    fns = {}
    for name, front in (("rear", False), ("front", True)):
        def call(front=front):
            cp.cp_attn_joint(path.attn_q, ki, vi, kj, vj, None, jm, joint_front=front, scale=path.scale, out=out)
        fns[name] = call
    fns["concatenated"] = path.attn
    return {f"{n}_us": ms * 1e3 for n, ms in time_together(fns, burst).items()}


def packed_varlen(path, n_docs=4, burst=10):
    """The AllGather-KV share with its sequence packed as n_docs documents (seeded cut
    points): for every AllGather-KV rank, the device-side remap of the global query
    boundaries to the rank's rows and the packed attention of its local rows over
    the global keys, each document attending to itself only."""
    import torch
    import workloads
    cp, wl = path.cp, path.wl
    Sl = wl.attn_rows
    A = wl.S // Sl
    cu = workloads.packed_boundaries(wl, n_docs)
    g = torch.tensor(cu, dtype=torch.int32, device=path.attn_q.device)
    q, k, v = path.attn_q[0], path.attn_k[0], path.attn_v[0]
    loc = torch.empty_like(g)
    out = torch.zeros_like(q)
    H, D = q.shape[1], q.shape[2]
    ranks = []
    for r in range(A):
        def call(r=r):
            cp.cp_varlen_remap_cu_seqlens_q(g, r, Sl, out=loc)
            cp.cp_attn_varlen(q, k, v, loc, g, scale=path.scale, out=out)
        call()
        torch.cuda.synchronize()
        lq = loc.cpu().tolist()
        flops = sum(4 * H * D * (lq[i + 1] - lq[i]) * (cu[i + 1] - cu[i]) for i in range(n_docs))
        us = time_burst(call, burst) * 1e3
        ranks.append({"rank": r, "local_cu_seqlens_q": lq, "us": us, "flops": flops,
                      "TFLOPs": flops / (us * 1e-6) / 1e12})
    return {"cu_seqlens": cu, "ranks": ranks}


def uaa_compare(seqs, heads=14, D=128, seed=1240):
    """Per-rank comparison of a padded Ulysses layout against the composed one, at the
    shapes of the pages' attention benchmark (heads 14, D 128, four ranks):

    usp4+uaa: Ulysses over 4 ranks; 14 heads padded to 16 (4 per rank).  Step: padded
              pack -> exchange -> unpack -> attention of 4 heads over all S rows -> send
              (identity, B = 1) -> exchange -> merge dropping the padding heads.  Also
              timed with the fused attention (recv -> send).
    cp2usp2:  Ulysses 2 x AllGather-KV 2; 7 heads per rank, S/2 query rows against the
              gathered S keys.  Step: pack -> exchange -> unpack (K/V into region 0 of the
              gathered K/V; region 1, the other AllGather rank's share, is resident) ->
              attention -> send -> exchange -> merge.
    Inputs are seeded N(0, 1) bf16 drawn on the GPU; every exchange partner's buffer is
    resident before timing.  Returns one record per sequence length."""
    import torch
    import context_attention_diffusion_amd as cp

    dev = torch.device("cuda:0")
    g = torch.Generator(device=dev)
    g.manual_seed(seed)

    def randn(*shape):
        return torch.randn(shape, generator=g, device=dev, dtype=torch.float32).to(torch.bfloat16)

    res = []
    for S in seqs:
        rec = {"S": S}
        scale = 1.0 / math.sqrt(D)
        # ---- usp4 + uaa
        W, Sl = 4, S // 4
        H_pad = -(-heads // W) * W
        Hl = H_pad // W
        x = [randn(1, Sl, heads, D) for _ in range(3)]
        st = [torch.empty((W, Sl, Hl, 3 * D), dtype=torch.bfloat16, device=dev) for _ in range(W)]
        for r in range(1, W):
            cp.cp_pack_qkv_dst_major_padded(*[randn(1, Sl, heads, D) for _ in range(3)], W, H_pad, staging=st[r])
        recv = torch.empty_like(st[0])
        hs = [torch.empty((1, S, Hl, D), dtype=torch.bfloat16, device=dev) for _ in range(3)]
        o = torch.empty((1, S, Hl, D), dtype=torch.bfloat16, device=dev)
        snd_f = torch.empty((W, 1, Sl, Hl, D), dtype=torch.bfloat16, device=dev)
        peers = [None] + [randn(W, 1, Sl, Hl, D) for _ in range(W - 1)]
        rcv = torch.empty((W, 1, Sl, Hl, D), dtype=torch.bfloat16, device=dev)
        out = torch.empty((1, Sl, heads, D), dtype=torch.bfloat16, device=dev)

        def u_front():
            cp.cp_pack_qkv_dst_major_padded(*x, W, H_pad, staging=st[0])
            cp.cp_sim_exchange(st, 0, recv=recv)

        def u_attn():
            cp.cp_attn_localq_globalkv(*hs, scale=scale, out=o)

        def u_back(snd):
            cp.cp_sim_exchange([snd] + peers[1:], 0, recv=rcv)
            cp.cp_output_merge_cropped(rcv, heads, out=out)

        def u_step():
            u_front()
            cp.cp_unpack_head_sharded(recv, 1, W, out=hs)
            u_attn()
            u_back(o.view(W, 1, Sl, Hl, D))

        def u_fused_step():
            u_front()
            cp.cp_attn_recv_to_send(recv, 1, W, scale=scale, out=snd_f)
            u_back(snd_f)

        u_step()
        u_fused_step()
        # ---- cp2usp2: Ulysses 2 inside an AllGather-KV pair (buffers of its own, so that
        # both layouts are timed side by side)
        U = 2
        Hu = heads // U
        cx = [randn(1, Sl, heads, D) for _ in range(3)]
        cst = [torch.empty((U, Sl, Hu, 3 * D), dtype=torch.bfloat16, device=dev) for _ in range(U)]
        cp.cp_pack_qkv_dst_major(*[randn(1, Sl, heads, D) for _ in range(3)], U, staging=cst[1])
        crecv = torch.empty_like(cst[0])
        q_hs = torch.empty((1, U * Sl, Hu, D), dtype=torch.bfloat16, device=dev)
        k_glob, v_glob = randn(1, S, Hu, D), randn(1, S, Hu, D)
        k_reg0, v_reg0 = k_glob[:, :U * Sl], v_glob[:, :U * Sl]
        co = torch.empty((1, U * Sl, Hu, D), dtype=torch.bfloat16, device=dev)
        cpeers = [None, randn(U, 1, Sl, Hu, D)]
        crcv = torch.empty((U, 1, Sl, Hu, D), dtype=torch.bfloat16, device=dev)
        cout = torch.empty((1, Sl, heads, D), dtype=torch.bfloat16, device=dev)

        def c_attn():
            cp.cp_attn_localq_globalkv(q_hs, k_glob, v_glob, scale=scale, out=co)

        def c_step():
            cp.cp_pack_qkv_dst_major(*cx, U, staging=cst[0])
            cp.cp_sim_exchange(cst, 0, recv=crecv)
            cp.cp_unpack_head_sharded(crecv, 1, U, out=(q_hs, k_reg0, v_reg0))
            c_attn()
            cp.cp_sim_exchange([co.view(U, 1, Sl, Hu, D)] + cpeers[1:], 0, recv=crcv)
            cp.cp_output_reverse(1, crcv, U, 1, out=cout)

        c_step()
        torch.cuda.synchronize()
        burst = 3 if S > 40000 else 5
        t = time_together({"u_attn": u_attn, "u_step": u_step, "u_fused_step": u_fused_step,
                           "c_attn": c_attn, "c_step": c_step}, burst)
        rec["uaa_usp4"] = {"heads_per_rank": Hl, "padded_heads": H_pad - heads,
                           "attn_us": t["u_attn"] * 1e3, "step_us": t["u_step"] * 1e3,
                           "fused_step_us": t["u_fused_step"] * 1e3,
                           "attn_flops": 4 * Hl * S * S * D}
        rec["cp2usp2"] = {"heads_per_rank": Hu, "attn_us": t["c_attn"] * 1e3, "step_us": t["c_step"] * 1e3,
                          "attn_flops": 4 * Hu * (S // 2) * S * D}
        del x, st, recv, hs, o, snd_f, peers, rcv, out
        del cx, cst, crecv, q_hs, k_glob, v_glob, k_reg0, v_reg0, co, cpeers, crcv, cout
        torch.cuda.empty_cache()
        u, c = rec["uaa_usp4"], rec["cp2usp2"]
        rec["attn_reduction"] = 1.0 - c["attn_us"] / u["attn_us"]
        rec["step_reduction"] = 1.0 - c["step_us"] / u["step_us"]
        rec["attn_TFLOPs"] = {"uaa_usp4": u["attn_flops"] / (u["attn_us"] * 1e-6) / 1e12,
                              "cp2usp2": c["attn_flops"] / (c["attn_us"] * 1e-6) / 1e12}
        res.append(rec)
    return res


ATTN_SRC = os.path.join(ROOT, "context_attention_diffusion_amd", "csrc", "cp_attention.hip")
# flags of the counter runs: only the attention kernel's launches, no extra sections
PROFILE_ATTN_FLAGS = "--only attn --steps 5 --warmup 1 --eager --no-cold --no-cpu-baseline --no-per-config"
CALIB_BYTES = 256 << 20


def src_sha256(path=ATTN_SRC):
    import hashlib
    return hashlib.sha256(open(path, "rb").read()).hexdigest()


def traffic_file(workload):
    return os.path.join(ROOT, "profiles", f"traffic_attn_fwd_{workload}.json")


def read_counter_by_kernel(d, counter, kernel_substr):
    """Mean per-dispatch value of `counter` for each kernel whose name contains kernel_substr."""
    import csv
    import glob
    vals = {}
    for f in glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True):
        for r in csv.DictReader(open(f)):
            if r["Counter_Name"] == counter and kernel_substr in r["Kernel_Name"]:
                vals.setdefault(r["Kernel_Name"], []).append(float(r["Counter_Value"]))
    return {k: float(np.mean(v)) for k, v in vals.items()}


def read_counter_csv(d, counter, kernel_substr):
    """Per-call value of `counter` over the kernels whose name contains kernel_substr:
    the sum of each kernel's mean per dispatch (an attention call launches each of its
    kernels once, e.g. a 256-row and a 128-row launch over different heads)."""
    per = read_counter_by_kernel(d, counter, kernel_substr)
    return float(sum(per.values())) if per else None


def summarize_traffic(fetch_dir, write_dir, out_json, workload):
    """FETCH_SIZE / WRITE_SIZE (KiB per dispatch) of the attention kernel, each scaled by
    what the same counter reads for the calibration copy (CALIB_BYTES read, CALIB_BYTES written)."""
    f_attn = read_counter_csv(os.path.join(fetch_dir, "attn"), "FETCH_SIZE", "attn_fwd")
    w_attn = read_counter_csv(os.path.join(write_dir, "attn"), "WRITE_SIZE", "attn_fwd")
    f_copy = read_counter_csv(os.path.join(fetch_dir, "copy"), "FETCH_SIZE", "copy")
    w_copy = read_counter_csv(os.path.join(write_dir, "copy"), "WRITE_SIZE", "copy")
    sf = (CALIB_BYTES / 1024.0) / f_copy
    sw = (CALIB_BYTES / 1024.0) / w_copy
    res = {"kernel": "attn_fwd_kernel", "workload": workload, "src_sha256": src_sha256(),
           "fetch_kib_raw": f_attn, "write_kib_raw": w_attn,
           "copy_fetch_kib_raw": f_copy, "copy_write_kib_raw": w_copy,
           "scale_fetch": sf, "scale_write": sw,
           "traffic_bytes": (f_attn * sf + w_attn * sw) * 1024.0,
           "commands": [
               f"rocprofv3 --pmc FETCH_SIZE -d {fetch_dir}/attn -o p --output-format csv -- python3 bench.py "
               f"--workload {workload} {PROFILE_ATTN_FLAGS}",
               f"rocprofv3 --pmc WRITE_SIZE -d {write_dir}/attn -o p --output-format csv -- python3 bench.py "
               f"--workload {workload} {PROFILE_ATTN_FLAGS}",
               f"rocprofv3 --pmc FETCH_SIZE -d {fetch_dir}/copy -o p --output-format csv -- python3 bench.py "
               "--calib-copy",
               f"rocprofv3 --pmc WRITE_SIZE -d {write_dir}/copy -o p --output-format csv -- python3 bench.py "
               "--calib-copy",
               f"python3 bench.py --workload {workload} --summarize-traffic {fetch_dir} {write_dir} {out_json}"]}
    with open(out_json, "w") as fh:
        json.dump(res, fh, indent=1)
    print(json.dumps(res))


def summarize_mfma(pmc_dir, out_md, workload):
    """MFMA utilisation of the attention kernel from one counter run: matrix-core busy cycles
    over (active cycles x SIMDs), the bf16 MFMA work the counters saw (512 flops per MOP)
    against the algorithmic count, and the share of CU-cycles with a workgroup resident."""
    import csv
    import glob
    import workloads
    wl = workloads.WORKLOADS[workload]
    n_xcd = 8
    n_cu = 256
    for f in glob.glob(os.path.join(pmc_dir, "**", "*agent_info.csv"), recursive=True):
        for r in csv.DictReader(open(f)):
            if r.get("Agent_Type", r.get("Type", "")).upper().endswith("GPU") or r.get("Name", "").startswith("gfx"):
                n_xcd = int(float(r.get("Num_Xcc", r.get("num_xcc", n_xcd)) or n_xcd))
                n_cu = int(float(r.get("Cu_Count", r.get("cu_count", n_cu)) or n_cu))
    busy = read_counter_csv(pmc_dir, "SQ_VALU_MFMA_BUSY_CYCLES", "attn_fwd")
    mops = read_counter_csv(pmc_dir, "SQ_INSTS_VALU_MFMA_MOPS_BF16", "attn_fwd")
    cu_busy = read_counter_csv(pmc_dir, "SQ_BUSY_CU_CYCLES", "attn_fwd")
    gui = read_counter_csv(pmc_dir, "GRBM_GUI_ACTIVE", "attn_fwd")
    cycles = gui / n_xcd                      # the counter is summed over the XCDs
    simds = 4 * n_cu
    flops_ctr = mops * 512.0
    flops_alg = float(wl.attn_flops_dense())
    lines = [
        f"# MFMA utilisation: attention kernel, workload {workload}",
        "",
        "Command (repository root, one MI355X):",
        "",
        "```",
        f"rocprofv3 --pmc SQ_VALU_MFMA_BUSY_CYCLES SQ_INSTS_VALU_MFMA_MOPS_BF16 SQ_BUSY_CU_CYCLES GRBM_GUI_ACTIVE "
        f"-d {pmc_dir} -o p --output-format csv -- python3 bench.py --workload {workload} {PROFILE_ATTN_FLAGS}",
        f"python3 bench.py --workload {workload} --summarize-mfma {pmc_dir} {out_md}",
        "```",
        "",
        f"Per attention call: each attn_fwd_kernel launch's mean per dispatch over the run, summed over the "
        f"launches of one call ({', '.join(sorted(short_kernel(k) for k in read_counter_by_kernel(pmc_dir, 'GRBM_GUI_ACTIVE', 'attn_fwd')))}; "
        f"{n_xcd} XCDs, {n_cu} CUs, {simds} SIMDs; the profiler serialises dispatches):",
        "",
        "| quantity | value |",
        "|---|---|",
        f"| active cycles (GRBM_GUI_ACTIVE / XCDs) | {cycles:.0f} |",
        f"| matrix-core busy cycles, all SIMDs (SQ_VALU_MFMA_BUSY_CYCLES) | {busy:.4g} |",
        f"| MFMA utilisation = busy / (active cycles x SIMDs) | {100.0 * busy / (cycles * simds):.1f}% |",
        f"| CU-cycles with a workgroup resident (SQ_BUSY_CU_CYCLES / (active cycles x CUs)) | "
        f"{100.0 * cu_busy / (cycles * n_cu):.1f}% |",
        f"| MFMA utilisation of the resident CUs = busy / (4 x SQ_BUSY_CU_CYCLES) | {100.0 * busy / (4.0 * cu_busy):.1f}% |",
        f"| bf16 MFMA flops counted (SQ_INSTS_VALU_MFMA_MOPS_BF16 x 512) | {flops_ctr:.6g} |",
        f"| algorithmic flops (4 B H Sq Skv D) | {flops_alg:.6g} |",
        "",
        "Busy cycles count the matrix pipe of a SIMD while it executes an MFMA; at the 2.5 PFLOP/s dense "
        "bf16 peak every SIMD would be busy every cycle, so the utilisation here is the fraction of that peak "
        "the kernel reaches at the clock it ran at.",
    ]
    with open(out_md, "w") as fh:
        fh.write("\n".join(lines) + "\n")
    print("\n".join(lines))


def short_kernel(name):
    return name.replace("void ", "").replace("cpattn::(anonymous namespace)::", "").split("(")[0]


def summarize_trace(db_path, out_md, command, workload):
    """Per-kernel launch counts and durations from a rocprofv3 kernel-trace database
    (its top_kernels view: durations in microseconds), with the attention call's
    algorithmic TFLOP/s and fraction of the dense bf16 peak: the call's time is the sum
    of the averages of its attn_fwd_kernel launches when they run equally often (one
    call launches each once), else the average of the busiest one."""
    import sqlite3
    import workloads
    wl = workloads.WORKLOADS[workload]
    mask = workloads.key_mask(wl)
    flops = attn_flops(wl, mask)
    con = sqlite3.connect(db_path)
    rows = list(con.execute("select name, total_calls, total_duration, average, percentage from top_kernels"))
    lines = [f"# Kernel trace: workload {workload}", "", "Command (repository root, one MI355X):", "", "```",
             command, f"python3 bench.py --workload {workload} --summarize-trace <trace db> <this file> '<command>'",
             "```", "", "| kernel | launches | total us | average us | share of GPU time |", "|---|---|---|---|---|"]
    for name, n, tot, avg, pct in rows:
        lines.append(f"| `{short_kernel(name)}` | {n} | {tot:.1f} | {avg:.3f} | {pct:.2f}% |")
    attn = [r for r in rows if "attn_fwd_kernel" in r[0]]
    if attn:
        if len({r[1] for r in attn}) == 1:
            used = attn
        else:
            used = [max(attn, key=lambda r: r[2])]
        avg = sum(r[3] for r in used)
        names = " + ".join(f"`{short_kernel(r[0])}`" for r in used)
        tf = flops / (avg * 1e-6) / 1e12
        lines += ["", f"Attention call ({names}): {flops / 1e9:.2f} GFLOP "
                  f"(4 B H Sq Skv D over valid keys) / {avg:.2f} us = {tf:.1f} TFLOP/s = "
                  f"{100.0 * tf / PEAK_BF16_TFLOPS:.1f}% of the 2.5 PFLOP/s dense bf16 peak."]
    with open(out_md, "w") as fh:
        fh.write("\n".join(lines) + "\n")
    print("\n".join(lines))


def calib_copy():
    import torch
    a = torch.empty(CALIB_BYTES // 2, dtype=torch.bfloat16, device="cuda:0").normal_()
    b = torch.empty_like(a)
    for _ in range(5):
        b.copy_(a)
    torch.cuda.synchronize()
    print(json.dumps({"calib_copy_bytes": CALIB_BYTES}))


def main():
    args = parse()
    if args.gpus != 1:
        print(json.dumps({"error": "the kernels run one rank's share on one GPU; --gpus must be 1 (the exchange is simulated on that GPU)",
                          "n_gpus": args.gpus}))
        sys.exit(2)
    if args.summarize_traffic:
        summarize_traffic(*args.summarize_traffic, args.workload)
        return
    if args.summarize_mfma:
        summarize_mfma(*args.summarize_mfma, args.workload)
        return
    if args.summarize_trace:
        summarize_trace(*args.summarize_trace, args.workload)
        return
    import torch

    if args.calib_copy:
        calib_copy()
        return
    if args.uaa:
        seqs = [int(x) for x in args.uaa_seqs.split(",")]
        recs = uaa_compare(seqs)
        print(json.dumps({"metric": "per-rank attention and step time, UAA head padding (usp4) vs "
                                    "composed Ulysses 2 x AllGather-KV 2; heads 14, D 128",
                          "unit": "us", "higher_is_better": False, "n_gpus": 1, "dtype": "bf16",
                          "data": "synthetic", "records": recs,
                          "ideal_attn_reduction": 1.0 - 3.5 / 4.0}), flush=True)
        return

    import workloads

    wl = workloads.WORKLOADS[args.workload]
    dev = torch.device("cuda:0")
    path = RankPath(wl, dev)
    for _ in range(args.warmup):
        run_steps(path, 1, only=args.only)
    torch.cuda.synchronize()

    graph = None
    if not args.eager:
        # One step captured into a HIP graph and replayed: the same kernels with
        # the host launch overhead taken out of the step.
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            run_steps(path, 1, only=args.only)
        for _ in range(2):
            graph.replay()
        torch.cuda.synchronize()
    # The clock rises over the first ~15 steps after idle (about 2.1 ms down to 1.75 ms
    # per video step): the untimed warm-up ends with about a second of steps, so that
    # the timed steps, like the per-kernel bursts below, run at the clock the GPU holds
    # under this load.
    warm_clock(graph.replay if graph is not None else (lambda: run_steps(path, 1, only=args.only)))

    # Timed region: exactly `steps` steps, synchronised on both sides.
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    if graph is not None:
        for _ in range(args.steps):
            graph.replay()
    else:
        run_steps(path, args.steps, only=args.only)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_per_step = wall * 1e3 / args.steps

    flops = attn_flops(wl, path.mask_np)
    value = flops / (ms_per_step * 1e-3) / 1e12 if args.only in (None, "attn") else None
    out = {
        "metric": METRIC,
        "value": value,
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "launch": "eager" if graph is None else "hip_graph_replay",
        "clock_warmup_s": CLOCK_WARMUP_S,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": config_of(wl),
    }
    step_fn = graph.replay if graph is not None else (lambda: run_steps(path, 1, only=args.only))
    rec = measure_config(path, args, step_fn)
    if "roofline" in rec:
        out["roofline"] = rec.pop("roofline")
    out.update(rec)
    if args.only is None:
        ref, secs = oracle_attention(wl, path.full, path.mask_np)
        out["parity"] = parity_whole(path, wl, ref)
        if not args.no_cpu_baseline:
            out["cpu_baseline"] = cpu_baseline(wl, flops, secs)
        del ref
    del graph, path
    torch.cuda.empty_cache()
    if args.only is None and not args.no_cold and not args.no_per_config:
        out["layout_ramp"] = layout_ramp(dev)
    if args.only is None and not args.no_per_config:
        per = {}
        for name in PER_CONFIG:
            if name == wl.name:
                continue
            w = workloads.WORKLOADS[name]
            p = RankPath(w, dev)
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                run_steps(p, 1)
            g.replay()
            torch.cuda.synchronize()
            r = measure_config(p, args, g.replay)
            r["config"] = config_of(w)
            ref, _ = oracle_attention(w, p.full, p.mask_np)
            r["parity"] = parity_whole(p, w, ref)
            per[name] = r
            del g, p, ref
            torch.cuda.empty_cache()
        out["per_config"] = per
    print(json.dumps(out), flush=True)


def config_of(wl):
    return {"workload": wl.name, "B": wl.B, "S_global": wl.S, "H": wl.H, "D": wl.D,
            "W": wl.W, "A": wl.A, "S_local": wl.S_local,
            "attn_q": [wl.B, wl.attn_rows, wl.attn_heads, wl.D],
            "attn_kv": [wl.B, wl.S, wl.attn_heads, wl.D], "masked": wl.masked,
            "parallelism": "one rank's share, exchange simulated on one GPU"}


def measure_config(path, args, step_fn):
    """Per-kernel durations (after a clock warm-up of step replays), the attention's
    roofline, the cold layout pass and the workload's extra sections."""
    import torch
    wl, dev = path.wl, path.dev
    warm_clock(step_fn)
    kms = kernel_bursts(path, only=args.only)
    flops = attn_flops(wl, path.mask_np)
    pack_bytes, merge_bytes = wl.pack_bytes(), wl.merge_bytes()
    kern = {}
    if "attn" in kms:
        t = kms["attn"] * 1e-3
        kern["attn"] = {"us": kms["attn"] * 1e3, "TFLOPs": flops / t / 1e12,
                        "frac_bf16_peak": flops / t / 1e12 / PEAK_BF16_TFLOPS,
                        "flops": flops, "flops_dense": wl.attn_flops_dense()}
    for name, nbytes in (("pack", pack_bytes), ("unpack", pack_bytes), ("merge", merge_bytes),
                         ("exchange_in", pack_bytes), ("exchange_out", merge_bytes),
                         ("send", merge_bytes)):
        if name in kms:
            t = kms[name] * 1e-3
            kern[name] = {"us": kms[name] * 1e3, "GBps_warm": nbytes / t / 1e9,
                          "frac_hbm_peak": nbytes / t / 1e9 / PEAK_HBM_GBPS, "bytes": nbytes}
    rec = {}
    if "attn" in kern:
        traffic = None
        tf = traffic_file(wl.name)
        if os.path.exists(tf):
            t = json.load(open(tf))
            if t.get("src_sha256") == src_sha256():   # counters taken on this kernel source
                traffic = t["traffic_bytes"]
        rec["roofline"] = {"bound": "mfma", "achieved": kern["attn"]["TFLOPs"],
                           "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                           "frac": kern["attn"]["TFLOPs"] / PEAK_BF16_TFLOPS, "traffic": traffic,
                           "kernel": "attn_fwd_kernel",
                           "algorithmic_flops_per_launch": flops,
                           "launches_per_timed_replay": KERNEL_BURST,
                           "note": "per cp_attn_localq_globalkv call: a call whose heads the library splits "
                                   "between 256-row and 128-row blocks launches attn_fwd_kernel twice, and "
                                   "achieved is over both"}
    rec["kernels"] = kern
    if args.only is None and not args.no_cold:
        pc, uc, cc = cold_layout_gbps(wl, dev)
        rec["layout_cold"] = {"pack_GBps": pc, "unpack_GBps": uc,
                              "pack_frac_hbm_peak": pc / PEAK_HBM_GBPS,
                              "unpack_frac_hbm_peak": uc / PEAK_HBM_GBPS,
                              "torch_copy_same_bytes_GBps": cc,
                              "note": "rotating buffer sets, over 600 MB of reads per pass (misses the 256 MB MALL)"}
    if args.only is None and not path.two_d and not args.no_extras:
        u = ulysses_chain(path)
        u["fused_attn_TFLOPs"] = flops / (u["fused_attn_us"] * 1e-6) / 1e12
        u["fused_step_TFLOPs"] = flops / (u["fused_step_us"] * 1e-6) / 1e12
        u["note"] = ("Ulysses-only rank step: attention of H/W heads over all W*S_l rows, "
                     "same FLOPs as the local-Q/global-KV share")
        rec["ulysses_fused"] = u
        c = chunked_kv(path)
        c["note"] = ("local-Q/global-KV share with K/V in W chunks: W partial attentions "
                     "(fp32 O + lse) and one merge, against the dense call timed beside them")
        rec["chunked_kv"] = c
    if args.only is None and path.two_d and not args.no_extras:
        u = ulysses_2d_chain(path)
        u["fused_attn_TFLOPs"] = flops / (u["fused_attn_us"] * 1e-6) / 1e12
        u["fused_step_TFLOPs"] = flops / (u["fused_step_us"] * 1e-6) / 1e12
        u["note"] = ("2D rank step: the unpack and the gathered-K/V attention against one fused call "
                     "over the received buffer and the other AllGather rank's resident K/V")
        rec["ulysses_2d_fused"] = u
    if args.only is None and not path.two_d and not wl.masked and wl.B == 1 and not args.no_extras:
        p = packed_varlen(path)
        p["dense_us"] = kern["attn"]["us"] if "attn" in kern else None
        p["note"] = ("AllGather-KV share with the sequence packed as 4 documents: per rank, the remap of "
                     "the packed query boundaries and the packed attention (both timed)")
        rec["packed_varlen"] = p
    if args.only is None and wl.masked and not args.no_extras:
        j = joint_segments(path)
        j["note"] = ("joint attention over image and text K/V segments (text mask only), "
                     "rear and front layouts, against the concatenated masked call")
        rec["joint_segments"] = j
    torch.cuda.synchronize()
    return rec


if __name__ == "__main__":
    main()
