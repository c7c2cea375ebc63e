#!/usr/bin/env python3
"""Benchmark of the quantized MTP draft-layer forward on one MI355X.

One step = one pass of the whole hot path over the dense draft workload:
a K=3 draft chain at m=1 (cache 4096 -> 4099), rollback, and one verify pass
at m=4 rows over positions 4096..4099 (hidden 2048, 16 query / 2 KV heads of
128, SwiGLU 6144, vocab 151936, 4-bit affine g32 weights, f32 KV cache).

Inputs are resident in HBM before the timed region.  To keep the 256 MB
Infinity Cache from serving repeated weight reads, R copies of the layer
weights and of the KV caches are rotated (step i uses copy i % R).

Printed: one JSON line with the weight-stream GB/s of the whole step
(algorithmic bytes / time of K steps launched back to back), per-step median
and p10/p90, draft steps/s (3 / time of the K=3 chain captured in a HIP graph
and replayed) and verify rows/s (4 / time of the captured m=4 pass), the same
for the MoE draft layer, the roofline of the dominant kernel (lm_head + argmax
at m=1: HIP events on its stream around K back-to-back launches), the measured
read-stream ceiling of the box, single-op GPU times (calls captured in graphs),
and the oracle's CPU baseline on one core and on all host cores.
"""
from __future__ import annotations

import argparse
import ctypes as C
import json
import os
import subprocess
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "quantized weight-stream GB/s (% of HBM peak); MTP draft steps/sec at m=1"
HBM_PEAK_GBS = 8000.0
HEAD_PROFILE = os.path.join(ROOT, "profiles", "lmhead_m1_vocab151936.md")
KERNEL_SOURCES = ["device.hpp", "launch.hpp", "gemv.hip"]


def kernel_source_hash() -> str:
    import hashlib
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        with open(os.path.join(ROOT, "mtp_speculative_draft_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def recorded_traffic():
    """HBM bytes per lm_head launch from the committed counter summary, or None
    when the kernel sources changed since those counters were taken."""
    try:
        text = open(HEAD_PROFILE).read()
    except OSError:
        return None
    want, got = None, None
    for line in text.splitlines():
        if line.startswith("kernel-source-sha256-16:"):
            want = line.split(":", 1)[1].split()[0]
        if line.startswith("traffic_bytes_per_launch:"):
            got = int(line.split(":", 1)[1].split()[0])
    return got if (want is not None and want == kernel_source_hash()) else None


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=30)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--copies", type=int, default=3, help="weight/cache copies rotated across steps")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-ops", action="store_true", help="skip the single-op timings")
    ap.add_argument("--no-moe", action="store_true", help="skip the MoE draft layer")
    ap.add_argument("--ops-only", action="store_true", help="only the single-op timings, for kernel traces")
    ap.add_argument("--cpu-seconds", type=float, default=12.0, help="budget of the oracle baseline samples")
    ap.add_argument("--head-only", action="store_true",
                    help="only the lm_head + argmax launches, for counter runs")
    ap.add_argument("--head-m", type=int, default=1, help="rows of the --head-only launches")
    ap.add_argument("--head-q8", action="store_true", help="--head-only over the 8-bit lm_head")
    ap.add_argument("--copy-ref", action="store_true",
                    help="only a plain device copy of 256 MiB, the reference for scaling byte counters")
    ap.add_argument("--moe-only", action="store_true", help="only the 8-bit MoE FFN at m=4 (counter runs)")
    ap.add_argument("--attn-only", action="store_true", help="only the attention block at m=1 (counter runs)")
    ap.add_argument("--step-only", action="store_true",
                    help="only the dense draft step, eager, --steps times (per-kernel counter runs)")
    return ap.parse_args()


# --------------------------------------------------------------------------
# timing helpers
# --------------------------------------------------------------------------
def capture(torch, fn):
    """A HIP graph of fn() (every libmtp call launches on torch's current
    stream, which is the capture stream inside the context)."""
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    return g


def replay_stats(torch, graphs, K, W, per_replay_units=1):
    """Replays graphs round robin: W untimed, then K timed between two
    synchronizations (the mean), then K with an event pair each (median,
    p10, p90).  Times are ms per replay / per_replay_units."""
    stream = torch.cuda.current_stream()
    for i in range(W):
        graphs[i % len(graphs)].replay()
    torch.cuda.synchronize()
    t = time.perf_counter()
    for i in range(K):
        graphs[i % len(graphs)].replay()
    torch.cuda.synchronize()
    mean = (time.perf_counter() - t) * 1e3 / K
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(K)]
    for i in range(K):
        evs[i][0].record(stream)
        graphs[i % len(graphs)].replay()
        evs[i][1].record(stream)
    torch.cuda.synchronize()
    ms = np.array([a.elapsed_time(b) for a, b in evs], dtype=np.float64)
    u = float(per_replay_units)
    return {"mean": mean / u, "median": float(np.median(ms)) / u, "p10": float(np.percentile(ms, 10)) / u,
            "p90": float(np.percentile(ms, 90)) / u}


def eager_region_us(torch, calls, n, W=3):
    """Average launch duration of a call that is one kernel: n back-to-back
    calls (fn(i)) on the stream between one event pair, / n.  (This is what
    the roofline quotes: it agrees with the kernel trace's average duration;
    the same launches replayed from a HIP graph measured several us longer
    per launch for the persistent lm_head.)"""
    for i in range(W):
        calls(i)
    stream = torch.cuda.current_stream()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    a.record(stream)
    for i in range(n):
        calls(i)
    b.record(stream)
    torch.cuda.synchronize()
    return float(a.elapsed_time(b)) * 1e3 / n


def graph_region_us(torch, calls, n, W=2):
    """GPU time per call: n calls (fn(i), i = 0..n-1) captured in one graph,
    replayed W times untimed, then once between an event pair on the stream;
    the region / n (no host work between the launches)."""
    for i in range(min(n, 4)):  # eager warm-up (lazy one-time setup, caches)
        calls(i)
    torch.cuda.synchronize()
    g = capture(torch, lambda: [calls(i) for i in range(n)])
    for _ in range(W):
        g.replay()
    stream = torch.cuda.current_stream()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    a.record(stream)
    g.replay()
    b.record(stream)
    torch.cuda.synchronize()
    us = float(a.elapsed_time(b)) * 1e3 / n
    del g
    return us


def r3(x):
    return round(float(x), 3)


def stats_ms(st):
    return {k: round(v, 5) for k, v in st.items()}


# --------------------------------------------------------------------------
# small modes (counter runs)
# --------------------------------------------------------------------------
def copy_ref(torch, dev, reps=4):
    """torch's device copy of a 256 MiB f32 tensor: reads and writes 268,435,456 bytes per launch."""
    src = torch.ones(64 << 20, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    for _ in range(reps):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_ref_bytes_per_launch": src.numel() * 4, "launches": reps}), flush=True)


def head_only(torch, mtp, synth, dev, reps, m, q8):
    """lm_head + argmax over 3 rotated copies of a 151936 x 2048 weight
    (4-bit, or 8-bit with --head-q8), eager launches."""
    if q8:
        lm = synth.q8_weight(synth.rng(8), 1, 151936, 2048)
        copies = [mtp.DeviceQ8(lm, dev) for _ in range(3)]
        call = mtp.mtp_lmhead_argmax_q8
        nbytes = 151936 * 2048 + 151936 * 64 * 4
    else:
        lm = synth.config2_head()[2]
        copies = [mtp.DeviceQ4(lm, dev) for _ in range(3)]
        call = mtp.mtp_lmhead_argmax
        nbytes = copies[0].nbytes
    gam = torch.ones(lm.k, device=dev)
    ws = torch.zeros(mtp.mtp_lmhead_workspace_size(lm.n, m), dtype=torch.uint8, device=dev)
    ids = torch.empty(m, dtype=torch.int32, device=dev)
    x = torch.randn((m, lm.k), device=dev)
    for i in range(reps):
        call(x, gam, 1e-6, copies[i % 3], ids_out=ids, ws=ws)
    torch.cuda.synchronize()
    print(json.dumps({"head_launches": reps, "rows": m, "bits": 8 if q8 else 4, "bytes_per_launch": nbytes}),
          flush=True)


def step_only(torch, mtp, synth, dev, reps, copies):
    """The dense draft step alone (K=3 chain at m=1 + verify at m=4, cache
    4096) over rotated layer/cache copies, eager launches, for per-kernel
    counter runs.  Prints the algorithmic bytes of each kernel role: the
    weights it streams once, the K/V rows read, and the partials."""
    S = synth.config4_step()
    L = S.layer
    R = max(1, copies)
    layers = [mtp.DeviceLayer(L, dev) for _ in range(R)]
    caches = [(torch.from_numpy(S.k_cache).to(dev), torch.from_numpy(S.v_cache).to(dev)) for _ in range(R)]
    chain, verify, _, _ = step_runner(torch, mtp, S, layers, caches, dev)
    for i in range(reps):
        chain(i)
        verify(i)
    torch.cuda.synchronize()
    q = layers[0].q4
    H, L0 = L.hidden, S.cache_len
    kvrow = L.n_kv_heads * L.head_dim * 4 * 2
    chunks = lambda m: (L0 + m + 31) // 32  # noqa: E731  (cache positions per partial block: 32)
    part = lambda m: chunks(m) * L.n_kv_heads * (L.n_heads // L.n_kv_heads) * m * (L.head_dim + 2) * 4  # noqa: E731
    roles = {}
    for m in (1, 4):
        roles[f"m{m}"] = {
            "eh_proj": q["eh_proj"].nbytes, "qkv": q["wq"].nbytes + q["wk"].nbytes + q["wv"].nbytes,
            "attn_partial_read": kvrow * L0, "attn_partial_write": part(m) + kvrow * m,
            "attn_combine_read": part(m), "wo": q["wo"].nbytes, "gate_up": q["gate"].nbytes + q["up"].nbytes,
            "down": q["down"].nbytes, "lm_head": q["lm_head"].nbytes}
    print(json.dumps({"step_calls": reps, "algorithmic_bytes": roles}), flush=True)


def moe_only(torch, mtp, synth, dev, reps):
    """The config-3 MoE FFN (256 experts, top-8 + shared) at m=4 over 3 rotated
    expert-stack copies, eager launches."""
    M = synth.config3_moe(4)
    copies = [{k: mtp.DeviceQ8(getattr(M, k), dev) for k in ("gate_exps", "up_exps", "down_exps", "sh_gate", "sh_up",
                                                               "sh_down")} for _ in range(3)]
    router, x = torch.from_numpy(M.router).to(dev), torch.from_numpy(M.x).to(dev)
    ws = torch.zeros(mtp.mtp_ffn_moe_workspace_size(2048, 256, M.top_k, 512, 512, 4), dtype=torch.uint8, device=dev)
    y = torch.empty((4, 2048), dtype=torch.float32, device=dev)
    for i in range(reps):
        c = copies[i % 3]
        mtp.mtp_ffn_moe_q(x, None, 1e-6, router, M.top_k, c["gate_exps"], c["up_exps"], c["down_exps"], c["sh_gate"],
                          c["sh_up"], c["sh_down"], y=y, ws=ws)
    torch.cuda.synchronize()
    print(json.dumps({"moe_m4_calls": reps}), flush=True)


def attn_only(torch, mtp, synth, dev, reps):
    """The attention block at m=1, cache 4096 (16 q / 2 kv heads x 128), over
    24 rotated layer/cache copies, eager launches."""
    g = synth.rng(40)
    Lh = synth.dense_layer(g, vocab=64)
    kc, vc = synth.kv_cache(g, Lh.n_kv_heads, 4096, 4112, 128)
    reps_ = [(mtp.DeviceLayer(Lh, dev), torch.from_numpy(kc).to(dev), torch.from_numpy(vc).to(dev)) for _ in range(24)]
    u = torch.randn((1, 2048), device=dev)
    o = torch.empty_like(u)
    ws = torch.zeros(mtp.mtp_attn_decode_workspace_size(reps_[0][0], 4096, 1), dtype=torch.uint8, device=dev)
    for i in range(reps):
        dl, dk, dv = reps_[i % 24]
        mtp.mtp_attn_decode(dl, u, dk, dv, 4096, out=o, ws=ws)
    torch.cuda.synchronize()
    print(json.dumps({"attn_m1_calls": reps}), flush=True)


# --------------------------------------------------------------------------
# the measured read ceiling (plain read stream, libmtp_bench.so)
# --------------------------------------------------------------------------
def read_ceiling(torch, dev, nbytes, K):
    """GB/s of plain nontemporal read streams over nbytes, three rotated
    buffers (past the Infinity Cache), K back-to-back launches between one
    event pair: a grid-stride kernel and two with contiguous per-wave shares
    (4 KB and 8 KB tiles) at a few grid sizes; the fastest is the ceiling."""
    path = os.path.join(ROOT, "mtp_speculative_draft_amd", "libmtp_bench.so")
    if not os.path.exists(path):
        return None
    lib = C.CDLL(path)
    lib.mtp_bench_read_stream.restype = C.c_int
    lib.mtp_bench_read_stream.argtypes = [C.c_void_p, C.c_size_t, C.c_void_p, C.c_int, C.c_int, C.c_void_p]
    nb = (nbytes + 15) // 16 * 16
    bufs = [torch.ones(nb // 4, dtype=torch.float32, device=dev) for _ in range(3)]
    cu = torch.cuda.get_device_properties(dev).multi_processor_count
    out = torch.empty(8 * cu, dtype=torch.float32, device=dev)
    variants = {}
    for mode, blocks in ((0, 8 * cu), (1, cu), (1, 2 * cu), (2, cu), (2, 2 * cu)):
        def call(i, mode=mode, blocks=blocks):
            rc = lib.mtp_bench_read_stream(C.c_void_p(bufs[i % 3].data_ptr()), nb, C.c_void_p(out.data_ptr()), blocks,
                                           mode, C.c_void_p(torch.cuda.current_stream().cuda_stream))
            if rc != 0:
                raise RuntimeError(f"read stream launch failed: {rc}")

        us = eager_region_us(torch, call, K)
        variants[f"{('grid_stride', 'chunks_4k', 'chunks_8k')[mode]}_b{blocks}"] = r3(us)
    del bufs
    best = min(variants, key=variants.get)
    us = variants[best]
    return {"GB/s": round(nb / us / 1e3, 1), "bytes": nb, "us": us, "best": best, "us_by_variant": variants,
            "kernel": "plain nontemporal float4 read streams (libmtp_bench.so), 3 rotated buffers, back-to-back "
                      "launches between one event pair; the fastest variant"}


# --------------------------------------------------------------------------
# draft steps (dense and MoE)
# --------------------------------------------------------------------------
def step_runner(torch, mtp, S, layers, caches, dev):
    """Callables for the K=3 chain at m=1 and the m=4 verify over copy c."""
    L = S.layer
    H, L0 = L.hidden, S.cache_len
    table = torch.from_numpy(S.table).to(dev)
    e0 = torch.from_numpy(S.e0).to(dev)
    e4 = e0.repeat(4, 1).contiguous()
    hbuf = torch.empty((4, H), dtype=torch.float32, device=dev)
    hbuf[0].copy_(torch.from_numpy(S.h0[0]).to(dev))
    tok = torch.full((4,), -1, dtype=torch.int32, device=dev)
    ids_v = torch.empty(4, dtype=torch.int32, device=dev)
    hid_v = torch.empty((4, H), dtype=torch.float32, device=dev)
    ws = torch.zeros(max(mtp.mtp_draft_step_workspace_size(layers[0], L0 + 3, 1),
                         mtp.mtp_draft_step_workspace_size(layers[0], L0, 4)), dtype=torch.uint8, device=dev)
    R = len(layers)

    def chain(c):
        dl = layers[c % R]
        kc, vc = caches[c % R]
        for k in range(3):
            mtp.mtp_draft_step(dl, e0, tok[k:k + 1], table, hbuf[k:k + 1], kc, vc, L0 + k,
                               ids_out=tok[k + 1:k + 2], hidden_out=hbuf[k + 1:k + 2], ws=ws)

    def verify(c):
        dl = layers[c % R]
        kc, vc = caches[c % R]
        mtp.mtp_draft_step(dl, e4, tok, table, hbuf, kc, vc, L0, ids_out=ids_v, hidden_out=hid_v, ws=ws)

    def outputs():
        torch.cuda.synchronize()
        return tok.cpu().numpy().copy(), ids_v.cpu().numpy().copy(), hid_v.cpu().numpy().copy()

    return chain, verify, outputs, table


def eager_stats(torch, fn, K, W):
    """fn(i) launched from the host: W untimed, K between two synchronizations
    (the mean), then K with an event pair each on the stream (median, p10,
    p90; the queue stays full, so these are device times)."""
    for i in range(W):
        fn(i)
    torch.cuda.synchronize()
    t = time.perf_counter()
    for i in range(K):
        fn(i)
    torch.cuda.synchronize()
    mean = (time.perf_counter() - t) * 1e3 / K
    stream = torch.cuda.current_stream()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(K)]
    for i in range(K):
        evs[i][0].record(stream)
        fn(i)
        evs[i][1].record(stream)
    torch.cuda.synchronize()
    ms = np.array([a.elapsed_time(b) for a, b in evs], dtype=np.float64)
    return {"mean": mean, "median": float(np.median(ms)), "p10": float(np.percentile(ms, 10)),
            "p90": float(np.percentile(ms, 90))}


def time_steps(torch, chain, verify, outputs, R, K, W):
    """Eager (host-launched) step timings, and graph-captured timings of the
    chain, the verify and the whole step; the graph replays must reproduce
    the eager outputs bit for bit."""
    eager = eager_stats(torch, lambda i: (chain(i), verify(i)), K, W)
    chain(0)
    verify(0)
    ref = outputs()
    g_chain = [capture(torch, lambda c=c: chain(c)) for c in range(R)]
    g_verify = [capture(torch, lambda c=c: verify(c)) for c in range(R)]
    g_step = [capture(torch, lambda c=c: (chain(c), verify(c))) for c in range(R)]
    g_step[0].replay()
    got = outputs()
    same = all(np.array_equal(a, b) for a, b in zip(ref, got))
    st_step = replay_stats(torch, g_step, K, W)
    st_chain = replay_stats(torch, g_chain, K, W)
    st_verify = replay_stats(torch, g_verify, K, W)
    del g_chain, g_verify, g_step
    return eager, st_step, st_chain, st_verify, same, ref


def stage_split(torch, mtp, S, layers, caches, dev, n):
    """One m = 1 draft step of the dense layer split into the stages the
    pages' draft profile reports (projection, attention, FFN, head), each run
    through its own libmtp call over the rotated weight copies and timed as
    graph GPU time per call; their sum is compared with the chain's per-draft
    time by the reader (each stage call carries its own launch boundary)."""
    L = S.layer
    H, V, L0 = L.hidden, L.vocab, S.cache_len
    R = len(layers)
    e = torch.from_numpy(S.e0).to(dev)
    h = torch.from_numpy(S.h0[:1]).to(dev)
    u = torch.empty((1, H), dtype=torch.float32, device=dev)
    r1 = torch.empty((1, H), dtype=torch.float32, device=dev)
    r2 = torch.empty((1, H), dtype=torch.float32, device=dev)
    ids = torch.empty(1, dtype=torch.int32, device=dev)
    ws_a = torch.zeros(mtp.mtp_attn_decode_workspace_size(layers[0], L0, 1), dtype=torch.uint8, device=dev)
    ws_f = torch.zeros(mtp.mtp_ffn_dense_workspace_size(L.ffn_inter, 1), dtype=torch.uint8, device=dev)
    ws_h = torch.zeros(mtp.mtp_lmhead_workspace_size(V, 1), dtype=torch.uint8, device=dev)
    mtp.mtp_norm_concat_proj(e, h, layers[0].gammas[0], layers[0].gammas[1], L.eps, layers[0].q4["eh_proj"], u=u)
    mtp.mtp_attn_decode(layers[0], u, caches[0][0], caches[0][1], L0, out=r1, ws=ws_a)
    mtp.mtp_ffn_dense_q(r1, layers[0].gammas[3], L.eps, layers[0].q4["gate"], layers[0].q4["up"],
                        layers[0].q4["down"], residual=r1, y=r2, ws=ws_f)

    def proj(i):
        dl = layers[i % R]
        mtp.mtp_norm_concat_proj(e, h, dl.gammas[0], dl.gammas[1], L.eps, dl.q4["eh_proj"], u=u)

    def attn(i):
        dl, (kc, vc) = layers[i % R], caches[i % R]
        mtp.mtp_attn_decode(dl, u, kc, vc, L0, out=r1, ws=ws_a)

    def ffn(i):
        dl = layers[i % R]
        mtp.mtp_ffn_dense_q(r1, dl.gammas[3], L.eps, dl.q4["gate"], dl.q4["up"], dl.q4["down"], residual=r1, y=r2,
                            ws=ws_f)

    def head(i):
        dl = layers[i % R]
        mtp.mtp_lmhead_argmax(r2, dl.gammas[4], L.eps, dl.q4["lm_head"], ids_out=ids, ws=ws_h)

    out = {"note": "GPU time per call of each stage's libmtp call (graph-captured, weights rotated); "
                   "proj = e/h norms + eh_proj, attn = attention norm + q/k/v + RoPE/append + SDPA + wo, "
                   "ffn = post-attention norm + gate/up + SwiGLU + down, head = final norm + lm_head + argmax"}
    total = 0.0
    for name, fn in (("proj", proj), ("attn", attn), ("ffn", ffn), ("head", head)):
        us = graph_region_us(torch, fn, max(n, 3 * R))
        out[f"{name}_us"] = r3(us)
        total += us
    out["sum_us"] = r3(total)
    return out


def moe_layer_bench(torch, mtp, synth, dev, K, W, q4=False):
    """The MoE draft layer at full size: the dense layer's attention, eh_proj
    and lm_head (vocab 151936) with the routed FFN (256 experts, top-8, shared
    expert, intermediate 512; 8-bit experts, or 4-bit with bf16 constants) in
    place of the SwiGLU; K=3 chain at m=1 and verify at m=4 over a 4096-row
    cache, two rotated copies."""
    S = synth.config4_step()
    moe = synth.moe_inputs(synth.rng(30, 0), 1, hidden=2048, n_experts=256, inter=512, top_k=8, shared_inter=512,
                           q4=q4)
    R = 2
    layers = [mtp.DeviceLayer(S.layer, dev, moe=moe) for _ in range(R)]
    caches = [(torch.from_numpy(S.k_cache).to(dev), torch.from_numpy(S.v_cache).to(dev)) for _ in range(R)]
    chain, verify, outputs, _ = step_runner(torch, mtp, S, layers, caches, dev)
    eager, st_step, st_chain, st_verify, same, _ = time_steps(torch, chain, verify, outputs, R, K, W)
    out = {"workload": "MoE draft layer: the dense layer's attention/eh_proj/lm_head, routed "
                       + ("4-bit (bf16 constants)" if q4 else "8-bit")
                       + " FFN 256 experts top-8 + shared (inter 512); K=3 chain at m=1 + verify at m=4, cache 4096",
           "graph_replay_equals_eager": bool(same),
           "draft_steps_per_s": round(3.0 / (st_chain["mean"] * 1e-3), 1),
           "verify_rows_per_s": round(4.0 / (st_verify["mean"] * 1e-3), 1),
           "ms_chain3_graph": stats_ms(st_chain), "ms_verify4_graph": stats_ms(st_verify),
           "ms_step_graph": stats_ms(st_step), "ms_step_eager": stats_ms(eager)}
    del layers, caches
    return out


# --------------------------------------------------------------------------
# main
# --------------------------------------------------------------------------
def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py: this build measures one GPU; --gpus {args.gpus} is not supported "
              "(the draft layer runs on a single MI355X; collectives and sharding are not part of it)", file=sys.stderr)
        sys.exit(2)

    import torch
    import mtp_speculative_draft_amd as mtp
    from mtp_speculative_draft_amd import synth

    assert torch.cuda.is_available(), "bench.py needs the GPU"
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    mtp.lib()
    if args.copy_ref:
        return copy_ref(torch, dev)
    if args.head_only:
        return head_only(torch, mtp, synth, dev, args.steps, args.head_m, args.head_q8)
    if args.moe_only:
        return moe_only(torch, mtp, synth, dev, args.steps)
    if args.attn_only:
        return attn_only(torch, mtp, synth, dev, args.steps)
    if args.step_only:
        return step_only(torch, mtp, synth, dev, args.steps, args.copies)
    if args.ops_only:
        print(json.dumps({"ops": op_timings(torch, mtp, synth, dev, args.steps, args.warmup)}), flush=True)
        return

    t0 = time.time()
    S = synth.config4_step()
    L = S.layer
    R = max(1, args.copies)
    layers = [mtp.DeviceLayer(L, dev) for _ in range(R)]
    caches = [(torch.from_numpy(S.k_cache).to(dev), torch.from_numpy(S.v_cache).to(dev)) for _ in range(R)]
    chain, verify, outputs, _ = step_runner(torch, mtp, S, layers, caches, dev)
    H, V, L0 = L.hidden, L.vocab, S.cache_len
    torch.cuda.synchronize()
    setup_s = time.time() - t0

    K, W = args.steps, args.warmup
    eager, st_step, st_chain, st_verify, same, ref = time_steps(torch, chain, verify, outputs, R, K, W)
    sec_step = eager["mean"] * 1e-3

    # algorithmic bytes: every weight byte once per call, the K/V rows read
    # (positions 0..cache_len+m-1, both heads, K and V) and the new rows written,
    # the embedding rows gathered and the f32 input/output rows
    wbytes = layers[0].weight_nbytes
    kvrow = L.n_kv_heads * L.head_dim * 4 * 2

    def call_bytes(cache_len, m):
        return wbytes + kvrow * (cache_len + m) + kvrow * m + m * H * 4 * 3

    step_bytes = sum(call_bytes(L0 + k, 1) for k in range(3)) + call_bytes(L0, 4)
    gbs = step_bytes / sec_step / 1e9

    # dominant kernel: lm_head + final norm + argmax (one launch per call),
    # K back-to-back launches over rotated copies between one event pair on
    # its stream; the average launch duration is region / K
    lm_copies = [dl.q4["lm_head"] for dl in layers]
    gam = layers[0].gammas[4]
    hws = torch.zeros(mtp.mtp_lmhead_workspace_size(V, 4), dtype=torch.uint8, device=dev)
    ids1 = torch.empty(4, dtype=torch.int32, device=dev)
    head_us = {}
    for m in (1, 4):
        xm = torch.randn((m, H), device=dev)
        head_us[m] = eager_region_us(
            torch, lambda i, xm=xm, m=m: mtp.mtp_lmhead_argmax(xm, gam, 1e-6, lm_copies[i % R], ids_out=ids1[:m],
                                                               ws=hws), K)
    lm_bytes = lm_copies[0].nbytes + 8 + H * 4  # weights + ids + gamma
    head_bytes_m1 = lm_bytes + 1 * H * 4
    achieved = head_bytes_m1 / (head_us[1] * 1e-6) / 1e9
    stages = stage_split(torch, mtp, S, layers, caches, dev, K)
    del layers, caches
    torch.cuda.empty_cache()
    ceiling = read_ceiling(torch, dev, head_bytes_m1, K)

    result = {
        "metric": METRIC,
        "value": round(gbs, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": W,
        "ms_per_step": round(eager["mean"], 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {
            "workload": "dense MTP draft step: K=3 chain at m=1 (cache 4096->4099) + verify at m=4; hidden 2048, "
                        "16 q / 2 kv heads x 128, SwiGLU 6144, vocab 151936, 4-bit affine g32 weights, f32 KV",
            "hidden": H, "vocab": V, "cache_len": L0, "verify_rows": 4, "draft_chain": 3,
            "weight_copies_rotated": R,
            "arithmetic": "f32 activations; codes enter exactly (f16 subnormals), products exact, f32 accumulation",
            "timing": "steps launched from the host back to back (value, ms_per_step, ms_step_stats); the K=3 "
                      "chain and the verify also captured in HIP graphs and replayed (draft_steps_per_s, "
                      "verify_rows_per_s)",
        },
        "pct_hbm_peak": round(100.0 * gbs / HBM_PEAK_GBS, 2),
        "ms_step_stats": stats_ms(eager),
        "ms_step_graph": stats_ms(st_step),
        "graph_replay_equals_eager": bool(same),
        "draft_steps_per_s": round(3.0 / (st_chain["mean"] * 1e-3), 1),
        "verify_rows_per_s": round(4.0 / (st_verify["mean"] * 1e-3), 1),
        "ms_chain3_graph": stats_ms(st_chain),
        "ms_verify4_graph": stats_ms(st_verify),
        "step_bytes": int(step_bytes),
        "chain_ids": ref[0][1:].tolist(),
        "verify_ids": ref[1].tolist(),
        "roofline": {
            "kernel": "mtp::k_gemv<0, 1, 1, 2, false> = mtp_lmhead_argmax (fused final RMSNorm + 4-bit lm_head GEMV + "
                      "argmax), m=1",
            "bound": "hbm",
            "achieved": round(achieved, 1),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4),
            "traffic": recorded_traffic(),
            "traffic_unit": "bytes per launch (FETCH_SIZE x2.0 + WRITE_SIZE x1.0, see profiles/)",
            "us_per_launch_m1": r3(head_us[1]),
            "us_per_launch_m4": r3(head_us[4]),
            "bytes_per_launch_m1": int(head_bytes_m1),
            "frac_of_measured_read_ceiling": (round(achieved / ceiling["GB/s"], 4) if ceiling else None),
        },
        "read_ceiling": ceiling,
        "draft_stages_m1": stages,
        "setup_s": round(setup_s, 1),
    }
    if not args.no_moe:
        torch.cuda.empty_cache()
        result["moe_layer"] = moe_layer_bench(torch, mtp, synth, dev, K, W)
        torch.cuda.empty_cache()
        result["moe_layer_q4"] = moe_layer_bench(torch, mtp, synth, dev, K, W, q4=True)
    if not args.no_ops:
        torch.cuda.empty_cache()
        result["ops"] = op_timings(torch, mtp, synth, dev, K, W)
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(S, step_bytes, args.cpu_seconds)
    print(json.dumps(result), flush=True)


# --------------------------------------------------------------------------
# single ops (GPU time per call from captured graphs)
# --------------------------------------------------------------------------
def op_entry(us, b):
    return {"us": r3(us), "bytes": int(b), "GB/s": round(b / us / 1e3, 1), "frac": round(b / us / 1e3 / HBM_PEAK_GBS, 4)}


def attn_catchup_stack_timings(torch, mtp, synth, dev, n):
    """Attention block (cache 4096, 16 q / 2 kv heads x 128; plain, with gated
    q, per-head q/k norms and rotary over 64 of 128 dims, with a 128-row
    sliding window and per-head sinks, and in MiMo's geometry: 16 query / 8 KV
    heads of 192 with V heads of 128, window 128, sinks) at m = 1 and 4, the
    cache catch-up of a 4-row target batch, and the three-layer draft stack
    (each layer catches up 4 rows, then drafts row t).  The attention and
    catch-up calls rotate over 24 layer/cache copies (about 18 MB read each)
    so that the 256 MB Infinity Cache cannot serve repeats; the stack's three
    layers stream 825 MB per call."""
    out = {}
    H, D, NKV, L0, CAP = 2048, 128, 2, 4096, 4112
    kvrow = NKV * D * 4 * 2  # K and V bytes of one position

    def q4_bytes(dl, names):
        return sum(dl.q4[k].nbytes for k in names)

    for name, kw in (("attn", {}), ("attn_variant", {"q_gated": True, "qk_norm": True, "rotary_dim": 64}),
                     ("attn_window128_sinks", {"window": 128, "sinks": True}),
                     ("attn_mimo_16x8_192v128_window128_sinks",
                      {"n_heads": 16, "n_kv_heads": 8, "head_dim": 192, "v_head_dim": 128, "window": 128,
                       "sinks": True})):
        g = synth.rng(40)
        Lh = synth.dense_layer(g, vocab=64, **kw)
        nkv, kd, vd = Lh.n_kv_heads, Lh.head_dim, Lh.v_head_dim or Lh.head_dim
        kc, vc = synth.kv_cache(g, nkv, L0, CAP, kd, v_dim=vd)
        row = nkv * (kd + vd) * 4  # K and V bytes of one position
        reps = [(mtp.DeviceLayer(Lh, dev), torch.from_numpy(kc).to(dev), torch.from_numpy(vc).to(dev))
                for _ in range(24)]
        wb = q4_bytes(reps[0][0], ("wq", "wk", "wv", "wo"))
        for m in (1, 4):
            u = torch.randn((m, H), device=dev)
            o = torch.empty_like(u)
            ws = torch.zeros(mtp.mtp_attn_decode_workspace_size(reps[0][0], L0, m), dtype=torch.uint8, device=dev)

            def call(i, u=u, o=o, ws=ws):
                dl, dk, dv = reps[i % len(reps)]
                mtp.mtp_attn_decode(dl, u, dk, dv, L0, out=o, ws=ws)

            us = graph_region_us(torch, call, n)
            seen = L0 + m if not kw.get("window") else min(L0 + m, kw["window"] + m - 1)  # K/V rows read
            b = wb + row * seen + row * m + m * H * 4 * 2
            out[f"{name}_cache4096_m{m}"] = op_entry(us, b)
        if name == "attn":
            # cache catch-up: shifted target hidden -> eh_proj -> K/V rows of 4 positions
            m = 4
            tab = torch.randn((64, H), device=dev)
            toks = torch.arange(m, dtype=torch.int32, device=dev)
            pend = torch.randn((1, H), device=dev)
            tgt = torch.randn((m, H), device=dev)
            ws = torch.zeros(mtp.mtp_append_kv_workspace_size(reps[0][0]), dtype=torch.uint8, device=dev)

            def catch_up(i):
                dl, dk, dv = reps[i % len(reps)]
                mtp.mtp_append_kv(dl, None, toks, tab, pend, tgt, dk, dv, L0, ws=ws)

            us = graph_region_us(torch, catch_up, n)
            b = q4_bytes(reps[0][0], ("eh_proj", "wk", "wv")) + m * H * 4 * 2 + H * 4 + kvrow * m
            out["append_kv_4rows_cache4096"] = op_entry(us, b)
        del reps
        torch.cuda.empty_cache()

    # three-layer draft stack, full vocabulary: t = L0 + 3, each layer
    # recomputes rows t - 4 .. t - 1 (catch-up) and drafts row t
    layers = [mtp.DeviceLayer(synth.dense_layer(synth.rng(41, k)), dev) for k in range(3)]
    V = layers[0].vocab
    t = L0 + 3
    caches = []
    for k in range(3):
        kc, vc = synth.kv_cache(synth.rng(42, k), NKV, t - 4, CAP, D)
        caches.append((torch.from_numpy(kc).to(dev), torch.from_numpy(vc).to(dev)))
    table = torch.randn((V, H), device=dev)
    target_h = torch.randn((t + 1, H), device=dev)
    tokens = torch.randint(0, V, (t + 2 + 3,), dtype=torch.int32, device=dev)
    starts = [t - 4] * 3
    ws = torch.zeros(mtp.mtp_stack_draft_workspace_size(layers, caches, starts, t), dtype=torch.uint8, device=dev)

    def stack(i):
        mtp.mtp_stack_draft(layers, caches, starts, tokens, table, target_h, t, ws=ws)

    us = graph_region_us(torch, stack, max(4, n // 4))
    per_layer = (layers[0].weight_nbytes + kvrow * (t + 1) + kvrow * 4
                 + q4_bytes(layers[0], ("eh_proj", "wk", "wv")))
    out["stack_draft_3layers_t4099"] = dict(op_entry(us, 3 * per_layer), us_per_layer=r3(us / 3))
    del layers, caches, table, target_h
    return out


def op_timings(torch, mtp, synth, dev, K, W):
    """The single-op workloads: 4-bit GEMV 1024x1024 (m=1), the e/h norm + concat
    + eh_proj 2048x4096 (m=1, 4), the attention block, catch-up and stack
    (above), the 8-bit lm_head (m=1, 4) and the MoE FFN (256 experts, top-8 +
    shared expert, m=1, 4) with 8-bit and with 4-bit experts.  Weight copies are rotated so that their
    total exceeds the 256 MB Infinity Cache; each entry is GPU time per call
    (n calls captured in one graph) and GB/s = algorithmic bytes / that time."""
    out = {"note": "us = GPU time per call: n calls captured in one HIP graph, events around one replay, / n"}
    n = max(K, 20)

    def rotated_q4(w, copies):
        base = mtp.DeviceQ4(w, dev)
        reps = [base]
        for _ in range(copies - 1):
            c = mtp.DeviceQ4.__new__(mtp.DeviceQ4)
            c.codes, c.scales, c.biases = base.codes.clone(), base.scales.clone(), base.biases.clone()
            c.n, c.k = base.n, base.k
            c.desc = mtp.MtpQ4(c.codes.data_ptr(), c.scales.data_ptr(), c.biases.data_ptr(), c.n, c.k)
            reps.append(c)
        return reps

    w0, x0 = synth.config0_gemv()
    c0 = rotated_q4(w0, 683)
    x = torch.from_numpy(x0).to(dev)
    y = torch.empty((1, w0.n), dtype=torch.float32, device=dev)
    us = graph_region_us(torch, lambda i: mtp.mtp_qgemv(c0[i % len(c0)], x, y=y), 200)
    out["qgemv_1024x1024_m1"] = op_entry(us, c0[0].nbytes + 2 * 1024 * 4)
    del c0
    torch.cuda.empty_cache()

    e, h, ge, gh, w1 = synth.config1_proj()
    c1 = rotated_q4(w1, 86)
    de, dh = torch.from_numpy(e).to(dev), torch.from_numpy(h).to(dev)
    dge, dgh = torch.from_numpy(ge).to(dev), torch.from_numpy(gh).to(dev)
    for m in (1, 4):
        u = torch.empty((m, w1.n), dtype=torch.float32, device=dev)
        em, hm = de[:m].contiguous(), dh[:m].contiguous()
        us = graph_region_us(torch, lambda i: mtp.mtp_norm_concat_proj(em, hm, dge, dgh, 1e-6, c1[i % len(c1)], u=u),
                             86)
        out[f"norm_concat_proj_2048x4096_m{m}"] = op_entry(us, c1[0].nbytes + 2 * 2048 * 4 + m * (2 * 2048 + 2048) * 4)
    del c1
    torch.cuda.empty_cache()
    out.update(attn_catchup_stack_timings(torch, mtp, synth, dev, n))
    torch.cuda.empty_cache()

    # 8-bit lm_head (vocab 151936 x 2048, int8 + one f32 scale per 32) with the
    # fused final norm and greedy pick, m = 1 and 4, two rotated copies (700 MB)
    g8 = synth.rng(8)
    lm8 = synth.q8_weight(g8, 1, 151936, 2048)
    c8 = [mtp.DeviceQ8(lm8, dev) for _ in range(2)]
    del lm8
    gam8 = torch.ones(2048, device=dev)
    ws8 = torch.zeros(mtp.mtp_lmhead_workspace_size(151936, 4), dtype=torch.uint8, device=dev)
    ids8 = torch.empty(4, dtype=torch.int32, device=dev)
    b8 = 151936 * 2048 + 151936 * 64 * 4
    for m in (1, 4):
        xm = torch.randn((m, 2048), device=dev)
        us = graph_region_us(torch, lambda i, xm=xm, m=m: mtp.mtp_lmhead_argmax_q8(xm, gam8, 1e-6, c8[i % 2],
                                                                                   ids_out=ids8[:m], ws=ws8), n)
        out[f"lmhead_q8_151936x2048_m{m}"] = op_entry(us, b8)
    del c8
    torch.cuda.empty_cache()

    out.update(moe_timings(torch, mtp, synth, dev, n, q4=False))
    torch.cuda.empty_cache()
    out.update(moe_timings(torch, mtp, synth, dev, n, q4=True))
    return out


def moe_timings(torch, mtp, synth, dev, n, q4):
    """The MoE FFN of the configuration (hidden 2048, 256 experts of 512,
    top-8 + shared) at m = 1 and 4: 8-bit experts (three rotated 906 MB
    stacks) or 4-bit experts with bf16 constants (two 505 MB stacks).  The
    bytes count the experts the call selected (read back from its ids)."""
    out = {}
    M = synth.config3_moe(4) if not q4 else synth.moe_inputs(synth.rng(3, 0), 4, q4=True)
    names = ("gate_exps", "up_exps", "down_exps", "sh_gate", "sh_up", "sh_down")
    R = 2 if q4 else 3
    copies = [{k: mtp.device_experts(getattr(M, k), dev) for k in names} for _ in range(R)]
    router = torch.from_numpy(M.router).to(dev)
    xm = torch.from_numpy(M.x).to(dev)
    per_expert = M.gate_exps.expert_nbytes * 3
    fn = mtp.mtp_ffn_moe_q4 if q4 else mtp.mtp_ffn_moe_q
    for m in (1, 4):
        xr = xm[:m].contiguous()
        y = torch.empty((m, 2048), dtype=torch.float32, device=dev)
        ids = torch.empty((m, M.top_k), dtype=torch.int32, device=dev)
        gts = torch.empty((m, M.top_k), dtype=torch.float32, device=dev)
        ws = torch.zeros(mtp.mtp_ffn_moe_workspace_size(2048, 256, M.top_k, 512, 512, m), dtype=torch.uint8,
                         device=dev)

        def call(i, m=m, xr=xr, y=y, ids=ids, gts=gts, ws=ws):
            c = copies[i % R]
            fn(xr, None, 1e-6, router, M.top_k, *(c[k] for k in names), y=y, expert_ids=ids, gates=gts, ws=ws)

        us = graph_region_us(torch, call, n)
        union = len(set(ids.cpu().numpy().ravel().tolist()))
        b = router.numel() * 4 + (union + 1) * per_expert + m * 2048 * 8
        out[f"moe_{'q4' if q4 else 'q8'}_256x8_m{m}"] = dict(op_entry(us, b), experts_touched=union + 1)
    del copies
    return out


# --------------------------------------------------------------------------
# CPU baseline: the oracle, timed as written
# --------------------------------------------------------------------------
def host_cpu():
    model = None
    try:
        for line in subprocess.run(["lscpu"], capture_output=True, text=True, timeout=20).stdout.splitlines():
            if line.lower().startswith("model name"):
                model = line.split(":", 1)[1].strip()
                break
    except Exception:
        pass
    try:
        usable = len(os.sched_getaffinity(0))
    except Exception:
        usable = os.cpu_count()
    return model, usable


def cpu_baseline(S, step_bytes, budget_s):
    """The scalar-C oracle on bounded samples of the same workload: the K=3
    chain (three m=1 drafts) and the m=4 verify, timed apart, repeated until
    half the budget is spent (at least once): first the plain build (one
    thread), then its OpenMP twin over all usable host cores (the same
    per-element sums, so the same bits)."""
    import oracle

    L = S.layer
    model, usable = host_cpu()
    threads = int(os.environ.get("OMP_NUM_THREADS") or usable or 1)

    def sample(limit):
        n, tc, tv = 0, 0.0, 0.0
        while True:
            kc, vc = S.k_cache.copy(), S.v_cache.copy()
            toks, hs = [-1], [S.h0[0]]
            t = time.perf_counter()
            for k in range(3):
                ids, hid, _ = oracle.draft_step(L, S.e0, np.array([toks[-1]], np.int32), S.table, hs[-1][None], kc, vc,
                                                S.cache_len + k, want_logits=False)
                toks.append(int(ids[0]))
                hs.append(hid[0])
            t1 = time.perf_counter()
            oracle.draft_step(L, np.repeat(S.e0, 4, 0), np.array(toks, np.int32), S.table, np.stack(hs), kc, vc,
                              S.cache_len, want_logits=False)
            tc += t1 - t
            tv += time.perf_counter() - t1
            n += 1
            if tc + tv >= limit or (tc + tv) / n * (n + 1) > 2.0 * limit:
                break
        return n, tc / n, tv / n

    out = {}
    for name, threaded in (("one_core", False), ("all_cores", True)):
        oracle.set_threaded(threaded)
        try:
            n, chain_s, verify_s = sample(budget_s / 2)
        finally:
            oracle.set_threaded(False)
        step_s = chain_s + verify_s
        out[name] = {"threads": threads if threaded else 1, "steps_sampled": n,
                     "ms_per_step": round(step_s * 1e3, 1), "GB/s": round(step_bytes / step_s / 1e9, 3),
                     "draft_steps_per_s": round(3.0 / chain_s, 3), "verify_rows_per_s": round(4.0 / verify_s, 3)}
    a = out["all_cores"]
    return {"value": a["GB/s"], "unit": "GB/s", "cores": a["threads"], "kind": "oracle",
            "sample": f"{a['steps_sampled']} whole step(s) (3 chained m=1 drafts + one m=4 verify, timed apart) of "
                      f"the same workload on {a['threads']} threads (OpenMP build of the oracle, same bits); "
                      f"{out['one_core']['steps_sampled']} on one thread (plain build)",
            "draft_steps_per_s": a["draft_steps_per_s"], "verify_rows_per_s": a["verify_rows_per_s"],
            "ms_per_step": a["ms_per_step"], "one_core": out["one_core"], "host_cpu_model": model,
            "host_cpus_usable": usable}


if __name__ == "__main__":
    main()
