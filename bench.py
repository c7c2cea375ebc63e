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
(algorithmic bytes / time), draft steps/s and verify rows/s, the roofline of
the dominant call (lm_head + argmax, timed with HIP events on its stream over the
K launches of its timed region) and
the oracle's CPU baseline.
"""
from __future__ import annotations

import argparse
import json
import os
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
    ap.add_argument("--no-ops", action="store_true", help="skip the single-op timings (GEMV, eh_proj, attention, catch-up, stack, 8-bit head, MoE)")
    ap.add_argument("--ops-only", action="store_true", help="only the single-op timings, for kernel traces")
    ap.add_argument("--cpu-seconds", type=float, default=12.0, help="budget of the oracle baseline sample")
    ap.add_argument("--head-only", action="store_true",
                    help="only the lm_head + argmax launches (m=1), for counter runs")
    ap.add_argument("--copy-ref", action="store_true",
                    help="only a plain device copy of 256 MiB, the reference for scaling byte counters")
    return ap.parse_args()


def copy_ref(torch, dev, reps=4):
    """torch's device copy of a 256 MiB f32 tensor: reads and writes 268,435,456 bytes per launch."""
    src = torch.ones(64 << 20, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    for _ in range(reps):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_ref_bytes_per_launch": src.numel() * 4, "launches": reps}), flush=True)


def head_only(torch, mtp, synth, dev, reps):
    """lm_head + argmax at m=1 over 3 rotated copies of a 151936 x 2048 4-bit weight."""
    lm = synth.config2_head()[2]
    copies = [mtp.DeviceQ4(lm, dev) for _ in range(3)]
    gam = torch.ones(lm.k, device=dev)
    ws = torch.zeros(mtp.mtp_lmhead_workspace_size(lm.n, 1), dtype=torch.uint8, device=dev)
    x = torch.randn((1, lm.k), device=dev)
    for i in range(reps):
        mtp.mtp_lmhead_argmax(x, gam, 1e-6, copies[i % 3], ws=ws)
    torch.cuda.synchronize()
    print(json.dumps({"head_launches": reps, "bytes_per_launch": copies[0].nbytes}), flush=True)


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
        return head_only(torch, mtp, synth, dev, args.steps)
    if args.ops_only:
        print(json.dumps({"ops": op_timings(torch, mtp, synth, dev, args.steps, args.warmup)}), flush=True)
        return

    t0 = time.time()
    S = synth.config4_step()
    L = S.layer
    R = max(1, args.copies)
    layers = [mtp.DeviceLayer(L, dev) for _ in range(R)]
    caches = [(torch.from_numpy(S.k_cache).to(dev), torch.from_numpy(S.v_cache).to(dev)) for _ in range(R)]
    table = torch.from_numpy(S.table).to(dev)
    e0 = torch.from_numpy(S.e0).to(dev)
    e4 = e0.repeat(4, 1).contiguous()
    h0 = torch.from_numpy(S.h0[0]).to(dev)
    H, V, L0 = L.hidden, L.vocab, S.cache_len
    hbuf = torch.empty((4, H), dtype=torch.float32, device=dev)
    tok = torch.full((4,), -1, dtype=torch.int32, device=dev)
    ids_v = torch.empty(4, dtype=torch.int32, device=dev)
    hid_v = torch.empty((4, H), dtype=torch.float32, device=dev)
    ws = torch.empty(max(mtp.mtp_draft_step_workspace_size(layers[0], L0 + 3, 1),
                         mtp.mtp_draft_step_workspace_size(layers[0], L0, 4)), dtype=torch.uint8, device=dev)
    hbuf[0].copy_(h0)
    torch.cuda.synchronize()
    setup_s = time.time() - t0

    def chain(i):
        dl = layers[i % R]
        kc, vc = caches[i % R]
        for k in range(3):
            mtp.mtp_draft_step(dl, e0, tok[k:k + 1], table, hbuf[k:k + 1], kc, vc, L0 + k,
                               ids_out=tok[k + 1:k + 2], hidden_out=hbuf[k + 1:k + 2], ws=ws)

    def verify(i):
        dl = layers[i % R]
        kc, vc = caches[i % R]
        mtp.mtp_draft_step(dl, e4, tok, table, hbuf, kc, vc, L0, ids_out=ids_v, hidden_out=hid_v, ws=ws)

    def step(i):
        chain(i)
        verify(i)

    def timed(fn, n, warm):
        for i in range(warm):
            fn(i)
        torch.cuda.synchronize()
        t = time.perf_counter()
        for i in range(n):
            fn(i)
        torch.cuda.synchronize()
        return (time.perf_counter() - t) / n

    K, W = args.steps, args.warmup
    sec_step = timed(step, K, W)
    sec_chain = timed(chain, K, W)
    sec_verify = timed(verify, K, W)

    # algorithmic bytes: every weight byte once per call, the K/V rows read
    # (positions 0..cache_len+m-1, both heads, K and V) and the new rows written,
    # the embedding rows gathered and the f32 input/output rows
    wbytes = layers[0].weight_nbytes
    kvrow = L.n_kv_heads * L.head_dim * 4 * 2

    def call_bytes(cache_len, m):
        return wbytes + kvrow * (cache_len + m) + kvrow * m + m * H * 4 * 3

    step_bytes = sum(call_bytes(L0 + k, 1) for k in range(3)) + call_bytes(L0, 4)
    gbs = step_bytes / sec_step / 1e9

    # dominant call: lm_head + final norm + argmax, events on its own stream
    lm_copies = [dl.q4["lm_head"] for dl in layers]
    gam = layers[0].gammas[4]
    hws = torch.zeros(mtp.mtp_lmhead_workspace_size(V, 4), dtype=torch.uint8, device=dev)
    ids1 = torch.empty(4, dtype=torch.int32, device=dev)
    stream = torch.cuda.current_stream(dev)
    # one event pair around the K back-to-back launches of the timed region
    # (rotated weight copies); the average launch duration is the region / K
    head_ms = {}
    for m in (1, 4):
        xm = torch.randn((m, H), device=dev)
        for i in range(W):
            mtp.mtp_lmhead_argmax(xm, gam, 1e-6, lm_copies[i % R], ids_out=ids1[:m], ws=hws)
        ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        ev0.record(stream)
        for i in range(K):
            mtp.mtp_lmhead_argmax(xm, gam, 1e-6, lm_copies[i % R], ids_out=ids1[:m], ws=hws)
        ev1.record(stream)
        torch.cuda.synchronize()
        head_ms[m] = float(ev0.elapsed_time(ev1)) / K
    lm_bytes = lm_copies[0].nbytes + 8 + H * 4  # weights + ids + gamma
    head_bytes_m1 = lm_bytes + 1 * H * 4
    achieved = head_bytes_m1 / (head_ms[1] * 1e-3) / 1e9

    result = {
        "metric": METRIC,
        "value": round(gbs, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": W,
        "ms_per_step": round(sec_step * 1e3, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "int8-dot/f32",
        "data": "synthetic",
        "config": {
            "workload": "dense MTP draft step: K=3 chain at m=1 (cache 4096->4099) + verify at m=4; hidden 2048, "
                        "16 q / 2 kv heads x 128, SwiGLU 6144, vocab 151936, 4-bit affine g32 weights, f32 KV",
            "hidden": H, "vocab": V, "cache_len": L0, "verify_rows": 4, "draft_chain": 3,
            "weight_copies_rotated": R,
        },
        "pct_hbm_peak": round(100.0 * gbs / HBM_PEAK_GBS, 2),
        "draft_steps_per_s": round(3.0 / sec_chain, 1),
        "verify_rows_per_s": round(4.0 / sec_verify, 1),
        "ms_chain3": round(sec_chain * 1e3, 4),
        "ms_verify4": round(sec_verify * 1e3, 4),
        "step_bytes": int(step_bytes),
        "roofline": {
            "kernel": "mtp_lmhead_argmax (fused final RMSNorm + 4-bit lm_head GEMV + argmax), m=1",
            "bound": "hbm",
            "achieved": round(achieved, 1),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4),
            "traffic": recorded_traffic(),
            "traffic_unit": "bytes per launch (FETCH_SIZE x2.0 + WRITE_SIZE x1.0, see profiles/)",
            "ms_per_launch_m1": round(head_ms[1], 5),
            "ms_per_launch_m4": round(head_ms[4], 5),
            "bytes_per_launch_m1": int(head_bytes_m1),
        },
        "setup_s": round(setup_s, 1),
    }

    if not args.no_ops:
        del layers, caches, table
        torch.cuda.empty_cache()
        result["ops"] = op_timings(torch, mtp, synth, dev, K, W)

    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(S, step_bytes, args.cpu_seconds)
    print(json.dumps(result), flush=True)


def event_us(torch, dev, fn, n, warm):
    """Mean duration of fn(i) in microseconds, from HIP events recorded on the
    current stream (the stream every libmtp call of the binding launches on)."""
    stream = torch.cuda.current_stream(dev)
    for i in range(warm):
        fn(i)
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n)]
    torch.cuda.synchronize()
    for i in range(n):
        evs[i][0].record(stream)
        fn(i)
        evs[i][1].record(stream)
    torch.cuda.synchronize()
    return float(np.mean([a.elapsed_time(b) for a, b in evs])) * 1e3


def attn_catchup_stack_timings(torch, mtp, synth, dev, n, W):
    """Attention block (cache 4096, 16 q / 2 kv heads x 128; plain, with gated
    q, per-head q/k norms and rotary over 64 of 128 dims, with a 128-row
    sliding window and per-head sinks, and in MiMo's geometry: 16 query / 8 KV
    heads of 192 with V heads of 128, window 128, sinks) at m = 1 and 4, the
    cache catch-up of a 4-row target batch, and the three-layer draft stack
    (each layer catches up 4 rows, then drafts row t).  The attention and
    catch-up loops rotate over 24 layer/cache copies (about 18 MB read each) so that
    the 256 MB Infinity Cache cannot serve repeats; the stack's three layers
    stream 825 MB per call."""
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
            ws = torch.empty(mtp.mtp_attn_decode_workspace_size(reps[0][0], L0, m), dtype=torch.uint8, device=dev)

            def call(i, u=u, o=o, ws=ws):
                dl, dk, dv = reps[i % len(reps)]
                mtp.mtp_attn_decode(dl, u, dk, dv, L0, out=o, ws=ws)

            us = event_us(torch, dev, call, n, W)
            seen = L0 + m if not kw.get("window") else min(L0 + m, kw["window"] + m - 1)  # K/V rows read
            b = wb + row * seen + row * m + m * H * 4 * 2
            out[f"{name}_cache4096_m{m}"] = {"us": round(us, 3), "bytes": b, "GB/s": round(b / us / 1e3, 1)}
        if name == "attn":
            # cache catch-up: shifted target hidden -> eh_proj -> K/V rows of 4 positions
            m = 4
            tab = torch.randn((64, H), device=dev)
            toks = torch.arange(m, dtype=torch.int32, device=dev)
            pend = torch.randn((1, H), device=dev)
            tgt = torch.randn((m, H), device=dev)
            ws = torch.empty(mtp.mtp_append_kv_workspace_size(reps[0][0]), dtype=torch.uint8, device=dev)

            def catch_up(i):
                dl, dk, dv = reps[i % len(reps)]
                mtp.mtp_append_kv(dl, None, toks, tab, pend, tgt, dk, dv, L0, ws=ws)

            us = event_us(torch, dev, catch_up, n, W)
            b = q4_bytes(reps[0][0], ("eh_proj", "wk", "wv")) + m * H * 4 * 2 + H * 4 + kvrow * m
            out["append_kv_4rows_cache4096"] = {"us": round(us, 3), "bytes": b, "GB/s": round(b / us / 1e3, 1)}
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
    ws = torch.empty(mtp.mtp_stack_draft_workspace_size(layers, caches, starts, t), dtype=torch.uint8, device=dev)

    def stack(i):
        mtp.mtp_stack_draft(layers, caches, starts, tokens, table, target_h, t, ws=ws)

    us = event_us(torch, dev, stack, n, W)
    per_layer = (layers[0].weight_nbytes + kvrow * (t + 1) + kvrow * 4
                 + q4_bytes(layers[0], ("eh_proj", "wk", "wv")))
    b = 3 * per_layer
    out["stack_draft_3layers_t4099"] = {"us": round(us, 3), "us_per_layer": round(us / 3, 3), "bytes": b,
                                        "GB/s": round(b / us / 1e3, 1)}
    del layers, caches, table, target_h
    return out


def op_timings(torch, mtp, synth, dev, K, W):
    """The single-op workloads: 4-bit GEMV 1024x1024 (m=1), the e/h norm + concat
    + eh_proj 2048x4096 (m=1, 4) and the 8-bit MoE FFN (256 experts, top-8 +
    shared expert, m=1, 4).  Weight copies are rotated so that their total
    exceeds the 256 MB Infinity Cache; GB/s = algorithmic bytes / event time."""
    out = {}
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
    us = event_us(torch, dev, lambda i: mtp.mtp_qgemv(c0[i % len(c0)], x, y=y), n, W)
    b = c0[0].nbytes + 2 * 1024 * 4
    out["qgemv_1024x1024_m1"] = {"us": round(us, 3), "bytes": b, "GB/s": round(b / us / 1e3, 1)}
    del c0
    torch.cuda.empty_cache()

    e, h, ge, gh, w1 = synth.config1_proj()
    c1 = rotated_q4(w1, 86)
    de, dh = torch.from_numpy(e).to(dev), torch.from_numpy(h).to(dev)
    dge, dgh = torch.from_numpy(ge).to(dev), torch.from_numpy(gh).to(dev)
    for m in (1, 4):
        u = torch.empty((m, w1.n), dtype=torch.float32, device=dev)
        em, hm = de[:m].contiguous(), dh[:m].contiguous()
        us = event_us(torch, dev, lambda i: mtp.mtp_norm_concat_proj(em, hm, dge, dgh, 1e-6, c1[i % len(c1)], u=u),
                      n, W)
        b = c1[0].nbytes + 2 * 2048 * 4 + m * (2 * 2048 + 2048) * 4
        out[f"norm_concat_proj_2048x4096_m{m}"] = {"us": round(us, 3), "bytes": b, "GB/s": round(b / us / 1e3, 1)}
    del c1
    torch.cuda.empty_cache()
    out.update(attn_catchup_stack_timings(torch, mtp, synth, dev, n, W))
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
        us = event_us(torch, dev, lambda i: mtp.mtp_lmhead_argmax_q8(xm, gam8, 1e-6, c8[i % 2], ids_out=ids8[:m],
                                                                      ws=ws8), n, W)
        out[f"lmhead_q8_151936x2048_m{m}"] = {"us": round(us, 3), "bytes": b8, "GB/s": round(b8 / us / 1e3, 1),
                                              "frac": round(b8 / us / 1e3 / HBM_PEAK_GBS, 4)}
    del c8
    torch.cuda.empty_cache()

    M = synth.config3_moe(4)
    copies = []
    for _ in range(3):  # 3 x 906 MB expert stacks
        copies.append({k: mtp.DeviceQ8(getattr(M, k), dev)
                       for k in ("gate_exps", "up_exps", "down_exps", "sh_gate", "sh_up", "sh_down")})
    router = torch.from_numpy(M.router).to(dev)
    xm = torch.from_numpy(M.x).to(dev)
    ones = torch.ones(2048, device=dev)
    per_expert = 3 * (512 * 2048 + 512 * 2048 // 32 * 4)
    for m in (1, 4):
        xr = xm[:m].contiguous()
        y = torch.empty((m, 2048), dtype=torch.float32, device=dev)
        ids = torch.empty((m, M.top_k), dtype=torch.int32, device=dev)
        gts = torch.empty((m, M.top_k), dtype=torch.float32, device=dev)
        ws = torch.empty(mtp.mtp_ffn_moe_workspace_size(2048, 256, M.top_k, 512, 512, m), dtype=torch.uint8,
                         device=dev)

        def call(i, m=m, xr=xr, y=y, ids=ids, gts=gts, ws=ws):
            c = copies[i % 3]
            mtp.mtp_ffn_moe_q(xr, None, 1e-6, router, M.top_k, c["gate_exps"], c["up_exps"], c["down_exps"],
                              c["sh_gate"], c["sh_up"], c["sh_down"], y=y, expert_ids=ids, gates=gts, ws=ws)

        us = event_us(torch, dev, call, n, W)
        union = len(set(ids.cpu().numpy().ravel().tolist()))
        b = router.numel() * 4 + (union + 1) * per_expert + m * 2048 * 8
        out[f"moe_q8_256x8_m{m}"] = {"us": round(us, 3), "experts_touched": union + 1, "bytes": b,
                                     "GB/s": round(b / us / 1e3, 1), "frac": round(b / us / 1e3 / HBM_PEAK_GBS, 4)}
    return out


def cpu_baseline(S, step_bytes, budget_s):
    """The scalar-C oracle (single thread, as written) on a bounded sample of
    the same workload: whole steps (chain of 3 + verify of 4) until the budget
    is spent, at least one."""
    import oracle

    L = S.layer
    n = 0
    t = time.perf_counter()
    while True:
        kc, vc = S.k_cache.copy(), S.v_cache.copy()
        toks, hs = [-1], [S.h0[0]]
        for k in range(3):
            ids, hid, _ = oracle.draft_step(L, S.e0, np.array([toks[-1]], np.int32), S.table, hs[-1][None], kc, vc,
                                            S.cache_len + k, want_logits=False)
            toks.append(int(ids[0]))
            hs.append(hid[0])
        oracle.draft_step(L, np.repeat(S.e0, 4, 0), np.array(toks, np.int32), S.table, np.stack(hs), kc, vc,
                          S.cache_len, want_logits=False)
        n += 1
        el = time.perf_counter() - t
        if el >= budget_s or el / n * (n + 1) > 2.5 * budget_s:
            break
    sec = el / n
    return {"value": round(step_bytes / sec / 1e9, 3), "unit": "GB/s", "cores": 1, "kind": "oracle",
            "sample": f"{n} whole step(s) (3 chained m=1 drafts + one m=4 verify) of the same workload",
            "ms_per_step": round(sec * 1e3, 1),
            # the oracle's loops are row-independent, so each of the 7 rows costs about the same
            "draft_steps_per_s": round(7.0 / sec, 3)}


if __name__ == "__main__":
    main()
