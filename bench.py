#!/usr/bin/env python3
"""Throughput of the slot-indexed gated delta rule on one MI355X.

Headline (the JSON line's `value`): the GDN decode step of a Qwen3-Next-like
linear layer: 32 heads, K = V = 128, conv width 12288, fp32 state pool of 512
slots, batch 128, one token per request, scalar decay per head, decode tracking
at interval 256.  A step is one gdn_decode_step over the batch (slot lookup,
conv, key norm, recurrence, output, track snapshot when a request reaches a
multiple of 256).  Steps rotate over three disjoint 128-slot batches so that
consecutive steps do not find the previous step's state in the last-level
cache.  Inputs are resident in HBM before timing starts.

Secondary lines (in "extra"): the KDA chunked prefill (12 heads, one request of
6144 tokens, snapshot every 64 tokens), the KDA decode with tracking over 69
layers, a prefix-hit restore across 24 layers followed by a warm prefill, a
speculative-decoding round (draft-tree verify in 32 layers, then the
accepted-step commit), and a ReplaySSM round (ring verify of a draft chain in
69 layers, then the exact-fold commit).

Run on one GPU only: --gpus N with N > 1 exits with a message.
"""
import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
MFMA_BF16_PEAK_TFLOPS = 2500.0  # dense bf16 / fp16


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def event_pair():
    import torch
    return torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)


# ------------------------------------------------------------------ decode --
def gdn_decode_setup(torch, gdn, wl, dev):
    cfg = wl.GDN_DECODE
    H, D, N, B = cfg.heads, cfg.head_k, cfg.slots, 128
    C = H * 3 * D
    g = torch.Generator(device=dev)
    g.manual_seed(cfg.seed)
    ssm = 0.25 * torch.randn(1, N, H, D, D, device=dev, generator=g)
    conv = torch.randn(1, N, 3, C, device=dev, generator=g).to(torch.bfloat16)
    err = torch.zeros(1, dtype=torch.int32, device=dev)
    pool = gdn.state_pool_create(ssm, conv, err)
    gc = wl.generator(cfg.seed)
    w = wl.conv_weights(gc, C).to(dev)
    perm = torch.randperm(N - 1, generator=gc) + 1
    tables = [perm[i * B:(i + 1) * B].to(torch.int32).to(dev) for i in range(3)]
    spare = perm[3 * B:]
    track = torch.stack([spare[(2 * torch.arange(B)) % spare.numel()],
                         spare[(2 * torch.arange(B) + 1) % spare.numel()]], 1).to(torch.int32).to(dev)
    inputs = [{k: v.to(dev) for k, v in wl.projected_inputs(gc, B, H, D, D, cfg.alpha_mode).items()}
              for _ in range(3)]
    base = (1 + 2 * torch.arange(B, dtype=torch.int32)).to(dev)   # distinct phases mod 256
    nxt = torch.zeros(B, dtype=torch.int32, device=dev)
    out = torch.empty(B, H, D, dtype=torch.bfloat16, device=dev)
    return dict(cfg=cfg, pool=pool, w=w, tables=tables, track=track, inputs=inputs, base=base,
                nxt=nxt, out=out, H=H, D=D, B=B, C=C)


def gdn_decode_launch(gdn, st, step, seq_len_after):
    i = step % 3
    inp = st["inputs"][i]
    gdn.gdn_decode_step(st["pool"], 0, st["tables"][i], inp["x"], st["w"], inp["alpha"],
                        st["cfg"].alpha_mode, inp["beta"], st["out"],
                        seq_len_after=seq_len_after, track_interval=256,
                        track_slots=st["track"], next_track_idx=st["nxt"])


def decode_bytes(B, H, D, C, state_bytes, alpha_per_channel, snapshots):
    """Algorithmic HBM bytes of one decode launch (each byte the method must move once)."""
    per_req = (2 * H * D * D * state_bytes      # state read + write
               + 2 * 3 * C * 2                  # conv rows read + write
               + C * 2                          # x
               + H * (D if alpha_per_channel else 1) * 4 + H * 4  # alpha, beta
               + H * D * 2                      # out
               + 4)                             # slot id
    snap = snapshots * (H * D * D * state_bytes + 3 * C * 2)
    return B * per_req + C * 4 * 2 + snap


def run_headline(torch, gdn, wl, dev, steps, warmup):
    st = gdn_decode_setup(torch, gdn, wl, dev)
    B, H, D, C = st["B"], st["H"], st["D"], st["C"]
    # per-step lengths after the step, prepared before timing
    seqs = [st["base"] + s for s in range(warmup + steps)]
    for s in range(warmup):
        gdn_decode_launch(gdn, st, s, seqs[s])
    torch.cuda.synchronize()
    start, end = event_pair()
    t0 = time.perf_counter()
    start.record()
    for k in range(steps):
        gdn_decode_launch(gdn, st, warmup + k, seqs[warmup + k])
    end.record()
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    # the stream holds nothing but the decode launches between the two events
    avg_kernel_s = start.elapsed_time(end) / steps / 1e3
    base = st["base"].cpu()
    snaps = sum(int(((base + warmup + k) % 256 == 0).sum()) for k in range(steps))
    total_bytes = steps * decode_bytes(B, H, D, C, 4, False, 0) + \
        snaps * (H * D * D * 4 + 3 * C * 2)
    achieved = total_bytes / steps / avg_kernel_s / 1e9
    assert int(st["pool"].err_word.item()) == 0
    return dict(elapsed=elapsed, tokens=B * steps, avg_kernel_s=avg_kernel_s,
                bytes_per_launch=total_bytes / steps, achieved_gbs=achieved, snapshots=snaps)


def measured_traffic():
    """HBM bytes per decode launch from the committed rocprofv3 counter runs, or None
    if the decode kernel's sources changed since those counters were taken."""
    import hashlib
    path = os.path.join(ROOT, "profiles", "gdn_decode_gdn32_b128_traffic.json")
    try:
        rec = json.load(open(path))
    except OSError:
        return None
    src = b"".join(open(os.path.join(ROOT, "gated_delta_rule_slot_amd", "csrc", f), "rb").read()
                   for f in ("decode.hip", "lanes.hpp", "common.hpp"))
    if hashlib.sha256(src).hexdigest() != rec.get("sources_sha256"):
        return None
    return rec["traffic_bytes_per_launch"]


def copy_calibration(torch, dev):
    """Achieved bandwidth of a plain 1 GiB device-to-device copy (context for % of peak)."""
    a = torch.ones(256 * 1024 * 1024, dtype=torch.float32, device=dev)
    b = torch.empty_like(a)
    for _ in range(3):
        b.copy_(a)
    s, e = event_pair()
    s.record()
    for _ in range(10):
        b.copy_(a)
    e.record()
    torch.cuda.synchronize()
    t = s.elapsed_time(e) / 10 / 1e3
    return 2 * a.numel() * 4 / t / 1e9


# ----------------------------------------------------------------- prefill --
def run_kda_prefill(torch, gdn, wl, dev, reps=5):
    cfg = wl.KDA_PREFILL
    H, D, T = cfg.heads, cfg.head_k, 6144
    C = H * 3 * D
    g = wl.generator(cfg.seed)
    inp = {k: v.to(dev) for k, v in wl.projected_inputs(g, T, H, D, D, cfg.alpha_mode).items()}
    w = wl.conv_weights(g, C).to(dev)
    ssm = torch.zeros(1, cfg.slots, H, D, D, dtype=torch.bfloat16, device=dev)
    conv = torch.zeros(1, cfg.slots, 3, C, dtype=torch.bfloat16, device=dev)
    pool = gdn.state_pool_create(ssm, conv, torch.zeros(1, dtype=torch.int32, device=dev))
    cu = torch.tensor([0, T], dtype=torch.int32, device=dev)
    slot = torch.tensor([1], dtype=torch.int32, device=dev)
    cold = torch.zeros(1, dtype=torch.int32, device=dev)
    start = torch.zeros(1, dtype=torch.int32, device=dev)
    track = torch.tensor([[2, 3]], dtype=torch.int32, device=dev)
    nxt = torch.zeros(1, dtype=torch.int32, device=dev)
    out = torch.empty(T, H, D, dtype=torch.bfloat16, device=dev)
    ws = torch.empty(gdn.gdn_prefill_workspace_bytes(pool, 1, T), dtype=torch.uint8, device=dev)

    def call(flags):
        gdn.conv_gdn_prefill_chunked(pool, 0, cu, slot, cold, inp["x"], w, inp["alpha"],
                                     cfg.alpha_mode, inp["beta"], out, T, start_len=start,
                                     flags=flags, snap_interval=64, track_slots=track,
                                     next_track_idx=nxt, workspace=ws)

    def timed(flags):
        call(flags)
        torch.cuda.synchronize()
        ms = []
        for _ in range(reps):
            a, b = event_pair()
            a.record()
            call(flags)
            b.record()
            torch.cuda.synchronize()
            ms.append(a.elapsed_time(b))
        return sorted(ms)[len(ms) // 2] / 1e3

    # every 64-token boundary's state is stored (the library's default); the
    # variant that stores only the last boundary of each ping-pong parity is
    # timed beside it
    t = timed(gdn.L2NORM_K)
    t_last = timed(gdn.L2NORM_K | gdn.SNAP_LAST_ONLY)
    flops = T * H * 140.6e3               # chunked-form algorithmic flops per (token, head)
    io = T * (C * 2 + H * D * 4 + H * 4 + H * D * 2) + C * 8
    snap_bytes = H * D * D * 2 + 3 * C * 2
    n_snap = T // 64
    byts = io + n_snap * snap_bytes + H * D * D * 2
    byts_last = io + 2 * snap_bytes + H * D * D * 2
    return {"workload": "KDA chunked prefill: 12 heads, K=V=128, 1 x 6144 tokens, snapshot every 64",
            "tokens_per_s": T / t, "ms": t * 1e3,
            "snapshots_written": n_snap, "snapshots_elided": 0,
            "mfma_util_vs_bf16_peak": flops / t / 1e12 / MFMA_BF16_PEAK_TFLOPS,
            "hbm_frac": byts / t / 1e9 / HBM_PEAK_GBS, "algorithmic_bytes": byts,
            "algorithmic_flops": flops,
            "last_only_snapshots": {"snapshots_written": 2, "snapshots_elided": n_snap - 2,
                                    "ms": t_last * 1e3, "algorithmic_bytes": byts_last,
                                    "hbm_frac": byts_last / t_last / 1e9 / HBM_PEAK_GBS},
            "cu_parallelism_ceiling": "serial scan over 96 chunks on 12 heads x 8 value tiles = 96 of 256 CUs"}


def run_kda_batch_prefill(torch, gdn, wl, dev, reps=3, B=64, ws_cap=8 << 30):
    """The KDA prefill shape (12 heads, K=V=128, per-channel decay, bf16 pool) for a
    batch of 64 requests x 6144 tokens, cold, every 64-token boundary stored to the
    request's ping-pong track slots.  The library's default path (768 (request, head)
    units: the one-kernel prefill) and the two-kernel path are timed on the same call."""
    cfg = wl.KDA_PREFILL
    H, D, Tr = cfg.heads, cfg.head_k, 6144
    C = H * 3 * D
    T = B * Tr
    g = torch.Generator(device=dev)
    g.manual_seed(cfg.seed + 1)
    x = torch.randn(T, C, generator=g, device=dev, dtype=torch.bfloat16)
    alpha = torch.sigmoid(torch.randn(T, H, D, generator=g, device=dev) + 3.0)
    beta = torch.sigmoid(torch.randn(T, H, generator=g, device=dev))
    w = wl.conv_weights(wl.generator(cfg.seed + 1), C).to(dev)
    N = 3 * B + 1
    ssm = torch.zeros(1, N, H, D, D, dtype=torch.bfloat16, device=dev)
    conv = torch.zeros(1, N, 3, C, dtype=torch.bfloat16, device=dev)
    pool = gdn.state_pool_create(ssm, conv, torch.zeros(1, dtype=torch.int32, device=dev))
    cu = wl.cu_seqlens([Tr] * B).to(dev)
    slots = torch.arange(1, B + 1, dtype=torch.int32, device=dev)
    track = torch.arange(B + 1, 3 * B + 1, dtype=torch.int32, device=dev).reshape(B, 2).contiguous()
    cold = torch.zeros(B, dtype=torch.int32, device=dev)
    start = torch.zeros(B, dtype=torch.int32, device=dev)
    nxt = torch.zeros(B, dtype=torch.int32, device=dev)
    out = torch.empty(T, H, D, dtype=torch.bfloat16, device=dev)
    ws = torch.empty(min(gdn.gdn_prefill_workspace_bytes(pool, B, Tr), ws_cap), dtype=torch.uint8, device=dev)

    def call(flags, workspace):
        gdn.conv_gdn_prefill_chunked(pool, 0, cu, slots, cold, x, w, alpha, cfg.alpha_mode, beta, out, Tr,
                                     start_len=start, flags=flags, snap_interval=64, track_slots=track,
                                     next_track_idx=nxt, workspace=workspace)

    def timed(flags, workspace):
        call(flags, workspace)
        torch.cuda.synchronize()
        ms = []
        for _ in range(reps):
            a, b = event_pair()
            a.record()
            call(flags, workspace)
            b.record()
            torch.cuda.synchronize()
            ms.append(a.elapsed_time(b))
        return sorted(ms)[len(ms) // 2] / 1e3

    t_one = timed(gdn.L2NORM_K, None)
    t_two = timed(gdn.L2NORM_K | gdn.PREFILL_TWO_KERNEL, ws)
    assert int(pool.err_word.item()) == 0
    flops = T * H * 140.6e3
    io = T * (C * 2 + H * D * 4 + H * 4 + H * D * 2) + C * 8
    byts = io + B * ((Tr // 64) * (H * D * D * 2 + 3 * C * 2) + H * D * D * 2 + 3 * C * 2)
    del pool, ssm, conv, x, alpha, out, ws
    torch.cuda.empty_cache()
    return {"workload": "KDA chunked prefill, batch: 12 heads, K=V=128, 64 x 6144 tokens, cold, "
                        "snapshot every 64, bf16 pool",
            "prefill_path": "one kernel (library default for 768 (request, head) units)",
            "tokens": T, "ms": t_one * 1e3, "tokens_per_s": T / t_one,
            "snapshots_written": B * (Tr // 64), "snapshots_elided": 0,
            "hbm_frac": byts / t_one / 1e9 / HBM_PEAK_GBS,
            "mfma_util_vs_bf16_peak": flops / t_one / 1e12 / MFMA_BF16_PEAK_TFLOPS,
            "algorithmic_bytes": byts, "algorithmic_flops": flops,
            "two_kernel_ms": t_two * 1e3, "two_kernel_tokens_per_s": T / t_two,
            "workspace_bytes_two_kernel": int(ws_cap)}


# ------------------------------------------------- KDA decode with tracking --
def run_kda_decode_tracking(torch, gdn, wl, dev, steps=16, warmup=2):
    """69 KDA layers per step, batch 256, bf16 pool of 1024 slots, per-channel decay,
    snapshot every 256 tokens into ping-pong track slots; the caller flips
    next_track_idx after the last layer.  Initial lengths ~ U[256, 8192), so the
    snapshots are spread over the steps.  The same steps are also timed without
    tracking to give the snapshot overhead."""
    cfg = wl.KDA_DECODE
    L, N, H, D, B = cfg.layers, cfg.slots, cfg.heads, cfg.head_k, 256
    C = H * 3 * D
    g = torch.Generator(device=dev)
    g.manual_seed(cfg.seed)
    ssm = torch.empty(L, N, H, D, D, dtype=torch.bfloat16, device=dev)
    conv = torch.empty(L, N, 3, C, dtype=torch.bfloat16, device=dev)
    for l in range(L):
        ssm[l].normal_(0.0, 0.25, generator=g)
        conv[l].normal_(0.0, 1.0, generator=g)
    pool = gdn.state_pool_create(ssm, conv, torch.zeros(1, dtype=torch.int32, device=dev))
    gc = wl.generator(cfg.seed)
    perm = (torch.randperm(N - 1, generator=gc) + 1).to(torch.int32)
    slots = perm[:B].to(dev)
    track = perm[B:3 * B].view(B, 2).contiguous().to(dev)
    len0 = torch.randint(256, 8192, (B,), generator=gc, dtype=torch.int32)
    w = wl.conv_weights(gc, C).to(dev)
    inputs = [{k: v.to(dev) for k, v in wl.projected_inputs(gc, B, H, D, D, cfg.alpha_mode).items()}
              for _ in range(3)]
    out = torch.empty(B, H, D, dtype=torch.bfloat16, device=dev)
    nxt = torch.zeros(B, dtype=torch.int32, device=dev)
    seqs = [(len0 + s + 1).to(dev) for s in range(warmup + steps)]
    flips = [(sq % 256 == 0).to(torch.int32) for sq in seqs]

    def step(s, interval):
        sq = seqs[s]
        for l in range(L):
            inp = inputs[l % 3]
            gdn.gdn_decode_step(pool, l, slots, inp["x"], w, inp["alpha"], cfg.alpha_mode, inp["beta"], out,
                                seq_len_after=sq, track_interval=interval, track_slots=track,
                                next_track_idx=nxt)
        if interval:
            nxt.bitwise_xor_(flips[s])

    res = {}
    for interval in (256, 0):
        for s in range(warmup):
            step(s, interval)
        torch.cuda.synchronize()
        a, b = event_pair()
        a.record()
        for s in range(warmup, warmup + steps):
            step(s, interval)
        b.record()
        torch.cuda.synchronize()
        res[interval] = a.elapsed_time(b) / 1e3
    assert int(pool.err_word.item()) == 0
    snaps = sum(int(f.sum()) for f in flips[warmup:])
    t = res[256]
    byts = steps * L * decode_bytes(B, H, D, C, 2, True, 0) + snaps * L * (H * D * D * 2 + 3 * C * 2)
    del pool, ssm, conv
    torch.cuda.empty_cache()
    return {"workload": "KDA decode with tracking: 12 heads, K=V=128, 69 layers, batch 256, "
                        "bf16 pool of 1024 slots, snapshot every 256 tokens",
            "steps": steps, "tokens_per_s": B * steps / t, "ms_per_step": t / steps * 1e3,
            "GB_per_s": byts / t / 1e9, "hbm_frac": byts / t / 1e9 / HBM_PEAK_GBS,
            "snapshots": snaps, "snapshot_overhead_frac": res[256] / res[0] - 1.0}


# ------------------------------------------------ prefix hit + warm prefill --
def run_warm_prefill(torch, gdn, wl, dev, ws_cap=8 << 30):
    import numpy as np
    """64 requests of 13600 tokens in 8 prefix groups over 24 GDN layers (32 heads,
    fp32 pool of 81 slots: 64 live + 8 groups x 2 checkpoints).  Each group's seed
    run left checkpoints at 6144 and 12288 tokens of the group's token sequence,
    stored in the host checkpoint index under their chained keys; a request shares
    the first P ~ U[0, 13600) tokens of its group's sequence.  The index plans the
    restores (deepest checkpoint strictly below the final token, so c = 6144 *
    min(2, P // 6144)), restore_slots copies them across all layers, then every
    request is prefilled from c to 13600 (cold on a miss).  Checkpoint contents
    are random (they stand for the seed runs); one x buffer serves every layer.
    The library's default path runs (64 x 32 (request, head) units: the one-kernel
    prefill); the same 24 layers on the two-kernel path are timed beside it."""
    cfg = wl.WARM_PREFILL
    L, N, H, D, B, T_full = cfg.layers, cfg.slots, cfg.heads, cfg.head_k, 64, 13600
    C = H * 3 * D
    g = torch.Generator(device=dev)
    g.manual_seed(cfg.seed)
    ssm = torch.empty(L, N, H, D, D, dtype=torch.float32, device=dev)
    conv = torch.empty(L, N, 3, C, dtype=torch.bfloat16, device=dev)
    for l in range(L):
        ssm[l].normal_(0.0, 0.25, generator=g)
        conv[l].normal_(0.0, 1.0, generator=g)
    pool = gdn.state_pool_create(ssm, conv, torch.zeros(1, dtype=torch.int32, device=dev))
    gc = wl.generator(cfg.seed)
    group = torch.randint(0, 8, (B,), generator=gc).tolist()
    prefix = torch.randint(0, T_full, (B,), generator=gc).tolist()
    # token sequences: the groups' seed sequences and the requests sharing P tokens of theirs
    seeds = torch.randint(0, 150000, (8, T_full), generator=gc, dtype=torch.int32).numpy()
    reqs = []
    for i in range(B):
        tail = torch.randint(150000, 160000, (T_full - prefix[i],), generator=gc, dtype=torch.int32).numpy()
        reqs.append(np.concatenate([seeds[group[i]][:prefix[i]], tail]))
    stride = 6144
    index = gdn.CheckpointIndex(64)
    for gi in range(8):
        keys = gdn.ckpt_chain_hashes(seeds[gi][:2 * stride], stride)
        for c, k in enumerate(keys):
            assert index.insert(int(k), 65 + 2 * gi + c) == ("stored", -1)
    t0 = time.perf_counter()
    ops, reach, hit_keys = index.plan_restores(reqs, stride, list(range(1, B + 1)))
    t_plan = time.perf_counter() - t0
    depth = [int(r) for r in reach]
    assert depth == [stride * min(2, p // stride) for p in prefix]
    lens = [T_full - c for c in depth]
    T = sum(lens)
    cu = wl.cu_seqlens(lens).to(dev)
    x = torch.randn(T, C, generator=g, device=dev, dtype=torch.bfloat16)
    alpha = torch.sigmoid(torch.randn(T, H, generator=g, device=dev) + 3.0)
    beta = torch.sigmoid(torch.randn(T, H, generator=g, device=dev))
    w = wl.conv_weights(gc, C).to(dev)
    out = torch.empty(T, H, D, dtype=torch.bfloat16, device=dev)
    slots = torch.arange(1, B + 1, dtype=torch.int32, device=dev)
    start = torch.tensor(depth, dtype=torch.int32, device=dev)
    # (the library's default path for this batch, one kernel, takes no workspace;
    # the two-kernel path timed afterwards gets one)
    ws = torch.empty(min(gdn.gdn_prefill_workspace_bytes(pool, B, max(lens)), ws_cap),
                     dtype=torch.uint8, device=dev)

    # warm up on one layer, then time the whole pass (restore + 24 layers)
    gdn.conv_gdn_prefill_chunked(pool, 0, cu, slots, torch.ones(B, dtype=torch.int32, device=dev), x, w,
                                 alpha, cfg.alpha_mode, beta, out, max(lens), start_len=start)
    torch.cuda.synchronize()
    a, m, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True), \
        torch.cuda.Event(enable_timing=True)
    # a short GPU spin ahead of the first event keeps the device busy while the host
    # prepares the restore call, so the events time the copy itself
    torch.cuda._sleep(4_000_000)
    a.record()
    hist = gdn.restore_slots(pool, ops, [0] * B)
    m.record()
    has = torch.tensor(hist, dtype=torch.int32, device=dev)
    for l in range(L):
        gdn.conv_gdn_prefill_chunked(pool, l, cu, slots, has, x, w, alpha, cfg.alpha_mode, beta, out,
                                     max(lens), start_len=start)
    b.record()
    torch.cuda.synchronize()
    for k, c in zip(hit_keys, depth):
        if c:
            index.release(int(k))   # the restore copies have run
    assert int(pool.err_word.item()) == 0
    t_restore = a.elapsed_time(m) / 1e3
    t_prefill = m.elapsed_time(b) / 1e3
    # the same layers on the two-kernel path (continuing from the states just written)
    c0, c1 = event_pair()
    c0.record()
    for l in range(L):
        gdn.conv_gdn_prefill_chunked(pool, l, cu, slots, has, x, w, alpha, cfg.alpha_mode, beta, out,
                                     max(lens), start_len=start, workspace=ws,
                                     flags=gdn.L2NORM_K | gdn.PREFILL_TWO_KERNEL)
    c1.record()
    torch.cuda.synchronize()
    t_two = c0.elapsed_time(c1) / 1e3
    n_restored = sum(1 for o in ops if o[2] >= 1)
    restore_bytes = 2 * n_restored * L * (H * D * D * 4 + 3 * C * 2)
    flops = T * L * H * 140.6e3
    # HBM bytes of the prefill: per (token, layer) x, decay, b and out; per
    # (request, layer) the fp32 state and the conv rows read (warm) and written
    n_warm = sum(hist)
    pbytes = T * L * (C * 2 + H * 4 * 2 + H * D * 2) + \
        L * (B + n_warm) * (H * D * D * 4 + 3 * C * 2) + L * C * 8
    del pool, ssm, conv, x, out, ws
    torch.cuda.empty_cache()
    return {"workload": "prefix-hit restore + warm prefill: 64 requests x 13600 tokens, 8 prefix groups, "
                        "24 GDN layers, 32 heads, K=V=128, fp32 pool of 81 slots",
            "restored_requests": n_restored, "restore_ms": t_restore * 1e3,
            "index_plan_ms": t_plan * 1e3,
            "index_plan_us_per_request": t_plan / B * 1e6,
            "restore_GB_per_s": restore_bytes / t_restore / 1e9,
            "prefill_path": "one kernel (library default for 2048 (request, head) units)",
            "prefill_tokens": T, "prefill_ms": t_prefill * 1e3,
            "prefill_tokens_per_s": T / t_prefill,
            "prefill_GB_per_s": pbytes / t_prefill / 1e9,
            "prefill_hbm_frac": pbytes / t_prefill / 1e9 / HBM_PEAK_GBS,
            "prefill_mfma_util_vs_bf16_peak": flops / t_prefill / 1e12 / MFMA_BF16_PEAK_TFLOPS,
            "prefill_algorithmic_bytes": pbytes,
            "two_kernel_prefill_ms": t_two * 1e3,
            "workspace_bytes_two_kernel": ws_cap}


# ----------------------------------------------------------------- restore --
def run_restore(torch, gdn, wl, dev, reps=5):
    cfg = wl.WARM_PREFILL
    L, N, H, D = cfg.layers, cfg.slots, cfg.heads, cfg.head_k
    C = H * 3 * D
    ssm = torch.empty(L, N, H, D, D, dtype=torch.float32, device=dev)
    conv = torch.empty(L, N, 3, C, dtype=torch.bfloat16, device=dev)
    ssm.fill_(0.5)
    conv.fill_(1.0)
    pool = gdn.state_pool_create(ssm, conv)
    # 35 restored requests (the expected count for the prefix mix): checkpoints 65..80 -> live 1..35
    n = 35
    ops = [(1 + i, 1, 65 + (i % 16)) for i in range(n)]
    gdn.restore_slots(pool, ops, [0] * n)
    torch.cuda.synchronize()
    ms = []
    for _ in range(reps):
        a, b = event_pair()
        torch.cuda._sleep(4_000_000)  # the device stays busy while the host prepares the call
        a.record()
        gdn.restore_slots(pool, ops, [0] * n)
        b.record()
        torch.cuda.synchronize()
        ms.append(a.elapsed_time(b))
    t = sorted(ms)[len(ms) // 2] / 1e3
    per_op = L * (H * D * D * 4 + 3 * C * 2)
    byts = 2 * n * per_op
    return {"workload": "prefix-hit restore: 35 requests x 24 layers, 32 heads, fp32 state",
            "GB_per_s": byts / t / 1e9, "ms": t * 1e3, "hbm_frac": byts / t / 1e9 / HBM_PEAK_GBS,
            "bytes": byts}


# ------------------------------------------------------ speculative verify --
def bfs_forest(topk, T):
    """Draft tree of T nodes: topk roots on the live state, then breadth-first
    topk children per node (topk 3 and 9 nodes is the tree the pages draw)."""
    return [-1 if n < topk else (n - topk) // topk for n in range(T)]


def run_spec_verify(torch, gdn, wl, dev, rounds=3, warmup=1):
    """One speculative-decoding round over 32 linear layers: every layer verifies
    a 63-node draft tree (4 roots, 4 children per node, breadth first) for 32
    requests and keeps its node states; then every layer commits the accepted
    node (depth 3) into the live slot, and into a track slot where the accepted
    tokens cross a multiple of 256.  32 heads, K = V = 128, bf16 state (524K
    elements per layer and request), scalar decay per head."""
    L, B, T, topk, H, D = 32, 32, 63, 4, 32, 128
    C = H * 3 * D
    N = 1 + 3 * B
    g = torch.Generator(device=dev)
    g.manual_seed(106)
    ssm = torch.empty(L, N, H, D, D, dtype=torch.bfloat16, device=dev).normal_(0.0, 0.25, generator=g)
    conv = torch.empty(L, N, 3, C, dtype=torch.bfloat16, device=dev).normal_(0.0, 1.0, generator=g)
    pool = gdn.state_pool_create(ssm, conv, torch.zeros(1, dtype=torch.int32, device=dev))
    gc = wl.generator(106)
    perm = (torch.randperm(N - 1, generator=gc) + 1).to(torch.int32)
    slots = perm[:B].to(dev)
    track = perm[B:3 * B].view(B, 2).contiguous().to(dev)
    parent = torch.tensor([bfs_forest(topk, T)] * B, dtype=torch.int32, device=dev)
    accepted = torch.randint(topk + topk * topk, T, (B,), generator=gc, dtype=torch.int32).to(dev)
    before = torch.randint(256, 8192, (B,), generator=gc, dtype=torch.int32).to(dev)
    nxt = torch.zeros(B, dtype=torch.int32, device=dev)
    inp = {k: v.to(dev) for k, v in wl.projected_inputs(gc, B * T, H, D, D, 0).items()}
    x = inp["x"].view(B, T, C)
    alpha, beta = inp["alpha"].view(B, T, H), inp["beta"].view(B, T, H)
    w = wl.conv_weights(gc, C).to(dev)
    out = torch.empty(B, T, H, D, dtype=torch.bfloat16, device=dev)
    node_ssm = [torch.empty(B, T, H, D, D, dtype=torch.bfloat16, device=dev) for _ in range(L)]
    node_conv = [torch.empty(B, T, 3, C, dtype=torch.bfloat16, device=dev) for _ in range(L)]

    def verify():
        for l in range(L):
            gdn.gdn_verify_tree(pool, l, slots, parent, x, w, alpha, 0, beta, out, node_ssm[l],
                                node_conv[l])

    def commit():
        for l in range(L):
            gdn.gdn_accept_scatter(pool, l, slots, parent, accepted, node_ssm[l], node_conv[l],
                                   seq_len_before=before, track_interval=256, track_slots=track,
                                   next_track_idx=nxt)

    for _ in range(warmup):
        verify()
        commit()
    torch.cuda.synchronize()
    ev = [event_pair() + event_pair() for _ in range(rounds)]
    for a, b, c, d in ev:
        a.record()
        verify()
        b.record()
        c.record()
        commit()
        d.record()
    torch.cuda.synchronize()
    tv = sorted(a.elapsed_time(b) for a, b, _, _ in ev)[rounds // 2] / 1e3
    tc = sorted(c.elapsed_time(d) for _, _, c, d in ev)[rounds // 2] / 1e3
    assert int(pool.err_word.item()) == 0
    # crossings per request: multiples of 256 in (before, before + 3]
    crossed = int(((before + 3) // 256 - before // 256).clamp(max=2).sum())
    state, rows = H * D * D * 2, 3 * C * 2
    v_bytes = (B * state + B * T * state + B * T * C * 2 + B * rows + B * T * rows +
               B * T * H * D * 2 + B * T * H * 8 + C * 8 + B * T * 4)
    c_bytes = 2 * (B + crossed) * (state + rows)
    res = {"workload": "speculative round: 32 layers, 32 requests, 63-node draft tree (topk 4, "
                       "breadth first), 32 heads, K=V=128, bf16 state, accept depth 3, "
                       "track every 256",
           "verify_ms_per_layer": tv / L * 1e3, "commit_ms_per_layer": tc / L * 1e3,
           "round_ms": (tv + tc) * 1e3,
           "draft_tokens_per_s": B * T / (tv + tc),
           "verify_GB_per_s": v_bytes * L / tv / 1e9,
           "verify_hbm_frac": v_bytes * L / tv / 1e9 / HBM_PEAK_GBS,
           "commit_GB_per_s": c_bytes * L / tc / 1e9,
           "verify_bytes_per_launch": v_bytes,
           "node_buffer_GB": L * (node_ssm[0].numel() + node_conv[0].numel()) * 2 / 1e9}
    del pool, ssm, conv, node_ssm, node_conv
    torch.cuda.empty_cache()
    return res


# ------------------------------------------------------------ ReplaySSM --
def run_replayssm(torch, gdn, wl, dev, rounds=5, warmup=1):
    """ReplaySSM speculative round on the KDA decode pool (69 layers, 1024 slots,
    12 heads, K = V = 128, bf16 state, per-channel decay) with the pages'
    16-position ring, batch 256.  Each round verifies a 4-token draft chain per
    request in every layer (outputs + ring, no state written), then commits 1..4
    accepted tokens per request in every layer (exact fold), with tracking every
    256 tokens into ping-pong track slots."""
    cfg = wl.KDA_DECODE
    L, N, H, D, B, T, P = cfg.layers, cfg.slots, cfg.heads, cfg.head_k, 256, 4, 16
    C = H * 3 * D
    g = torch.Generator(device=dev)
    g.manual_seed(107)
    ssm = torch.empty(L, N, H, D, D, dtype=torch.bfloat16, device=dev).normal_(0.0, 0.25, generator=g)
    conv = torch.empty(L, N, 3, C, dtype=torch.bfloat16, device=dev).normal_(0.0, 1.0, generator=g)
    pool = gdn.state_pool_create(ssm, conv, torch.zeros(1, dtype=torch.int32, device=dev))
    ring = gdn.ReplayRing(pool, P, gdn.ALPHA_PER_CHANNEL)
    gc = wl.generator(107)
    perm = (torch.randperm(N - 1, generator=gc) + 1).to(torch.int32)
    slots = perm[:B].to(dev)
    track = perm[B:3 * B].view(B, 2).contiguous().to(dev)
    accepted = torch.randint(1, T + 1, (B,), generator=gc, dtype=torch.int32).to(dev)
    before = torch.randint(256, 8192, (B,), generator=gc, dtype=torch.int32).to(dev)
    inp = {k: v.to(dev) for k, v in wl.projected_inputs(gc, B * T, H, D, D, gdn.ALPHA_PER_CHANNEL).items()}
    x = inp["x"].view(B, T, C)
    alpha, beta = inp["alpha"].view(B, T, H, D), inp["beta"].view(B, T, H)
    w = wl.conv_weights(gc, C).to(dev)
    out = torch.empty(B, T, H, D, dtype=torch.bfloat16, device=dev)
    nxt = torch.zeros(B, dtype=torch.int32, device=dev)

    def verify():
        for l in range(L):
            gdn.replayssm_verify(pool, ring, l, slots, x, w, alpha, beta, out)

    def commit():
        for l in range(L):
            gdn.replayssm_commit(pool, ring, l, slots, accepted, seq_len_before=before,
                                 track_interval=256, track_slots=track, next_track_idx=nxt)

    for _ in range(warmup):
        verify()
        commit()
    torch.cuda.synchronize()
    ev = [event_pair() + event_pair() for _ in range(rounds)]
    for a, b, c, d in ev:
        a.record()
        verify()
        b.record()
        c.record()
        commit()
        d.record()
    torch.cuda.synchronize()
    tv = sorted(a.elapsed_time(b) for a, b, _, _ in ev)[rounds // 2] / 1e3
    tc = sorted(c.elapsed_time(d) for _, _, c, d in ev)[rounds // 2] / 1e3
    assert int(pool.err_word.item()) == 0
    state, rows = H * D * D * 2, 3 * C * 2
    ring_pos = H * D * 2 * 2 + H * D * 4 + H * 4 + C * 2          # rawk, rawv, g, beta, xrow
    v_bytes = B * (state + rows + T * (C * 2 + H * D * 4 + H * 4 + ring_pos + H * D * 2)) + C * 8
    n_acc = int(accepted.sum())
    c_bytes = B * 2 * (state + rows) + n_acc * ring_pos
    crossed = int(((before + accepted) // 256 - before // 256).clamp(max=2).sum())
    c_bytes += crossed * (state + rows)
    res = {"workload": "ReplaySSM round: KDA pool (69 layers, 1024 slots, 12 heads, K=V=128, bf16 "
                       "state), 16-position ring, 256 requests, 4-token draft chain, 1..4 accepted, "
                       "track every 256",
           "verify_ms_per_layer": tv / L * 1e3, "commit_ms_per_layer": tc / L * 1e3,
           "round_ms": (tv + tc) * 1e3, "draft_tokens_per_s": B * T / (tv + tc),
           "verify_GB_per_s": v_bytes * L / tv / 1e9, "verify_hbm_frac": v_bytes * L / tv / 1e9 / HBM_PEAK_GBS,
           "commit_GB_per_s": c_bytes * L / tc / 1e9, "commit_hbm_frac": c_bytes * L / tc / 1e9 / HBM_PEAK_GBS,
           "verify_bytes_per_launch": v_bytes, "commit_bytes_per_launch": c_bytes,
           "ring_GB": sum(t.numel() * t.element_size() for t in (ring.rawk, ring.rawv, ring.g, ring.beta,
                                                                    ring.xrow)) / 1e9}
    del pool, ssm, conv, ring
    torch.cuda.empty_cache()
    return res


# ------------------------------------------------------------ cpu baseline --
def cpu_baseline(wl, seconds=10.0):
    import numpy as np
    import oracle
    cfg = wl.GDN_DECODE
    H, D, B = cfg.heads, cfg.head_k, 128
    g = wl.generator(cfg.seed)
    pool = oracle.Pool(1, 2 * B + 1, H, D, D, oracle.SSM_F32)
    pool.ssm()[:] = 0.25
    w = wl.bf16_bits(wl.conv_weights(g, H * 3 * D))
    inp = wl.projected_inputs(g, B, H, D, D, cfg.alpha_mode)
    x, a, b = wl.bf16_bits(inp["x"]), inp["alpha"].numpy(), inp["beta"].numpy()
    slots = np.arange(1, B + 1, dtype=np.int32)
    steps = 0
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < seconds:
        oracle.decode_step(pool, 0, slots, x, w, a, cfg.alpha_mode, b, precision="f32")
        steps += 1
    t = time.perf_counter() - t0
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            model = next(l.split(":", 1)[1].strip() for l in f if l.startswith("model name"))
    except (OSError, StopIteration):
        pass
    return {"value": B * steps / t, "unit": "tokens/s", "cores": oracle.num_threads("f32"),
            "kind": "oracle",
            "sample": f"{steps} GDN decode steps (128 requests x 32 heads, K=V=128, fp32) "
                      f"of the fp32 oracle in {t:.1f} s",
            "cpu": f"{model}; {os.cpu_count()} logical CPUs visible"}


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=60)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--no-extra", action="store_true", help="skip the secondary workloads")
    ap.add_argument("--extra", default="kda_prefill,kda_batch_prefill,restore,kda_decode_tracking,"
                    "warm_prefill,spec_verify,replayssm", help="comma-separated secondary workloads to run")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: the hot path has no cross-GPU step (heads shard "
              "with no exchange); rerun with --gpus 1", file=sys.stderr)
        sys.exit(2)

    import torch
    import gated_delta_rule_slot_amd as gdn
    import workloads as wl

    dev = torch.device("cuda:0")
    log("headline: GDN decode")
    r = run_headline(torch, gdn, wl, dev, args.steps, args.warmup)
    value = r["tokens"] / r["elapsed"]
    extra = {"hbm_copy_calibration_GBps": copy_calibration(torch, dev)}
    runs = {"kda_prefill": ("KDA prefill", run_kda_prefill),
            "kda_batch_prefill": ("KDA prefill, batch of 64 requests", run_kda_batch_prefill),
            "restore": ("restore", run_restore),
            "kda_decode_tracking": ("KDA decode with tracking (69 layers)", run_kda_decode_tracking),
            "warm_prefill": ("prefix-hit restore + warm prefill (24 layers)", run_warm_prefill),
            "spec_verify": ("speculative verify + commit (32 layers)", run_spec_verify),
            "replayssm": ("ReplaySSM verify + exact-fold commit (69 layers)", run_replayssm)}
    chosen = [] if args.no_extra else [n for n in args.extra.split(",") if n]
    for name in chosen:
        if name not in runs:
            sys.exit(f"unknown --extra workload {name!r}; choose from {', '.join(runs)}")
        log(f"extra: {runs[name][0]}")
        extra[name] = runs[name][1](torch, gdn, wl, dev)
    cpu = None
    if not args.no_cpu_baseline:
        log("cpu baseline (oracle)")
        cpu = cpu_baseline(wl, args.cpu_seconds)
    line = {
        "metric": "gated-delta tokens/s (prefill, decode) + state-copy GB/s, % of HBM/MFMA peak",
        "value": value,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": r["elapsed"] / args.steps * 1e3,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": "GDN decode step: 32 heads, K=V=128, conv width 12288, fp32 pool "
                               "of 512 slots, batch 128, 1 token/request, tracking every 256",
                   "batch": 128, "heads": 32, "head_dim": 128, "pool_slots": 512},
        "roofline": {"bound": "hbm", "achieved": r["achieved_gbs"], "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": r["achieved_gbs"] / HBM_PEAK_GBS,
                     "traffic": measured_traffic()},
        "kernel_avg_us": r["avg_kernel_s"] * 1e6,
        "bytes_per_launch": r["bytes_per_launch"],
        "cpu_baseline": cpu,
        "extra": extra,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
