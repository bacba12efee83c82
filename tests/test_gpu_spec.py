"""GPU parity of gdn_verify_tree and gdn_accept_scatter against the oracle.

Verify: outputs (bf16) and node states (pool dtype) as relative L2 per
(request, node, head) unit, tolerance 2e-3; node conv rows bit-exact (they are
copies of x and live rows); the live pool bit-exact untouched.  Scatter: the
slots it writes are the ones the oracle writes, each a byte copy of the GPU's
own node buffer, values within tolerance of the oracle's, everything else
untouched.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads as wl
from tests.helpers import (REL_L2_TOL, bf16_np, device_ssm_values, pool_bytes_equal, pool_to_oracle,
                           ssm_values, unit_rel_l2, widen, worst_unit_rel_l2)

pytestmark = pytest.mark.gpu


def _spec_inputs(seed, L, N, H, D, bf16, B, T, alpha_mode):
    g = wl.generator(seed)
    ssm, conv = wl.warm_pool(g, L, N, H, D, D, bf16)
    w = wl.conv_weights(g, H * 3 * D)
    inp = wl.projected_inputs(g, B * T, H, D, D, alpha_mode)
    slots = wl.distinct_slots(g, B, N)
    return g, ssm, conv, w, inp, slots


def _verify_both(ssm, conv, w, inp, slots, parent, alpha_mode, layer, scale=1.0, flags=1):
    import gated_delta_rule_slot_amd as gdn
    B, T = parent.shape
    H, D = ssm.shape[2], ssm.shape[3]
    C = H * 3 * D
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    pool = gdn.state_pool_create(ssm.cuda(), conv.cuda(), err)
    out = torch.full((B, T, H, D), 7.0, dtype=torch.bfloat16, device="cuda")
    ns = torch.zeros((B, T, H, D, D), dtype=ssm.dtype, device="cuda")
    nc = torch.zeros((B, T, 3, C), dtype=torch.bfloat16, device="cuda")
    a = inp["alpha"].reshape(B, T, *inp["alpha"].shape[1:])
    gdn.gdn_verify_tree(pool, layer, slots.cuda(), parent.cuda(), inp["x"].reshape(B, T, C).cuda(),
                        w.cuda(), a.contiguous().cuda(), alpha_mode,
                        inp["beta"].reshape(B, T, H).contiguous().cuda(), out, ns, nc,
                        scale=scale, flags=flags)
    ref = pool_to_oracle(ssm, conv)
    o_ref, ns_ref, nc_ref, e = oracle.verify_tree(
        ref, layer, slots.numpy(), parent.numpy(), wl.bf16_bits(inp["x"]).reshape(B, T, C),
        wl.bf16_bits(w), a.numpy(), alpha_mode, inp["beta"].numpy().reshape(B, T, H),
        scale=scale, flags=flags)
    torch.cuda.synchronize()
    return pool, out, ns, nc, ref, o_ref, ns_ref, nc_ref, e


def _node_values(ns_dev, ns_ref):
    got = ns_dev.detach().cpu().to(torch.float64).numpy()
    want = ns_ref.astype(np.float64) if ns_ref.dtype == np.float32 else widen(ns_ref)
    return got, want


def _assert_verify(ssm, conv, pool, out, ns, nc, o_ref, ns_ref, nc_ref):
    eo = worst_unit_rel_l2(widen(bf16_np(out)), widen(o_ref), 3)
    got, want = _node_values(ns, ns_ref)
    es = worst_unit_rel_l2(got, want, 3)
    print(f"  worst unit rel-L2: out {eo:.2e}  node state {es:.2e}", flush=True)
    assert eo <= REL_L2_TOL and es <= REL_L2_TOL
    assert np.array_equal(bf16_np(nc), nc_ref)
    # the live pool is only read
    assert torch.equal(pool.ssm.cpu(), ssm) and torch.equal(pool.conv.cpu(), conv)


def bfs_forest(topk, T):
    """Complete topk-ary forest in breadth-first order: topk roots on the live
    state, node n >= topk under node (n - topk) // topk.  topk 3 and 9 nodes is
    the pages' tree."""
    return [-1 if n < topk else (n - topk) // topk for n in range(T)]


def random_tree(g, T):
    return [int(torch.randint(-1, n, (1,), generator=g)) if n else -1 for n in range(T)]


@pytest.mark.parametrize("name,seed,L,N,H,D,bf16,B,T,amode,kind", [
    ("D16 fp32 KDA, the pages' tree", 11, 1, 12, 2, 16, False, 3, 9, 1, "page"),
    ("D32 bf16 GDN, chains", 12, 2, 30, 4, 32, True, 5, 6, 0, "chain"),
    ("D64 fp32 KDA, random trees", 13, 1, 40, 6, 64, False, 7, 13, 1, "random"),
    ("D128 fp32 GDN, topk-2 forest", 14, 1, 48, 8, 128, False, 6, 7, 0, "bfs2"),
    ("D128 bf16 KDA, random trees", 15, 2, 40, 12, 128, True, 3, 21, 1, "random"),
    ("D64 bf16 GDN, stars", 16, 1, 20, 3, 64, True, 4, 5, 0, "star"),
])
def test_verify_parity(name, seed, L, N, H, D, bf16, B, T, amode, kind):
    print(f"verify parity: {name}", flush=True)
    g, ssm, conv, w, inp, slots = _spec_inputs(seed, L, N, H, D, bf16, B, T, amode)
    trees = {
        "page": lambda: bfs_forest(3, T),
        "chain": lambda: list(range(-1, T - 1)),
        "star": lambda: [-1] * T,
        "bfs2": lambda: bfs_forest(2, T),
        "random": lambda: random_tree(g, T),
    }
    parent = torch.tensor([trees[kind]() for _ in range(B)], dtype=torch.int32)
    layer = L - 1
    pool, out, ns, nc, ref, o_ref, ns_ref, nc_ref, e = _verify_both(
        ssm, conv, w, inp, slots, parent, amode, layer, scale=0.8)
    _assert_verify(ssm, conv, pool, out, ns, nc, o_ref, ns_ref, nc_ref)
    assert e == 0 and int(pool.err_word.item()) == 0


def test_verify_skips_bad_trees_and_slots():
    """An invalid tree (bit 8), a live slot past the pool (bit 1) and slot 0
    (padding) give zero outputs and no node writes; the others are computed."""
    print("verify: bad trees and slots", flush=True)
    B, T, H, D, N = 5, 4, 2, 32, 16
    g, ssm, conv, w, inp, slots = _spec_inputs(21, 1, N, H, D, False, B, T, 1)
    parent = torch.tensor([[-1, 0, 1, 0], [-1, 0, 3, 1], [-1, -1, 0, 1], [-1, 0, 0, 2],
                           [-1, 0, 1, 2]], dtype=torch.int32)
    slots[3] = N + 4
    slots[4] = 0
    pool, out, ns, nc, ref, o_ref, ns_ref, nc_ref, e = _verify_both(
        ssm, conv, w, inp, slots, parent, 1, 0)
    assert e == 8 | 1
    assert int(pool.err_word.item()) == 8 | 1
    _assert_verify(ssm, conv, pool, out, ns, nc, o_ref, ns_ref, nc_ref)
    for b in (1, 3, 4):
        assert not bf16_np(out[b]).any()
        assert not ns[b].any() and not nc[b].any()
    assert bf16_np(out[0]).any() and bf16_np(out[2]).any()


def test_verify_max_tree_nodes_chain():
    """A chain of the largest accepted length: deep carried state and the
    parent list at the shared-memory limit."""
    import gated_delta_rule_slot_amd as gdn
    print("verify: chain of MAX_TREE_NODES nodes", flush=True)
    B, T, H, D, N = 1, gdn.MAX_TREE_NODES, 1, 16, 4
    g, ssm, conv, w, inp, slots = _spec_inputs(22, 1, N, H, D, False, B, T, 0)
    parent = torch.arange(-1, T - 1, dtype=torch.int32)[None]
    pool, out, ns, nc, ref, o_ref, ns_ref, nc_ref, e = _verify_both(
        ssm, conv, w, inp, slots, parent, 0, 0)
    _assert_verify(ssm, conv, pool, out, ns, nc, o_ref, ns_ref, nc_ref)


def _changed_slots(before, after):
    """(layer, slot) pairs whose ssm or conv bytes differ."""
    L, N = before.ssm().shape[:2]
    sb = before.ssm_bytes.reshape(L, N, -1) != after.ssm_bytes.reshape(L, N, -1)
    cb = before.conv_bytes.reshape(L, N, -1) != after.conv_bytes.reshape(L, N, -1)
    return {(l, n) for l in range(L) for n in range(N) if sb[l, n].any() or cb[l, n].any()}


@pytest.mark.parametrize("bf16", [False, True])
def test_accept_scatter_parity(bf16):
    """Verify, then commit: accepted -1 (nothing), roots, deep nodes, with the
    accepted tokens crossing a multiple of the tracking interval (3) zero, one
    or two times, and one crossing onto a masked track entry.  The GPU writes
    exactly the slots the oracle writes, each a byte copy of its node buffer."""
    import gated_delta_rule_slot_amd as gdn
    print(f"accept scatter parity (bf16 state: {bf16})", flush=True)
    B, T, H, D, N, L = 8, 15, 4, 64, 40, 2
    g, ssm, conv, w, inp, slots = _spec_inputs(31 + bf16, L, N, H, D, bf16, B, T, 1)
    parent = torch.tensor([bfs_forest(2, T)] * B, dtype=torch.int32)   # depths 1..4
    layer = 1
    pool, out, ns, nc, ref, o_ref, ns_ref, nc_ref, e = _verify_both(
        ssm, conv, w, inp, slots, parent, 1, layer)
    used = set(slots.tolist())
    free = [s for s in range(1, N) if s not in used]
    track = torch.tensor(free[:2 * B], dtype=torch.int32).reshape(B, 2)
    track[5, 1] = 0                      # a masked track entry
    accepted = torch.tensor([-1, 0, 1, 14, 7, 13, 2, 10], dtype=torch.int32)
    before = torch.tensor([5, 6, 5, 2, 7, 15, 0, 14], dtype=torch.int32)
    nxt = torch.tensor([0, 1, 0, 1, 1, 1, 1, 0], dtype=torch.int32)
    gdn.gdn_accept_scatter(pool, layer, slots.cuda(), parent.cuda(), accepted.cuda(), ns, nc,
                           seq_len_before=before.cuda(), track_interval=3,
                           track_slots=track.cuda(), next_track_idx=nxt.cuda())
    ref0 = ref.copy()
    e2 = oracle.accept_scatter(ref, layer, slots.numpy(), parent.numpy(), accepted.numpy(), ns_ref,
                               nc_ref, seq_len_before=before.numpy(), track_interval=3,
                               track_slots=track.numpy(), next_track_idx=nxt.numpy())
    torch.cuda.synchronize()
    assert e2 == 0 and int(pool.err_word.item()) == 0
    gpu = pool_to_oracle(pool.ssm, pool.conv)
    want = _changed_slots(ref0, ref)
    got = _changed_slots(ref0, gpu)
    assert got == want and len(want) == 12, (sorted(got), sorted(want))
    # each written slot is a byte copy of one of the GPU's node buffers of its request
    nsb = ns.cpu().contiguous().view(torch.uint8).numpy().reshape(B, T, -1)
    ssb = gpu.ssm_bytes.reshape(L, N, -1)
    for b in range(B):
        s, n = int(slots[b]), int(accepted[b])
        if n >= 0:
            assert np.array_equal(ssb[layer, s], nsb[b, n])
            assert np.array_equal(gpu.conv()[layer, s], bf16_np(nc[b, n]))
    # the two crossings of request 3 (lengths 3 and 6): depth-1 node 0 to
    # track[(1 + 0) & 1], the accepted node 14 to track[(1 + 1) & 1]
    assert np.array_equal(ssb[layer, int(track[3, 1])], nsb[3, 0])
    assert np.array_equal(ssb[layer, int(track[3, 0])], nsb[3, 14])
    es = worst_unit_rel_l2(ssm_values(gpu)[layer], ssm_values(ref)[layer], 2)
    print(f"  worst slot rel-L2 after commit: {es:.2e}", flush=True)
    assert es <= REL_L2_TOL
    assert np.array_equal(gpu.conv(), ref.conv())


def test_accept_scatter_flags_bad_input():
    import gated_delta_rule_slot_amd as gdn
    print("accept scatter: bad input", flush=True)
    B, T, H, D, N = 3, 4, 2, 16, 12
    g, ssm, conv, w, inp, slots = _spec_inputs(41, 1, N, H, D, False, B, T, 0)
    parent = torch.tensor([[-1, 0, 1, 2]] * B, dtype=torch.int32)
    pool, out, ns, nc, ref, o_ref, ns_ref, nc_ref, e = _verify_both(
        ssm, conv, w, inp, slots, parent, 0, 0)
    snap = (pool.ssm.clone(), pool.conv.clone())
    bad_parent = parent.clone()
    bad_parent[1, 2] = 3
    gdn.gdn_accept_scatter(pool, 0, slots.cuda(), bad_parent.cuda(),
                           torch.tensor([3, 3, 4], dtype=torch.int32).cuda(), ns, nc)
    torch.cuda.synchronize()
    assert int(pool.err_word.item()) == gdn.ERRW_BAD_TREE
    # request 0 committed, 1 (bad tree) and 2 (accepted past the tree) untouched
    s = slots.tolist()
    assert torch.equal(pool.ssm[0, s[0]], ns[0, 3])
    assert torch.equal(pool.ssm[0, s[1]], snap[0][0, s[1]])
    assert torch.equal(pool.ssm[0, s[2]], snap[0][0, s[2]])
    pool.err_word.zero_()
    tr = torch.tensor([[N + 1, N + 2]] * B, dtype=torch.int32).cuda()
    gdn.gdn_accept_scatter(pool, 0, slots.cuda(), parent.cuda(),
                           torch.tensor([-1, 2, -1], dtype=torch.int32).cuda(), ns, nc,
                           seq_len_before=torch.tensor([0, 1, 0], dtype=torch.int32).cuda(),
                           track_interval=2, track_slots=tr,
                           next_track_idx=torch.zeros(B, dtype=torch.int32).cuda())
    torch.cuda.synchronize()
    assert int(pool.err_word.item()) == gdn.ERRW_BAD_TRACK_SLOT
    assert torch.equal(pool.ssm[0, s[1]], ns[1, 2])


@pytest.mark.timeout(600)
def test_verify_full_size_tree_every_unit():
    """The benchmark's draft-tree verify launch: 32 requests, a 63-node breadth-first
    tree of topk 4, 32 heads, K = V = 128, bf16 state, decay per head.  Every
    (request, node, head) unit of the launch is compared with the oracle, twice:

    * step by step: the oracle takes each node's token from the GPU's own stored
      parent state and conv rows (the live slot's for a root), as one decode step.
      This isolates the kernel's step; every unit must be within 2e-3.
    * end to end: the oracle walks the whole tree from the live slots.  Both sides
      round every node state to bf16 before its children read it, and where the
      GPU's fp32 and the oracle's fp64 values fall on two sides of a bf16 rounding
      boundary the two trees carry different parents from then on, so the
      difference grows with depth (worst output unit 4.1e-4, 1.2e-3 and 1.8e-3 at
      depths 1, 2 and 3).  Every unit must be within 2e-3.

    Conv rows of every node are bit-exact copies of inputs on both sides."""
    import gated_delta_rule_slot_amd as gdn
    print("verify: full-size tree launch, every unit", flush=True)
    B, T, H, D = 32, 63, 32, 128
    N, C = 1 + 3 * B, H * 3 * D
    g, ssm, conv, w, inp, slots = _spec_inputs(106, 1, N, H, D, True, B, T, 0)
    parent = torch.tensor([bfs_forest(4, T)] * B, dtype=torch.int32)
    x = inp["x"].reshape(B, T, C).contiguous()
    a = inp["alpha"].reshape(B, T, H).contiguous()
    bt = inp["beta"].reshape(B, T, H).contiguous()
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    pool = gdn.state_pool_create(ssm.cuda(), conv.cuda(), err)
    out = torch.empty((B, T, H, D), dtype=torch.bfloat16, device="cuda")
    ns = torch.empty((B, T, H, D, D), dtype=torch.bfloat16, device="cuda")
    nc = torch.empty((B, T, 3, C), dtype=torch.bfloat16, device="cuda")
    gdn.gdn_verify_tree(pool, 0, slots.cuda(), parent.cuda(), x.cuda(), w.cuda(), a.cuda(), 0, bt.cuda(),
                        out, ns, nc)
    torch.cuda.synchronize()
    assert int(err.item()) == 0
    assert torch.equal(pool.ssm.cpu(), ssm) and torch.equal(pool.conv.cpu(), conv)  # live slots only read
    out_h, ns_h, nc_h = bf16_np(out), bf16_np(ns), bf16_np(nc)
    par = parent[0].tolist()
    depth = np.array([1 if p < 0 else 0 for p in par])
    for n, p in enumerate(par):
        if p >= 0:
            depth[n] = depth[p] + 1

    # step by step: node (b, n) from the GPU's stored parent, one oracle decode step
    cond = oracle.Pool(1, 1 + B * T, H, D, D, oracle.SSM_BF16)
    ssm_b, conv_b = bf16_np(ssm), bf16_np(conv)
    pidx = np.array(par)
    for b in range(B):
        rows = slice(1 + b * T, 1 + (b + 1) * T)
        live = int(slots[b])
        cond.ssm()[0, rows] = np.where((pidx < 0)[:, None, None, None], ssm_b[0, live][None],
                                       ns_h[b, np.maximum(pidx, 0)])
        cond.conv()[0, rows] = np.where((pidx < 0)[:, None, None], conv_b[0, live][None],
                                        nc_h[b, np.maximum(pidx, 0)])
    o_c, e_c = oracle.decode_step(cond, 0, np.arange(1, 1 + B * T, dtype=np.int32),
                                  wl.bf16_bits(x).reshape(B * T, C), wl.bf16_bits(w),
                                  a.numpy().reshape(B * T, H), 0, bt.numpy().reshape(B * T, H))
    assert e_c == 0
    eo_c = unit_rel_l2(out_h.reshape(B * T, H, D), o_c, 2)
    es_c = unit_rel_l2(ns_h.reshape(B * T, H, D, D), cond.ssm()[0, 1:], 2)
    assert np.array_equal(nc_h.reshape(B * T, 3, C), cond.conv()[0, 1:])
    print(f"  step by step, all {B * T * H} units: worst out {eo_c.max():.2e}  state {es_c.max():.2e}",
          flush=True)
    del cond

    # end to end: the oracle's own tree walk from the live slots
    ref = pool_to_oracle(ssm, conv)
    o_ref, ns_ref, nc_ref, e = oracle.verify_tree(
        ref, 0, slots.numpy(), parent.numpy(), wl.bf16_bits(x), wl.bf16_bits(w), a.numpy(), 0,
        bt.numpy())
    assert e == 0
    assert np.array_equal(nc_h, nc_ref)
    eo = unit_rel_l2(out_h, o_ref, 3)            # [B, T, H]
    es = unit_rel_l2(ns_h, ns_ref, 3)
    del ns_ref
    worst = {}
    for d in sorted(set(depth.tolist())):
        sel = depth == d
        worst[d] = (float(eo[:, sel].max()), float(es[:, sel].max()))
        print(f"  end to end, depth {d} ({int(sel.sum())} nodes x {B} requests x {H} heads): "
              f"worst out {worst[d][0]:.2e}  state {worst[d][1]:.2e}", flush=True)
    assert eo_c.max() <= REL_L2_TOL and es_c.max() <= REL_L2_TOL
    for d, (wo, ws) in worst.items():
        assert wo <= REL_L2_TOL and ws <= REL_L2_TOL, (d, wo, ws)

    # the benchmark's commit of that launch (a depth-3 node per request, tracking every
    # 256; three requests cross a multiple of 256 at depths 1, 2 and 3): the pool must
    # equal, byte for byte, what the oracle's scatter makes of the GPU's node buffers
    used = set(slots.tolist())
    track = torch.tensor([s for s in range(1, N) if s not in used][:2 * B], dtype=torch.int32).reshape(B, 2)
    accepted = torch.randint(4 + 16, T, (B,), generator=g, dtype=torch.int32)
    before = torch.randint(256, 8192, (B,), generator=g, dtype=torch.int32)
    before[0], before[1], before[2] = 255, 510, 1021
    nxt = torch.zeros(B, dtype=torch.int32)
    ref2 = pool_to_oracle(pool.ssm, pool.conv)
    gdn.gdn_accept_scatter(pool, 0, slots.cuda(), parent.cuda(), accepted.cuda(), ns, nc,
                           seq_len_before=before.cuda(), track_interval=256, track_slots=track.cuda(),
                           next_track_idx=nxt.cuda())
    e3 = oracle.accept_scatter(ref2, 0, slots.numpy(), parent.numpy(), accepted.numpy(), ns_h,
                               nc_h, seq_len_before=before.numpy(), track_interval=256,
                               track_slots=track.numpy(), next_track_idx=nxt.numpy())
    torch.cuda.synchronize()
    assert e3 == 0 and int(err.item()) == 0
    assert pool_bytes_equal(pool.ssm, pool.conv, ref2)
    # the first crossing of requests 0..2 goes to track slot (next_track_idx + 0) & 1 = 0
    assert {(0, int(track[i, 0])) for i in range(3)} <= _changed_slots(pool_to_oracle(ssm, conv), ref2)
