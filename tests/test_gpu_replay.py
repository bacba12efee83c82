"""GPU parity of the ReplaySSM ring verify and exact-fold commit against the oracle.

Verify: outputs (bf16) as relative L2 per (request, position, head) unit,
tolerance 2e-3; the ring's k and v (bf16 roundings of conv outputs, which the two
sides may round one ulp apart) as relative L2 per unit; decay, beta and conv
input rows bit-exact; the live pool bit-exact untouched.  Commit: each side
folds its own ring; the slots written are the ones the oracle writes, states
within tolerance per (slot, head), conv rows bit-exact, everything else
untouched.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads as wl
from tests.helpers import (REL_L2_TOL, bf16_np, device_ssm_values, pool_to_oracle, ssm_values,
                           widen, worst_unit_rel_l2)

pytestmark = pytest.mark.gpu


def _setup(seed, L, N, H, D, bf16, B, T, amode):
    g = wl.generator(seed)
    ssm, conv = wl.warm_pool(g, L, N, H, D, D, bf16)
    w = wl.conv_weights(g, H * 3 * D)
    inp = wl.projected_inputs(g, B * T, H, D, D, amode)
    slots = wl.distinct_slots(g, B, N)
    return g, ssm, conv, w, inp, slots


def _verify_both(ssm, conv, w, inp, slots, B, T, P, amode, layer, scale=1.0, flags=1):
    import gated_delta_rule_slot_amd as gdn
    H, D = ssm.shape[2], ssm.shape[3]
    C = H * 3 * D
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    pool = gdn.state_pool_create(ssm.cuda(), conv.cuda(), err)
    ring = gdn.ReplayRing(pool, P, amode)
    out = torch.full((B, T, H, D), 7.0, dtype=torch.bfloat16, device="cuda")
    a = inp["alpha"].reshape(B, T, *inp["alpha"].shape[1:]).contiguous()
    bt = inp["beta"].reshape(B, T, H).contiguous()
    x = inp["x"].reshape(B, T, C).contiguous()
    gdn.replayssm_verify(pool, ring, layer, slots.cuda(), x.cuda(), w.cuda(), a.cuda(), bt.cuda(), out,
                         scale=scale, flags=flags)
    ref = pool_to_oracle(ssm, conv)
    rref = oracle.Ring(ref, P, amode)
    o_ref, e = oracle.replay_verify(ref, rref, layer, slots.numpy(), wl.bf16_bits(x), wl.bf16_bits(w),
                                    a.numpy(), amode, bt.numpy(), scale=scale, flags=flags)
    torch.cuda.synchronize()
    return pool, ring, out, ref, rref, o_ref, e


def _assert_ring(ring, rref, layer, slots, T):
    s = [int(v) for v in slots if 0 < int(v) < rref.rawk.shape[1]]
    for name in ("rawk", "rawv"):
        got = widen(bf16_np(getattr(ring, name)))[layer, s, :, :T]
        want = widen(getattr(rref, name))[layer, s, :, :T]
        e = worst_unit_rel_l2(got, want, 3)
        print(f"  ring {name} worst unit rel-L2 {e:.2e}", flush=True)
        assert e <= 1e-2   # a few one-ulp bf16 differences
    assert np.array_equal(ring.g.cpu().numpy()[layer, s][:, :, :T], rref.g[layer, s][:, :, :T])
    assert np.array_equal(ring.beta.cpu().numpy()[layer, s][:, :, :T], rref.beta[layer, s][:, :, :T])
    assert np.array_equal(bf16_np(ring.xrow)[layer, s, :T], rref.xrow[layer, s, :T])


@pytest.mark.parametrize("name,seed,L,N,H,D,bf16,B,T,P,amode", [
    ("D16 fp32 KDA", 61, 1, 10, 2, 16, False, 3, 4, 4, 1),
    ("D32 bf16 GDN", 62, 2, 24, 4, 32, True, 6, 5, 8, 0),
    ("D64 fp32 KDA", 63, 1, 30, 6, 64, False, 5, 3, 16, 1),
    ("D64 bf16 GDN", 64, 1, 30, 3, 64, True, 4, 6, 6, 0),
    ("D128 fp32 GDN", 65, 1, 40, 8, 128, False, 7, 4, 16, 0),
    ("D128 bf16 KDA", 66, 2, 40, 12, 128, True, 5, 7, 16, 1),
])
def test_replay_verify_parity(name, seed, L, N, H, D, bf16, B, T, P, amode):
    print(f"replay verify parity: {name}", flush=True)
    g, ssm, conv, w, inp, slots = _setup(seed, L, N, H, D, bf16, B, T, amode)
    layer = L - 1
    pool, ring, out, ref, rref, o_ref, e = _verify_both(ssm, conv, w, inp, slots, B, T, P, amode, layer,
                                                        scale=0.7)
    eo = worst_unit_rel_l2(widen(bf16_np(out)), widen(o_ref), 3)
    print(f"  worst unit rel-L2: out {eo:.2e}", flush=True)
    assert eo <= REL_L2_TOL and e == 0 and int(pool.err_word.item()) == 0
    _assert_ring(ring, rref, layer, slots.numpy(), T)
    assert torch.equal(pool.ssm.cpu(), ssm) and torch.equal(pool.conv.cpu(), conv)


# Drafts of up to 8 tokens at head dims 32..128 run the MFMA form of the verify
# (in two sizes: up to 4 and up to 8 tokens); longer drafts and head dim 16 run
# the token-by-token kernel.  Both against the same oracle.
@pytest.mark.parametrize("name,seed,H,D,bf16,B,T,P,amode,flags", [
    ("D64 bf16 KDA T1", 91, 4, 64, True, 3, 1, 4, 1, 1),
    ("D128 fp32 GDN T12 q-norm silu (token by token)", 92, 4, 128, False, 4, 12, 16, 0, 7),
    ("D128 bf16 KDA T16 (token by token)", 93, 12, 128, True, 5, 16, 16, 1, 1),
    ("D32 fp32 KDA T9 (token by token)", 94, 3, 32, False, 4, 9, 12, 1, 3),
    ("D128 bf16 KDA T8 q-norm", 95, 6, 128, True, 6, 8, 8, 1, 3),
    ("D128 fp32 GDN T5 q-norm silu", 90, 4, 128, False, 4, 5, 8, 0, 7),
    ("D32 fp32 KDA T2 q-norm", 89, 3, 32, False, 4, 2, 4, 1, 3),
    ("D128 bf16 KDA T24 (token by token)", 96, 4, 128, True, 3, 24, 32, 1, 1),
    ("D32 fp32 GDN T64 (token by token)", 97, 2, 32, False, 2, 64, 64, 0, 1),
    ("D16 bf16 KDA T6 (token by token)", 98, 3, 16, True, 4, 6, 8, 1, 1),
])
def test_replay_verify_forms(name, seed, H, D, bf16, B, T, P, amode, flags):
    print(f"replay verify: {name}", flush=True)
    N = 3 * B + 4
    g, ssm, conv, w, inp, slots = _setup(seed, 1, N, H, D, bf16, B, T, amode)
    pool, ring, out, ref, rref, o_ref, e = _verify_both(ssm, conv, w, inp, slots, B, T, P, amode, 0,
                                                        scale=0.8, flags=flags)
    eo = worst_unit_rel_l2(widen(bf16_np(out)), widen(o_ref), 3)
    print(f"  worst unit rel-L2: out {eo:.2e}", flush=True)
    assert eo <= REL_L2_TOL and e == 0 and int(pool.err_word.item()) == 0
    _assert_ring(ring, rref, 0, slots.numpy(), T)
    assert torch.equal(pool.ssm.cpu(), ssm) and torch.equal(pool.conv.cpu(), conv)


@pytest.mark.parametrize("D,T", [(128, 4), (128, 8), (128, 12), (16, 3)])
def test_replay_verify_skips_bad_slots(D, T):
    """Slot 0 and an id past the pool skip their request (zero outputs, bit 1 for
    the out-of-range id); the other requests match the oracle."""
    print(f"replay verify: bad slots, D {D}, T {T}", flush=True)
    import gated_delta_rule_slot_amd as gdn
    B, H, N = 5, 4, 20
    g, ssm, conv, w, inp, slots = _setup(99 + D + T, 1, N, H, D, True, B, T, 1)
    slots[1] = 0
    slots[3] = N + 5
    pool, ring, out, ref, rref, o_ref, e = _verify_both(ssm, conv, w, inp, slots, B, T, T, 1, 0)
    got = widen(bf16_np(out))
    assert int(pool.err_word.item()) == gdn.ERRW_BAD_SLOT
    assert not got[[1, 3]].any()
    good = [0, 2, 4]
    eo = worst_unit_rel_l2(got[good], widen(o_ref)[good], 3)
    print(f"  worst unit rel-L2 (valid requests): {eo:.2e}", flush=True)
    assert eo <= REL_L2_TOL


def _changed(before, after):
    L, N = before.ssm().shape[:2]
    sb = before.ssm_bytes.reshape(L, N, -1) != after.ssm_bytes.reshape(L, N, -1)
    cb = before.conv_bytes.reshape(L, N, -1) != after.conv_bytes.reshape(L, N, -1)
    return {(l, n) for l in range(L) for n in range(N) if sb[l, n].any() or cb[l, n].any()}


@pytest.mark.parametrize("bf16,amode", [(False, 1), (True, 0), (True, 1)])
def test_replay_commit_parity(bf16, amode):
    """Verify 6 draft tokens, then commit 0..6 of them per request, with tracking
    every 4 tokens: zero, one and two crossings, and a masked track entry."""
    import gated_delta_rule_slot_amd as gdn
    print(f"replay commit parity (bf16 {bf16}, alpha mode {amode})", flush=True)
    B, T, P, H, D, N, L = 8, 6, 8, 4, 64, 40, 2
    g, ssm, conv, w, inp, slots = _setup(71 + bf16 + 2 * amode, L, N, H, D, bf16, B, T, amode)
    layer = 1
    pool, ring, out, ref, rref, o_ref, e = _verify_both(ssm, conv, w, inp, slots, B, T, P, amode, layer)
    used = set(slots.tolist())
    free = [s for s in range(1, N) if s not in used]
    track = torch.tensor(free[:2 * B], dtype=torch.int32).reshape(B, 2)
    track[6, 0] = 0
    accepted = torch.tensor([0, 1, 2, 3, 4, 5, 6, 6], dtype=torch.int32)
    before = torch.tensor([5, 3, 2, 1, 7, 0, 2, 9], dtype=torch.int32)
    nxt = torch.tensor([0, 1, 1, 0, 1, 0, 0, 1], dtype=torch.int32)
    gdn.replayssm_commit(pool, ring, layer, slots.cuda(), accepted.cuda(), seq_len_before=before.cuda(),
                         track_interval=4, track_slots=track.cuda(), next_track_idx=nxt.cuda())
    ref0 = ref.copy()
    e2 = oracle.replay_commit(ref, rref, layer, slots.numpy(), accepted.numpy(), amode,
                              seq_len_before=before.numpy(), track_interval=4,
                              track_slots=track.numpy(), next_track_idx=nxt.numpy())
    torch.cuda.synchronize()
    assert e2 == 0 and int(pool.err_word.item()) == 0
    gpu = pool_to_oracle(pool.ssm, pool.conv)
    want, got = _changed(ref0, ref), _changed(ref0, gpu)
    assert got == want and len(want) >= 12, (sorted(got), sorted(want))
    es = worst_unit_rel_l2(ssm_values(gpu)[layer], ssm_values(ref)[layer], 2)
    print(f"  worst (slot, head) rel-L2 after commit: {es:.2e}", flush=True)
    assert es <= REL_L2_TOL
    assert np.array_equal(gpu.conv(), ref.conv())


def test_replay_commit_flags_bad_input():
    import gated_delta_rule_slot_amd as gdn
    print("replay commit: bad input", flush=True)
    B, T, P, H, D, N = 3, 2, 4, 2, 16, 12
    g, ssm, conv, w, inp, slots = _setup(81, 1, N, H, D, False, B, T, 1)
    pool, ring, out, ref, rref, o_ref, e = _verify_both(ssm, conv, w, inp, slots, B, T, P, 1, 0)
    snap = pool.ssm.clone()
    gdn.replayssm_commit(pool, ring, 0, slots.cuda(), torch.tensor([2, 5, -1], dtype=torch.int32).cuda())
    torch.cuda.synchronize()
    assert int(pool.err_word.item()) == gdn.ERRW_BAD_TREE
    s = slots.tolist()
    assert not torch.equal(pool.ssm[0, s[0]], snap[0, s[0]])
    assert torch.equal(pool.ssm[0, s[1]], snap[0, s[1]]) and torch.equal(pool.ssm[0, s[2]], snap[0, s[2]])
    pool.err_word.zero_()
    bad = slots.clone()
    bad[1] = N + 3
    gdn.replayssm_commit(pool, ring, 0, bad.cuda(), torch.tensor([0, 1, 1], dtype=torch.int32).cuda(),
                         seq_len_before=torch.zeros(B, dtype=torch.int32).cuda(), track_interval=1,
                         track_slots=torch.full((B, 2), N + 1, dtype=torch.int32).cuda(),
                         next_track_idx=torch.zeros(B, dtype=torch.int32).cuda())
    torch.cuda.synchronize()
    assert int(pool.err_word.item()) == gdn.ERRW_BAD_SLOT | gdn.ERRW_BAD_TRACK_SLOT


def test_replay_full_size_round():
    """The benchmark's ReplaySSM launches on one layer of the KDA pool (12 heads,
    K = V = 128, bf16 state, 1024 slots, per-channel decay): verify of 4-token
    draft chains for 256 requests into a 16-position ring, then the commit of 1..4
    accepted tokens with tracking every 256 (request 137's replay crosses 1024 at
    its second token).  Every request is checked against the oracle: all outputs
    per (request, token, head) unit, then the whole pool after the commit (the
    same slots written, states within tolerance, conv rows bit-exact)."""
    import gated_delta_rule_slot_amd as gdn
    print("replay: full-size round, every request", flush=True)
    H, D, N, B, T, P, amode = 12, 128, 1024, 256, 4, 16, 1
    C = H * 3 * D
    g, ssm, conv, w, inp, _ = _setup(107, 1, N, H, D, True, B, T, amode)
    ids = wl.distinct_slots(g, 3 * B, N)
    slots, track = ids[:B].contiguous(), ids[B:].reshape(B, 2).contiguous()
    accepted = torch.randint(1, T + 1, (B,), generator=g, dtype=torch.int32)
    before = torch.randint(256, 8192, (B,), generator=g, dtype=torch.int32)
    nxt = torch.randint(0, 2, (B,), generator=g, dtype=torch.int32)
    accepted[137], before[137] = 4, 1022   # the replay reaches 1024 at its second token
    x = inp["x"].reshape(B, T, C).contiguous()
    a = inp["alpha"].reshape(B, T, H, D).contiguous()
    bt = inp["beta"].reshape(B, T, H).contiguous()
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    pool = gdn.state_pool_create(ssm.cuda(), conv.cuda(), err)
    ring = gdn.ReplayRing(pool, P, amode)
    out = torch.empty((B, T, H, D), dtype=torch.bfloat16, device="cuda")
    gdn.replayssm_verify(pool, ring, 0, slots.cuda(), x.cuda(), w.cuda(), a.cuda(), bt.cuda(), out)
    gdn.replayssm_commit(pool, ring, 0, slots.cuda(), accepted.cuda(), seq_len_before=before.cuda(),
                         track_interval=256, track_slots=track.cuda(), next_track_idx=nxt.cuda())
    torch.cuda.synchronize()
    assert int(err.item()) == 0

    ref = pool_to_oracle(ssm, conv)
    rref = oracle.Ring(ref, P, amode)
    o_ref, e = oracle.replay_verify(ref, rref, 0, slots.numpy(), wl.bf16_bits(x), wl.bf16_bits(w),
                                    a.numpy(), amode, bt.numpy())
    assert e == 0
    eo = worst_unit_rel_l2(widen(bf16_np(out)), widen(o_ref), 3)
    ref0 = ref.copy()
    e2 = oracle.replay_commit(ref, rref, 0, slots.numpy(), accepted.numpy(), amode,
                              seq_len_before=before.numpy(), track_interval=256,
                              track_slots=track.numpy(), next_track_idx=nxt.numpy())
    assert e2 == 0
    gpu = pool_to_oracle(pool.ssm, pool.conv)
    want_changed = _changed(ref0, ref)
    assert _changed(ref0, gpu) == want_changed
    assert {(0, int(s)) for s in slots} <= want_changed and len(want_changed) > B  # + track slots
    es = worst_unit_rel_l2(widen(gpu.ssm()[0]), widen(ref.ssm()[0]), 2)
    print(f"  worst unit rel-L2 over {B} requests: out {eo:.2e}  pool state {es:.2e} "
          f"({len(want_changed) - B} snapshots)", flush=True)
    assert eo <= REL_L2_TOL and es <= REL_L2_TOL
    assert np.array_equal(gpu.conv(), ref.conv())
