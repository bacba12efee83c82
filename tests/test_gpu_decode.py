"""GPU parity of gdn_decode_step against the oracle.

Outputs are compared as bf16 (GPU) against the oracle's bf16-rounded outputs,
states in the pool dtype, each as relative L2 per (request, head) unit
(tolerance 2e-3); conv rows, slot selection and untouched slots bit-exact.
"""
import json
import os

import numpy as np
import pytest
import torch

import oracle
import workloads as wl
from tests.helpers import (REL_L2_TOL, bf16_np, device_ssm_values, pool_to_oracle, ssm_values,
                           widen, worst_unit_rel_l2)

pytestmark = pytest.mark.gpu


def _setup(seed, L, N, H, D, bf16, B, alpha_mode):
    g = wl.generator(seed)
    ssm, conv = wl.warm_pool(g, L, N, H, D, D, bf16)
    w = wl.conv_weights(g, H * 3 * D)
    inp = wl.projected_inputs(g, B, H, D, D, alpha_mode)
    slots = wl.distinct_slots(g, B, N)
    return ssm, conv, w, inp, slots


def _run_both(ssm, conv, w, inp, slots, alpha_mode, layer=0, scale=1.0, flags=1,
              seq_len_after=None, interval=0, track=None, nxt=None):
    import gated_delta_rule_slot_amd as gdn
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    pool = gdn.state_pool_create(ssm.cuda(), conv.cuda(), err)
    B = slots.numel()
    H, D = ssm.shape[2], ssm.shape[3]
    out = torch.empty(B, H, D, dtype=torch.bfloat16, device="cuda")
    dev = lambda t: None if t is None else t.cuda()
    gdn.gdn_decode_step(pool, layer, dev(slots), dev(inp["x"]), dev(w), dev(inp["alpha"]),
                        alpha_mode, dev(inp["beta"]), out, scale=scale, flags=flags,
                        seq_len_after=dev(seq_len_after), track_interval=interval,
                        track_slots=dev(track), next_track_idx=dev(nxt))
    ref = pool_to_oracle(ssm, conv)
    o_ref, e = oracle.decode_step(
        ref, layer, slots.numpy(), wl.bf16_bits(inp["x"]), wl.bf16_bits(w), inp["alpha"].numpy(),
        alpha_mode, inp["beta"].numpy(), scale=scale, flags=flags,
        seq_len_after=None if seq_len_after is None else seq_len_after.numpy(),
        track_interval=interval, track_slots=None if track is None else track.numpy(),
        next_track_idx=None if nxt is None else nxt.numpy())
    torch.cuda.synchronize()
    return pool, out, ref, o_ref, e


def _assert_parity(pool, out, ref, o_ref, layer, live, extra_written=()):
    got_o = widen(bf16_np(out))
    want_o = widen(o_ref)
    eo = worst_unit_rel_l2(got_o, want_o, 2)
    gs, ws = device_ssm_values(pool.ssm), ssm_values(ref)
    written = list(live) + list(extra_written)
    es = worst_unit_rel_l2(gs[layer, written], ws[layer, written], 2)
    print(f"  worst unit rel-L2: out {eo:.2e}  state {es:.2e}", flush=True)
    assert eo <= REL_L2_TOL and es <= REL_L2_TOL
    # conv rows are byte copies of inputs: exact
    assert np.array_equal(bf16_np(pool.conv), ref.conv())
    # every other slot untouched (bit-exact)
    mask = np.ones(gs.shape[:2], bool)
    mask[layer, written] = False
    a = pool.ssm.cpu().contiguous().view(torch.uint8).numpy().reshape(gs.shape[0], gs.shape[1], -1)
    b = ref.ssm_bytes.reshape(gs.shape[0], gs.shape[1], -1)
    assert np.array_equal(a[mask], b[mask])


@pytest.mark.parametrize("name,seed,L,N,H,D,bf16,B,amode", [
    ("tiny D16 fp32 KDA", 1, 1, 8, 2, 16, False, 3, 1),
    ("D32 bf16 GDN", 2, 2, 30, 4, 32, True, 9, 0),
    ("D64 fp32 KDA", 3, 1, 40, 6, 64, False, 17, 1),
    ("D128 fp32 GDN", 4, 1, 64, 8, 128, False, 33, 0),
    ("D128 bf16 KDA", 5, 3, 64, 12, 128, True, 20, 1),
    ("D128 bf16 KDA every slot live", 6, 1, 600, 3, 128, True, 599, 1),
])
def test_decode_parity(name, seed, L, N, H, D, bf16, B, amode):
    print(f"decode parity: {name}", flush=True)
    ssm, conv, w, inp, slots = _setup(seed, L, N, H, D, bf16, B, amode)
    layer = L - 1
    pool, out, ref, o_ref, e = _run_both(ssm, conv, w, inp, slots, amode, layer=layer, scale=0.75)
    _assert_parity(pool, out, ref, o_ref, layer, slots.numpy())
    assert int(pool.err_word.item()) == 0 and e == 0


def test_decode_full_size_gdn_config():
    """The 32-head, K=V=128 decode step on a 512-slot fp32 pool, batch 128, checked in full."""
    cfg = wl.GDN_DECODE
    print("decode parity: full GDN decode workload", flush=True)
    ssm, conv, w, inp, slots = _setup(cfg.seed, 1, cfg.slots, cfg.heads, cfg.head_k, False, 128,
                                      cfg.alpha_mode)
    pool, out, ref, o_ref, e = _run_both(ssm, conv, w, inp, slots, cfg.alpha_mode)
    _assert_parity(pool, out, ref, o_ref, 0, slots.numpy())


def test_decode_tracking_snapshots():
    """Requests whose length reaches a multiple of 256 also write the track slot
    named by next_track_idx; others do not."""
    print("decode tracking", flush=True)
    H, D, B, N = 4, 128, 12, 64
    ssm, conv, w, inp, slots = _setup(9, 1, N, H, D, True, B, 1)
    g = wl.generator(10)
    free = [s for s in range(1, N) if s not in set(slots.tolist())]
    track = torch.tensor(free[:2 * B], dtype=torch.int32).reshape(B, 2)
    nxt = torch.randint(0, 2, (B,), generator=g, dtype=torch.int32)
    seq = torch.tensor([256 * (i + 1) if i % 3 == 0 else 256 * i + 17 for i in range(B)],
                       dtype=torch.int32)
    track[1, 0] = 0   # a masked track entry: no snapshot even at the boundary
    pool, out, ref, o_ref, e = _run_both(ssm, conv, w, inp, slots, 1, seq_len_after=seq,
                                         interval=256, track=track, nxt=nxt)
    hit = [int(track[i, int(nxt[i])]) for i in range(B)
           if seq[i] % 256 == 0 and int(track[i, int(nxt[i])]) > 0]
    assert len(hit) >= 3
    _assert_parity(pool, out, ref, o_ref, 0, slots.numpy(), extra_written=hit)
    # the snapshot is the updated live state, byte for byte
    for i in range(B):
        t = int(track[i, int(nxt[i])])
        if seq[i] % 256 == 0 and t > 0:
            assert torch.equal(pool.ssm[0, t], pool.ssm[0, int(slots[i])])
            assert torch.equal(pool.conv[0, t], pool.conv[0, int(slots[i])])


def test_decode_full_size_kda_tracking_config():
    """One layer of the 69-layer KDA decode in its launch configuration: 12 heads,
    K=V=128, bf16 pool of 1024 slots, batch 256, per-channel decay, tracking every
    256 tokens into ping-pong track slots with lengths ~ U[256, 8192) (about one
    request in 256 reaches a boundary; some are forced to), checked in full."""
    cfg = wl.KDA_DECODE
    print("decode parity: full KDA decode-with-tracking layer", flush=True)
    B, N = 256, cfg.slots
    ssm, conv, w, inp, slots = _setup(cfg.seed, 1, N, cfg.heads, cfg.head_k, True, B, cfg.alpha_mode)
    g = wl.generator(cfg.seed + 1)
    free = [s for s in range(1, N) if s not in set(slots.tolist())]
    track = torch.tensor(free[:2 * B], dtype=torch.int32).reshape(B, 2)
    nxt = torch.randint(0, 2, (B,), generator=g, dtype=torch.int32)
    seq = torch.randint(256, 8192, (B,), generator=g, dtype=torch.int32)
    seq[::16] = 256 * torch.randint(1, 32, (B // 16,), generator=g, dtype=torch.int32)
    pool, out, ref, o_ref, e = _run_both(ssm, conv, w, inp, slots, cfg.alpha_mode, seq_len_after=seq,
                                         interval=256, track=track, nxt=nxt)
    hit = [int(track[i, int(nxt[i])]) for i in range(B) if seq[i] % 256 == 0]
    assert len(hit) >= 16
    _assert_parity(pool, out, ref, o_ref, 0, slots.numpy(), extra_written=hit)
    assert e == 0 and int(pool.err_word.item()) == 0


def test_decode_skips_reserved_and_bad_slots():
    print("decode slot skipping", flush=True)
    H, D, B, N = 2, 64, 4, 16
    ssm, conv, w, inp, slots = _setup(11, 1, N, H, D, False, B, 0)
    slots = torch.tensor([0, 5, -3, 16], dtype=torch.int32)
    pool, out, ref, o_ref, e = _run_both(ssm, conv, w, inp, slots, 0)
    assert e == 1 and (int(pool.err_word.item()) & 1)
    o = bf16_np(out)
    assert not o[[0, 2, 3]].any()
    _assert_parity(pool, out, ref, o_ref, 0, [5])


def test_hand_worked_step_bitexact_on_gpu(golden_dir):
    """The 2x2 hand-worked step, embedded in a 16-dim head (zero padding), is
    reproduced bit-exactly by the decode kernel."""
    import gated_delta_rule_slot_amd as gdn
    case = json.load(open(os.path.join(golden_dir, "rank1_step_2x2.json")))
    D = 16
    ssm = torch.zeros(1, 2, 1, D, D)
    ssm[0, 1, 0, :2, :2] = torch.tensor(case["S0"], dtype=torch.float32)
    conv = torch.zeros(1, 2, 3, 3 * D, dtype=torch.bfloat16)
    w = torch.zeros(3 * D, 4)
    w[:, 3] = 1.0
    x = torch.zeros(1, 3 * D)
    x[0, 0:2] = torch.tensor(case["q"], dtype=torch.float32)
    x[0, D:D + 2] = torch.tensor(case["k"], dtype=torch.float32)
    x[0, 2 * D:2 * D + 2] = torch.tensor(case["v"], dtype=torch.float32)
    alpha = torch.ones(1, 1, D)
    alpha[0, 0, :2] = torch.tensor(case["alpha"])
    beta = torch.tensor([[case["beta"]]], dtype=torch.float32)
    pool = gdn.state_pool_create(ssm.cuda(), conv.cuda())
    out = torch.empty(1, 1, D, dtype=torch.bfloat16, device="cuda")
    gdn.gdn_decode_step(pool, 0, torch.tensor([1], dtype=torch.int32).cuda(),
                        x.to(torch.bfloat16).cuda(), w.to(torch.bfloat16).cuda(), alpha.cuda(),
                        gdn.ALPHA_PER_CHANNEL, beta.cuda(), out, scale=1.0, flags=0)
    torch.cuda.synchronize()
    S1 = pool.ssm[0, 1, 0].cpu()
    assert torch.equal(S1[:2, :2], torch.tensor(case["S1"], dtype=torch.float32))
    assert not S1[2:].any() and not S1[:, 2:].any()
    assert out[0, 0, :2].float().cpu().tolist() == case["o"]


def test_decode_extreme_decay_finite():
    print("decode extreme decay", flush=True)
    H, D, B, N = 4, 128, 8, 20
    ssm, conv, w, inp, slots = _setup(12, 1, N, H, D, False, B, 1)
    inp["alpha"][:, :, :32] = 1e-3
    inp["alpha"][:, 1, :] = 1e-30
    pool, out, ref, o_ref, e = _run_both(ssm, conv, w, inp, slots, 1)
    assert torch.isfinite(out.float()).all() and torch.isfinite(pool.ssm).all()
    _assert_parity(pool, out, ref, o_ref, 0, slots.numpy())
