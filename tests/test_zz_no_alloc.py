"""GPU: the allocation-free prefill entry point against the workspace entry point.

conv_gdn_prefill_chunked_noalloc runs the same kernels as conv_gdn_prefill_chunked
in the library's fixed per-device scratch (the two-kernel path in windows of as
many chunks as the scratch holds; the one-kernel paths, for a decay per head and per
channel, need no scratch).  Windows
leave the result bit-identical, so each call is compared bit for bit with the
workspace entry point on an identical pool (outputs, every slot's state and conv
rows), and with the oracle to the stated tolerance.  Two calls run in a row, the
second with a smaller input, so the second starts on the scratch contents the
first left behind.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads as wl
from tests.helpers import REL_L2_TOL, bf16_np, pool_to_oracle, widen, worst_unit_rel_l2

pytestmark = pytest.mark.gpu


def _inputs(seed, H, D, lens, amode, bf16, N):
    g = wl.generator(seed)
    ssm, conv = wl.warm_pool(g, 1, N, H, D, D, bf16)
    w = wl.conv_weights(g, 3 * H * D)
    inp = wl.projected_inputs(g, sum(lens), H, D, D, amode)
    perm = (torch.randperm(N - 1, generator=g) + 1).to(torch.int32)
    B = len(lens)
    slots, track = perm[:B].contiguous(), perm[B:3 * B].reshape(B, 2).contiguous()
    warm = torch.randint(0, 2, (B,), generator=g, dtype=torch.int32)
    start = (64 * torch.randint(0, 4, (B,), generator=g, dtype=torch.int32)) * warm
    nxt = torch.randint(0, 2, (B,), generator=g, dtype=torch.int32)
    return dict(ssm=ssm, conv=conv, w=w, inp=inp, cu=wl.cu_seqlens(lens), slots=slots, track=track,
                warm=warm, start=start, nxt=nxt, lens=lens, H=H, D=D, amode=amode)


def _run(c, noalloc, snap, flags=1):
    import gated_delta_rule_slot_amd as gdn
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    pool = gdn.state_pool_create(c["ssm"].cuda(), c["conv"].cuda(), err)
    T = int(c["cu"][-1])
    out = torch.full((T, c["H"], c["D"]), -7.0, dtype=torch.bfloat16, device="cuda")
    args = (pool, 0, c["cu"].cuda(), c["slots"].cuda(), c["warm"].cuda(), c["inp"]["x"].cuda(),
            c["w"].cuda(), c["inp"]["alpha"].cuda(), c["amode"], c["inp"]["beta"].cuda(), out,
            max(c["lens"]))
    kw = dict(start_len=c["start"].cuda(), snap_interval=snap, track_slots=c["track"].cuda(),
              next_track_idx=c["nxt"].cuda(), flags=flags)
    if noalloc:
        gdn.conv_gdn_prefill_chunked_noalloc(*args, **kw)
    else:
        ws = torch.empty(gdn.gdn_prefill_workspace_bytes(pool, len(c["lens"]), max(c["lens"])),
                         dtype=torch.uint8, device="cuda")
        gdn.conv_gdn_prefill_chunked(*args, workspace=ws, **kw)
    torch.cuda.synchronize()
    assert int(err.item()) == 0
    return pool, out


def _check_against_oracle(c, pool, out, snap):
    ref = pool_to_oracle(c["ssm"], c["conv"])
    o_ref, e = oracle.prefill(ref, 0, c["cu"].numpy(), c["slots"].numpy(), wl.bf16_bits(c["inp"]["x"]),
                              wl.bf16_bits(c["w"]), c["inp"]["alpha"].numpy(), c["amode"],
                              c["inp"]["beta"].numpy(), has_initial_state=c["warm"].numpy(),
                              start_len=c["start"].numpy(), snap_interval=snap,
                              track_slots=c["track"].numpy(), next_track_idx=c["nxt"].numpy())
    assert e == 0
    H, D = c["H"], c["D"]
    go, wo = widen(bf16_np(out)), widen(o_ref)
    eo = 0.0
    for b in range(len(c["lens"])):
        s0, s1 = int(c["cu"][b]), int(c["cu"][b + 1])
        if s1 > s0:
            eo = max(eo, worst_unit_rel_l2(go[s0:s1].transpose(1, 0, 2), wo[s0:s1].transpose(1, 0, 2), 1))
    gs = pool.ssm.cpu().to(torch.float64).numpy()[0]
    ws = ref.ssm()[0].astype(np.float64) if ref.ssm_dtype == oracle.SSM_F32 else widen(ref.ssm()[0])
    es = worst_unit_rel_l2(gs, ws, 2)
    assert np.array_equal(bf16_np(pool.conv), ref.conv())
    return eo, es


@pytest.mark.timeout(300)
def test_noalloc_prefill_matches_workspace_entry_on_two_calls():
    import gated_delta_rule_slot_amd as gdn
    # call 1: 12 KDA heads, bf16 pool, 3 requests up to 3000 tokens with snapshots
    # every 64: 36 (request, head) units take the two-kernel path, and the 64 MiB
    # scratch holds 12 chunks of records per window, so the call runs in 4 windows
    # call 2: a smaller input on the same scratch, 1 request of 300 tokens
    # call 3: a GDN batch of 128 units on the one-kernel path (no scratch)
    # call 4: a KDA batch of 132 units on the one-kernel path (no scratch)
    calls = [
        ("two-kernel, windows", _inputs(71, 12, 128, [3000, 1700, 64], 1, True, 16), 64),
        ("two-kernel, smaller", _inputs(72, 12, 128, [300], 1, True, 8), 64),
        ("one-kernel", _inputs(73, 4, 128, [200] * 32, 0, False, 100), 128),
        ("one-kernel, KDA", _inputs(75, 12, 128, [150, 64, 1, 200, 90, 65, 130, 7, 64, 300, 40], 1, True, 40), 64),
    ]
    for name, c, snap in calls:
        print(f"no-alloc prefill: {name}", flush=True)
        p_ref, o_ref = _run(c, False, snap)
        p_na, o_na = _run(c, True, snap)
        assert torch.equal(o_na, o_ref)
        assert torch.equal(p_na.ssm, p_ref.ssm) and torch.equal(p_na.conv, p_ref.conv)
        eo, es = _check_against_oracle(c, p_na, o_na, snap)
        print(f"  bit-identical to the workspace entry; oracle worst unit rel-L2 out {eo:.2e} "
              f"state {es:.2e}", flush=True)
        assert eo <= REL_L2_TOL and es <= REL_L2_TOL
    # a two-kernel batch beyond the scratch is refused before any launch (the batch
    # would take the one-kernel path by default, which needs no scratch; the path is
    # forced)
    c = _inputs(74, 12, 128, [64] * 400, 1, True, 1300)
    with pytest.raises(gdn.GdnError, match="scratch"):
        _run(c, True, 0, flags=1 | gdn.PREFILL_TWO_KERNEL)
