"""GPU parity of conv_gdn_prefill_chunked against the oracle.

Outputs: GPU bf16 against the oracle's bf16-rounded outputs; states: in the pool
dtype; both as relative L2 per (request, head) unit, tolerance 2e-3.  Conv rows,
snapshot placement and untouched slots: bit-exact.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads as wl
from tests.helpers import (REL_L2_TOL, bf16_np, device_ssm_values, output_unit_ok, pool_to_oracle,
                           ssm_values, widen, worst_unit_rel_l2)

pytestmark = pytest.mark.gpu


class Case:
    def __init__(self, seed, H, D, lens, bf16=False, amode=1, slots=None, N=None, L=1,
                 warm=None, start=None, flags=1, scale=1.0, snap=0, path=0):
        g = wl.generator(seed)
        self.path = path  # GDN_F_PREFILL_* bit passed to the library only
        B = len(lens)
        self.H, self.D, self.lens, self.amode, self.flags, self.scale = H, D, lens, amode, flags, scale
        self.L = L
        self.layer = L - 1
        self.N = N or (3 * B + 2)
        self.ssm, self.conv = wl.warm_pool(g, L, self.N, H, D, D, bf16)
        self.w = wl.conv_weights(g, 3 * H * D)
        self.inp = wl.projected_inputs(g, max(sum(lens), 1), H, D, D, amode)
        self.cu = wl.cu_seqlens(lens)
        perm = torch.randperm(self.N - 1, generator=g) + 1
        self.slots = (perm[:B] if slots is None else torch.tensor(slots)).to(torch.int32)
        self.track = perm[B:3 * B].reshape(B, 2).to(torch.int32).contiguous()
        self.nxt = torch.randint(0, 2, (B,), generator=g, dtype=torch.int32)
        self.warm = torch.tensor(warm if warm is not None else [1] * B, dtype=torch.int32)
        self.start = torch.tensor(start if start is not None else [0] * B, dtype=torch.int32)
        self.snap = snap

    def run_gpu(self, workspace_bytes=None):
        import gated_delta_rule_slot_amd as gdn
        err = torch.zeros(1, dtype=torch.int32, device="cuda")
        pool = gdn.state_pool_create(self.ssm.cuda(), self.conv.cuda(), err)
        T = int(self.cu[-1])
        out = torch.full((max(T, 1), self.H, self.D), -7.0, dtype=torch.bfloat16, device="cuda")
        maxlen = max(self.lens) if self.lens else 0
        need = gdn.gdn_prefill_workspace_bytes(pool, len(self.lens), maxlen)
        ws = torch.empty(workspace_bytes or need, dtype=torch.uint8, device="cuda")
        gdn.conv_gdn_prefill_chunked(
            pool, self.layer, self.cu.cuda(), self.slots.cuda(), self.warm.cuda(),
            self.inp["x"].cuda(), self.w.cuda(), self.inp["alpha"].cuda(), self.amode,
            self.inp["beta"].cuda(), out, maxlen, start_len=self.start.cuda(), scale=self.scale,
            flags=self.flags | self.path, snap_interval=self.snap, track_slots=self.track.cuda(),
            next_track_idx=self.nxt.cuda(), workspace=ws)
        torch.cuda.synchronize()
        return pool, out[:T]

    def run_oracle(self, exact=False):
        ref = pool_to_oracle(self.ssm, self.conv)
        res = oracle.prefill(
            ref, self.layer, self.cu.numpy(), self.slots.numpy(), wl.bf16_bits(self.inp["x"]),
            wl.bf16_bits(self.w), self.inp["alpha"].numpy(), self.amode, self.inp["beta"].numpy(),
            has_initial_state=self.warm.numpy(), start_len=self.start.numpy(), scale=self.scale,
            flags=self.flags, snap_interval=self.snap,
            track_slots=self.track.numpy() if self.snap else None,
            next_track_idx=self.nxt.numpy() if self.snap else None, exact=exact)
        if exact:
            o, e, oe, _ = res
            return ref, o, e, oe
        o, e = res
        return ref, o, e

    def written_slots(self):
        s = [int(v) for v in self.slots if 0 < int(v) < self.N]
        if self.snap:
            for b, n in enumerate(self.lens):
                if not (0 < int(self.slots[b]) < self.N):
                    continue
                st = int(self.start[b])
                if any((st + i + 1) % self.snap == 0 for i in range(n)):
                    s += [int(v) for v in self.track[b] if 0 < int(v) < self.N]
        return sorted(set(s))


def check(case, pool, out, ref, o_ref, tol=REL_L2_TOL, o_exact=None):
    """Outputs per (request, head) unit, states per (slot, head) unit, conv rows and
    untouched slots.  With o_exact (the oracle's f64 outputs) an output unit may
    also pass as a set of valid bf16 roundings (helpers.output_unit_ok)."""
    T = int(case.cu[-1])
    go = widen(bf16_np(out)).reshape(T, case.H, case.D)
    wo = widen(o_ref).reshape(T, case.H, case.D)
    eo = 0.0
    for b in range(len(case.lens)):   # units: (request, head)
        s0, s1 = int(case.cu[b]), int(case.cu[b + 1])
        if s1 <= s0:
            continue
        if o_exact is None:
            eo = max(eo, worst_unit_rel_l2(go[s0:s1].transpose(1, 0, 2), wo[s0:s1].transpose(1, 0, 2), 1))
            continue
        gb = bf16_np(out).reshape(T, case.H, case.D)
        wb = np.asarray(o_ref).reshape(T, case.H, case.D)
        ex = np.asarray(o_exact).reshape(T, case.H, case.D)
        for h in range(case.H):
            ok, stated, excess = output_unit_ok(gb[s0:s1, h], wb[s0:s1, h], ex[s0:s1, h], tol)
            if stated > tol:
                print(f"  request {b} head {h}: bf16 outputs {stated:.2e} apart; excess over the "
                      f"rounding of the exact outputs {excess:.2e}, valid roundings: {ok}", flush=True)
            assert ok, (b, h, stated, excess)
            eo = max(eo, min(stated, tol))
    written = case.written_slots()
    gs, ws = device_ssm_values(pool.ssm), ssm_values(ref)
    es = worst_unit_rel_l2(gs[case.layer, written], ws[case.layer, written], 2) if written else 0.0
    print(f"  worst unit rel-L2: out {eo:.2e}  state {es:.2e}", flush=True)
    assert np.all(np.isfinite(widen(bf16_np(out))))
    assert np.all(np.isfinite(gs[case.layer, written]))
    assert eo <= tol, eo
    assert es <= tol, es
    assert np.array_equal(bf16_np(pool.conv), ref.conv()), "conv rows differ"
    L, N = gs.shape[:2]
    mask = np.ones((L, N), bool)
    mask[case.layer, written] = False
    a = pool.ssm.cpu().contiguous().view(torch.uint8).numpy().reshape(L, N, -1)
    b = ref.ssm_bytes.reshape(L, N, -1)
    assert np.array_equal(a[mask], b[mask]), "a slot that the call does not name changed"
    return eo, es


@pytest.mark.parametrize("name,kw", [
    ("tiny D16 fp32 KDA, snapshots every 64", dict(seed=101, H=2, D=16, lens=[256, 256], snap=64,
                                                   warm=[0, 0], N=8)),
    ("D32 bf16 GDN ragged", dict(seed=3, H=3, D=32, lens=[1, 63, 64, 65, 130], bf16=True, amode=0)),
    ("D64 fp32 KDA warm/cold", dict(seed=4, H=4, D=64, lens=[200, 7, 129], warm=[1, 0, 1],
                                    scale=0.5)),
    ("D128 bf16 KDA snapshots, unaligned start", dict(seed=5, H=4, D=128, lens=[300, 70, 2],
                                                      bf16=True, snap=64, start=[64, 37, 126],
                                                      warm=[1, 1, 1])),
    ("D128 fp32 GDN silu + q norm", dict(seed=6, H=6, D=128, lens=[190, 64], amode=0, flags=7)),
    ("D128 empty and bad slots", dict(seed=7, H=2, D=128, lens=[0, 40, 0, 33], slots=[3, 0, 4, 5],
                                      warm=[1, 1, 0, 1], N=14)),
])
def test_prefill_parity(name, kw):
    print(f"prefill parity: {name}", flush=True)
    case = Case(**kw)
    pool, out = case.run_gpu()
    ref, o_ref, e = case.run_oracle()
    check(case, pool, out, ref, o_ref)
    assert int(pool.err_word.item()) == 0


ONE, TWO = 8, 16  # GDN_F_PREFILL_ONE_KERNEL, GDN_F_PREFILL_TWO_KERNEL

GDN_CASES = [
    ("fp32 ragged warm/cold, scale", dict(seed=11, H=3, D=128, lens=[1, 63, 64, 65, 130, 200],
                                          amode=0, warm=[1, 0, 1, 1, 0, 1], scale=0.5)),
    ("bf16 snapshots, unaligned start", dict(seed=12, H=4, D=128, lens=[300, 70, 2, 129],
                                             bf16=True, amode=0, snap=64,
                                             start=[64, 37, 126, 0], warm=[1, 1, 1, 0])),
    ("fp32 silu + q norm", dict(seed=13, H=5, D=128, lens=[190, 64, 17], amode=0, flags=7)),
    ("empty and bad slots", dict(seed=14, H=2, D=128, lens=[0, 40, 0, 33, 5],
                                 slots=[3, 0, 4, 5, 20], warm=[1, 1, 0, 1, 1], N=20, amode=0)),
    ("snapshots every 128 across several chunks", dict(seed=15, H=2, D=128, lens=[640, 333],
                                                       amode=0, snap=128, start=[0, 192],
                                                       warm=[0, 1])),
]


@pytest.mark.parametrize("path", [ONE, TWO], ids=["one-kernel", "two-kernel"])
@pytest.mark.parametrize("name,kw", GDN_CASES, ids=[c[0] for c in GDN_CASES])
def test_prefill_gdn_paths_parity(name, kw, path):
    """Decay per head at head dim 128: each prefill path against the oracle."""
    print(f"prefill GDN parity ({'one' if path == ONE else 'two'}-kernel): {name}", flush=True)
    case = Case(path=path, **kw)
    pool, out = case.run_gpu()
    ref, o_ref, e = case.run_oracle()
    check(case, pool, out, ref, o_ref)
    assert int(pool.err_word.item()) == e


def test_prefill_one_kernel_extreme_decay():
    """Decays of 1e-3, 1e-20 and exactly 0 on the one-kernel path: finite and
    matching (every decay factor is applied as a number <= 1)."""
    print("prefill one-kernel extreme decay", flush=True)
    case = Case(seed=16, H=3, D=128, lens=[150, 64, 100], amode=0, path=ONE)
    case.inp["alpha"][:, 0] = 1e-3
    case.inp["alpha"][40:90, 1] = 1e-20
    case.inp["alpha"][200:210, 2] = 0.0
    pool, out = case.run_gpu()
    ref, o_ref, e = case.run_oracle()
    check(case, pool, out, ref, o_ref)


KDA_ONE_CASES = [
    ("fp32 ragged warm/cold, scale", dict(seed=31, H=3, D=128, lens=[1, 63, 64, 65, 130, 200],
                                          warm=[1, 0, 1, 1, 0, 1], scale=0.5)),
    ("bf16 snapshots, unaligned start", dict(seed=32, H=4, D=128, lens=[300, 70, 2, 129],
                                             bf16=True, snap=64, start=[64, 37, 126, 0],
                                             warm=[1, 1, 1, 0])),
    ("fp32 silu + q and k norms", dict(seed=33, H=5, D=128, lens=[190, 64, 17], flags=7)),
    ("bf16 no norms", dict(seed=34, H=2, D=128, lens=[150, 90], bf16=True, flags=0)),
    ("empty and bad slots", dict(seed=35, H=2, D=128, lens=[0, 40, 0, 33, 5],
                                 slots=[3, 0, 4, 5, 20], warm=[1, 1, 0, 1, 1], N=20)),
    ("snapshots every 128 across several chunks", dict(seed=36, H=2, D=128, lens=[640, 333],
                                                       snap=128, start=[0, 192], warm=[0, 1])),
]


@pytest.mark.parametrize("name,kw", KDA_ONE_CASES, ids=[c[0] for c in KDA_ONE_CASES])
def test_prefill_kda_one_kernel_parity(name, kw):
    """Decay per channel at head dim 128 on the one-kernel path against the oracle."""
    print(f"prefill KDA parity (one-kernel): {name}", flush=True)
    case = Case(path=ONE, amode=1, **kw)
    pool, out = case.run_gpu()
    ref, o_ref, e = case.run_oracle()
    check(case, pool, out, ref, o_ref)
    assert int(pool.err_word.item()) == e


def test_prefill_kda_one_kernel_extreme_decay():
    """Decays per channel that leave the range of the decay-factor planes: chunks in
    which a channel decays below 2^-96 are run token by token.  Channels at 1e-3
    everywhere in the first request (every chunk token by token), a head at 1e-20
    and exact zeros in the second, and one channel at 0.3 over tokens 64..127 of the
    third (2^-111 in its second chunk only, the other chunks on the planes)."""
    print("prefill KDA one-kernel extreme decay", flush=True)
    case = Case(seed=37, H=3, D=128, lens=[150, 64, 260], amode=1, path=ONE, warm=[1, 0, 1])
    a = case.inp["alpha"]
    a[:150, :, :16] = 1e-3
    a[150 + 20:150 + 50, 1, :] = 1e-20
    a[150 + 5:150 + 9, 2, 7] = 0.0
    a[214 + 64:214 + 128, 0, 100] = 0.3
    pool, out = case.run_gpu()
    ref, o_ref, e = case.run_oracle()
    check(case, pool, out, ref, o_ref)


def test_prefill_kda_one_kernel_choice_and_agreement():
    """A batch of many KDA requests (8 x 16 = 128 units) takes the one-kernel path by
    default: bit for bit the forced one-kernel run, and within the tolerance of the
    two-kernel path."""
    print("prefill KDA path choice", flush=True)
    kw = dict(seed=38, H=16, D=128, lens=[64, 100, 37, 200, 1, 64, 129, 90], amode=1,
              snap=64, warm=[1, 0, 1, 1, 0, 1, 1, 1])
    d_pool, d_out = Case(**kw).run_gpu()
    o_pool, o_out = Case(path=ONE, **kw).run_gpu()
    t_pool, t_out = Case(path=TWO, **kw).run_gpu()
    assert torch.equal(d_out, o_out) and torch.equal(d_pool.ssm, o_pool.ssm)
    assert torch.equal(d_pool.conv, t_pool.conv)
    T, H, D = d_out.shape
    a = widen(bf16_np(o_out)).reshape(T, H, D).transpose(1, 0, 2)
    b = widen(bf16_np(t_out)).reshape(T, H, D).transpose(1, 0, 2)
    assert worst_unit_rel_l2(a, b, 1) <= REL_L2_TOL
    assert worst_unit_rel_l2(device_ssm_values(o_pool.ssm)[0], device_ssm_values(t_pool.ssm)[0], 2) <= REL_L2_TOL


def test_prefill_one_kernel_default_choice_and_agreement():
    """A batch of many GDN requests takes the one-kernel path by default; its
    result equals the forced one-kernel run bit for bit and agrees with the
    two-kernel path within the tolerance."""
    print("prefill path choice", flush=True)
    kw = dict(seed=17, H=16, D=128, lens=[64, 100, 37, 200, 1, 64, 129, 90], amode=0,
              snap=64, warm=[1, 0, 1, 1, 0, 1, 1, 1])
    d_pool, d_out = Case(**kw).run_gpu()            # 8 x 16 = 128 units: one kernel
    o_pool, o_out = Case(path=ONE, **kw).run_gpu()
    t_pool, t_out = Case(path=TWO, **kw).run_gpu()
    assert torch.equal(d_out, o_out) and torch.equal(d_pool.ssm, o_pool.ssm)
    assert torch.equal(d_pool.conv, t_pool.conv)
    T, H, D = d_out.shape
    a = widen(bf16_np(o_out)).reshape(T, H, D).transpose(1, 0, 2)
    b = widen(bf16_np(t_out)).reshape(T, H, D).transpose(1, 0, 2)
    assert worst_unit_rel_l2(a, b, 1) <= REL_L2_TOL
    assert worst_unit_rel_l2(device_ssm_values(o_pool.ssm)[0], device_ssm_values(t_pool.ssm)[0], 2) <= REL_L2_TOL


@pytest.mark.parametrize("path", [ONE, TWO], ids=["one-kernel", "two-kernel"])
def test_prefill_request_over_max_seqlen_is_skipped(path):
    """A request longer than max_seqlen sets error bit 4 and is skipped (its slot
    and output rows untouched); the others equal the oracle run without it."""
    import gated_delta_rule_slot_amd as gdn
    print(f"prefill bad seqlens, path {path}", flush=True)
    case = Case(seed=19, H=4, D=128, lens=[100, 300, 64], amode=0, warm=[1, 1, 0], path=path)
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    pool = gdn.state_pool_create(case.ssm.cuda(), case.conv.cuda(), err)
    T = int(case.cu[-1])
    out = torch.full((T, case.H, case.D), -7.0, dtype=torch.bfloat16, device="cuda")
    ws = torch.empty(gdn.gdn_prefill_workspace_bytes(pool, 3, 300), dtype=torch.uint8, device="cuda")
    gdn.conv_gdn_prefill_chunked(pool, 0, case.cu.cuda(), case.slots.cuda(), case.warm.cuda(),
                                 case.inp["x"].cuda(), case.w.cuda(), case.inp["alpha"].cuda(), 0,
                                 case.inp["beta"].cuda(), out, 200, start_len=case.start.cuda(),
                                 flags=1 | path, workspace=ws)
    torch.cuda.synchronize()
    assert int(err.item()) == 4
    keep = [0, 2]
    rows = torch.cat([torch.arange(0, 100), torch.arange(400, 464)])
    ref = pool_to_oracle(case.ssm, case.conv)
    o_ref, e = oracle.prefill(
        ref, 0, wl.cu_seqlens([100, 64]).numpy(), case.slots[keep].numpy(),
        wl.bf16_bits(case.inp["x"][rows]), wl.bf16_bits(case.w), case.inp["alpha"][rows].numpy(), 0,
        case.inp["beta"][rows].numpy(), has_initial_state=case.warm[keep].numpy())
    assert e == 0
    got = widen(bf16_np(out[rows.cuda()])).reshape(-1, case.H, case.D)
    want = widen(o_ref).reshape(-1, case.H, case.D)
    eo = max(worst_unit_rel_l2(got[:100].transpose(1, 0, 2), want[:100].transpose(1, 0, 2), 1),
             worst_unit_rel_l2(got[100:].transpose(1, 0, 2), want[100:].transpose(1, 0, 2), 1))
    assert eo <= REL_L2_TOL, eo
    skipped = bf16_np(out[100:400])
    assert np.all(skipped == bf16_np(torch.full((1,), -7.0, dtype=torch.bfloat16))[0])
    s_bad = int(case.slots[1])
    gs = device_ssm_values(pool.ssm)
    assert np.array_equal(gs[0, s_bad], case.ssm.double().numpy()[0, s_bad])
    assert torch.equal(pool.conv[0, s_bad].cpu(), case.conv[0, s_bad])
    sk = [int(case.slots[i]) for i in keep]
    assert worst_unit_rel_l2(gs[0, sk], ssm_values(ref)[0, sk], 2) <= REL_L2_TOL
    assert np.array_equal(bf16_np(pool.conv[0, sk]), ref.conv()[0, sk])


def test_prefill_small_workspace_windows_match_single_pass():
    """A workspace that holds one chunk per request forces many windows; the
    fp32 carry between windows makes the result identical bit for bit."""
    print("prefill windows", flush=True)
    import gated_delta_rule_slot_amd as gdn
    case = Case(seed=8, H=3, D=64, lens=[333, 64, 129], amode=1, bf16=True, snap=128,
                start=[0, 64, 128])
    p1, o1 = case.run_gpu()
    H, D, B = case.H, case.D, 3
    minimum = gdn.gdn_prefill_workspace_bytes(p1, B, 64)
    p2, o2 = case.run_gpu(workspace_bytes=minimum)
    assert torch.equal(o1, o2)
    assert torch.equal(p1.ssm, p2.ssm) and torch.equal(p1.conv, p2.conv)
    ref, o_ref, e = case.run_oracle()
    check(case, p2, o2, ref, o_ref)


def test_prefill_long_request_windows_match_single_pass():
    """A request of 25+ chunks, per-channel decay, bf16 pool, snapshots: one window
    for all chunks against one chunk per window (minimum workspace).  The fp32
    carry between windows makes both bit-identical, snapshots included."""
    print("prefill long-request windows", flush=True)
    import gated_delta_rule_slot_amd as gdn
    case = Case(seed=18, H=3, D=128, lens=[1500, 700, 0, 64], amode=1, bf16=True, snap=64,
                start=[0, 128, 0, 64], warm=[0, 1, 1, 1], path=TWO)
    p1, o1 = case.run_gpu()
    p2, o2 = case.run_gpu(workspace_bytes=gdn.gdn_prefill_workspace_bytes(p1, 4, 64))
    assert torch.equal(o1, o2)
    assert torch.equal(p1.ssm, p2.ssm) and torch.equal(p1.conv, p2.conv)
    ref, o_ref, e = case.run_oracle()
    check(case, p1, o1, ref, o_ref)


def test_prefill_very_long_request():
    """One request of 100,000 tokens (1,563 chunks, a partial last one) beside a
    short one, warm start, per-channel decay, bf16 pool, a snapshot every 4096
    tokens from an unaligned-to-4096 start: the whole result against the oracle."""
    print("prefill parity: 100k-token request", flush=True)
    case = Case(seed=31, H=2, D=16, lens=[100_000, 37], bf16=True, amode=1, snap=4096,
                start=[1024, 64], warm=[1, 1], path=TWO)
    pool, out = case.run_gpu()
    assert int(pool.err_word.item()) == 0
    ref, o_ref, e = case.run_oracle()
    check(case, pool, out, ref, o_ref)


LAST_ONLY = 32  # GDN_F_SNAP_LAST_ONLY


@pytest.mark.parametrize("name,kw", [
    ("D128 bf16 KDA, two kernels", dict(seed=5, H=4, D=128, lens=[300, 70, 2], bf16=True, snap=64,
                                        start=[64, 37, 126], warm=[1, 1, 1])),
    ("D128 bf16 GDN, two kernels", dict(seed=12, H=4, D=128, lens=[300, 70, 2, 129], bf16=True,
                                        amode=0, snap=64, start=[64, 37, 126, 0], warm=[1, 1, 1, 0],
                                        path=TWO)),
    ("D128 bf16 GDN, one kernel", dict(seed=12, H=4, D=128, lens=[300, 70, 2, 129], bf16=True,
                                       amode=0, snap=64, start=[64, 37, 126, 0], warm=[1, 1, 1, 0],
                                       path=ONE)),
])
def test_prefill_snapshots_last_only(name, kw):
    """GDN_F_SNAP_LAST_ONLY stores only the last boundary of each ping-pong parity;
    the pool after the call is the one the oracle's every-boundary definition
    gives (slots, states and conv rows)."""
    print(f"prefill snapshots, last of each parity only: {name}", flush=True)
    case = Case(**kw)
    case.path |= LAST_ONLY
    pool, out = case.run_gpu()
    ref, o_ref, e = case.run_oracle()
    check(case, pool, out, ref, o_ref)
    assert int(pool.err_word.item()) == 0


def test_prefill_full_kda_workload():
    """12 heads, K=V=128, one request of 6144 tokens, per-channel decay, bf16
    pool, snapshot at every 64-token boundary: checked in full."""
    print("prefill parity: full KDA prefill workload", flush=True)
    cfg = wl.KDA_PREFILL
    case = Case(seed=cfg.seed, H=cfg.heads, D=cfg.head_k, lens=[6144], bf16=True, amode=1,
                snap=64, warm=[0], N=cfg.slots)
    pool, out = case.run_gpu()
    assert int(pool.err_word.item()) == 0
    ref, o_ref, e = case.run_oracle()
    check(case, pool, out, ref, o_ref)


def test_prefill_kda_batch_launch():
    """The KDA prefill shape for a batch, in the launch configuration the benchmark
    times: 64 cold requests x 6144 tokens, 12 heads, K=V=128, per-channel decay, bf16
    pool, every 64-token boundary stored to the requests' track slots, the library's
    default path (768 units: one kernel).  Inputs are drawn on the device.  Three
    requests (first, middle, last) against the oracle: outputs, live states, both
    track slots and conv rows.  Every (request, head) unit against the two-kernel
    path on the same inputs: outputs and live states within the tolerance."""
    import gated_delta_rule_slot_amd as gdn
    print("prefill parity: KDA batch launch", flush=True)
    cfg = wl.KDA_PREFILL
    H, D, B, Tr = cfg.heads, cfg.head_k, 64, 6144
    C, T, N = 3 * H * D, B * Tr, 3 * B + 1
    dev = torch.device("cuda")
    gd = torch.Generator(device=dev)
    gd.manual_seed(cfg.seed + 7)
    x = torch.randn(T, C, generator=gd, device=dev).to(torch.bfloat16)
    k = x[:, H * D:2 * H * D].view(T, H, D).float()         # keys L2-normalised per head
    x[:, H * D:2 * H * D] = (k / k.norm(dim=-1, keepdim=True)).to(torch.bfloat16).view(T, H * D)
    del k
    alpha = torch.sigmoid(torch.randn(T, H, D, generator=gd, device=dev) + 3.0)
    beta = torch.sigmoid(torch.randn(T, H, generator=gd, device=dev))
    w = wl.conv_weights(wl.generator(cfg.seed + 7), C).to(dev)
    g = wl.generator(cfg.seed + 8)
    ssm0 = (0.25 * torch.randn(1, N, H, D, D, generator=g)).to(torch.bfloat16)
    conv0 = torch.randn(1, N, 3, C, generator=g).to(torch.bfloat16)
    cu = wl.cu_seqlens([Tr] * B)
    slots = torch.arange(1, B + 1, dtype=torch.int32)
    track = torch.arange(B + 1, 3 * B + 1, dtype=torch.int32).reshape(B, 2).contiguous()
    nxt = torch.randint(0, 2, (B,), generator=g, dtype=torch.int32)
    zeros = torch.zeros(B, dtype=torch.int32)

    def run(flags, workspace=None):
        err = torch.zeros(1, dtype=torch.int32, device=dev)
        pool = gdn.state_pool_create(ssm0.to(dev), conv0.to(dev), err)
        out = torch.empty(T, H, D, dtype=torch.bfloat16, device=dev)
        gdn.conv_gdn_prefill_chunked(pool, 0, cu.to(dev), slots.to(dev), zeros.to(dev), x, w, alpha,
                                     cfg.alpha_mode, beta, out, Tr, start_len=zeros.to(dev),
                                     flags=flags, snap_interval=64, track_slots=track.to(dev),
                                     next_track_idx=nxt.to(dev), workspace=workspace)
        torch.cuda.synchronize()
        assert int(err.item()) == 0
        return pool, out

    pool, out = run(gdn.L2NORM_K)
    ws = torch.empty(min(gdn.gdn_prefill_workspace_bytes(pool, B, Tr), 8 << 30), dtype=torch.uint8,
                     device=dev)
    pool2, out2 = run(gdn.L2NORM_K | gdn.PREFILL_TWO_KERNEL, ws)
    del ws
    # every unit against the two-kernel path (on the device, in fp32)
    a, b = out.float().view(B, Tr, H, D), out2.float().view(B, Tr, H, D)
    rel = ((a - b).square().sum(dim=(1, 3)) / b.square().sum(dim=(1, 3))).sqrt()
    sa = pool.ssm[0, 1:B + 1].float()
    sb = pool2.ssm[0, 1:B + 1].float()
    rels = ((sa - sb).square().sum(dim=(2, 3)) / sb.square().sum(dim=(2, 3))).sqrt()
    print(f"  one kernel against two kernels, all {B * H} units: out {rel.max().item():.2e}  "
          f"state {rels.max().item():.2e}", flush=True)
    assert rel.max().item() <= REL_L2_TOL and rels.max().item() <= REL_L2_TOL
    del a, b, out2, pool2
    # three requests against the oracle
    pick = [0, B // 2, B - 1]
    idx = torch.cat([torch.arange(int(cu[i]), int(cu[i + 1])) for i in pick]).to(dev)
    ref = pool_to_oracle(ssm0, conv0)
    o_ref, e = oracle.prefill(
        ref, 0, wl.cu_seqlens([Tr] * 3).numpy(), slots[pick].numpy(), wl.bf16_bits(x[idx].cpu()),
        wl.bf16_bits(w.cpu()), alpha[idx].cpu().numpy(), cfg.alpha_mode, beta[idx].cpu().numpy(),
        has_initial_state=np.zeros(3, np.int32), start_len=np.zeros(3, np.int32), snap_interval=64,
        track_slots=track[pick].numpy(), next_track_idx=nxt[pick].numpy())
    assert e == 0
    got = widen(bf16_np(out[idx])).reshape(-1, H, D)
    want = widen(o_ref).reshape(-1, H, D)
    eo = max(worst_unit_rel_l2(got[i * Tr:(i + 1) * Tr].transpose(1, 0, 2),
                               want[i * Tr:(i + 1) * Tr].transpose(1, 0, 2), 1) for i in range(3))
    sp = [int(slots[i]) for i in pick] + [int(t) for i in pick for t in track[i]]
    es = worst_unit_rel_l2(device_ssm_values(pool.ssm)[0, sp], ssm_values(ref)[0, sp], 2)
    print(f"  requests {pick} against the oracle: worst unit rel-L2 out {eo:.2e}  state {es:.2e} "
          f"(live and track slots)", flush=True)
    assert eo <= REL_L2_TOL and es <= REL_L2_TOL
    assert np.array_equal(bf16_np(pool.conv[0, sp]), ref.conv()[0, sp])


def test_prefill_single_pass_matches_scratch_windows():
    """The full KDA workload shape (12 heads, one request, snapshots every 64) in one
    pass over a full workspace equals, bit for bit, the no-alloc entry point, whose
    64 MiB scratch holds 37 chunks per window (three windows with the fp32 carry
    between them), and the oracle; a second call on a warm, unaligned request
    follows on the same scratch."""
    import gated_delta_rule_slot_amd as gdn
    print("prefill: single pass against scratch windows", flush=True)
    for seed, lens, start, warm in ((31, [6144], [0], [0]), (32, [2500], [192], [1])):
        case = Case(seed=seed, H=12, D=128, lens=lens, bf16=True, amode=1, snap=64, start=start,
                    warm=warm, N=8)
        p1, o1 = case.run_gpu()
        err = torch.zeros(1, dtype=torch.int32, device="cuda")
        p2 = gdn.state_pool_create(case.ssm.cuda(), case.conv.cuda(), err)
        o2 = torch.full_like(o1, -7.0)
        gdn.conv_gdn_prefill_chunked_noalloc(
            p2, case.layer, case.cu.cuda(), case.slots.cuda(), case.warm.cuda(), case.inp["x"].cuda(),
            case.w.cuda(), case.inp["alpha"].cuda(), case.amode, case.inp["beta"].cuda(), o2,
            max(lens), start_len=case.start.cuda(), snap_interval=case.snap,
            track_slots=case.track.cuda(), next_track_idx=case.nxt.cuda())
        torch.cuda.synchronize()
        assert torch.equal(o1, o2)
        assert torch.equal(p1.ssm, p2.ssm) and torch.equal(p1.conv, p2.conv)
        ref, o_ref, e = case.run_oracle()
        check(case, p1, o1, ref, o_ref)


@pytest.mark.parametrize("path", [ONE, TWO], ids=["one-kernel", "two-kernel"])
def test_prefill_warm_gdn_subset(path):
    """32 heads, K=V=128, scalar decay, fp32 pool, warm starts at a 6144
    boundary followed by ragged remainders (a sample of the prefix-hit workload)."""
    print(f"prefill parity: warm GDN sample, path {path}", flush=True)
    cfg = wl.WARM_PREFILL
    case = Case(seed=cfg.seed, H=cfg.heads, D=cfg.head_k, lens=[1312, 700, 2048], amode=0,
                start=[12288, 6144, 6144], warm=[1, 1, 1], N=12, snap=6144, path=path)
    pool, out = case.run_gpu()
    ref, o_ref, e = case.run_oracle()
    check(case, pool, out, ref, o_ref)


@pytest.mark.timeout(600)
def test_prefill_warm_workload_launch():
    """The prefix-hit warm prefill in the launch configuration the benchmark times:
    64 requests whose remaining lengths follow the benchmark's seeded prefix mix
    (13600 - 6144 * min(2, P // 6144), P ~ U[0, 13600)), 32 heads, K=V=128, scalar
    decay, fp32 pool of 81 slots, restored requests warm, the library's default
    path (64 x 32 units: one kernel, called without a workspace).  Inputs are
    drawn on the device.  Checked against the oracle, every head: the two
    shortest requests, a middle one, the first and the last cold 13,600-token
    request (the longest, which the kernel's longest-first order starts first and
    last among equals) and the first warm 7,456-token one."""
    import gated_delta_rule_slot_amd as gdn
    print("prefill parity: warm-prefill launch", flush=True)
    cfg = wl.WARM_PREFILL
    H, D, N, B, T_full = cfg.heads, cfg.head_k, cfg.slots, 64, 13600
    C = 3 * H * D
    gc = wl.generator(cfg.seed)
    torch.randint(0, 8, (B,), generator=gc)                   # prefix groups (unused here)
    prefix = torch.randint(0, T_full, (B,), generator=gc).tolist()
    depth = [6144 * min(2, p // 6144) for p in prefix]
    lens = [T_full - c for c in depth]
    warm = [1 if c > 0 else 0 for c in depth]
    dev = torch.device("cuda")
    gd = torch.Generator(device=dev)
    gd.manual_seed(cfg.seed)
    ssm = torch.empty(1, N, H, D, D, dtype=torch.float32, device=dev).normal_(0.0, 0.25, generator=gd)
    conv = torch.empty(1, N, 3, C, dtype=torch.float32, device=dev).normal_(0.0, 1.0, generator=gd)
    conv = conv.to(torch.bfloat16)
    T = sum(lens)
    x = torch.randn(T, C, generator=gd, device=dev).to(torch.bfloat16)
    k = x[:, H * D:2 * H * D].view(T, H, D).float()         # keys L2-normalised per head
    x[:, H * D:2 * H * D] = (k / k.norm(dim=-1, keepdim=True)).to(torch.bfloat16).view(T, H * D)
    del k
    alpha = torch.sigmoid(torch.randn(T, H, generator=gd, device=dev) + 3.0)
    beta = torch.sigmoid(torch.randn(T, H, generator=gd, device=dev))
    w = wl.conv_weights(gc, C).to(dev)
    cu = wl.cu_seqlens(lens)
    slots = torch.arange(1, B + 1, dtype=torch.int32)
    ssm_host, conv_host = ssm.cpu(), conv.cpu()
    err = torch.zeros(1, dtype=torch.int32, device=dev)
    pool = gdn.state_pool_create(ssm, conv, err)
    out = torch.empty(T, H, D, dtype=torch.bfloat16, device=dev)
    gdn.conv_gdn_prefill_chunked(pool, 0, cu.to(dev), slots.to(dev),
                                 torch.tensor(warm, dtype=torch.int32, device=dev), x, w, alpha,
                                 cfg.alpha_mode, beta, out, max(lens),
                                 start_len=torch.tensor(depth, dtype=torch.int32, device=dev))
    torch.cuda.synchronize()
    assert int(err.item()) == 0
    order = sorted(range(B), key=lambda i: lens[i])
    cold = [i for i in range(B) if lens[i] == T_full]
    warm1 = [i for i in range(B) if lens[i] == T_full - 6144]
    assert cold and warm1
    pick = sorted({order[0], order[1], order[B // 2], cold[0], cold[-1], warm1[0]})
    sub = [(int(cu[i]), int(cu[i + 1])) for i in pick]
    sl = [lens[i] for i in pick]
    idx = torch.cat([torch.arange(a, b) for a, b in sub]).to(dev)
    ref = pool_to_oracle(ssm_host, conv_host)
    o_ref, e = oracle.prefill(
        ref, 0, wl.cu_seqlens(sl).numpy(), slots[pick].numpy(), wl.bf16_bits(x[idx].cpu()),
        wl.bf16_bits(w.cpu()), alpha[idx].cpu().numpy(), cfg.alpha_mode, beta[idx].cpu().numpy(),
        has_initial_state=np.array([warm[i] for i in pick], np.int32),
        start_len=np.array([depth[i] for i in pick], np.int32))
    assert e == 0
    got = widen(bf16_np(out[idx])).reshape(-1, H, D)
    want = widen(o_ref).reshape(-1, H, D)
    eo, s0 = 0.0, 0
    for n in sl:
        eo = max(eo, worst_unit_rel_l2(got[s0:s0 + n].transpose(1, 0, 2), want[s0:s0 + n].transpose(1, 0, 2), 1))
        s0 += n
    sp = [int(slots[i]) for i in pick]
    es = worst_unit_rel_l2(device_ssm_values(pool.ssm)[0, sp], ssm_values(ref)[0, sp], 2)
    print(f"  requests {pick} (lengths {sl}): worst unit rel-L2 out {eo:.2e}  state {es:.2e}", flush=True)
    assert eo <= REL_L2_TOL and es <= REL_L2_TOL
    assert np.array_equal(bf16_np(pool.conv[0, sp]), ref.conv()[0, sp])


def test_prefill_extreme_decay():
    """Channels with alpha = 1e-3 (and a head at 1e-20) stay finite and match."""
    print("prefill extreme decay", flush=True)
    case = Case(seed=9, H=3, D=128, lens=[150, 64], amode=1)
    case.inp["alpha"][:, :, :16] = 1e-3
    case.inp["alpha"][40:90, 1, :] = 1e-20
    pool, out = case.run_gpu()
    ref, o_ref, e = case.run_oracle()
    check(case, pool, out, ref, o_ref)


def test_prefill_then_restore_then_resume():
    """Tiny workload end to end: prefill 256 tokens with a snapshot every 64,
    restore each boundary's snapshot into a fresh slot, resume to 256, and land
    on the uninterrupted state (GPU against the oracle at every step)."""
    import gated_delta_rule_slot_amd as gdn
    print("prefill + restore + resume", flush=True)
    case = Case(seed=101, H=2, D=16, lens=[256, 256], snap=64, warm=[0, 0], N=8, slots=[1, 2])
    case.track = torch.tensor([[3, 4], [5, 6]], dtype=torch.int32)
    case.nxt = torch.zeros(2, dtype=torch.int32)
    full_pool, full_out = case.run_gpu()
    ref_full, o_full, _ = case.run_oracle()
    check(case, full_pool, full_out, ref_full, o_full)
    # prefill to 192 (snapshots at 64, 128, 192: the last lands in track[0])
    part = Case(seed=101, H=2, D=16, lens=[256, 256], snap=64, warm=[0, 0], N=8, slots=[1, 2])
    part.track, part.nxt = case.track, case.nxt
    x, al, be = part.inp["x"], part.inp["alpha"], part.inp["beta"]
    idx = torch.cat([torch.arange(0, 192), torch.arange(256, 448)])
    part.inp = {"x": x[idx].contiguous(), "alpha": al[idx].contiguous(), "beta": be[idx].contiguous()}
    part.lens, part.cu = [192, 192], wl.cu_seqlens([192, 192])
    pool, _ = part.run_gpu()
    ref, _, _ = part.run_oracle()
    # preemption: live slots overwritten with garbage, then restore 192's snapshot into 7 and 1
    pool.ssm[0, 1].fill_(float("nan"))
    pool.ssm[0, 2].fill_(float("nan"))
    ref.ssm()[0, 1] = np.nan
    ref.ssm()[0, 2] = np.nan
    ops = [(7, 1, 3), (1, 1, 5)]
    hi = gdn.restore_slots(pool, ops, [0, 0])
    hi_ref = oracle.restore_slots(ref, ops, np.zeros(2, dtype=np.int64))
    assert hi == hi_ref.tolist() == [1, 1]
    torch.cuda.synchronize()
    # resume the last 64 tokens of each request from the restored slots
    res = Case(seed=101, H=2, D=16, lens=[64, 64], N=8, slots=[7, 1], warm=[1, 1], start=[192, 192])
    res.ssm = pool.ssm.cpu()
    res.conv = pool.conv.cpu()
    idx = torch.cat([torch.arange(192, 256), torch.arange(448, 512)])
    res.inp = {"x": x[idx].contiguous(), "alpha": al[idx].contiguous(), "beta": be[idx].contiguous()}
    rpool, rout = res.run_gpu()
    rref, ro, _ = res.run_oracle()
    check(res, rpool, rout, rref, ro)
    # and the resumed state equals the uninterrupted run's, within tolerance
    a = device_ssm_values(rpool.ssm)[0, [7, 1]]
    b = device_ssm_values(full_pool.ssm)[0, [1, 2]]
    assert worst_unit_rel_l2(a, b, 2) <= REL_L2_TOL
    got_o = widen(bf16_np(rout)).reshape(2, 64, 2, 16)
    want_o = widen(bf16_np(full_out)).reshape(2, 256, 2, 16)[:, 192:]
    assert worst_unit_rel_l2(got_o.transpose(0, 2, 1, 3), want_o.transpose(0, 2, 1, 3), 2) <= REL_L2_TOL
