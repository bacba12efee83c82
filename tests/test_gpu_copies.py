"""GPU parity of the slot copies (track_snapshot, restore_slots): byte-exact
pool images against the oracle after random sequences of copies."""
import numpy as np
import pytest
import torch

import oracle
import workloads as wl
from tests.helpers import pool_bytes_equal, pool_to_oracle

pytestmark = pytest.mark.gpu


def _pool(g, L, N, H, D, bf16):
    import gated_delta_rule_slot_amd as gdn
    ssm, conv = wl.warm_pool(g, L, N, H, D, D, bf16)
    ssm_d, conv_d = ssm.cuda(), conv.cuda()
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    return gdn.state_pool_create(ssm_d, conv_d, err), ssm, conv


@pytest.mark.parametrize("L,N,H,D,bf16", [(1, 8, 2, 16, False), (3, 40, 12, 128, True),
                                          (2, 20, 32, 128, False), (4, 9, 3, 64, True)])
def test_random_copy_sequences_bitexact(L, N, H, D, bf16):
    import gated_delta_rule_slot_amd as gdn
    g = wl.generator(1000 + L * N)
    pool, ssm, conv = _pool(g, L, N, H, D, bf16)
    ref = pool_to_oracle(ssm, conv)
    rng = np.random.default_rng(L * 7 + N)
    print(f"copies L={L} N={N} H={H} D={D} bf16={bf16}", flush=True)
    for step in range(6):
        if step % 2 == 0:
            n = int(rng.integers(1, N // 2))
            perm = rng.permutation(np.arange(1, N))
            src = perm[:n].astype(np.int32)
            dst = perm[n:2 * n].astype(np.int32)
            dst[rng.random(n) < 0.25] = 0          # masked entries
            l0 = int(rng.integers(0, L))
            l1 = int(rng.integers(l0, L + 1))
            gdn.track_snapshot(pool, l0, l1, torch.from_numpy(src).cuda(),
                               torch.from_numpy(dst).cuda())
            oracle.track_snapshot(ref, l0, l1, src, dst)
        else:
            n = int(rng.integers(1, N // 2))
            perm = rng.permutation(np.arange(1, N))
            ops = [(int(perm[n + i]), int(rng.random() < 0.8), int(perm[i])) for i in range(n)]
            ops.append((int(perm[0]), 1, -1))      # no source -> cold
            hi = [5] * len(ops)
            got = gdn.restore_slots(pool, ops, hi)
            want = oracle.restore_slots(ref, ops, np.array([5] * len(ops), dtype=np.int64))
            assert got == want.tolist()
        torch.cuda.synchronize()
        assert pool_bytes_equal(pool.ssm, pool.conv, ref), f"step {step}"
    assert int(pool.err_word.item()) == 0


def test_bad_track_slots_set_error_word_and_skip():
    import gated_delta_rule_slot_amd as gdn
    g = wl.generator(77)
    pool, ssm, conv = _pool(g, 2, 10, 2, 32, False)
    ref = pool_to_oracle(ssm, conv)
    src = torch.tensor([1, 2, 0, 3], dtype=torch.int32, device="cuda")
    dst = torch.tensor([4, 10, 5, -1], dtype=torch.int32, device="cuda")
    gdn.track_snapshot(pool, 0, 2, src, dst)
    oracle.track_snapshot(ref, 0, 2, src.cpu().numpy(), dst.cpu().numpy())
    torch.cuda.synchronize()
    assert pool_bytes_equal(pool.ssm, pool.conv, ref)
    assert int(pool.err_word.item()) & gdn.ERRW_BAD_TRACK_SLOT


def test_restore_across_many_ops_and_layers():
    """More ops than fit in one launch's argument block; every layer copied."""
    import gated_delta_rule_slot_amd as gdn
    g = wl.generator(88)
    L, N = 3, 700
    pool, ssm, conv = _pool(g, L, N, 1, 16, True)
    ref = pool_to_oracle(ssm, conv)
    ops = [(i + 350, 1, i + 1) for i in range(300)]
    got = gdn.restore_slots(pool, ops, [0] * 300)
    want = oracle.restore_slots(ref, ops, np.zeros(300, dtype=np.int64))
    torch.cuda.synchronize()
    assert got == want.tolist() == [1] * 300
    assert pool_bytes_equal(pool.ssm, pool.conv, ref)


def test_restore_full_size_workload():
    """The benchmark's restore launch: 35 requests restored across all 24 layers of a
    32-head, K = V = 128 fp32 pool of 81 slots (2 MiB of state and 72 KiB of conv rows
    per layer and slot) from 16 checkpoint slots, plus a requested restore without a
    source, one onto its own slot and one not requested.  Every copied (layer, slot)
    equals its source byte for byte and every other slot is untouched (checked on the
    device); the outcomes are the oracle's, whose rules do not depend on the state's
    size (a one-head pool of the same slot count decides them)."""
    import gated_delta_rule_slot_amd as gdn
    print("restore: full-size launch", flush=True)
    cfg = wl.WARM_PREFILL
    L, N, H, D = cfg.layers, cfg.slots, cfg.heads, cfg.head_k
    C = 3 * H * D
    gd = torch.Generator(device="cuda")
    gd.manual_seed(91)
    ssm = torch.empty(L, N, H, D, D, dtype=torch.float32, device="cuda").normal_(generator=gd)
    conv = torch.empty(L, N, 3, C, dtype=torch.float32, device="cuda").normal_(generator=gd).to(torch.bfloat16)
    ssm0, conv0 = ssm.clone(), conv.clone()
    pool = gdn.state_pool_create(ssm, conv, torch.zeros(1, dtype=torch.int32, device="cuda"))
    ops = [(1 + i, 1, 65 + (i % 16)) for i in range(35)] + [(40, 1, -1), (41, 1, 41), (42, 0, 70)]
    got = gdn.restore_slots(pool, ops, [0] * len(ops))
    want = oracle.restore_slots(oracle.Pool(1, N, 1, 16, 16, oracle.SSM_F32), ops,
                                np.zeros(len(ops), dtype=np.int64))
    torch.cuda.synchronize()
    assert got == want.tolist() and got[:35] == [1] * 35 and got[35:] == [0, 1, 0]
    copied = {d: s for (d, r, s) in ops if r and 0 < s < N and s != d}
    for n in range(N):
        s = copied.get(n, n)
        assert torch.equal(ssm[:, n], ssm0[:, s]) and torch.equal(conv[:, n], conv0[:, s]), n
