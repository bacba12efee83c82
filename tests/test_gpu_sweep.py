"""Seeded random sweep of the GPU paths against the oracle.

Each case draws its shape from a seeded generator: head dim, heads, batch,
lengths (empty, single tokens, ragged tails, several chunks), warm or cold
starts at arbitrary positions, decay per head or per channel, fp32 or bf16
pool, key/query norm and SiLU flags, output scale, snapshot interval and the
prefill path, and for the draft-tree verify random trees.  The comparison
rules are those of the targeted tests: floats within 2e-3 relative L2 per
unit, conv rows and untouched slots bit-exact.  Prefill units here can be a few
hundred outputs, where one output that the two sides round to neighbouring bf16
values weighs more than 2e-3; such a unit passes as a set of valid roundings of
the oracle's exact outputs (helpers.output_unit_ok).
"""
import numpy as np
import pytest
import torch

import workloads as wl
from tests.test_gpu_decode import _assert_parity, _run_both
from tests.test_gpu_prefill import ONE, TWO, Case, check
from tests.test_gpu_spec import _assert_verify, _spec_inputs, _verify_both, random_tree

pytestmark = pytest.mark.gpu

LENGTHS = [0, 1, 2, 3, 17, 63, 64, 65, 127, 128, 129, 200, 300]


@pytest.mark.parametrize("i", range(24))
def test_prefill_random_cases(i):
    import gated_delta_rule_slot_amd as gdn
    r = np.random.default_rng(5000 + i)
    D = int(r.choice([16, 32, 64, 128]))
    H = int(r.integers(1, 5))
    B = int(r.integers(1, 5))
    lens = [int(v) for v in r.choice(LENGTHS, size=B)]
    amode = int(r.integers(0, 2))
    bf16 = bool(r.integers(0, 2))
    flags = int(r.choice([1, 3, 5, 7]))
    snap = int(r.choice([0, 64, 128]))
    warm = [int(v) for v in r.integers(0, 2, size=B)]
    start = [int(v) for v in r.integers(0, 400, size=B)]
    scale = float(r.choice([1.0, 0.5, 1.75]))
    paths = [0, TWO] + ([ONE] if amode == 0 and D == 128 else [])
    path = int(r.choice(paths)) | (32 if r.integers(0, 4) == 0 else 0)  # GDN_F_SNAP_LAST_ONLY
    small_ws = bool(r.integers(0, 2))
    print(f"prefill sweep {i}: D={D} H={H} lens={lens} amode={amode} bf16={bf16} flags={flags} "
          f"snap={snap} warm={warm} start={start} scale={scale} path={path} small_ws={small_ws}",
          flush=True)
    case = Case(seed=6000 + i, H=H, D=D, lens=lens, bf16=bf16, amode=amode, warm=warm, start=start,
                flags=flags, scale=scale, snap=snap, path=path)
    ws = None
    if small_ws:
        import gated_delta_rule_slot_amd as gdn
        err = torch.zeros(1, dtype=torch.int32, device="cuda")
        probe = gdn.state_pool_create(case.ssm.cuda(), case.conv.cuda(), err)
        ws = gdn.gdn_prefill_workspace_bytes(probe, B, 64)
    pool, out = case.run_gpu(workspace_bytes=ws)
    assert int(pool.err_word.item()) == 0
    ref, o_ref, e, o_exact = case.run_oracle(exact=True)
    assert e == 0
    if int(case.cu[-1]) > 0:
        check(case, pool, out, ref, o_ref, o_exact=o_exact)


ONE_KERNEL_LENGTHS = [1, 5, 63, 64, 65, 130, 257, 400, 700]


@pytest.mark.parametrize("i", range(32))
def test_prefill_one_kernel_random_cases(i):
    """The one-kernel path (decay per head, head dim 128) on random batches of
    longer requests: warm and cold starts at arbitrary positions, fp32 or bf16
    pool, norm and SiLU flags, snapshots every boundary or the last of each parity."""
    r = np.random.default_rng(90000 + i)
    H = int(r.integers(1, 5))
    B = int(r.integers(1, 7))
    lens = [int(v) for v in r.choice(ONE_KERNEL_LENGTHS, size=B)]
    bf16 = bool(r.integers(0, 2))
    flags = int(r.choice([1, 3, 5, 7]))
    snap = int(r.choice([0, 64, 128]))
    warm = [int(v) for v in r.integers(0, 2, size=B)]
    start = [int(v) for v in r.integers(0, 400, size=B)]
    path = ONE | (32 if r.integers(0, 3) == 0 else 0)  # GDN_F_SNAP_LAST_ONLY
    print(f"one-kernel sweep {i}: H={H} lens={lens} bf16={bf16} flags={flags} snap={snap} "
          f"warm={warm} start={start} path={path}", flush=True)
    case = Case(seed=91000 + i, H=H, D=128, lens=lens, bf16=bf16, amode=0, warm=warm, start=start,
                flags=flags, scale=0.75, snap=snap, path=path)
    pool, out = case.run_gpu()
    assert int(pool.err_word.item()) == 0
    ref, o_ref, e, o_exact = case.run_oracle(exact=True)
    assert e == 0
    check(case, pool, out, ref, o_ref, o_exact=o_exact)


@pytest.mark.parametrize("i", range(24))
def test_prefill_kda_one_kernel_random_cases(i):
    """The one-kernel path with a decay per channel on random batches: warm and cold
    starts at arbitrary positions, fp32 or bf16 pool, norm and SiLU flags, snapshot
    modes; in a third of the cases some channels of one request decay hard enough
    (a = 0.2 .. 0.35 over a stretch) that chunks run token by token."""
    r = np.random.default_rng(92000 + i)
    H = int(r.integers(1, 5))
    B = int(r.integers(1, 7))
    lens = [int(v) for v in r.choice(ONE_KERNEL_LENGTHS, size=B)]
    bf16 = bool(r.integers(0, 2))
    flags = int(r.choice([0, 1, 3, 5, 7]))
    snap = int(r.choice([0, 64, 128]))
    warm = [int(v) for v in r.integers(0, 2, size=B)]
    start = [int(v) for v in r.integers(0, 400, size=B)]
    path = ONE | (32 if r.integers(0, 3) == 0 else 0)  # GDN_F_SNAP_LAST_ONLY
    hard = r.integers(0, 3) == 0
    print(f"KDA one-kernel sweep {i}: H={H} lens={lens} bf16={bf16} flags={flags} snap={snap} "
          f"warm={warm} start={start} path={path} hard={hard}", flush=True)
    case = Case(seed=93000 + i, H=H, D=128, lens=lens, bf16=bf16, amode=1, warm=warm, start=start,
                flags=flags, scale=0.75, snap=snap, path=path)
    if hard:
        b = int(r.integers(0, B))
        s0 = int(case.cu[b])
        n = lens[b]
        t0 = int(r.integers(0, n))
        t1 = min(n, t0 + int(r.integers(1, 160)))
        chans = r.choice(128, size=int(r.integers(1, 9)), replace=False)
        hh = int(r.integers(0, H))
        case.inp["alpha"][s0 + t0:s0 + t1, hh, chans] = float(r.uniform(0.2, 0.35))
    pool, out = case.run_gpu()
    assert int(pool.err_word.item()) == 0
    ref, o_ref, e, o_exact = case.run_oracle(exact=True)
    assert e == 0
    check(case, pool, out, ref, o_ref, o_exact=o_exact)


@pytest.mark.parametrize("i", range(12))
def test_decode_random_cases(i):
    r = np.random.default_rng(7000 + i)
    D = int(r.choice([16, 32, 64, 128]))
    H = int(r.integers(1, 9))
    B = int(r.integers(1, 40))
    N = B * 3 + 2
    L = int(r.integers(1, 3))
    amode = int(r.integers(0, 2))
    bf16 = bool(r.integers(0, 2))
    flags = int(r.choice([1, 3, 5, 7]))
    interval = int(r.choice([0, 2, 4, 256]))
    print(f"decode sweep {i}: D={D} H={H} B={B} L={L} amode={amode} bf16={bf16} flags={flags} "
          f"interval={interval}", flush=True)
    g = wl.generator(8000 + i)
    ssm, conv = wl.warm_pool(g, L, N, H, D, D, bf16)
    w = wl.conv_weights(g, H * 3 * D)
    inp = wl.projected_inputs(g, B, H, D, D, amode)
    ids = wl.distinct_slots(g, 3 * B, N)
    slots, track = ids[:B].contiguous(), ids[B:].reshape(B, 2).contiguous()
    seq = torch.randint(1, 600, (B,), generator=g, dtype=torch.int32)
    nxt = torch.randint(0, 2, (B,), generator=g, dtype=torch.int32)
    layer = L - 1
    kw = dict(seq_len_after=seq, interval=interval, track=track, nxt=nxt) if interval else {}
    pool, out, ref, o_ref, e = _run_both(ssm, conv, w, inp, slots, amode, layer=layer, scale=0.9,
                                         flags=flags, **kw)
    extra = []
    if interval:
        hit = (seq % interval == 0).numpy()
        extra = [int(track[b, int(nxt[b])]) for b in range(B) if hit[b]]
    _assert_parity(pool, out, ref, o_ref, layer, slots.numpy(), extra_written=extra)
    assert e == 0 and int(pool.err_word.item()) == 0


@pytest.mark.parametrize("i", range(10))
def test_verify_random_cases(i):
    r = np.random.default_rng(9100 + i)
    D = int(r.choice([16, 32, 64, 128]))
    H = int(r.integers(1, 7))
    B = int(r.integers(1, 6))
    T = int(r.integers(1, 40))
    amode = int(r.integers(0, 2))
    bf16 = bool(r.integers(0, 2))
    flags = int(r.choice([1, 3, 5, 7]))
    N = B + 3
    print(f"verify sweep {i}: D={D} H={H} B={B} T={T} amode={amode} bf16={bf16} flags={flags}", flush=True)
    g, ssm, conv, w, inp, slots = _spec_inputs(9200 + i, 1, N, H, D, bf16, B, T, amode)
    parent = torch.tensor([random_tree(g, T) for _ in range(B)], dtype=torch.int32)
    pool, out, ns, nc, ref, o_ref, ns_ref, nc_ref, e = _verify_both(
        ssm, conv, w, inp, slots, parent, amode, 0, scale=1.25, flags=flags)
    _assert_verify(ssm, conv, pool, out, ns, nc, o_ref, ns_ref, nc_ref)
    assert e == 0 and int(pool.err_word.item()) == 0
