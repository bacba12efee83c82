"""The C++ checkpoint index (include/gdn_ckpt.h) against its oracle, on the CPU.

Every result must match exactly: keys, hits, reaches, slots, insert outcomes,
evicted slots and sizes, over random operation sequences that force evictions
and pinning."""
import json
import os

import numpy as np
import pytest

import gated_delta_rule_slot_amd as gdn
from gated_delta_rule_slot_amd import _binding as B
from oracle import ckpt_index as ci
from tests.test_ckpt_pins import _sglang_policy_walkthrough


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_chain_hashes_match_the_oracle(seed):
    rng = np.random.default_rng(seed)
    for _ in range(20):
        stride = int(rng.integers(1, 300))
        n = int(rng.integers(0, 3000))
        t = rng.integers(-2 ** 31, 2 ** 31, n, dtype=np.int64).astype(np.int32)
        want = ci.chain_hashes(t.tolist(), stride)
        assert [int(x) for x in gdn.ckpt_chain_hashes(t, stride)] == want
        if len(want) > 2:   # incremental extension from a recorded key
            tail = gdn.ckpt_chain_hashes(t, stride, first_chunk=2, prev_key=want[1])
            assert [int(x) for x in tail] == want[2:]


@pytest.mark.parametrize("seed,capacity", [(3, 1), (4, 3), (5, 8), (6, 40)])
def test_random_operation_sequences_match_the_oracle(seed, capacity):
    rng = np.random.default_rng(seed)
    stride = 16
    # a small family of sequences sharing prefixes, so keys repeat and hits happen
    base = [rng.integers(0, 50, 160).astype(np.int32) for _ in range(4)]
    seqs = []
    for _ in range(24):
        b = base[int(rng.integers(0, 4))].copy()
        cut = int(rng.integers(0, 160))
        b[cut:] = rng.integers(0, 50, 160 - cut)
        seqs.append(b[: int(rng.integers(1, 161))])
    cpp, ref = gdn.CheckpointIndex(capacity), ci.CheckpointIndex(capacity)
    pinned = []
    next_slot = 1
    for step in range(600):
        op = rng.random()
        s = seqs[int(rng.integers(0, len(seqs)))]
        keys = ci.chain_hashes(s.tolist(), stride)
        if op < 0.45 and keys:
            k = keys[int(rng.integers(0, len(keys)))]
            got, want = cpp.insert(k, next_slot), ref.insert(k, next_slot)
            assert got == want, (step, got, want)
            next_slot += 1
        elif op < 0.8:
            got = cpp.match(np.array(keys, dtype=np.uint64), len(s), stride)
            want = ref.match(keys, len(s), stride)
            assert got == want, (step, got, want)
            if want[2] is not None:
                pinned.append(want[2])
        elif op < 0.95 and pinned:
            k = pinned.pop(int(rng.integers(0, len(pinned))))
            cpp.release(k)
            ref.release(k)
        else:
            k = keys[0] if keys else 12345
            assert cpp.contains(k) == ref.contains(k)
        assert len(cpp) == len(ref)


def test_plan_restores_matches_per_request_matching():
    rng = np.random.default_rng(9)
    stride = 32
    prefix = rng.integers(0, 1000, 200).astype(np.int32)
    cpp, ref = gdn.CheckpointIndex(16), ci.CheckpointIndex(16)
    pk = ci.chain_hashes(prefix.tolist(), stride)
    for i, k in enumerate(pk[:5]):
        assert cpp.insert(k, 10 + i) == ref.insert(k, 10 + i)
    reqs = [np.concatenate([prefix[:n], rng.integers(0, 1000, m).astype(np.int32)])
            for n, m in ((0, 50), (40, 5), (100, 100), (200, 1), (64, 0), (65, 0), (31, 0))]
    live = list(range(1, len(reqs) + 1))
    ops, reach, keys = cpp.plan_restores(reqs, stride, live)
    for i, r in enumerate(reqs):
        want = ref.match(ci.chain_hashes(r.tolist(), stride), len(r), stride)
        assert (int(reach[i]), ops[i][2]) == want[:2]
        assert ops[i][:2] == (live[i], 1)
        assert (int(keys[i]) if want[2] is not None else None) == (want[2] if want[2] is not None else None)
    # 200 + 1 tokens: chunks 0..5 end below the final token, the deepest stored is chunk 4
    assert int(reach[3]) == 160 and ops[3][2] == 14
    assert int(reach[4]) == 32 and int(reach[5]) == 64 and ops[6][2] == -1
    # the restores then follow restore_slots' host rules: a miss is a cold start
    assert [o[2] >= 1 for o in ops] == [False, True, True, True, True, True, False]


def test_edge_cases_and_errors():
    idx = gdn.CheckpointIndex(1)
    assert idx.insert(7, 3) == ("stored", -1)
    assert idx.match(np.array([7], dtype=np.uint64), 33, 32) == (32, 3, 7)
    assert idx.insert(8, 4) == ("full", 4)          # the only entry is pinned
    idx.release(7)
    with pytest.raises(gdn.GdnError):
        idx.release(7)                                 # not pinned any more
    with pytest.raises(gdn.GdnError):
        idx.release(99)                                # not held
    assert idx.insert(8, 4) == ("stored", 3)
    assert idx.match(np.array([], dtype=np.uint64), 5, 32) == (0, -1, None)
    with pytest.raises(gdn.GdnError):
        gdn.CheckpointIndex(0)
    with pytest.raises(gdn.GdnError):
        gdn.ckpt_chain_hashes([1, 2, 3], 0)


def test_prefix_walkthrough_through_the_library(golden_dir):
    spec = json.load(open(os.path.join(golden_dir, "prefix_walkthrough.json")))
    idx = gdn.CheckpointIndex(64)
    slots = iter(range(1, 64))

    def index_match(keys, n, blk):
        reach, slot, key = idx.match(np.array(keys, dtype=np.uint64), n, blk)
        if key is not None:
            idx.release(key)
        return reach, key

    got = []
    for reach, save_key in _sglang_policy_walkthrough(spec, index_match):
        got.append(reach)
        if save_key is not None:
            idx.insert(save_key, next(slots))
    assert got[:7] == spec["prefix"][:7] and got[7] == 256


def test_finish_request_matches_the_oracle():
    rng = np.random.default_rng(11)
    cpp, ref = gdn.CheckpointIndex(5), ci.CheckpointIndex(5)
    for step in range(300):
        key = None if rng.random() < 0.2 else int(rng.integers(1, 12))
        live = int(rng.integers(0, 40))
        track = [int(rng.integers(0, 40)), int(rng.integers(0, 40))]
        nxt = int(rng.integers(0, 2))
        if rng.random() < 0.3 and len(ref):
            k = next(iter(ref.entries))   # pin one entry now and then
            assert cpp.match(np.array([k], dtype=np.uint64), 2, 1) == ref.match([k], 2, 1)
        assert cpp.finish_request(key, live, track, nxt) == ci.finish_request(ref, key, live, track, nxt), step
        assert len(cpp) == len(ref)
