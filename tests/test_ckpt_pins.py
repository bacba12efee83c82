"""Pins of the checkpoint-index oracle (CPU): the hash against its published
test vectors, the match rules of the page "Qwen3.5 Linear-State Prefix Cache"
(section 6.2), the recency and reference-count rules, and the prefix-sharing
walk-through of the page "SGLang Mamba Radix Cache 深度解析" under that page's
save policy."""
import json
import os

import pytest

from oracle import ckpt_index as ci


def test_fnv1a64_published_vectors():
    """FNV-1a 64-bit test vectors of the FNV reference (empty string, 'a', 'foobar')."""
    assert ci.fnv1a64(b"") == 0xCBF29CE484222325
    assert ci.fnv1a64(b"a") == 0xAF63DC4C8601EC8C
    assert ci.fnv1a64(b"foobar") == 0x85944171F73967E8


def test_chain_keys_cover_the_whole_prefix_and_extend_incrementally():
    a = list(range(1000))
    b = a[:512] + [7] * 488
    ka, kb = ci.chain_hashes(a, 128), ci.chain_hashes(b, 128)
    assert len(ka) == 7 and ka[:4] == kb[:4] and all(x != y for x, y in zip(ka[4:], kb[4:]))
    # chunk 4 differs, so every later key differs although chunks 5, 6 of b equal each other
    head = ci.chain_hashes(a[:300], 128)
    assert head == ka[:2]
    assert head + ci.chain_hashes(a, 128, first_chunk=2, prev_key=head[-1]) == ka
    # a partial last chunk has no key
    assert len(ci.chain_hashes(a[:255], 128)) == 1


def _index_with(keys_slots, capacity=16):
    idx = ci.CheckpointIndex(capacity)
    for k, s in keys_slots:
        assert idx.insert(k, s) == ("stored", -1)
    return idx


def test_match_only_below_the_final_token():
    """A chunk counts only if it ends strictly below the final token."""
    keys = ci.chain_hashes(list(range(512)), 256)
    idx = _index_with([(keys[0], 3), (keys[1], 5)])
    assert idx.match(keys, 512, 256)[:2] == (256, 3)       # chunk 1 ends at the final token
    assert idx.match(keys, 513, 256)[:2] == (512, 5)
    assert idx.match(keys, 256, 256) == (0, -1, None)      # one chunk, not below the final token


def test_match_allows_gaps_and_takes_only_the_deepest_hit():
    keys = ci.chain_hashes(list(range(1024)), 128)
    idx = _index_with([(keys[0], 1), (keys[3], 2), (keys[5], 4)])
    reach, slot, key = idx.match(keys, 1024, 128)
    assert (reach, slot, key) == (768, 4, keys[5])          # misses at 1, 2, 4 are skipped
    assert idx.entries[keys[5]][1] == 1
    assert idx.entries[keys[0]][1] == 0 and idx.entries[keys[3]][1] == 0
    idx.release(keys[5])
    assert idx.entries[keys[5]][1] == 0
    with pytest.raises(ValueError):
        idx.release(keys[5])


def test_probing_keeps_the_recency_order_and_taking_pins():
    """contains() leaves the LRU order, find() promotes and pins: eviction takes
    the least recent unpinned entry."""
    k = [101, 102, 103]
    idx = _index_with([(k[0], 1), (k[1], 2), (k[2], 3)], capacity=3)
    assert idx.contains(k[0])                  # probe only
    assert idx.insert(104, 4) == ("stored", 1)   # k0 still least recent -> evicted
    idx.find(k[1])                             # k1 most recent and pinned
    assert idx.insert(105, 5) == ("stored", 3)   # k2 is now the least recent
    assert idx.insert(106, 6) == ("stored", 4)   # 104 next; k1 pinned
    assert idx.insert(k[1], 9) == ("present", 9)
    idx2 = _index_with([(1, 1)], capacity=1)
    idx2.find(1)
    assert idx2.insert(2, 2) == ("full", 2)


def _sglang_policy_walkthrough(spec, index_match):
    """Run the page's requests through an index with the page's save policy: a
    request is served from the deepest checkpoint below its final token; it then
    keeps one state, at the aligned fork point if its path forked beyond the
    served prefix (the longest aligned prefix shared with an earlier request),
    otherwise at its own last aligned point."""
    blk = spec["block"]
    ids = {}
    seqs, got = [], []
    for blocks in spec["requests"]:
        toks = [ids.setdefault(name, len(ids) + 1) for name in blocks for _ in range(blk)]
        keys = ci.chain_hashes(toks, blk)
        reach, key = index_match(keys, len(toks), blk)
        got.append(reach)
        shared = 0
        for s in seqs:
            n = 0
            while n < min(len(s), len(toks)) and s[n] == toks[n]:
                n += 1
            shared = max(shared, n // blk * blk)
        save = shared if shared > reach else len(toks) // blk * blk
        seqs.append(toks)
        yield got[-1], keys[save // blk - 1] if save else None


def test_prefix_walkthrough_from_the_page(golden_dir):
    """R1..R7 get the cached prefixes the page prints; R8 (the same 512 tokens as
    R7) gets 256 here because a checkpoint must end strictly below the final
    token, where the page's tree gives 512 (reading recorded in the design notes)."""
    spec = json.load(open(os.path.join(golden_dir, "prefix_walkthrough.json")))
    idx = ci.CheckpointIndex(64)
    slots = iter(range(1, 64))

    def index_match(keys, n, blk):
        reach, slot, key = idx.match(keys, n, blk)
        if key is not None:
            idx.release(key)
        return reach, key

    got = []
    for reach, save_key in _sglang_policy_walkthrough(spec, index_match):
        got.append(reach)
        if save_key is not None:
            idx.insert(save_key, next(slots))
    assert got[:7] == spec["prefix"][:7]
    assert got[7] == 256 and spec["prefix"][7] == 512


def test_finish_keeps_the_other_track_slot_as_the_page_shows():
    """extra_buffer mode: track slots [B, C] with next = 1 -> slot B (index 0) goes
    to the cache, C and the live slot A are released; without a tracked boundary
    everything is released; a key already held sends the kept slot back too."""
    A, Bs, Cs = 3, 7, 9
    idx = ci.CheckpointIndex(4)
    assert ci.finish_request(idx, 111, A, [Bs, Cs], 1) == [A, Cs]
    assert idx.entries[111][0] == Bs
    assert ci.finish_request(idx, None, A, [Bs, Cs], 0) == [A, Bs, Cs]
    assert ci.finish_request(idx, 111, A, [5, 6], 0) == [A, 5, 6]
