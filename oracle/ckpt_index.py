"""Plain-Python oracle of the host checkpoint index of linear states.

TEST INFRASTRUCTURE, NOT PRODUCT CODE.  Only ``tests/`` and the benchmark may
import this module; the library never does.  It restates the rules of the page
"Qwen3.5 Linear-State Prefix Cache" (sections 4, 5.1, 5.2 and 6.2) as directly
as possible: a dict from key to entry, a Python list for the recency order.

* Keys are chained per-chunk hashes: the key of chunk i covers tokens
  [0, (i + 1) * stride) and is computed from the key of chunk i - 1 and the
  chunk's own tokens (section 4: a hash domain of its own, step chunk_stride,
  precomputed once and extended as the sequence grows).  The hash is 64-bit
  FNV-1a (Fowler, Noll, Vo; offset basis 14695981039346656037, prime
  1099511628211) over the previous key's 8 little-endian bytes followed by the
  chunk's tokens as 4 little-endian bytes each; chunk 0 starts from the offset
  basis alone.
* match (section 6.2): probe every whole chunk that ends strictly below the
  final token, i.e. (i + 1) * stride <= n_tokens - 1; gaps are allowed; the
  deepest hit wins and only it is taken: reach = (i + 1) * stride.  Probing
  does not touch the recency order (contains); taking the hit does (find:
  reference count + 1, most recent).
* insert (section 5.2, insert_with_recorded_hash): a checkpoint is stored under
  the key recorded at its boundary.  A key already present keeps its slot and
  the offered slot comes back to the caller.  A full index evicts the least
  recently used entry whose reference count is 0 and returns its slot; if every
  entry is pinned the insert is refused.
* release: reference count - 1 once the restore copied from the slot.
* finish (page "SGLang Mamba Radix Cache 深度解析", cache_finished_req and
  free_mamba_cache in extra_buffer mode): the track slot other(next) holds the
  last tracked boundary and goes to the index under that boundary's key, no
  copy; the live slot and track slot next are freed, and so is the kept slot
  when the index does not take it (key already held, or every entry pinned),
  together with any slot an insert evicts.
"""
from __future__ import annotations

FNV_OFFSET = 14695981039346656037
FNV_PRIME = 1099511628211
MASK64 = (1 << 64) - 1


def fnv1a64(data: bytes, h: int = FNV_OFFSET) -> int:
    for byte in data:
        h ^= byte
        h = (h * FNV_PRIME) & MASK64
    return h


def chain_hashes(tokens, stride, first_chunk=0, prev_key=None):
    """Keys of the whole chunks first_chunk .. len(tokens)//stride - 1."""
    out = []
    key = prev_key
    for i in range(first_chunk, len(tokens) // stride):
        data = b"" if key is None else key.to_bytes(8, "little")
        for t in tokens[i * stride:(i + 1) * stride]:
            data += (int(t) & 0xFFFFFFFF).to_bytes(4, "little")
        key = fnv1a64(data)
        out.append(key)
    return out


class CheckpointIndex:
    def __init__(self, capacity):
        self.capacity = capacity
        self.entries = {}      # key -> [slot, refs]
        self.order = []        # least recent first

    def __len__(self):
        return len(self.entries)

    def contains(self, key):
        return key in self.entries

    def find(self, key):
        e = self.entries[key]
        e[1] += 1
        self.order.remove(key)
        self.order.append(key)
        return e[0]

    def match(self, keys, n_tokens, stride):
        """Returns (reach_tokens, slot, key); (0, -1, None) on a miss."""
        best = -1
        for i, k in enumerate(keys):
            if (i + 1) * stride > n_tokens - 1:
                break
            if self.contains(k):
                best = i
        if best < 0:
            return 0, -1, None
        key = keys[best]
        return (best + 1) * stride, self.find(key), key

    def release(self, key):
        e = self.entries[key]
        if e[1] <= 0:
            raise ValueError("release without a matching find")
        e[1] -= 1

    def insert(self, key, slot):
        """Returns (status, slot_back): status 'stored' (slot_back = evicted slot
        or -1), 'present' (slot_back = the offered slot), 'full' (refused)."""
        if key in self.entries:
            return "present", slot
        evicted = -1
        if len(self.entries) >= self.capacity:
            victim = next((k for k in self.order if self.entries[k][1] == 0), None)
            if victim is None:
                return "full", slot
            evicted = self.entries.pop(victim)[0]
            self.order.remove(victim)
        self.entries[key] = [slot, 0]
        self.order.append(key)
        return "stored", evicted


def finish_request(index, key, live_slot, track_slots, next_track_idx):
    """Slots the caller frees when a request finishes (see the module notes);
    key None means no boundary was tracked, so every slot is freed."""
    keep = track_slots[1 - (next_track_idx & 1)]
    freed = [live_slot, track_slots[next_track_idx & 1]]
    if key is None:
        freed.append(keep)
    else:
        status, back = index.insert(key, keep)
        if status == "stored":
            if back >= 0:
                freed.append(back)
        else:
            freed.append(back)
    return [s for s in freed if s > 0]
