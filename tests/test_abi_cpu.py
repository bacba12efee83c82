"""Host-side checks of the C ABI that need no GPU: the library loads, exports
every entry point the header declares, sizes pools like the oracle and the
pages, and rejects bad arguments before launching anything."""
import ctypes as ct
import os
import re

import pytest

import gated_delta_rule_slot_amd as gdn
from gated_delta_rule_slot_amd import _binding as B
import oracle

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def header_functions():
    text = "".join(open(os.path.join(ROOT, "include", f)).read()
                   for f in sorted(os.listdir(os.path.join(ROOT, "include"))) if f.endswith(".h"))
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?[a-z_0-9]+\s*\*?\s*([a-z_0-9]+)\s*\(", text, flags=re.M)))


def test_library_exports_every_declared_function():
    names = header_functions()
    assert {"state_pool_bytes", "state_pool_create", "state_pool_destroy", "gdn_last_error",
            "conv_gdn_prefill_chunked", "gdn_prefill_workspace_bytes", "gdn_decode_step",
            "track_snapshot", "restore_slots", "gdn_verify_tree",
            "gdn_accept_scatter", "replayssm_ring_bytes", "replayssm_verify",
            "replayssm_commit", "ckpt_chain_hashes", "ckpt_index_create", "ckpt_index_destroy",
            "ckpt_index_size", "ckpt_index_contains", "ckpt_index_match", "ckpt_index_release",
            "ckpt_index_insert", "ckpt_plan_restores", "ckpt_finish_request"} <= set(names)
    lib = ct.CDLL(B.LIB_PATH)
    for n in names:
        assert hasattr(lib, n), n


@pytest.mark.parametrize("shape", [
    (69, 52, 12, 128, 128, 0), (69, 81, 12, 128, 128, 1), (1, 8, 2, 16, 16, 0),
    (24, 81, 32, 128, 128, 0), (1, 512, 32, 128, 128, 0), (69, 1024, 12, 128, 128, 1)])
def test_pool_bytes_match_oracle(shape):
    L, N, H, K, V, dt = shape
    assert gdn.state_pool_bytes(L, N, H, K, V, dt) == oracle.pool_bytes(L, N, H, K, V, dt)


def _desc(**kw):
    d = dict(layers=1, slots=8, heads=2, head_k=16, head_v=16, conv_kernel=4,
             ssm_dtype=B.GDN_F32, conv_dtype=B.GDN_BF16, ssm_base=0x10000, conv_base=0x20000,
             err_word=None)
    d.update(kw)
    return B.PoolDesc(*[d[f] for f, _ in B.PoolDesc._fields_])


def _create(**kw):
    h = ct.c_void_p()
    st = B._lib.state_pool_create(ct.byref(_desc(**kw)), ct.byref(h))
    return st, h


@pytest.mark.parametrize("kw,status", [
    (dict(), 0),
    (dict(conv_kernel=3), -3),
    (dict(head_k=16, head_v=32), -3),
    (dict(head_k=48, head_v=48), -3),
    (dict(ssm_dtype=7), -1),
    (dict(conv_dtype=B.GDN_F32), -3),
    (dict(slots=1), -1),
    (dict(ssm_base=0x10008), -3),
    (dict(conv_base=None), -1),
])
def test_pool_create_validation(kw, status):
    st, h = _create(**kw)
    assert st == status, B.last_error()
    if st == 0:
        B._lib.state_pool_destroy(h)
    else:
        assert B.last_error()


def test_calls_reject_bad_arguments_before_launch():
    st, h = _create()
    assert st == 0
    try:
        fake = ct.c_void_p(0x30000)
        # bad layer
        assert B._lib.gdn_decode_step(h, 1, 1, fake, fake, fake, fake, 0, fake, 1.0, 1, fake,
                                      None, 0, None, None, None) == -2
        # unknown alpha mode, unknown flag bits
        assert B._lib.gdn_decode_step(h, 0, 1, fake, fake, fake, fake, 5, fake, 1.0, 1, fake,
                                      None, 0, None, None, None) == -1
        assert B._lib.gdn_decode_step(h, 0, 1, fake, fake, fake, fake, 0, fake, 1.0, 64, fake,
                                      None, 0, None, None, None) == -1
        # tracking without its tables
        assert B._lib.gdn_decode_step(h, 0, 1, fake, fake, fake, fake, 0, fake, 1.0, 1, fake,
                                      None, 256, None, None, None) == -1
        # snapshot interval not a multiple of 64
        assert B._lib.conv_gdn_prefill_chunked(
            h, 0, 1, 64, 64, fake, fake, fake, fake, fake, fake, fake, 0, fake, 1.0, 1, fake,
            32, fake, fake, fake, 1 << 30, None) == -1
        # workspace below the minimum
        assert B._lib.conv_gdn_prefill_chunked(
            h, 0, 1, 64, 64, fake, fake, fake, fake, fake, fake, fake, 0, fake, 1.0, 1, fake,
            0, None, None, fake, 16, None) == -1
        assert "workspace" in B.last_error()
        # prefill path bits: both at once, and the one-kernel path at head dim 16
        # (it serves head dim 128 only)
        assert B._lib.conv_gdn_prefill_chunked(
            h, 0, 1, 64, 64, fake, fake, fake, fake, fake, fake, fake, 0, fake, 1.0,
            1 | B.PREFILL_ONE_KERNEL | B.PREFILL_TWO_KERNEL, fake, 0, None, None, fake, 1 << 30,
            None) == -1
        assert B._lib.conv_gdn_prefill_chunked(
            h, 0, 1, 64, 64, fake, fake, fake, fake, fake, fake, fake, 1, fake, 1.0,
            1 | B.PREFILL_ONE_KERNEL, fake, 0, None, None, fake, 1 << 30, None) == -3
        assert "one-kernel" in B.last_error()
        assert B._lib.conv_gdn_prefill_chunked(
            h, 0, 1, 64, 64, fake, fake, fake, fake, fake, fake, fake, 0, fake, 1.0, 1 | 64, fake,
            0, None, None, fake, 1 << 30, None) == -1
        # the two-kernel path needs its workspace (tiny batch: the library's choice)
        assert B._lib.conv_gdn_prefill_chunked(
            h, 0, 1, 64, 64, fake, fake, fake, fake, fake, fake, fake, 0, fake, 1.0,
            1 | B.SNAP_LAST_ONLY, fake, 0, None, None, None, 0, None) == -1
        assert "workspace" in B.last_error()
        # the allocation-free prefill refuses a two-kernel batch beyond its fixed scratch
        # (before touching the device)
        assert B._lib.conv_gdn_prefill_chunked_noalloc(
            h, 0, 65535, 64, 64, fake, fake, fake, fake, fake, fake, fake, 0, fake, 1.0, 1, fake,
            0, None, None, None) == -2
        assert "scratch" in B.last_error()
        assert B._lib.conv_gdn_prefill_chunked_noalloc(
            h, 0, 1, 64, 64, fake, fake, fake, fake, fake, fake, fake, 0, fake, 1.0, 1, fake,
            32, fake, fake, None) == -1
        # layer range for copies
        assert B._lib.track_snapshot(h, 0, 2, 1, fake, fake, None) == -2
        # draft trees: node count range, required buffers, alignment of node buffers
        v = B._lib.gdn_verify_tree
        args = [fake, fake, fake, fake, fake, 0, fake, 1.0, 1, fake, fake, fake, None]
        assert v(h, 0, 1, 0, *args) == -2
        assert v(h, 0, 1, B.MAX_TREE_NODES + 1, *args) == -2
        assert v(h, 1, 1, 4, *args) == -2
        bad = list(args)
        bad[11] = None      # node_conv
        assert v(h, 0, 1, 4, *bad) == -1
        bad = list(args)
        bad[10] = ct.c_void_p(0x30008)  # node_ssm not 16-byte aligned
        assert v(h, 0, 1, 4, *bad) == -3
        assert v(h, 0, 0, 4, *args) == 0    # empty batch launches nothing
        sc = B._lib.gdn_accept_scatter
        assert sc(h, 0, 1, 4, fake, fake, fake, fake, -1, fake, fake, fake, fake, None) == -1
        assert sc(h, 0, 1, 4, fake, fake, fake, None, 256, fake, fake, fake, fake, None) == -1
        assert sc(h, 0, 1, 4, fake, fake, None, None, 0, None, None, fake, fake, None) == -1
        assert sc(h, 0, 1, 2000, fake, fake, fake, None, 0, None, None, fake, fake, None) == -2
        assert sc(h, 0, 0, 4, fake, fake, fake, None, 0, None, None, fake, fake, None) == 0
        # ReplaySSM: ring shape, draft range, alignment, tracking tables
        ring = B.RingDesc(16, 1, 0x40000, 0x50000, 0x60000, 0x70000, 0x80000)
        rv, rc = B._lib.replayssm_verify, B._lib.replayssm_commit
        vargs = [fake, fake, fake, fake, fake, 1.0, 1, fake, None]
        assert rv(h, ct.byref(ring), 0, 1, 17, *vargs) == -2
        assert rv(h, ct.byref(ring), 0, 1, 0, *vargs) == -2
        assert rv(h, None, 0, 1, 4, *vargs) == -1
        bad = B.RingDesc(0, 1, 0x40000, 0x50000, 0x60000, 0x70000, 0x80000)
        assert rv(h, ct.byref(bad), 0, 1, 1, *vargs) == -2
        bad = B.RingDesc(16, 3, 0x40000, 0x50000, 0x60000, 0x70000, 0x80000)
        assert rv(h, ct.byref(bad), 0, 1, 1, *vargs) == -1
        bad = B.RingDesc(16, 1, 0x40008, 0x50000, 0x60000, 0x70000, 0x80000)
        assert rv(h, ct.byref(bad), 0, 1, 1, *vargs) == -3
        assert rv(h, ct.byref(ring), 0, 0, 4, *vargs) == 0
        assert rc(h, ct.byref(ring), 0, 1, fake, fake, 1, None, 256, None, None, None) == -1
        assert rc(h, ct.byref(ring), 0, 1, fake, None, 1, None, 0, None, None, None) == -1
        assert rc(h, ct.byref(ring), 0, 1, fake, fake, 1, None, -1, None, None, None) == -1
        assert rc(h, ct.byref(ring), 0, 0, fake, fake, 1, None, 0, None, None, None) == 0
    finally:
        B._lib.state_pool_destroy(h)


def test_restore_rules_without_copies_are_host_only():
    """Ops that need no copy are decided on the host (no GPU needed): not
    requested -> unchanged, bad source or destination -> COLD_START (0),
    src == dst -> RESTORED (1)."""
    st, h = _create()
    assert st == 0
    try:
        pool = B.StatePool(h, None, None, None, (1, 8, 2, 16, 16))
        ops = [(3, 0, 2), (3, 1, -1), (3, 1, 8), (0, 1, 2), (4, 1, 4)]
        got = B.restore_slots(pool, ops, [7, 7, 7, 7, 7], stream=type("S", (), {"cuda_stream": 0})())
        assert got == [7, 0, 0, 0, 1]
        pool.handle = None
    finally:
        B._lib.state_pool_destroy(h)


def test_restore_rejects_chained_and_duplicate_copies():
    """The copies of one restore call run in parallel, so a call where a copy
    reads a slot another copy writes, or two copies write one slot, is rejected
    on the host with has_initial_state untouched (nothing is launched)."""
    st, h = _create()
    assert st == 0
    try:
        S = type("S", (), {"cuda_stream": 0})()
        pool = B.StatePool(h, None, None, None, (1, 8, 2, 16, 16))
        for ops in ([(3, 1, 2), (5, 1, 3)],           # 2 -> 3 and 3 -> 5: a chain
                    [(5, 1, 3), (3, 1, 2)],           # the same, listed the other way
                    [(3, 1, 2), (3, 1, 4)],           # two copies into slot 3
                    [(4, 1, 6), (6, 1, 4)]):          # a swap
            with pytest.raises(RuntimeError, match="restore_slots"):
                B.restore_slots(pool, ops, [7] * len(ops), stream=S)
        hi = (ct.c_int64 * 2)(7, 7)
        arr = (B.RestoreOp * 2)(B.RestoreOp(3, 1, 2), B.RestoreOp(5, 1, 3))
        assert B._lib.restore_slots(h, 2, arr, hi, None) == -1
        assert list(hi) == [7, 7]
        # no copy is involved when src == dst, a request is off or a source is
        # missing, so these do not conflict with the copy into 3
        got = B.restore_slots(pool, [(3, 1, 3), (2, 0, 3), (3, 1, -1)], [7, 7, 7], stream=S)
        assert got == [1, 7, 0]
        pool.handle = None
    finally:
        B._lib.state_pool_destroy(h)


def test_workspace_query():
    st, h = _create()
    assert st == 0
    try:
        n = ct.c_size_t()
        assert B._lib.gdn_prefill_workspace_bytes(h, 2, 256, ct.byref(n)) == 0
        m = ct.c_size_t()
        assert B._lib.gdn_prefill_workspace_bytes(h, 2, 64, ct.byref(m)) == 0
        assert n.value > m.value > 0
    finally:
        B._lib.state_pool_destroy(h)


def test_prefill_argument_checks_before_launch():
    """Range, pointer, enum and alignment checks of conv_gdn_prefill_chunked, each
    answered on the host with the status the header documents (nothing launches)."""
    st, h = _create()
    assert st == 0
    fake, odd = ct.c_void_p(0x30000), ct.c_void_p(0x30008)  # 16-byte aligned / not

    def call(**kw):
        a = dict(layer=0, batch=1, total=64, maxlen=64, cu=fake, slots=fake, has=fake, start=fake,
                 x=fake, w=fake, alpha=fake, amode=0, beta=fake, flags=1, out=fake, snap=0,
                 track=None, nxt=None, ws=fake, wsb=1 << 30)
        a.update(kw)
        return B._lib.conv_gdn_prefill_chunked(
            h, a["layer"], a["batch"], a["total"], a["maxlen"], a["cu"], a["slots"], a["has"],
            a["start"], a["x"], a["w"], a["alpha"], a["amode"], a["beta"], 1.0, a["flags"], a["out"],
            a["snap"], a["track"], a["nxt"], a["ws"], a["wsb"], None)

    try:
        assert call(batch=70000) == -2                 # batch outside [0, 65535]
        assert call(total=-1) == -2                    # negative token count
        assert call(batch=0, cu=None, x=None) == 0     # an empty batch launches nothing
        assert call(cu=None) == -1                     # a required pointer is NULL
        assert call(x=None) == -1                      # x is NULL with tokens to read
        assert call(amode=7) == -1                     # unknown decay layout
        assert call(w=odd) == -3                       # conv_w not 16-byte aligned
        assert call(x=odd) == -3
        assert call(out=odd) == -3
        assert call(alpha=odd) == -3
        assert "aligned" in B.last_error()
        # the two-kernel path: a workspace that is not 256-byte aligned
        assert call(ws=ct.c_void_p(0x30010)) == -3
        assert "workspace" in B.last_error()
        assert call(layer=5) == -2                     # layer outside the pool
    finally:
        B._lib.state_pool_destroy(h)


def test_decode_argument_checks_before_launch():
    """The decode entry's range, pointer, enum and alignment checks (nothing launches)."""
    st, h = _create()
    assert st == 0
    fake, odd = ct.c_void_p(0x30000), ct.c_void_p(0x30008)

    def call(**kw):
        a = dict(batch=1, slots=fake, x=fake, w=fake, alpha=fake, amode=0, beta=fake, out=fake,
                 ti=0)
        a.update(kw)
        return B._lib.gdn_decode_step(h, 0, a["batch"], a["slots"], a["x"], a["w"], a["alpha"],
                                      a["amode"], a["beta"], 1.0, 1, a["out"], None, a["ti"], None,
                                      None, None)

    try:
        assert call(batch=70000) == -2
        assert call(batch=0, x=None) == 0
        assert call(out=None) == -1
        assert call(amode=7) == -1
        assert call(ti=-1) == -1
        assert call(w=odd) == -3
        assert call(x=odd) == -3
        assert call(alpha=odd) == -3
    finally:
        B._lib.state_pool_destroy(h)
