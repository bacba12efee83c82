"""numpy/ctypes front end of the CPU oracle.

TEST INFRASTRUCTURE, NOT PRODUCT CODE.  Only ``tests/``, the package smoke
check and the benchmark's CPU-baseline leg may import this module.  It never
touches a GPU and shares no code with the HIP library; the product path does
not import it.

Arrays are numpy.  bf16 data travels as ``uint16`` bit patterns.  The pool is
held in host memory with exactly the byte layout of the device pool:

    ssm  [layers][slots][heads][head_v][head_k]  float32 or bf16
    conv [layers][slots][3][C]                   bf16,  C = heads*(2*head_k+head_v)
"""
from __future__ import annotations

import ctypes as ct
import os

import numpy as np

from . import build as _build

SSM_F32, SSM_BF16 = 0, 1
ALPHA_PER_HEAD, ALPHA_PER_CHANNEL = 0, 1
L2NORM_K, L2NORM_Q, CONV_SILU = 1, 2, 4

_i32p = ct.POINTER(ct.c_int32)
_i64p = ct.POINTER(ct.c_int64)
_u16p = ct.POINTER(ct.c_uint16)
_f32p = ct.POINTER(ct.c_float)
_f64p = ct.POINTER(ct.c_double)


class _Pool(ct.Structure):
    _fields_ = [
        ("layers", ct.c_int32), ("slots", ct.c_int32), ("heads", ct.c_int32),
        ("head_k", ct.c_int32), ("head_v", ct.c_int32), ("ssm_dtype", ct.c_int32),
        ("ssm", ct.c_void_p), ("conv", _u16p),
    ]


class _Ring(ct.Structure):
    _fields_ = [
        ("positions", ct.c_int32), ("alpha_mode", ct.c_int32), ("rawk", _u16p), ("rawv", _u16p),
        ("g", _f32p), ("beta", _f32p), ("xrow", _u16p),
    ]


class RestoreOp(ct.Structure):
    _fields_ = [
        ("linear_state_id", ct.c_int32),
        ("restore_requested", ct.c_int32),
        ("restore_src_slot_id", ct.c_int32),
    ]


_LIBS: dict = {}


def lib(precision: str = "f64"):
    """Load liboracle_<precision>.so, building it if it is absent."""
    if precision not in ("f64", "f32"):
        raise ValueError(precision)
    if precision in _LIBS:
        return _LIBS[precision]
    path = _build.lib_path(precision)
    if not os.path.exists(path):
        _build.build()
    L = ct.CDLL(path)
    L.oracle_real_bytes.restype = ct.c_int
    L.oracle_num_threads.restype = ct.c_int
    L.oracle_pool_bytes.argtypes = [ct.c_int32] * 6 + [ct.POINTER(ct.c_size_t)] * 2
    L.oracle_prefill.argtypes = [
        ct.POINTER(_Pool), ct.c_int32, ct.c_int32, _i32p, _i32p, _i32p, _i32p,
        _u16p, _u16p, _f32p, ct.c_int32, _f32p, ct.c_float, ct.c_uint32, _u16p,
        ct.c_int32, _i32p, _i32p, _f64p, _f64p,
    ]
    L.oracle_decode_step.argtypes = [
        ct.POINTER(_Pool), ct.c_int32, ct.c_int32, _i32p, _u16p, _u16p, _f32p,
        ct.c_int32, _f32p, ct.c_float, ct.c_uint32, _u16p, _i32p, ct.c_int32,
        _i32p, _i32p, _f64p, _f64p,
    ]
    L.oracle_track_snapshot.argtypes = [ct.POINTER(_Pool), ct.c_int32, ct.c_int32,
                                        ct.c_int32, _i32p, _i32p]
    L.oracle_restore_slots.argtypes = [ct.POINTER(_Pool), ct.c_int32,
                                       ct.POINTER(RestoreOp), _i64p]
    L.oracle_verify_tree.argtypes = [
        ct.POINTER(_Pool), ct.c_int32, ct.c_int32, ct.c_int32, _i32p, _i32p, _u16p, _u16p,
        _f32p, ct.c_int32, _f32p, ct.c_float, ct.c_uint32, _u16p, ct.c_void_p, _u16p, _f64p,
    ]
    L.oracle_accept_scatter.argtypes = [
        ct.POINTER(_Pool), ct.c_int32, ct.c_int32, ct.c_int32, _i32p, _i32p, _i32p, _i32p,
        ct.c_int32, _i32p, _i32p, ct.c_void_p, _u16p,
    ]
    L.oracle_ring_bytes.argtypes = [ct.POINTER(_Pool), ct.c_int32, ct.c_int32, ct.POINTER(ct.c_size_t)]
    L.oracle_replay_verify.argtypes = [
        ct.POINTER(_Pool), ct.POINTER(_Ring), ct.c_int32, ct.c_int32, ct.c_int32, _i32p, _u16p,
        _u16p, _f32p, ct.c_int32, _f32p, ct.c_float, ct.c_uint32, _u16p, _f64p,
    ]
    L.oracle_replay_commit.argtypes = [
        ct.POINTER(_Pool), ct.POINTER(_Ring), ct.c_int32, ct.c_int32, _i32p, _i32p, ct.c_int32,
        ct.c_uint32, _i32p, ct.c_int32, _i32p, _i32p,
    ]
    L.oracle_recurrence_head.argtypes = [ct.c_int32] * 3 + [_f64p] * 5 + [ct.c_double, _f64p, _f64p]
    L.oracle_recurrence_head.restype = None
    L.oracle_chunked_head_f64.argtypes = [ct.c_int32] * 4 + [_f64p] * 5 + [ct.c_double, _f64p, _f64p]
    L.oracle_chunked_head_f64.restype = None
    L.oracle_bf16_round.argtypes = [ct.c_double]
    L.oracle_bf16_round.restype = ct.c_uint16
    L.oracle_bf16_widen.argtypes = [ct.c_uint16]
    L.oracle_bf16_widen.restype = ct.c_double
    _LIBS[precision] = L
    return L


def _p(a, typ):
    if a is None:
        return None
    return a.ctypes.data_as(typ)


def _c(a, dtype):
    """Contiguous array of the exact dtype (no silent value conversion for bf16)."""
    a = np.asarray(a)
    if a.dtype != np.dtype(dtype):
        if dtype == np.uint16:
            raise TypeError("bf16 data must be passed as uint16 bit patterns")
        a = a.astype(dtype)
    return np.ascontiguousarray(a)


def num_threads(precision="f64") -> int:
    return lib(precision).oracle_num_threads()


def pool_bytes(layers, slots, heads, head_k, head_v, ssm_dtype, precision="f64"):
    s, c = ct.c_size_t(), ct.c_size_t()
    rc = lib(precision).oracle_pool_bytes(layers, slots, heads, head_k, head_v, ssm_dtype,
                                          ct.byref(s), ct.byref(c))
    if rc:
        raise ValueError("bad pool shape")
    return s.value, c.value


class Pool:
    """Host image of the state pool."""

    def __init__(self, layers, slots, heads, head_k, head_v, ssm_dtype=SSM_F32):
        self.layers, self.slots, self.heads = layers, slots, heads
        self.head_k, self.head_v, self.ssm_dtype = head_k, head_v, ssm_dtype
        sb, cb = pool_bytes(layers, slots, heads, head_k, head_v, ssm_dtype)
        self.ssm_bytes = np.zeros(sb, dtype=np.uint8)
        self.conv_bytes = np.zeros(cb, dtype=np.uint8)

    @property
    def channels(self):
        return self.heads * (2 * self.head_k + self.head_v)

    def ssm(self):
        """Typed view [L][N][H][V][K]: float32, or uint16 bf16 bits."""
        dt = np.float32 if self.ssm_dtype == SSM_F32 else np.uint16
        return self.ssm_bytes.view(dt).reshape(self.layers, self.slots, self.heads,
                                               self.head_v, self.head_k)

    def conv(self):
        """uint16 (bf16 bits) view [L][N][3][C]."""
        return self.conv_bytes.view(np.uint16).reshape(self.layers, self.slots, 3, self.channels)

    def copy(self):
        p = Pool(self.layers, self.slots, self.heads, self.head_k, self.head_v, self.ssm_dtype)
        p.ssm_bytes[:] = self.ssm_bytes
        p.conv_bytes[:] = self.conv_bytes
        return p

    def _struct(self):
        return _Pool(self.layers, self.slots, self.heads, self.head_k, self.head_v,
                     self.ssm_dtype, self.ssm_bytes.ctypes.data_as(ct.c_void_p),
                     self.conv_bytes.ctypes.data_as(_u16p))


def prefill(pool: Pool, layer, cu_seqlens, slot_table, x, conv_w, alpha, alpha_mode, beta,
            has_initial_state=None, start_len=None, scale=1.0, flags=L2NORM_K,
            snap_interval=0, track_slots=None, next_track_idx=None, exact=False,
            precision="f64"):
    """Fold each request's tokens into its live slot (modifies ``pool``).

    Returns ``(out_bf16_bits[T,H,V], err)`` or, with ``exact=True``,
    ``(out, err, out_exact[T,H,V], state_exact[B,H,V,K])``."""
    cu = _c(cu_seqlens, np.int32)
    B = cu.shape[0] - 1
    T = int(cu[-1])
    H, V, K = pool.heads, pool.head_v, pool.head_k
    st = _c(slot_table, np.int32)
    hi = _c(has_initial_state if has_initial_state is not None else np.ones(B), np.int32)
    sl = _c(start_len if start_len is not None else np.zeros(B), np.int32)
    xs, w = _c(x, np.uint16), _c(conv_w, np.uint16)
    a, bt = _c(alpha, np.float32), _c(beta, np.float32)
    ts = _c(track_slots, np.int32) if track_slots is not None else None
    nt = _c(next_track_idx, np.int32) if next_track_idx is not None else None
    out = np.zeros((T, H, V), dtype=np.uint16)
    oe = np.zeros((T, H, V), dtype=np.float64) if exact else None
    se = np.zeros((B, H, V, K), dtype=np.float64) if exact else None
    ps = pool._struct()
    err = lib(precision).oracle_prefill(
        ct.byref(ps), layer, B, _p(cu, _i32p), _p(st, _i32p), _p(hi, _i32p), _p(sl, _i32p),
        _p(xs, _u16p), _p(w, _u16p), _p(a, _f32p), alpha_mode, _p(bt, _f32p), scale, flags,
        _p(out, _u16p), snap_interval, _p(ts, _i32p), _p(nt, _i32p), _p(oe, _f64p),
        _p(se, _f64p))
    if err & 4:
        raise ValueError("oracle_prefill: bad argument")
    return (out, err, oe, se) if exact else (out, err)


def decode_step(pool: Pool, layer, slot_table, x, conv_w, alpha, alpha_mode, beta,
                scale=1.0, flags=L2NORM_K, seq_len_after=None, track_interval=0,
                track_slots=None, next_track_idx=None, exact=False, precision="f64"):
    """One token per request; returns like :func:`prefill`."""
    st = _c(slot_table, np.int32)
    B = st.shape[0]
    H, V, K = pool.heads, pool.head_v, pool.head_k
    xs, w = _c(x, np.uint16), _c(conv_w, np.uint16)
    a, bt = _c(alpha, np.float32), _c(beta, np.float32)
    sla = _c(seq_len_after if seq_len_after is not None else np.ones(B), np.int32)
    ts = _c(track_slots, np.int32) if track_slots is not None else None
    nt = _c(next_track_idx, np.int32) if next_track_idx is not None else None
    out = np.zeros((B, H, V), dtype=np.uint16)
    oe = np.zeros((B, H, V), dtype=np.float64) if exact else None
    se = np.zeros((B, H, V, K), dtype=np.float64) if exact else None
    ps = pool._struct()
    err = lib(precision).oracle_decode_step(
        ct.byref(ps), layer, B, _p(st, _i32p), _p(xs, _u16p), _p(w, _u16p), _p(a, _f32p),
        alpha_mode, _p(bt, _f32p), scale, flags, _p(out, _u16p), _p(sla, _i32p),
        track_interval, _p(ts, _i32p), _p(nt, _i32p), _p(oe, _f64p), _p(se, _f64p))
    if err & 4:
        raise ValueError("oracle_decode_step: bad argument")
    return (out, err, oe, se) if exact else (out, err)


def track_snapshot(pool: Pool, layer_begin, layer_end, src_slots, dst_slots, precision="f64"):
    s, d = _c(src_slots, np.int32), _c(dst_slots, np.int32)
    ps = pool._struct()
    err = lib(precision).oracle_track_snapshot(ct.byref(ps), layer_begin, layer_end, s.shape[0],
                                               _p(s, _i32p), _p(d, _i32p))
    if err & 4:
        raise ValueError("oracle_track_snapshot: bad argument")
    return err


def restore_slots(pool: Pool, ops, has_initial_state, precision="f64"):
    """``ops``: list of (linear_state_id, restore_requested, restore_src_slot_id).
    ``has_initial_state``: int64 array, updated in place (also returned)."""
    arr = (RestoreOp * max(len(ops), 1))(*[RestoreOp(*o) for o in ops])
    hi = np.asarray(has_initial_state)
    if hi.dtype != np.int64 or not hi.flags.c_contiguous:
        raise TypeError("has_initial_state must be a contiguous int64 array")
    ps = pool._struct()
    err = lib(precision).oracle_restore_slots(ct.byref(ps), len(ops), arr, _p(hi, _i64p))
    if err & 4:
        raise ValueError("oracle_restore_slots: bad argument")
    return hi


def node_buffers(pool: Pool, batch, nodes):
    """Zeroed per-node buffers of a draft tree: (node_ssm [B][T][H][V][K] in the
    pool's ssm dtype, node_conv uint16 [B][T][3][C])."""
    dt = np.float32 if pool.ssm_dtype == SSM_F32 else np.uint16
    return (np.zeros((batch, nodes, pool.heads, pool.head_v, pool.head_k), dtype=dt),
            np.zeros((batch, nodes, 3, pool.channels), dtype=np.uint16))


def verify_tree(pool: Pool, layer, slot_table, parent, x, conv_w, alpha, alpha_mode, beta,
                scale=1.0, flags=L2NORM_K, exact=False, precision="f64"):
    """Verify a draft tree per request without touching the live slots.

    ``parent`` int [B][T] (-1 = the live slot), ``x`` uint16 [B][T][C], ``alpha``
    [B][T][H] or [B][T][H][K], ``beta`` [B][T][H].  Returns ``(out[B,T,H,V],
    node_ssm, node_conv, err)``, plus ``out_exact`` with ``exact=True``."""
    st = _c(slot_table, np.int32)
    par = _c(parent, np.int32)
    B, T = par.shape
    if st.shape != (B,):
        raise ValueError("slot_table must have one entry per request")
    H, V = pool.heads, pool.head_v
    xs, w = _c(x, np.uint16), _c(conv_w, np.uint16)
    a, bt = _c(alpha, np.float32), _c(beta, np.float32)
    out = np.zeros((B, T, H, V), dtype=np.uint16)
    oe = np.zeros((B, T, H, V), dtype=np.float64) if exact else None
    ns, nc = node_buffers(pool, B, T)
    ps = pool._struct()
    err = lib(precision).oracle_verify_tree(
        ct.byref(ps), layer, B, T, _p(st, _i32p), _p(par, _i32p), _p(xs, _u16p), _p(w, _u16p),
        _p(a, _f32p), alpha_mode, _p(bt, _f32p), scale, flags, _p(out, _u16p),
        ns.ctypes.data_as(ct.c_void_p), _p(nc, _u16p), _p(oe, _f64p))
    if err & 4:
        raise ValueError("oracle_verify_tree: bad argument")
    return (out, ns, nc, err, oe) if exact else (out, ns, nc, err)


def accept_scatter(pool: Pool, layer, slot_table, parent, accepted, node_ssm, node_conv,
                   seq_len_before=None, track_interval=0, track_slots=None,
                   next_track_idx=None, precision="f64"):
    """Copy each request's accepted node into its live slot (modifies ``pool``)
    and, across a multiple of ``track_interval``, into its ping-pong track slot.
    Returns the error bits."""
    st = _c(slot_table, np.int32)
    par = _c(parent, np.int32)
    B, T = par.shape
    acc = _c(accepted, np.int32)
    sb = _c(seq_len_before if seq_len_before is not None else np.zeros(B), np.int32)
    ts = _c(track_slots, np.int32) if track_slots is not None else None
    nt = _c(next_track_idx, np.int32) if next_track_idx is not None else None
    ns, nc = np.ascontiguousarray(node_ssm), _c(node_conv, np.uint16)
    ps = pool._struct()
    err = lib(precision).oracle_accept_scatter(
        ct.byref(ps), layer, B, T, _p(st, _i32p), _p(par, _i32p), _p(acc, _i32p), _p(sb, _i32p),
        track_interval, _p(ts, _i32p), _p(nt, _i32p), ns.ctypes.data_as(ct.c_void_p),
        _p(nc, _u16p))
    if err & 4:
        raise ValueError("oracle_accept_scatter: bad argument")
    return err


def ring_bytes(pool: Pool, positions, alpha_mode, precision="f64"):
    """Byte sizes (rawk, rawv, g, beta, xrow) of a ReplaySSM ring for the pool's shape."""
    b = (ct.c_size_t * 5)()
    ps = pool._struct()
    if lib(precision).oracle_ring_bytes(ct.byref(ps), positions, alpha_mode, b):
        raise ValueError("bad ring shape")
    return tuple(b[i] for i in range(5))


class Ring:
    """Host image of a ReplaySSM ring for a pool (zero-filled)."""

    def __init__(self, pool: Pool, positions, alpha_mode):
        L, N, H, K, V = pool.layers, pool.slots, pool.heads, pool.head_k, pool.head_v
        self.positions, self.alpha_mode = positions, alpha_mode
        self.rawk = np.zeros((L, N, H, positions, K), dtype=np.uint16)
        self.rawv = np.zeros((L, N, H, positions, V), dtype=np.uint16)
        gshape = (L, N, H, positions, K) if alpha_mode == ALPHA_PER_CHANNEL else (L, N, H, positions)
        self.g = np.zeros(gshape, dtype=np.float32)
        self.beta = np.zeros((L, N, H, positions), dtype=np.float32)
        self.xrow = np.zeros((L, N, positions, pool.channels), dtype=np.uint16)

    def copy(self):
        r = object.__new__(Ring)
        r.positions, r.alpha_mode = self.positions, self.alpha_mode
        for n in ("rawk", "rawv", "g", "beta", "xrow"):
            setattr(r, n, getattr(self, n).copy())
        return r

    def _struct(self):
        return _Ring(self.positions, self.alpha_mode, _p(self.rawk, _u16p), _p(self.rawv, _u16p),
                     _p(self.g, _f32p), _p(self.beta, _f32p), _p(self.xrow, _u16p))


def replay_verify(pool: Pool, ring: Ring, layer, slot_table, x, conv_w, alpha, alpha_mode, beta,
                  scale=1.0, flags=L2NORM_K, exact=False, precision="f64"):
    """Verify a draft chain of D tokens per request (x [B][D][C], alpha [B][D][H](,K), beta
    [B][D][H]) from the live slots, which stay as they are; fills ring positions 0..D-1.
    Returns ``(out[B,D,H,V], err)`` or, with ``exact=True``, ``(out, err, out_exact)``."""
    st = _c(slot_table, np.int32)
    xs = _c(x, np.uint16)
    B, D = xs.shape[0], xs.shape[1]
    H, V = pool.heads, pool.head_v
    w = _c(conv_w, np.uint16)
    a, bt = _c(alpha, np.float32), _c(beta, np.float32)
    out = np.zeros((B, D, H, V), dtype=np.uint16)
    oe = np.zeros((B, D, H, V), dtype=np.float64) if exact else None
    ps, rs = pool._struct(), ring._struct()
    err = lib(precision).oracle_replay_verify(
        ct.byref(ps), ct.byref(rs), layer, B, D, _p(st, _i32p), _p(xs, _u16p), _p(w, _u16p),
        _p(a, _f32p), alpha_mode, _p(bt, _f32p), scale, flags, _p(out, _u16p), _p(oe, _f64p))
    if err & 4:
        raise ValueError("oracle_replay_verify: bad argument")
    return (out, err, oe) if exact else (out, err)


def replay_commit(pool: Pool, ring: Ring, layer, slot_table, accepted, alpha_mode, flags=L2NORM_K,
                  seq_len_before=None, track_interval=0, track_slots=None, next_track_idx=None,
                  precision="f64"):
    """Fold ring positions 0..accepted[b]-1 into each live slot (modifies ``pool``)."""
    st = _c(slot_table, np.int32)
    B = st.shape[0]
    acc = _c(accepted, np.int32)
    sb = _c(seq_len_before if seq_len_before is not None else np.zeros(B), np.int32)
    ts = _c(track_slots, np.int32) if track_slots is not None else None
    nt = _c(next_track_idx, np.int32) if next_track_idx is not None else None
    ps, rs = pool._struct(), ring._struct()
    err = lib(precision).oracle_replay_commit(
        ct.byref(ps), ct.byref(rs), layer, B, _p(st, _i32p), _p(acc, _i32p), alpha_mode, flags,
        _p(sb, _i32p), track_interval, _p(ts, _i32p), _p(nt, _i32p))
    if err & 4:
        raise ValueError("oracle_replay_commit: bad argument")
    return err


def recurrence_head(q, k, v, alpha, beta, S0, scale=1.0, precision="f64"):
    """Bare recurrence for one head over prepared tokens. Returns (o[T,V], S[V,K])."""
    q, k, v = (_c(t, np.float64) for t in (q, k, v))
    alpha, beta = _c(alpha, np.float64), _c(beta, np.float64)
    T, K = k.shape
    V = v.shape[1]
    if alpha.ndim == 1:
        alpha = np.ascontiguousarray(np.repeat(alpha[:, None], K, axis=1))
    S = _c(S0, np.float64).copy()
    o = np.zeros((T, V), dtype=np.float64)
    lib(precision).oracle_recurrence_head(T, K, V, _p(q, _f64p), _p(k, _f64p), _p(v, _f64p),
                                          _p(alpha, _f64p), _p(beta, _f64p), scale,
                                          _p(S, _f64p), _p(o, _f64p))
    return o, S


def chunked_head_f64(q, k, v, alpha, beta, S0, chunk=64, scale=1.0):
    """WY chunked form of :func:`recurrence_head`, in double."""
    q, k, v = (_c(t, np.float64) for t in (q, k, v))
    alpha, beta = _c(alpha, np.float64), _c(beta, np.float64)
    T, K = k.shape
    V = v.shape[1]
    if alpha.ndim == 1:
        alpha = np.ascontiguousarray(np.repeat(alpha[:, None], K, axis=1))
    S = _c(S0, np.float64).copy()
    o = np.zeros((T, V), dtype=np.float64)
    lib("f64").oracle_chunked_head_f64(T, K, V, chunk, _p(q, _f64p), _p(k, _f64p),
                                       _p(v, _f64p), _p(alpha, _f64p), _p(beta, _f64p),
                                       scale, _p(S, _f64p), _p(o, _f64p))
    return o, S


def bf16_round(x, precision="f64"):
    f = lib(precision).oracle_bf16_round
    return np.array([f(float(v)) for v in np.asarray(x, dtype=np.float64).ravel()],
                    dtype=np.uint16).reshape(np.shape(x))


def bf16_widen(bits):
    b = np.asarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
