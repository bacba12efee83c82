"""ctypes binding of libgdnslot.so (include/gdn_slot.h), argument marshalling only.

Each function carries the C entry point's name and takes torch tensors that
live on the current HIP device.  Nothing here computes: every step runs in the
library's kernels.  PyTorch provides the device memory and the stream.  If the
shared library is missing, importing this module raises; there is no fallback.
"""
from __future__ import annotations

import ctypes as ct
import os

import torch

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libgdnslot.so")

GDN_F32, GDN_BF16 = 0, 1
ALPHA_PER_HEAD, ALPHA_PER_CHANNEL = 0, 1
L2NORM_K, L2NORM_Q, CONV_SILU = 1, 2, 4
PREFILL_ONE_KERNEL, PREFILL_TWO_KERNEL = 8, 16
SNAP_LAST_ONLY = 32
NOALLOC_SCRATCH_BYTES = 64 << 20  # GDN_NOALLOC_SCRATCH_BYTES
ERRW_BAD_SLOT, ERRW_BAD_TRACK_SLOT, ERRW_BAD_SEQLENS, ERRW_BAD_TREE = 1, 2, 4, 8
MAX_TREE_NODES = 1024
MAX_RING_POSITIONS = 64


class GdnError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"gdn status {status}: {message}")
        self.status = status


class PoolDesc(ct.Structure):
    _fields_ = [
        ("layers", ct.c_int32), ("slots", ct.c_int32), ("heads", ct.c_int32),
        ("head_k", ct.c_int32), ("head_v", ct.c_int32), ("conv_kernel", ct.c_int32),
        ("ssm_dtype", ct.c_int32), ("conv_dtype", ct.c_int32),
        ("ssm_base", ct.c_void_p), ("conv_base", ct.c_void_p), ("err_word", ct.c_void_p),
    ]


class RingDesc(ct.Structure):
    _fields_ = [("positions", ct.c_int32), ("alpha_mode", ct.c_int32), ("rawk", ct.c_void_p),
                ("rawv", ct.c_void_p), ("g", ct.c_void_p), ("beta", ct.c_void_p),
                ("xrow", ct.c_void_p)]


class RestoreOp(ct.Structure):
    _fields_ = [("linear_state_id", ct.c_int32), ("restore_requested", ct.c_int32),
                ("restore_src_slot_id", ct.c_int32)]


if not os.path.exists(LIB_PATH):
    raise ImportError(f"{LIB_PATH} is not built; run gated_delta_rule_slot_amd/build.py")

_lib = ct.CDLL(LIB_PATH)
_vp, _i32, _u32, _f32, _sz = ct.c_void_p, ct.c_int32, ct.c_uint32, ct.c_float, ct.c_size_t
_lib.state_pool_bytes.argtypes = [ct.POINTER(PoolDesc), ct.POINTER(_sz), ct.POINTER(_sz)]
_lib.state_pool_create.argtypes = [ct.POINTER(PoolDesc), ct.POINTER(_vp)]
_lib.state_pool_destroy.argtypes = [_vp]
_lib.state_pool_destroy.restype = None
_lib.gdn_last_error.restype = ct.c_char_p
_lib.conv_gdn_prefill_chunked.argtypes = [
    _vp, _i32, _i32, _i32, _i32, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _i32, _vp, _f32, _u32,
    _vp, _i32, _vp, _vp, _vp, _sz, _vp]
_lib.conv_gdn_prefill_chunked_noalloc.argtypes = [
    _vp, _i32, _i32, _i32, _i32, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _i32, _vp, _f32, _u32,
    _vp, _i32, _vp, _vp, _vp]
_lib.gdn_prefill_workspace_bytes.argtypes = [_vp, _i32, _i32, ct.POINTER(_sz)]
_lib.gdn_decode_step.argtypes = [
    _vp, _i32, _i32, _vp, _vp, _vp, _vp, _i32, _vp, _f32, _u32, _vp, _vp, _i32, _vp, _vp, _vp]
_lib.track_snapshot.argtypes = [_vp, _i32, _i32, _i32, _vp, _vp, _vp]
_lib.restore_slots.argtypes = [_vp, _i32, ct.POINTER(RestoreOp), ct.POINTER(ct.c_int64), _vp]
_lib.gdn_verify_tree.argtypes = [
    _vp, _i32, _i32, _i32, _vp, _vp, _vp, _vp, _vp, _i32, _vp, _f32, _u32, _vp, _vp, _vp, _vp]
_lib.gdn_accept_scatter.argtypes = [
    _vp, _i32, _i32, _i32, _vp, _vp, _vp, _vp, _i32, _vp, _vp, _vp, _vp, _vp]
_lib.replayssm_ring_bytes.argtypes = [_vp, _i32, _i32, ct.POINTER(_sz)]
_i64, _u64 = ct.c_int64, ct.c_uint64
_lib.ckpt_chain_hashes.argtypes = [_vp, _i64, _i32, _i64, _u64, _vp, _i64, ct.POINTER(_i64)]
_lib.ckpt_index_create.argtypes = [_i32, ct.POINTER(_vp)]
_lib.ckpt_index_destroy.argtypes = [_vp]
_lib.ckpt_index_destroy.restype = None
_lib.ckpt_index_size.argtypes = [_vp]
_lib.ckpt_index_size.restype = _i32
_lib.ckpt_index_contains.argtypes = [_vp, _u64]
_lib.ckpt_index_contains.restype = _i32
_lib.ckpt_index_match.argtypes = [_vp, _vp, _i64, _i64, _i32, ct.POINTER(_i64), ct.POINTER(_i32),
                                  ct.POINTER(_u64)]
_lib.ckpt_index_release.argtypes = [_vp, _u64]
_lib.ckpt_index_insert.argtypes = [_vp, _u64, _i32, ct.POINTER(_i32), ct.POINTER(_i32)]
_lib.ckpt_plan_restores.argtypes = [_vp, _i32, _vp, _vp, _i32, _vp, ct.POINTER(RestoreOp), _vp, _vp]
_lib.ckpt_finish_request.argtypes = [_vp, _i32, _u64, _i32, ct.POINTER(_i32), _i32, ct.POINTER(_i32),
                                     ct.POINTER(_i32)]
_lib.replayssm_verify.argtypes = [
    _vp, ct.POINTER(RingDesc), _i32, _i32, _i32, _vp, _vp, _vp, _vp, _vp, _f32, _u32, _vp, _vp]
_lib.replayssm_commit.argtypes = [
    _vp, ct.POINTER(RingDesc), _i32, _i32, _vp, _vp, _u32, _vp, _i32, _vp, _vp, _vp]
for _f in ("state_pool_bytes", "state_pool_create", "conv_gdn_prefill_chunked",
           "conv_gdn_prefill_chunked_noalloc",
           "gdn_prefill_workspace_bytes", "gdn_decode_step", "track_snapshot", "restore_slots",
           "gdn_verify_tree", "gdn_accept_scatter", "replayssm_ring_bytes", "replayssm_verify",
           "replayssm_commit", "ckpt_chain_hashes", "ckpt_index_create", "ckpt_index_match",
           "ckpt_index_release", "ckpt_index_insert", "ckpt_plan_restores", "ckpt_finish_request"):
    getattr(_lib, _f).restype = ct.c_int


def _check(status: int) -> None:
    if status != 0:
        raise GdnError(status, _lib.gdn_last_error().decode(errors="replace"))


def _ptr(t) -> int | None:
    if t is None:
        return None
    if not isinstance(t, torch.Tensor):
        raise TypeError("expected a torch.Tensor")
    if not t.is_cuda:
        raise ValueError("tensor must be on the GPU")
    if not t.is_contiguous():
        raise ValueError("tensor must be contiguous")
    return t.data_ptr()


def _need(t, dtype, numel=None, name="tensor"):
    if t is None:
        return
    if t.dtype != dtype:
        raise TypeError(f"{name}: expected {dtype}, got {t.dtype}")
    if numel is not None and t.numel() < numel:
        raise ValueError(f"{name}: needs at least {numel} elements, has {t.numel()}")


def _stream(stream) -> int:
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream


def last_error() -> str:
    return _lib.gdn_last_error().decode(errors="replace")


def state_pool_bytes(layers, slots, heads, head_k, head_v, ssm_dtype):
    d = PoolDesc(layers, slots, heads, head_k, head_v, 4, ssm_dtype, GDN_BF16, None, None, None)
    s, c = _sz(), _sz()
    _check(_lib.state_pool_bytes(ct.byref(d), ct.byref(s), ct.byref(c)))
    return s.value, c.value


class StatePool:
    """Handle over caller-owned pool tensors (see state_pool_create)."""

    def __init__(self, handle, ssm, conv, err_word, shape):
        self.handle = handle
        self.ssm, self.conv, self.err_word = ssm, conv, err_word
        self.layers, self.slots, self.heads, self.head_k, self.head_v = shape

    @property
    def channels(self):
        return self.heads * (2 * self.head_k + self.head_v)

    def destroy(self):
        if self.handle:
            _lib.state_pool_destroy(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.destroy()
        except Exception:
            pass


def state_pool_create(ssm: torch.Tensor, conv: torch.Tensor, err_word: torch.Tensor | None = None):
    """Wrap ``ssm`` [L,N,H,V,K] (float32|bfloat16) and ``conv`` [L,N,3,C] (bfloat16)."""
    if ssm.dim() != 5 or conv.dim() != 4:
        raise ValueError("ssm must be [L,N,H,V,K] and conv [L,N,3,C]")
    L, N, H, V, K = ssm.shape
    if ssm.dtype == torch.float32:
        sd = GDN_F32
    elif ssm.dtype == torch.bfloat16:
        sd = GDN_BF16
    else:
        raise TypeError("ssm must be float32 or bfloat16")
    if conv.dtype != torch.bfloat16 or tuple(conv.shape) != (L, N, 3, H * (2 * K + V)):
        raise ValueError("conv must be bfloat16 [L, N, 3, H*(2K+V)]")
    if err_word is not None:
        _need(err_word, torch.int32, 1, "err_word")
    d = PoolDesc(L, N, H, K, V, 4, sd, GDN_BF16, _ptr(ssm), _ptr(conv), _ptr(err_word))
    h = _vp()
    _check(_lib.state_pool_create(ct.byref(d), ct.byref(h)))
    return StatePool(h, ssm, conv, err_word, (L, N, H, K, V))


def gdn_prefill_workspace_bytes(pool: StatePool, batch: int, max_seqlen: int) -> int:
    n = _sz()
    _check(_lib.gdn_prefill_workspace_bytes(pool.handle, batch, max_seqlen, ct.byref(n)))
    return n.value


def conv_gdn_prefill_chunked(pool: StatePool, layer, cu_seqlens, slot_table, has_initial_state,
                             x, conv_w, alpha, alpha_mode, beta, out, max_seqlen,
                             start_len=None, scale=1.0, flags=L2NORM_K, snap_interval=0,
                             track_slots=None, next_track_idx=None, workspace=None,
                             stream=None):
    B = slot_table.numel()
    T = x.shape[0] if x is not None else 0
    H, V, K = pool.heads, pool.head_v, pool.head_k
    _need(cu_seqlens, torch.int32, B + 1, "cu_seqlens")
    _need(slot_table, torch.int32, B, "slot_table")
    _need(has_initial_state, torch.int32, B, "has_initial_state")
    _need(start_len, torch.int32, B, "start_len")
    _need(x, torch.bfloat16, T * pool.channels, "x")
    _need(conv_w, torch.bfloat16, pool.channels * 4, "conv_w")
    _need(alpha, torch.float32, T * H * (K if alpha_mode == ALPHA_PER_CHANNEL else 1), "alpha")
    _need(beta, torch.float32, T * H, "beta")
    _need(out, torch.bfloat16, T * H * V, "out")
    _need(track_slots, torch.int32, 2 * B, "track_slots")
    _need(next_track_idx, torch.int32, B, "next_track_idx")
    if workspace is not None:
        _need(workspace, torch.uint8, None, "workspace")
    ws_bytes = workspace.numel() if workspace is not None else 0
    _check(_lib.conv_gdn_prefill_chunked(
        pool.handle, layer, B, T, int(max_seqlen), _ptr(cu_seqlens), _ptr(slot_table),
        _ptr(has_initial_state), _ptr(start_len), _ptr(x), _ptr(conv_w), _ptr(alpha), alpha_mode,
        _ptr(beta), float(scale), flags, _ptr(out), snap_interval, _ptr(track_slots),
        _ptr(next_track_idx), _ptr(workspace), ws_bytes, _stream(stream)))


def conv_gdn_prefill_chunked_noalloc(pool: StatePool, layer, cu_seqlens, slot_table,
                                     has_initial_state, x, conv_w, alpha, alpha_mode, beta, out,
                                     max_seqlen, start_len=None, scale=1.0, flags=L2NORM_K,
                                     snap_interval=0, track_slots=None, next_track_idx=None,
                                     stream=None):
    """conv_gdn_prefill_chunked without a workspace: the library's fixed per-device
    scratch serves the two-kernel path and nothing is allocated."""
    B = slot_table.numel()
    T = x.shape[0] if x is not None else 0
    H, V, K = pool.heads, pool.head_v, pool.head_k
    _need(cu_seqlens, torch.int32, B + 1, "cu_seqlens")
    _need(slot_table, torch.int32, B, "slot_table")
    _need(has_initial_state, torch.int32, B, "has_initial_state")
    _need(start_len, torch.int32, B, "start_len")
    _need(x, torch.bfloat16, T * pool.channels, "x")
    _need(conv_w, torch.bfloat16, pool.channels * 4, "conv_w")
    _need(alpha, torch.float32, T * H * (K if alpha_mode == ALPHA_PER_CHANNEL else 1), "alpha")
    _need(beta, torch.float32, T * H, "beta")
    _need(out, torch.bfloat16, T * H * V, "out")
    _need(track_slots, torch.int32, 2 * B, "track_slots")
    _need(next_track_idx, torch.int32, B, "next_track_idx")
    _check(_lib.conv_gdn_prefill_chunked_noalloc(
        pool.handle, layer, B, T, int(max_seqlen), _ptr(cu_seqlens), _ptr(slot_table),
        _ptr(has_initial_state), _ptr(start_len), _ptr(x), _ptr(conv_w), _ptr(alpha), alpha_mode,
        _ptr(beta), float(scale), flags, _ptr(out), snap_interval, _ptr(track_slots),
        _ptr(next_track_idx), _stream(stream)))


def gdn_decode_step(pool: StatePool, layer, slot_table, x, conv_w, alpha, alpha_mode, beta, out,
                    scale=1.0, flags=L2NORM_K, seq_len_after=None, track_interval=0,
                    track_slots=None, next_track_idx=None, stream=None):
    B = slot_table.numel()
    H, V, K = pool.heads, pool.head_v, pool.head_k
    _need(slot_table, torch.int32, B, "slot_table")
    _need(x, torch.bfloat16, B * pool.channels, "x")
    _need(conv_w, torch.bfloat16, pool.channels * 4, "conv_w")
    _need(alpha, torch.float32, B * H * (K if alpha_mode == ALPHA_PER_CHANNEL else 1), "alpha")
    _need(beta, torch.float32, B * H, "beta")
    _need(out, torch.bfloat16, B * H * V, "out")
    _need(seq_len_after, torch.int32, B, "seq_len_after")
    _need(track_slots, torch.int32, 2 * B, "track_slots")
    _need(next_track_idx, torch.int32, B, "next_track_idx")
    _check(_lib.gdn_decode_step(
        pool.handle, layer, B, _ptr(slot_table), _ptr(x), _ptr(conv_w), _ptr(alpha), alpha_mode,
        _ptr(beta), float(scale), flags, _ptr(out), _ptr(seq_len_after), track_interval,
        _ptr(track_slots), _ptr(next_track_idx), _stream(stream)))


def track_snapshot(pool: StatePool, layer_begin, layer_end, src_slots, dst_slots, stream=None):
    n = src_slots.numel()
    _need(src_slots, torch.int32, n, "src_slots")
    _need(dst_slots, torch.int32, n, "dst_slots")
    _check(_lib.track_snapshot(pool.handle, layer_begin, layer_end, n, _ptr(src_slots),
                               _ptr(dst_slots), _stream(stream)))


def restore_slots(pool: StatePool, ops, has_initial_state, stream=None):
    """``ops``: sequence of (linear_state_id, restore_requested, restore_src_slot_id);
    ``has_initial_state``: host int64 tensor or list, updated and returned as a list."""
    n = len(ops)
    arr = (RestoreOp * max(n, 1))(*[RestoreOp(*map(int, o)) for o in ops])
    hi = (ct.c_int64 * max(n, 1))(*[int(v) for v in has_initial_state])
    _check(_lib.restore_slots(pool.handle, n, arr, hi, _stream(stream)))
    return [hi[i] for i in range(n)]


def gdn_verify_tree(pool: StatePool, layer, slot_table, parent, x, conv_w, alpha, alpha_mode, beta,
                    out, node_ssm, node_conv, scale=1.0, flags=L2NORM_K, stream=None):
    """``parent`` int32 [B, T]; ``x`` bf16 [B, T, C]; ``alpha`` fp32 [B, T, H(, K)];
    ``beta`` fp32 [B, T, H]; ``out`` bf16 [B, T, H, V]; ``node_ssm`` [B, T, H, V, K]
    in the pool's ssm dtype; ``node_conv`` bf16 [B, T, 3, C]."""
    B = slot_table.numel()
    if parent.dim() != 2 or parent.shape[0] != B:
        raise ValueError("parent must be [batch, tree_nodes]")
    T = parent.shape[1]
    H, V, K = pool.heads, pool.head_v, pool.head_k
    _need(slot_table, torch.int32, B, "slot_table")
    _need(parent, torch.int32, B * T, "parent")
    _need(x, torch.bfloat16, B * T * pool.channels, "x")
    _need(conv_w, torch.bfloat16, pool.channels * 4, "conv_w")
    _need(alpha, torch.float32, B * T * H * (K if alpha_mode == ALPHA_PER_CHANNEL else 1), "alpha")
    _need(beta, torch.float32, B * T * H, "beta")
    _need(out, torch.bfloat16, B * T * H * V, "out")
    _need(node_ssm, pool.ssm.dtype, B * T * H * V * K, "node_ssm")
    _need(node_conv, torch.bfloat16, B * T * 3 * pool.channels, "node_conv")
    _check(_lib.gdn_verify_tree(
        pool.handle, layer, B, T, _ptr(slot_table), _ptr(parent), _ptr(x), _ptr(conv_w),
        _ptr(alpha), alpha_mode, _ptr(beta), float(scale), flags, _ptr(out), _ptr(node_ssm),
        _ptr(node_conv), _stream(stream)))


def gdn_accept_scatter(pool: StatePool, layer, slot_table, parent, accepted, node_ssm, node_conv,
                       seq_len_before=None, track_interval=0, track_slots=None,
                       next_track_idx=None, stream=None):
    """Commit node ``accepted[b]`` (-1: none) of each request's verified tree."""
    B = slot_table.numel()
    if parent.dim() != 2 or parent.shape[0] != B:
        raise ValueError("parent must be [batch, tree_nodes]")
    T = parent.shape[1]
    H, V, K = pool.heads, pool.head_v, pool.head_k
    _need(slot_table, torch.int32, B, "slot_table")
    _need(parent, torch.int32, B * T, "parent")
    _need(accepted, torch.int32, B, "accepted")
    _need(seq_len_before, torch.int32, B, "seq_len_before")
    _need(track_slots, torch.int32, 2 * B, "track_slots")
    _need(next_track_idx, torch.int32, B, "next_track_idx")
    _need(node_ssm, pool.ssm.dtype, B * T * H * V * K, "node_ssm")
    _need(node_conv, torch.bfloat16, B * T * 3 * pool.channels, "node_conv")
    _check(_lib.gdn_accept_scatter(
        pool.handle, layer, B, T, _ptr(slot_table), _ptr(parent), _ptr(accepted),
        _ptr(seq_len_before), track_interval, _ptr(track_slots), _ptr(next_track_idx),
        _ptr(node_ssm), _ptr(node_conv), _stream(stream)))


def replayssm_ring_bytes(pool: StatePool, positions, alpha_mode):
    """Byte sizes (rawk, rawv, g, beta, xrow) of a ReplaySSM ring for the pool."""
    b = (_sz * 5)()
    _check(_lib.replayssm_ring_bytes(pool.handle, positions, alpha_mode, b))
    return tuple(b[i] for i in range(5))


class ReplayRing:
    """Caller-owned ReplaySSM ring tensors (see gdn_replay_ring in the header)."""

    def __init__(self, pool: StatePool, positions, alpha_mode, device=None):
        L, N, H, K, V = pool.layers, pool.slots, pool.heads, pool.head_k, pool.head_v
        dev = device if device is not None else pool.ssm.device
        self.positions, self.alpha_mode = positions, alpha_mode
        self.rawk = torch.zeros(L, N, H, positions, K, dtype=torch.bfloat16, device=dev)
        self.rawv = torch.zeros(L, N, H, positions, V, dtype=torch.bfloat16, device=dev)
        gshape = (L, N, H, positions, K) if alpha_mode == ALPHA_PER_CHANNEL else (L, N, H, positions)
        self.g = torch.zeros(gshape, dtype=torch.float32, device=dev)
        self.beta = torch.zeros(L, N, H, positions, dtype=torch.float32, device=dev)
        self.xrow = torch.zeros(L, N, positions, pool.channels, dtype=torch.bfloat16, device=dev)

    def desc(self):
        return RingDesc(self.positions, self.alpha_mode, _ptr(self.rawk), _ptr(self.rawv),
                        _ptr(self.g), _ptr(self.beta), _ptr(self.xrow))


def replayssm_verify(pool: StatePool, ring: ReplayRing, layer, slot_table, x, conv_w, alpha, beta,
                     out, scale=1.0, flags=L2NORM_K, stream=None):
    """``x`` bf16 [B, D, C]; ``alpha`` fp32 [B, D, H(, K)]; ``beta`` fp32 [B, D, H];
    ``out`` bf16 [B, D, H, V].  The live slots are only read."""
    B = slot_table.numel()
    if x.dim() != 3 or x.shape[0] != B:
        raise ValueError("x must be [batch, draft, C]")
    D = x.shape[1]
    H, V, K = pool.heads, pool.head_v, pool.head_k
    _need(slot_table, torch.int32, B, "slot_table")
    _need(x, torch.bfloat16, B * D * pool.channels, "x")
    _need(conv_w, torch.bfloat16, pool.channels * 4, "conv_w")
    _need(alpha, torch.float32, B * D * H * (K if ring.alpha_mode == ALPHA_PER_CHANNEL else 1), "alpha")
    _need(beta, torch.float32, B * D * H, "beta")
    _need(out, torch.bfloat16, B * D * H * V, "out")
    d = ring.desc()
    _check(_lib.replayssm_verify(pool.handle, ct.byref(d), layer, B, D, _ptr(slot_table), _ptr(x),
                                 _ptr(conv_w), _ptr(alpha), _ptr(beta), float(scale), flags,
                                 _ptr(out), _stream(stream)))


def replayssm_commit(pool: StatePool, ring: ReplayRing, layer, slot_table, accepted, flags=L2NORM_K,
                     seq_len_before=None, track_interval=0, track_slots=None, next_track_idx=None,
                     stream=None):
    """Fold ring positions 0..accepted[b]-1 into each live slot."""
    B = slot_table.numel()
    _need(slot_table, torch.int32, B, "slot_table")
    _need(accepted, torch.int32, B, "accepted")
    _need(seq_len_before, torch.int32, B, "seq_len_before")
    _need(track_slots, torch.int32, 2 * B, "track_slots")
    _need(next_track_idx, torch.int32, B, "next_track_idx")
    d = ring.desc()
    _check(_lib.replayssm_commit(pool.handle, ct.byref(d), layer, B, _ptr(slot_table), _ptr(accepted),
                                 flags, _ptr(seq_len_before), track_interval, _ptr(track_slots),
                                 _ptr(next_track_idx), _stream(stream)))


# ------------------------------------------------------- checkpoint index --
CKPT_STORED, CKPT_PRESENT, CKPT_FULL = 0, 1, 2


def ckpt_chain_hashes(tokens, stride, first_chunk=0, prev_key=0):
    """Chained keys of the whole chunks first_chunk.. of an int32 token sequence
    (numpy array or list); returns a numpy uint64 array."""
    import numpy as np
    t = np.ascontiguousarray(tokens, dtype=np.int32)
    cap = max(t.shape[0] // stride - first_chunk, 0) if stride > 0 else 0  # the library rejects stride < 1
    keys = np.zeros(max(cap, 1), dtype=np.uint64)
    n = ct.c_int64()
    _check(_lib.ckpt_chain_hashes(t.ctypes.data, t.shape[0], stride, first_chunk, prev_key,
                                  keys.ctypes.data, cap, ct.byref(n)))
    return keys[:n.value]


class CheckpointIndex:
    """The host checkpoint index (include/gdn_ckpt.h)."""

    def __init__(self, capacity):
        h = _vp()
        _check(_lib.ckpt_index_create(capacity, ct.byref(h)))
        self.handle = h

    def __del__(self):
        try:
            if self.handle:
                _lib.ckpt_index_destroy(self.handle)
                self.handle = None
        except Exception:
            pass

    def __len__(self):
        return _lib.ckpt_index_size(self.handle)

    def contains(self, key):
        return bool(_lib.ckpt_index_contains(self.handle, int(key)))

    def match(self, keys, n_tokens, stride):
        """(reach_tokens, slot, key); (0, -1, None) on a miss."""
        import numpy as np
        k = np.ascontiguousarray(keys, dtype=np.uint64)
        reach, slot, key = ct.c_int64(), ct.c_int32(), ct.c_uint64()
        _check(_lib.ckpt_index_match(self.handle, k.ctypes.data if k.size else None, k.size, n_tokens,
                                     stride, ct.byref(reach), ct.byref(slot), ct.byref(key)))
        return (reach.value, slot.value, key.value) if slot.value >= 0 else (0, -1, None)

    def release(self, key):
        _check(_lib.ckpt_index_release(self.handle, int(key)))

    def insert(self, key, slot):
        """('stored' | 'present' | 'full', slot_back)."""
        out, back = ct.c_int32(), ct.c_int32()
        _check(_lib.ckpt_index_insert(self.handle, int(key), slot, ct.byref(out), ct.byref(back)))
        return ("stored", "present", "full")[out.value], back.value

    def plan_restores(self, token_lists, stride, live_slots):
        """Hash, match and pin for a batch; returns (ops, reach, hit_keys) where ops
        are (linear_state_id, restore_requested, restore_src_slot_id) tuples."""
        import numpy as np
        n = len(token_lists)
        cu = np.zeros(n + 1, dtype=np.int64)
        for i, t in enumerate(token_lists):
            cu[i + 1] = cu[i] + len(t)
        toks = np.ascontiguousarray(np.concatenate([np.asarray(t, dtype=np.int32) for t in token_lists])
                                    if n else np.zeros(1, dtype=np.int32))
        live = np.ascontiguousarray(live_slots, dtype=np.int32)
        ops = (RestoreOp * max(n, 1))()
        reach = np.zeros(max(n, 1), dtype=np.int64)
        keys = np.zeros(max(n, 1), dtype=np.uint64)
        _check(_lib.ckpt_plan_restores(self.handle, n, toks.ctypes.data, cu.ctypes.data, stride,
                                       live.ctypes.data, ops, reach.ctypes.data, keys.ctypes.data))
        return ([(ops[i].linear_state_id, ops[i].restore_requested, ops[i].restore_src_slot_id)
                 for i in range(n)], reach[:n], keys[:n])

    def finish_request(self, key, live_slot, track_slots, next_track_idx):
        """Hand the tracked boundary's slot to the index; returns the slots to free
        (key None: nothing was tracked)."""
        tr = (ct.c_int32 * 2)(*[int(v) for v in track_slots])
        freed, n = (ct.c_int32 * 4)(), ct.c_int32()
        _check(_lib.ckpt_finish_request(self.handle, 0 if key is None else 1, 0 if key is None else int(key),
                                        int(live_slot), tr, int(next_track_idx), freed, ct.byref(n)))
        return [freed[i] for i in range(n.value)]
