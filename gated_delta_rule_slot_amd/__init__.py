"""MI355X (gfx950) slot-indexed gated delta rule: HIP kernels behind a C ABI.

The entry points mirror include/gdn_slot.h one to one:

  state_pool_bytes, state_pool_create, gdn_prefill_workspace_bytes,
  conv_gdn_prefill_chunked, conv_gdn_prefill_chunked_noalloc, gdn_decode_step,
  track_snapshot, restore_slots,
  gdn_verify_tree, gdn_accept_scatter, replayssm_ring_bytes, replayssm_verify,
  replayssm_commit

and the host checkpoint index of include/gdn_ckpt.h (CheckpointIndex,
ckpt_chain_hashes).

Importing the package loads ``libgdnslot.so`` (built by ``build.py``); if it is
missing the import fails.  There is no CPU fallback.
"""
from ._binding import (  # noqa: F401
    ALPHA_PER_CHANNEL, ALPHA_PER_HEAD, CONV_SILU, ERRW_BAD_SEQLENS, ERRW_BAD_SLOT,
    ERRW_BAD_TRACK_SLOT, ERRW_BAD_TREE, GDN_BF16, GDN_F32, L2NORM_K, L2NORM_Q, LIB_PATH,
    CKPT_FULL, CKPT_PRESENT, CKPT_STORED, MAX_RING_POSITIONS, MAX_TREE_NODES, CheckpointIndex,
    GdnError, PREFILL_ONE_KERNEL, PREFILL_TWO_KERNEL, SNAP_LAST_ONLY, ReplayRing, StatePool,
    ckpt_chain_hashes,
    NOALLOC_SCRATCH_BYTES, conv_gdn_prefill_chunked, conv_gdn_prefill_chunked_noalloc,
    gdn_accept_scatter, gdn_decode_step, gdn_prefill_workspace_bytes, gdn_verify_tree, last_error,
    replayssm_commit, replayssm_ring_bytes, replayssm_verify, restore_slots, state_pool_bytes,
    state_pool_create, track_snapshot,
)
