// slot_copy.hip -- byte-exact copies of whole (layer, slot) state blocks.
//
// One kernel serves the track snapshot (the masked copy of the active slot into
// a track slot, page "企业官网建设流程全解析", section "--mamba-track-interval"),
// copy_from / fork (page "SGLang之MambaRadixCache机制", section 3.2) and the
// checkpoint restore (page "Qwen3.5 Linear-State Prefix Cache", section 6.4).
//
// A (layer, slot) block is the ssm block followed, logically, by the conv block;
// the two live in different buffers.  The grid is
//   x: 16 KiB tiles over the concatenated block, y: layer, z: pair,
// and every thread moves four 16-byte vectors: all four loads are issued before
// the first store so each wave keeps 4 KiB in flight.  Block sizes are
// multiples of 16 bytes for every supported shape (checked at pool creation).
#include "common.hpp"

namespace gdn {
namespace {

constexpr int kThreads = 256;
constexpr int kVecPerThread = 4;
constexpr int64_t kTileBytes = int64_t(kThreads) * kVecPerThread * 16;
constexpr int kMaxHostPairs = 256;  // 2 KiB of kernel arguments per launch

struct CopyGeom {
  char *ssm;
  char *conv;
  int64_t ssm_block, conv_block;   // bytes of one (layer, slot) block
  int64_t ssm_layer, conv_layer;   // bytes of one layer (slots * block)
  int32_t slots;
  int32_t layer_begin;
  int32_t ssm_tiles;               // tiles covering the ssm part
  int32_t *err;
};

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

struct HostPairs {
  int32_t src[kMaxHostPairs];
  int32_t dst[kMaxHostPairs];
};

__device__ __forceinline__ void copy_tile(const char *src_block, char *dst_block,
                                          int64_t block_bytes, int64_t tile_off) {
  const u32x4 *src = reinterpret_cast<const u32x4 *>(src_block);
  u32x4 *dst = reinterpret_cast<u32x4 *>(dst_block);
  const int64_t nvec = block_bytes >> 4;
  const int64_t v0 = (tile_off >> 4) + threadIdx.x;
  u32x4 buf[kVecPerThread];
#pragma unroll
  for (int u = 0; u < kVecPerThread; ++u) {
    int64_t v = v0 + int64_t(u) * kThreads;
    if (v < nvec) buf[u] = __builtin_nontemporal_load(src + v);
  }
#pragma unroll
  for (int u = 0; u < kVecPerThread; ++u) {
    int64_t v = v0 + int64_t(u) * kThreads;
    if (v < nvec) __builtin_nontemporal_store(buf[u], dst + v);
  }
}

template <bool kFromDevice>
__global__ __launch_bounds__(kThreads) void slot_copy_kernel(CopyGeom g, const int32_t *src_dev,
                                                             const int32_t *dst_dev, HostPairs hp) {
  const int pair = blockIdx.z;
  int src, dst;
  if (kFromDevice) {
    src = src_dev[pair];
    dst = dst_dev[pair];
    if (dst <= 0) return;
    if (src <= 0 || src >= g.slots || dst >= g.slots) {
      if (g.err && blockIdx.x == 0 && blockIdx.y == 0 && threadIdx.x == 0)
        atomicOr(g.err, GDN_ERRW_BAD_TRACK_SLOT);
      return;
    }
    if (src == dst) return;
  } else {
    src = hp.src[pair];
    dst = hp.dst[pair];
  }
  const int64_t layer = g.layer_begin + blockIdx.y;
  const int tile = blockIdx.x;
  if (tile < g.ssm_tiles) {
    copy_tile(g.ssm + layer * g.ssm_layer + src * g.ssm_block,
              g.ssm + layer * g.ssm_layer + dst * g.ssm_block, g.ssm_block,
              int64_t(tile) * kTileBytes);
  } else {
    copy_tile(g.conv + layer * g.conv_layer + src * g.conv_block,
              g.conv + layer * g.conv_layer + dst * g.conv_block, g.conv_block,
              int64_t(tile - g.ssm_tiles) * kTileBytes);
  }
}

// Accepted-step scatter (page "SGLang之MambaRadixCache机制解析", section 8.4: the
// slot takes the intermediate state of the request's last accepted step;
// section 8.6: when the accepted tokens cross a track-interval boundary the
// ping-pong track slot is written too; section 9.10 places the snapshot at the
// token that completes the multiple).  Grid: x tiles of the (ssm + conv)
// block, y request, z job.  Job 0 copies the accepted node into the live slot.
// Jobs 1 and 2 copy the nodes at the last and the second-to-last crossing: the
// j-th crossing of the call goes to track slot (next_track_idx + j) & 1, so
// earlier crossings would be overwritten and only these two decide the result.
__global__ __launch_bounds__(kThreads) void accept_scatter_kernel(CopyGeom g, ScatterArgs a) {
  const int tile = blockIdx.x, b = blockIdx.y, job = blockIdx.z;
  const int acc = a.accepted[b];
  if (acc == -1) return;
  const int T = a.nodes;
  __shared__ int spar[kMaxTreeNodes];
  const int32_t *par = a.parent + int64_t(b) * T;
  int bad = acc < -1 || acc >= T;
  for (int i = threadIdx.x; i < T; i += kThreads) {
    const int p = par[i];
    spar[i] = p;
    bad |= (p < -1 || p >= i);
  }
  bad = __syncthreads_or(bad);
  const bool reporter = g.err && tile == 0 && threadIdx.x == 0;
  if (bad) {
    if (reporter && job == 0) atomicOr(g.err, GDN_ERRW_BAD_TREE);
    return;
  }
  const int slot = a.slot_table[b];
  if (slot <= 0 || slot >= g.slots) {
    if (reporter && job == 0 && slot >= g.slots) atomicOr(g.err, GDN_ERRW_BAD_SLOT);
    return;
  }
  int node = acc, dst = slot;
  if (job > 0) {
    if (a.track_interval <= 0) return;
    int depth = 0;  // tokens the accepted node folds beyond the live state
    for (int n = acc; n >= 0; n = spar[n]) ++depth;
    const int64_t before = a.seq_len_before[b];
    int crossings = 0, last = 0, prev = 0;  // count and depths of the last two crossings
    for (int i = 1; i <= depth; ++i)
      if ((before + i) % a.track_interval == 0) {
        prev = last;
        last = i;
        ++crossings;
      }
    const int j = crossings - job;
    if (j < 0) return;
    const int at = job == 1 ? last : prev;
    for (int s = depth; s > at; --s) node = spar[node];
    dst = a.track_slots[2 * b + ((a.next_track_idx[b] + j) & 1)];
    if (dst <= 0) return;
    if (dst >= g.slots) {
      if (reporter) atomicOr(g.err, GDN_ERRW_BAD_TRACK_SLOT);
      return;
    }
  }
  const int64_t layer = a.layer;
  const int64_t src_node = int64_t(b) * T + node;
  if (tile < g.ssm_tiles) {
    copy_tile(static_cast<const char *>(a.node_ssm) + src_node * g.ssm_block,
              g.ssm + layer * g.ssm_layer + dst * g.ssm_block, g.ssm_block,
              int64_t(tile) * kTileBytes);
  } else {
    copy_tile(reinterpret_cast<const char *>(a.node_conv) + src_node * g.conv_block,
              g.conv + layer * g.conv_layer + dst * g.conv_block, g.conv_block,
              int64_t(tile - g.ssm_tiles) * kTileBytes);
  }
}

CopyGeom make_geom(const gdn_pool *p, int layer_begin) {
  CopyGeom g;
  g.ssm = static_cast<char *>(p->d.ssm_base);
  g.conv = static_cast<char *>(p->d.conv_base);
  g.ssm_block = p->ssm_block_bytes;
  g.conv_block = p->conv_block_bytes;
  g.ssm_layer = p->ssm_block_bytes * p->d.slots;
  g.conv_layer = p->conv_block_bytes * p->d.slots;
  g.slots = p->d.slots;
  g.layer_begin = layer_begin;
  g.ssm_tiles = static_cast<int32_t>((g.ssm_block + kTileBytes - 1) / kTileBytes);
  g.err = p->d.err_word;
  return g;
}

int tiles_total(const CopyGeom &g) {
  return g.ssm_tiles + static_cast<int>((g.conv_block + kTileBytes - 1) / kTileBytes);
}

}  // namespace

hipError_t launch_copy_device_pairs(const gdn_pool *p, int layer_begin, int layer_end, int n,
                                    const int32_t *src, const int32_t *dst, hipStream_t s) {
  if (n == 0 || layer_end == layer_begin) return hipSuccess;
  CopyGeom g = make_geom(p, layer_begin);
  HostPairs none{};
  for (int first = 0; first < n; first += 65535) {
    int cnt = n - first < 65535 ? n - first : 65535;
    dim3 grid(tiles_total(g), layer_end - layer_begin, cnt);
    hipLaunchKernelGGL(slot_copy_kernel<true>, grid, dim3(kThreads), 0, s, g, src + first,
                       dst + first, none);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

hipError_t launch_accept_scatter(const gdn_pool *p, const ScatterArgs &a, hipStream_t s) {
  if (a.batch == 0) return hipSuccess;
  CopyGeom g = make_geom(p, 0);
  dim3 grid(tiles_total(g), a.batch, 3);
  hipLaunchKernelGGL(accept_scatter_kernel, grid, dim3(kThreads), 0, s, g, a);
  return hipGetLastError();
}

hipError_t launch_copy_host_pairs(const gdn_pool *p, int n, const int32_t *src, const int32_t *dst,
                                  hipStream_t s) {
  CopyGeom g = make_geom(p, 0);
  for (int first = 0; first < n; first += kMaxHostPairs) {
    int cnt = n - first < kMaxHostPairs ? n - first : kMaxHostPairs;
    HostPairs hp{};
    for (int i = 0; i < cnt; ++i) {
      hp.src[i] = src[first + i];
      hp.dst[i] = dst[first + i];
    }
    dim3 grid(tiles_total(g), p->d.layers, cnt);
    hipLaunchKernelGGL(slot_copy_kernel<false>, grid, dim3(kThreads), 0, s, g, nullptr, nullptr,
                       hp);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace gdn
