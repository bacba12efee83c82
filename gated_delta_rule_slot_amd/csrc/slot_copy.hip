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

__device__ __forceinline__ void copy_tile(char *base, int64_t block_bytes, int64_t src_off,
                                          int64_t dst_off, int64_t tile_off) {
  const u32x4 *src = reinterpret_cast<const u32x4 *>(base + src_off);
  u32x4 *dst = reinterpret_cast<u32x4 *>(base + dst_off);
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
    copy_tile(g.ssm, g.ssm_block, layer * g.ssm_layer + src * g.ssm_block,
              layer * g.ssm_layer + dst * g.ssm_block, int64_t(tile) * kTileBytes);
  } else {
    copy_tile(g.conv, g.conv_block, layer * g.conv_layer + src * g.conv_block,
              layer * g.conv_layer + dst * g.conv_block, int64_t(tile - g.ssm_tiles) * kTileBytes);
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
