// Host-side helpers of the kernel launchers: the region table passed to the kernels.
#pragma once

#include "device_common.h"
#include "pool_internal.h"

namespace kvattn {

// Region table of `pool` for the kernel arguments; `bases` (optional) replaces the regions'
// addresses, e.g. by the device-mapped addresses of pinned host regions.
inline RegionTable region_table(const kvattn_pool* pool, void* const* bases = nullptr) {
  RegionTable rt{};
  for (int r = 0; r < KVATTN_MAX_REGIONS; ++r) {
    const int src = r < pool->n_regions ? r : 0;
    rt.base[r] = static_cast<const char*>(bases ? bases[src] : pool->base[src]);
    rt.first[r] = pool->first_id[r];
    rt.first32[r] = static_cast<int32_t>(pool->first_id[r]);
    rt.adj[r] = reinterpret_cast<uint64_t>(rt.base[r]) -
                static_cast<uint64_t>(pool->first_id[r]) * static_cast<uint64_t>(pool->block_bytes);
  }
  rt.first[KVATTN_MAX_REGIONS] = pool->first_id[KVATTN_MAX_REGIONS];
  rt.block_bytes = pool->block_bytes;
  rt.n = pool->n_regions;
  rt.total = (int32_t)pool->total_blocks;
  return rt;
}

}  // namespace kvattn
