// Reserved device address ranges whose physical pages can be mapped, and moved from one range to
// another, with HIP's virtual memory management.
//
// "Dynamic HBM Repartitioning for Multi-Turn MoE Serving": §IV-C, the physical pages behind a
// group of expert weights are unmapped and remapped into the KV-cache pool while the experts'
// address ranges stay reserved; §V-A, the remap unit is a multiple of the allocation
// granularity, the reclaimed pages join the free-block pool at once, and the primitive also
// runs in reverse.  Here a range is reserved once (hipMemAddressReserve) and backed chunk by
// chunk, a chunk being the remap unit (a multiple of the allocation granularity; by default the
// runtime's recommended one), with hipMemCreate + hipMemMap + hipMemSetAccess; a move unmaps
// chunks from one range and maps the same physical allocations into another, so their contents
// travel with them and nothing is copied.  Growing a pool by a moved range is then kvattn_pool_add_region or
// kvattn_pool_resize_last_region over the destination addresses.

#include <hip/hip_runtime_api.h>

#include <new>
#include <string>
#include <vector>

#include "pool_internal.h"

struct kvattn_vmm {
  int device = 0;
  char* base = nullptr;
  uint64_t va_bytes = 0, gran = 0, mapped = 0;
  std::vector<hipMemGenericAllocationHandle_t> chunk;  // one per chunk of `gran` bytes
  std::vector<unsigned char> live;                     // chunk mapped
};

namespace kvattn {
namespace {

kvattn_status hip_fail(hipError_t e, const char* what) {
  return set_error(KVATTN_E_HIP, std::string(what) + ": " + hipGetErrorString(e));
}

hipMemAllocationProp alloc_prop(int device) {
  hipMemAllocationProp prop{};
  prop.type = hipMemAllocationTypePinned;
  prop.location.type = hipMemLocationTypeDevice;
  prop.location.id = device;
  return prop;
}

// Read-write access for the device over [off, off + bytes): one call for the whole range,
// else (if the runtime refuses a range spanning several mappings) one call per chunk.
kvattn_status set_rw(const kvattn_vmm* v, uint64_t off, uint64_t bytes) {
  hipMemAccessDesc desc{};
  desc.location.type = hipMemLocationTypeDevice;
  desc.location.id = v->device;
  desc.flags = hipMemAccessFlagsProtReadWrite;
  if (hipMemSetAccess(v->base + off, bytes, &desc, 1) == hipSuccess) return KVATTN_OK;
  (void)hipGetLastError();
  for (uint64_t o = off; o < off + bytes; o += v->gran) {
    const hipError_t e = hipMemSetAccess(v->base + o, v->gran, &desc, 1);
    if (e != hipSuccess) return hip_fail(e, "vmm: hipMemSetAccess");
  }
  return KVATTN_OK;
}

bool range_ok(const kvattn_vmm* v, uint64_t off, uint64_t bytes) {
  return bytes > 0 && off % v->gran == 0 && bytes % v->gran == 0 && off <= v->va_bytes &&
         bytes <= v->va_bytes - off;
}

// Runs with v's device current, restoring the caller's afterwards.
struct DeviceScope {
  int prev = -1;
  explicit DeviceScope(int dev) {
    if (hipGetDevice(&prev) != hipSuccess) prev = -1;
    if (prev != dev) (void)hipSetDevice(dev);
  }
  ~DeviceScope() {
    if (prev >= 0) (void)hipSetDevice(prev);
  }
};

}  // namespace
}  // namespace kvattn

using kvattn::set_error;

extern "C" {

kvattn_status kvattn_vmm_create(int32_t device, uint64_t va_bytes, uint64_t chunk_bytes,
                                kvattn_vmm** out) {
  kvattn::clear_error();
  if (!out) return set_error(KVATTN_E_INVAL, "vmm_create: null output");
  *out = nullptr;
  if (va_bytes == 0) return set_error(KVATTN_E_INVAL, "vmm_create: va_bytes must be > 0");
  int supported = 0;
  hipError_t e = hipDeviceGetAttribute(
      &supported, hipDeviceAttributeVirtualMemoryManagementSupported, device);
  if (e != hipSuccess) return kvattn::hip_fail(e, "vmm_create: device query");
  if (!supported)
    return set_error(KVATTN_E_UNSUPPORTED, "vmm_create: the device has no virtual memory management");
  const hipMemAllocationProp prop = kvattn::alloc_prop(device);
  size_t min_gran = 0, gran = 0;
  e = hipMemGetAllocationGranularity(&min_gran, &prop, hipMemAllocationGranularityMinimum);
  if (e != hipSuccess || min_gran == 0) return kvattn::hip_fail(e, "vmm_create: granularity");
  if (chunk_bytes == 0) {
    e = hipMemGetAllocationGranularity(&gran, &prop, hipMemAllocationGranularityRecommended);
    if (e != hipSuccess || gran == 0 || gran % min_gran != 0) gran = min_gran;
  } else {
    if (chunk_bytes % min_gran != 0)
      return set_error(KVATTN_E_INVAL, "vmm_create: chunk_bytes must be a multiple of " +
                                           std::to_string(min_gran));
    gran = chunk_bytes;
  }
  const uint64_t va = (va_bytes + gran - 1) / gran * gran;
  void* base = nullptr;
  e = hipMemAddressReserve(&base, va, gran, nullptr, 0);
  if (e != hipSuccess) return kvattn::hip_fail(e, "vmm_create: hipMemAddressReserve");
  kvattn_vmm* v = new (std::nothrow) kvattn_vmm();
  if (!v) {
    (void)hipMemAddressFree(base, va);
    return set_error(KVATTN_E_INVAL, "vmm_create: out of host memory");
  }
  v->device = device;
  v->base = static_cast<char*>(base);
  v->va_bytes = va;
  v->gran = gran;
  v->chunk.assign(va / gran, hipMemGenericAllocationHandle_t{});
  v->live.assign(va / gran, 0);
  *out = v;
  return KVATTN_OK;
}

uint64_t kvattn_vmm_granularity(const kvattn_vmm* v) { return v ? v->gran : 0; }
void* kvattn_vmm_base(const kvattn_vmm* v) { return v ? v->base : nullptr; }
uint64_t kvattn_vmm_mapped_bytes(const kvattn_vmm* v) { return v ? v->mapped : 0; }

kvattn_status kvattn_vmm_map_new(kvattn_vmm* v, uint64_t offset, uint64_t bytes) {
  kvattn::clear_error();
  if (!v) return set_error(KVATTN_E_INVAL, "vmm_map_new: null range");
  if (!kvattn::range_ok(v, offset, bytes))
    return set_error(KVATTN_E_INVAL, "vmm_map_new: offset and size must be granularity multiples inside the range");
  for (uint64_t o = offset; o < offset + bytes; o += v->gran)
    if (v->live[o / v->gran]) return set_error(KVATTN_E_STATE, "vmm_map_new: part of the range is mapped");
  kvattn::DeviceScope scope(v->device);
  const hipMemAllocationProp prop = kvattn::alloc_prop(v->device);
  for (uint64_t o = offset; o < offset + bytes; o += v->gran) {
    hipMemGenericAllocationHandle_t h{};
    hipError_t e = hipMemCreate(&h, v->gran, &prop, 0);
    if (e != hipSuccess) return kvattn::hip_fail(e, "vmm_map_new: hipMemCreate");
    e = hipMemMap(v->base + o, v->gran, 0, h, 0);
    if (e != hipSuccess) {
      (void)hipMemRelease(h);
      return kvattn::hip_fail(e, "vmm_map_new: hipMemMap");
    }
    v->chunk[o / v->gran] = h;
    v->live[o / v->gran] = 1;
    v->mapped += v->gran;
  }
  return kvattn::set_rw(v, offset, bytes);
}

kvattn_status kvattn_vmm_move(kvattn_vmm* src, uint64_t src_offset, kvattn_vmm* dst,
                              uint64_t dst_offset, uint64_t bytes, int32_t sync_device) {
  kvattn::clear_error();
  if (!src || !dst) return set_error(KVATTN_E_INVAL, "vmm_move: null range");
  if (src->device != dst->device || src->gran != dst->gran)
    return set_error(KVATTN_E_INVAL, "vmm_move: both ranges must be on one device with one chunk size");
  if (!kvattn::range_ok(src, src_offset, bytes) || !kvattn::range_ok(dst, dst_offset, bytes))
    return set_error(KVATTN_E_INVAL, "vmm_move: offsets and size must be granularity multiples inside the ranges");
  if (src == dst && src_offset < dst_offset + bytes && dst_offset < src_offset + bytes)
    return set_error(KVATTN_E_INVAL, "vmm_move: overlapping source and destination");
  for (uint64_t i = 0; i < bytes; i += src->gran) {
    if (!src->live[(src_offset + i) / src->gran])
      return set_error(KVATTN_E_STATE, "vmm_move: part of the source is not mapped");
    if (dst->live[(dst_offset + i) / dst->gran])
      return set_error(KVATTN_E_STATE, "vmm_move: part of the destination is mapped");
  }
  kvattn::DeviceScope scope(src->device);
  if (sync_device) {
    const hipError_t e = hipDeviceSynchronize();
    if (e != hipSuccess) return kvattn::hip_fail(e, "vmm_move: hipDeviceSynchronize");
  }
  // unmap the whole source range at once (one TLB shoot-down), else chunk by chunk
  bool whole = hipMemUnmap(src->base + src_offset, bytes) == hipSuccess;
  if (!whole) (void)hipGetLastError();
  for (uint64_t i = 0; i < bytes; i += src->gran) {
    const uint64_t s = (src_offset + i) / src->gran, d = (dst_offset + i) / dst->gran;
    const hipMemGenericAllocationHandle_t h = src->chunk[s];
    if (!whole) {
      const hipError_t e = hipMemUnmap(src->base + src_offset + i, src->gran);
      if (e != hipSuccess) return kvattn::hip_fail(e, "vmm_move: hipMemUnmap");
    }
    src->live[s] = 0;
    src->mapped -= src->gran;
    const hipError_t e = hipMemMap(dst->base + dst_offset + i, dst->gran, 0, h, 0);
    if (e != hipSuccess) {
      (void)hipMemRelease(h);  // the allocation would otherwise be lost with no mapping
      return kvattn::hip_fail(e, "vmm_move: hipMemMap");
    }
    dst->chunk[d] = h;
    dst->live[d] = 1;
    dst->mapped += dst->gran;
  }
  return kvattn::set_rw(dst, dst_offset, bytes);
}

void kvattn_vmm_free(kvattn_vmm* v) {
  if (!v) return;
  {
    kvattn::DeviceScope scope(v->device);
    (void)hipDeviceSynchronize();
    for (size_t g = 0; g < v->live.size(); ++g) {
      if (!v->live[g]) continue;
      (void)hipMemUnmap(v->base + g * v->gran, v->gran);
      (void)hipMemRelease(v->chunk[g]);
    }
    (void)hipMemAddressFree(v->base, v->va_bytes);
  }
  delete v;
}

}  // extern "C"
