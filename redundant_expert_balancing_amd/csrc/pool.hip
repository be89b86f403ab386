// Process-global pool of prefetch slots, shared by every layer of one projection
// type, through HIP virtual memory.
//
// The pages want two things at once: each projection's weights form ONE
// contiguous [E+B, H, H'] tensor that the grouped GEMM addresses by row index,
// and the B prefetch slots come from a process-global pool shared by all
// layers, so the extra memory is B expert weights per projection in total, not
// per layer [ai-maestro.online "Moonshot AI open-sources MoonEP", section "The
// memory contract"; the same section of the noticiai.com.br page]. Virtual
// memory gives both: a layer's view is one reserved address range whose first
// E rows map the layer's own home-weight allocation and whose remaining R*B rows
// map the pool's physical slot memory. Every kernel sees a plain contiguous
// tensor; no kernel knows about the pool.
//
// Host code only. These calls allocate (they are the allocator); every other
// entry point of the library allocates nothing.
#include <new>

#include "common.h"

struct moonep_pool {
  int device;
  int32_t R, B, H, Hp, dtype;
  size_t row_bytes;   // one expert weight row, H * Hp * element size
  size_t set_bytes;   // R * B rows rounded up to the granularity
  size_t gran;
  int32_t nsets;
  hipMemGenericAllocationHandle_t* sets;
};

struct moonep_view {
  int32_t set;
  void* va;
  size_t va_bytes;
  size_t home_bytes;
  size_t slot_bytes;   // a copy: destroying the view never reads the pool
  hipMemGenericAllocationHandle_t home;
};

namespace moonep {

static hipMemAllocationProp device_prop(int dev) {
  hipMemAllocationProp p{};
  p.type = hipMemAllocationTypePinned;
  p.location.type = hipMemLocationTypeDevice;
  p.location.id = dev;
  return p;
}

static size_t round_up(size_t x, size_t g) { return (x + g - 1) / g * g; }

static size_t granularity(int dev) {
  int vmm = 0;
  if (hipDeviceGetAttribute(&vmm, hipDeviceAttributeVirtualMemoryManagementSupported, dev) !=
          hipSuccess ||
      !vmm)
    return 0;
  hipMemAllocationProp p = device_prop(dev);
  size_t g = 0;
  if (hipMemGetAllocationGranularity(&g, &p, hipMemAllocationGranularityMinimum) != hipSuccess)
    return 0;
  return g;
}

}  // namespace moonep

using namespace moonep;

extern "C" size_t moonep_vm_granularity(void) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 0;
  return granularity(dev);
}

extern "C" int moonep_pool_create(const moonep_shape* shape, int32_t nsets, moonep_pool** pool) {
  if (!pool) return MOONEP_EINVAL;
  *pool = nullptr;
  int st = validate(shape);
  if (st) return st;
  const moonep_shape& s = *shape;
  if (s.B < 1 || nsets < 1 || nsets > 64) return MOONEP_EINVAL;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return MOONEP_EHIP;
  const size_t gran = granularity(dev);
  if (gran == 0) return MOONEP_EHIP;
  moonep_pool* p = new (std::nothrow) moonep_pool{};
  if (!p) return MOONEP_EHIP;
  p->sets = new (std::nothrow) hipMemGenericAllocationHandle_t[nsets]();
  if (!p->sets) {
    delete p;
    return MOONEP_EHIP;
  }
  p->device = dev;
  p->R = s.R; p->B = s.B; p->H = s.H; p->Hp = s.Hp; p->dtype = s.dtype;
  p->row_bytes = size_t(s.H) * s.Hp * elem_bytes(s);
  p->gran = gran;
  p->set_bytes = round_up(size_t(s.R) * s.B * p->row_bytes, gran);
  const hipMemAllocationProp prop = device_prop(dev);
  for (int i = 0; i < nsets; ++i) {
    if (hipMemCreate(&p->sets[i], p->set_bytes, &prop, 0) != hipSuccess) {
      for (int j = 0; j < i; ++j) (void)hipMemRelease(p->sets[j]);
      delete[] p->sets;
      delete p;
      return MOONEP_EHIP;
    }
    p->nsets = i + 1;
  }
  *pool = p;
  return MOONEP_OK;
}

extern "C" int moonep_pool_destroy(moonep_pool* pool) {
  if (!pool) return MOONEP_EINVAL;
  int st = MOONEP_OK;
  for (int i = 0; i < pool->nsets; ++i)
    if (hipMemRelease(pool->sets[i]) != hipSuccess) st = MOONEP_EHIP;
  delete[] pool->sets;
  delete pool;
  return st;
}

extern "C" size_t moonep_pool_bytes(const moonep_pool* pool) {
  return pool ? pool->set_bytes * size_t(pool->nsets) : 0;
}

extern "C" int moonep_view_create(const moonep_shape* shape, moonep_pool* pool, int32_t set,
                                  moonep_view** view, void** w_all) {
  if (!view || !w_all || !pool) return MOONEP_EINVAL;
  *view = nullptr;
  *w_all = nullptr;
  int st = validate(shape);
  if (st) return st;
  const moonep_shape& s = *shape;
  if (set < 0 || set >= pool->nsets) return MOONEP_EINVAL;
  // the slot rows of every view of a pool have one size and count
  if (s.R != pool->R || s.B != pool->B || s.H != pool->H || s.Hp != pool->Hp ||
      s.dtype != pool->dtype)
    return MOONEP_EINVAL;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return MOONEP_EHIP;
  if (dev != pool->device) return MOONEP_EINVAL;
  const size_t home_bytes = size_t(s.E) * pool->row_bytes;
  // the slot mapping starts right after the home rows: that boundary must be a
  // mapping boundary
  if (home_bytes == 0 || home_bytes % pool->gran) return MOONEP_EINVAL;
  moonep_view* v = new (std::nothrow) moonep_view{};
  if (!v) return MOONEP_EHIP;
  v->set = set;
  v->home_bytes = home_bytes;
  v->slot_bytes = pool->set_bytes;
  v->va_bytes = home_bytes + pool->set_bytes;
  const hipMemAllocationProp prop = device_prop(dev);
  bool reserved = false, created = false, home_mapped = false, slots_mapped = false;
  do {
    if (hipMemAddressReserve(&v->va, v->va_bytes, pool->gran, nullptr, 0) != hipSuccess) break;
    reserved = true;
    if (hipMemCreate(&v->home, home_bytes, &prop, 0) != hipSuccess) break;
    created = true;
    if (hipMemMap(v->va, home_bytes, 0, v->home, 0) != hipSuccess) break;
    home_mapped = true;
    if (hipMemMap(static_cast<char*>(v->va) + home_bytes, pool->set_bytes, 0, pool->sets[set], 0) !=
        hipSuccess)
      break;
    slots_mapped = true;
    hipMemAccessDesc acc{};
    acc.location.type = hipMemLocationTypeDevice;
    acc.location.id = dev;
    acc.flags = hipMemAccessFlagsProtReadWrite;
    if (hipMemSetAccess(v->va, v->va_bytes, &acc, 1) != hipSuccess) break;
    *view = v;
    *w_all = v->va;
    return MOONEP_OK;
  } while (false);
  if (slots_mapped) (void)hipMemUnmap(static_cast<char*>(v->va) + home_bytes, pool->set_bytes);
  if (home_mapped) (void)hipMemUnmap(v->va, home_bytes);
  if (created) (void)hipMemRelease(v->home);
  if (reserved) (void)hipMemAddressFree(v->va, v->va_bytes);
  delete v;
  return MOONEP_EHIP;
}

extern "C" int moonep_view_destroy(moonep_view* view) {
  if (!view) return MOONEP_EINVAL;
  // no kernel may still read the range being unmapped
  int st = hipDeviceSynchronize() == hipSuccess ? MOONEP_OK : MOONEP_EHIP;
  char* va = static_cast<char*>(view->va);
  if (hipMemUnmap(va + view->home_bytes, view->slot_bytes) != hipSuccess) st = MOONEP_EHIP;
  if (hipMemUnmap(va, view->home_bytes) != hipSuccess) st = MOONEP_EHIP;
  if (hipMemRelease(view->home) != hipSuccess) st = MOONEP_EHIP;
  if (hipMemAddressFree(view->va, view->va_bytes) != hipSuccess) st = MOONEP_EHIP;
  delete view;
  return st;
}
