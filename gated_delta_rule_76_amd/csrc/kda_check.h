// Bounds checks of the checked build (libkda_checked.so, compiled with
// KDA_CHECKED=1 from the same sources as libkda.so).
//
// In the checked build every index a kernel forms into a global buffer, and
// every run-time LDS destination of a direct global->LDS load, is compared
// with the extent of the buffer it addresses before the access happens.  An
// index outside it sets the bit of its check site in a device word of its
// translation unit and the access does not happen: a load is redirected to
// element 0 of the same buffer, a store is dropped.  The host reads and
// clears the word after each call (the checked entry points synchronise their
// stream) and returns KDA_ERR_CHECK, so a wrong index shows up as a status
// instead of a stray access.  In the normal build every check compiles to
// nothing: chk() returns its index and chk_ok() returns true.
//
// Each .hip file that launches kernels includes this header once and gets its
// own device word; the sites of the prefill, decode and AttnRes units occupy
// bits 0-15, 16-23 and 24-31 of the combined mask the API reports.
#pragma once

#include <hip/hip_runtime.h>

#ifndef KDA_CHECKED
#define KDA_CHECKED 0
#endif

namespace kda {

constexpr bool kChecked = KDA_CHECKED != 0;

#if KDA_CHECKED
// The unit's failed check sites (one bit per site).  Internal linkage: one
// word per translation unit, per device.
static __device__ unsigned int g_check_sites;

__device__ __forceinline__ void check_fail(int site) {
  __hip_atomic_fetch_or(&g_check_sites, 1u << site, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Host: the unit's failed sites on the current device, then cleared.  The
// caller has synchronised the stream the unit's kernels ran on.  All ones if
// the word cannot be read.
static unsigned check_take() {
  void* p = nullptr;
  if (hipGetSymbolAddress(&p, HIP_SYMBOL(g_check_sites)) != hipSuccess) return ~0u;
  unsigned v = 0;
  if (hipMemcpy(&v, p, sizeof(v), hipMemcpyDeviceToHost) != hipSuccess) return ~0u;
  if (v != 0 && hipMemset(p, 0, sizeof(v)) != hipSuccess) return ~0u;
  return v;
}
#else
static inline unsigned check_take() { return 0; }
#endif

// Element index idx of an access `width` elements wide into a buffer of n
// elements, at check site `site`: idx itself when [idx, idx + width) lies in
// [0, n); otherwise (checked build) the site is flagged and 0 comes back.
__device__ __forceinline__ long chk(long idx, long n, int site, int width = 1) {
#if KDA_CHECKED
  if (idx < 0 || idx + width > n) {
    check_fail(site);
    return 0;
  }
#else
  (void)n;
  (void)site;
  (void)width;
#endif
  return idx;
}

// Whether a store of `width` elements at idx into n elements may proceed
// (always true in the normal build).
__device__ __forceinline__ bool chk_ok(long idx, long n, int site, int width = 1) {
#if KDA_CHECKED
  if (idx < 0 || idx + width > n) {
    check_fail(site);
    return false;
  }
#else
  (void)idx;
  (void)n;
  (void)site;
  (void)width;
#endif
  return true;
}

}  // namespace kda
