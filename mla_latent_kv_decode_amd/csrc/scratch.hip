// scratch.hip -- the static device scratch of mla_decode_step_noalloc.
//
// Callers that cannot allocate device memory (code under graph capture, tight
// serving loops, harnesses that forbid hipMalloc) get a decode step whose
// workspace lives in this file-scope array instead of a caller buffer.  Every
// GPU the library runs on holds its own copy, at its own address, from the
// moment the code object is loaded until the process ends.  In host code the
// array's name is only a host-side stand-in: its device address comes from
// hipGetSymbolAddress, taken once per device at mla_create (with that device
// current) and kept by the host library.

#include <hip/hip_runtime.h>

#include "mla.h"

static __device__ __align__(256) unsigned char scratch[MLA_NOALLOC_SCRATCH_BYTES];

namespace mla {

// Device address of the current device's copy of `scratch`; the HIP status of
// the lookup.
hipError_t noalloc_scratch_address(void** out) {
  void* p = nullptr;
  const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
  if (e == hipSuccess) *out = p;
  return e;
}

}  // namespace mla
