// One (pipeline depth, weight format) instance of the decode kernel, single
// step and greedy multi-step; the build compiles this file once per pair
// (AMK_INST_DEPTH, AMK_INST_WFMT) so the instances compile in parallel.
#include "vm.h"

#if !defined(AMK_INST_DEPTH) || !defined(AMK_INST_WFMT)
#error "AMK_INST_DEPTH and AMK_INST_WFMT must be defined"
#endif

namespace amk {

template __global__ void amk_vm<AMK_INST_DEPTH, AMK_INST_WFMT, false>(VmParams);
template __global__ void amk_vm<AMK_INST_DEPTH, AMK_INST_WFMT, true>(VmParams);

template <>
const void* vm_kernel<AMK_INST_DEPTH, AMK_INST_WFMT>(bool multi) {
  return multi ? reinterpret_cast<const void*>(&amk_vm<AMK_INST_DEPTH, AMK_INST_WFMT, true>)
               : reinterpret_cast<const void*>(&amk_vm<AMK_INST_DEPTH, AMK_INST_WFMT, false>);
}

}  // namespace amk
