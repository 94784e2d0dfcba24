// Launch of the paged-attention kernels (decode*.hip), with the kernel-timing
// events of mla_time_attention when the calling thread armed them.
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>

#include <tuple>

#include "mla_internal.h"

namespace mla {

// Launch an attention kernel (grid, block, no dynamic LDS) through the
// runtime's launch call, with the arguments converted to the kernel's
// parameter types.  With events armed, the dispatch itself records them
// (hipExtLaunchKernel): the kernel's own start and end times, and no timing
// packets queued between the kernels of the stream.
template <class... P, class... A>
hipError_t launch_attention(void (*kernel)(P...), dim3 grid, dim3 block, hipStream_t stream,
                            A... args) {
  static_assert(sizeof...(P) == sizeof...(A), "argument count");
  std::tuple<P...> formals{static_cast<P>(args)...};
  void* ptrs[sizeof...(P)];
  std::apply([&ptrs](auto&... f) {
    int i = 0;
    ((ptrs[i++] = const_cast<void*>(static_cast<const void*>(&f))), ...);
  }, formals);
  const KernelEvents ev = take_attention_events();
  const void* fn = reinterpret_cast<const void*>(kernel);
  if (ev.start != nullptr || ev.stop != nullptr)
    return hipExtLaunchKernel(fn, grid, block, ptrs, 0, stream, ev.start, ev.stop, 0);
  return hipLaunchKernel(fn, grid, block, ptrs, 0, stream);
}

}  // namespace mla
