// Host-side runtime queries shared by the libpa launchers (HIP calls, cached
// per device where they cost a driver round trip), the checked kernel launch
// every launcher goes through, and the one launcher one source file lends
// another.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <tuple>
#include <type_traits>
#include <utility>

#include "pa.h"

namespace pa {

// Compute units of the current device, or -1.
int device_cu_count();
// Workgroups of kernel `fn` with `threads` threads that fit one compute unit
// at once (cached per device and kernel), or 0 on failure.
int resident_per_cu(const void* fn, int threads);

// A launch the hardware can address: every grid dimension at least 1 and its
// work-items (workgroups x threads) within 32 bits, which is how the dispatch
// counts them.  Pure host arithmetic.
inline bool grid_fits(dim3 grid, dim3 block) {
  const uint64_t lim = 0xffffffffull;
  return grid.x > 0 && grid.y > 0 && grid.z > 0 && (uint64_t)grid.x * block.x <= lim &&
         (uint64_t)grid.y * block.y <= lim && (uint64_t)grid.z * block.z <= lim;
}

// Launch `fn` with `args` converted to its parameter types: PA_ERR_INVALID_ARG
// (nothing enqueued) for a grid outside grid_fits, PA_ERR_HIP when the runtime
// refuses the launch, else PA_OK.  The status is the launch call's own return
// value, so an error some earlier call left pending in the runtime neither
// fails this launch nor gets consumed by it.
template <typename... P, typename... A>
int launch_kernel(void (*fn)(P...), dim3 grid, dim3 block, hipStream_t stream, A&&... args) {
  static_assert(sizeof...(P) == sizeof...(A), "argument count");
  if (!grid_fits(grid, block)) return PA_ERR_INVALID_ARG;
  std::tuple<std::decay_t<P>...> vals(std::forward<A>(args)...);
  void* ptrs[sizeof...(P) > 0 ? sizeof...(P) : 1] = {};
  std::apply([&ptrs](auto&... v) {
    int i = 0;
    ((ptrs[i++] = static_cast<void*>(&v)), ...);
  }, vals);
  return hipLaunchKernel(reinterpret_cast<const void*>(fn), grid, block, ptrs, 0, stream) == hipSuccess
             ? PA_OK
             : PA_ERR_HIP;
}

struct PrefillShape;
struct PoolView;
// The fp32 column tile over the new tokens of a varlen batch (fp32
// prefill): the kernel for shape `s` and its workgroup size, then the
// launch (query_start_loc [num_seqs + 1]), partials into
// ws_acc [rows, H, parts, D] / ws_ml [rows, H, parts] for rows whose keys span
// several partitions.
const void* columns_kernel(const PrefillShape& s, int* threads);
int launch_columns(void* out, const void* query, const PoolView& pv, const int32_t* block_tables,
                   const int32_t* context_lens, const int32_t* query_start_loc, const PrefillShape& s, float scale,
                   void* ws_acc, void* ws_ml, int part_tokens, int num_parts, void* stream);

struct DecodeShape;
// Shared-prefix decode in one launch (shared_prefix_grid); PA_ERR_UNSUPPORTED,
// with nothing enqueued, when the batch does not fit that form.
int launch_shared_prefix_single(void* out, const void* query, const PoolView& pv, const int32_t* block_tables,
                                const int32_t* context_lens, const int32_t* group_start, const int32_t* prefix_lens,
                                const DecodeShape& s, int num_groups, int max_group_size, float scale,
                                void* stream);

}  // namespace pa
