// Host-side runtime queries shared by the libpa launchers (HIP calls, cached
// per device where they cost a driver round trip).
#pragma once

namespace pa {

// Compute units of the current device, or -1.
int device_cu_count();
// Workgroups of kernel `fn` with `threads` threads that fit one compute unit
// at once (cached per device and kernel), or 0 on failure.
int resident_per_cu(const void* fn, int threads);
// PA_OK, or PA_ERR_HIP if the last launch failed.
int launch_status();

}  // namespace pa
