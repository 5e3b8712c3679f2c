// Launcher of the read-bandwidth measurement kernel (stream_read.hip).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace pkv {

// Read bytes (a multiple of 16) of src with `workgroups` workgroups; out gets
// stream_read_waves_per_workgroup() words per workgroup.
int stream_read_waves_per_workgroup();
hipError_t launch_stream_read(uint32_t* out, const void* src, size_t bytes, int workgroups,
                              hipStream_t stream);

}  // namespace pkv
