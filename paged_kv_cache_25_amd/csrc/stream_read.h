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
// Read the 4 KiB chunks ids[0 .. num_ids) of src (bytes long), per_workgroup
// of them per one-wave workgroup (num_ids a multiple of it); out gets 64
// words per workgroup.
hipError_t launch_gather_read(uint32_t* out, const void* src, size_t bytes, const int32_t* ids,
                              int num_ids, int per_workgroup, hipStream_t stream);

}  // namespace pkv
