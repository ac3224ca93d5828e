// Host-side interface of the streaming-read ceiling kernel.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace pa {

// Workgroups a streaming read is launched with on the current device (0 if it cannot be queried);
// the sink needs one uint32 per workgroup.
int stream_read_grid();
hipError_t launch_stream_read(const void* src, size_t bytes, uint32_t* sink, int grid,
                              hipStream_t stream);

}  // namespace pa
