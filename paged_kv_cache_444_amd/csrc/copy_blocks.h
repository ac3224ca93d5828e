// Host-side interface of the whole-block copy used for copy-on-write.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pa {

struct CopyBlocksParams {
  uint16_t* kpool;
  uint16_t* vpool;
  const int64_t* mapping;  // [num_pairs][2] (source, destination) block ids
  int64_t num_blocks;
  int64_t block_vec16;     // 16-byte vectors in one block of one pool
  int num_pairs;
};

hipError_t launch_copy_blocks(const CopyBlocksParams& p, hipStream_t stream);

}  // namespace pa
