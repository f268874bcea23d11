// pkv_noalloc.h -- internal: the static decode scratch of paged_attn_decode_noalloc.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>

namespace pkv {

// Bytes of the static scratch every GPU holds for paged_attn_decode_noalloc:
// 32 MiB.  A balanced split needs (waves + sequences x kv heads) rows of
// (q heads per kv head) x (head_dim + 1) floats: on a full MI355X grid (2048
// waves) with 8 kv heads, a kv group of 4 and head_dim 128 that is 5.3 MB for
// 64 sequences and 8.5 MB for 256, and 32 MiB holds up to about 1500.
constexpr size_t kScratchBytes = size_t(32) << 20;
constexpr int kMaxDevices = 64;

// Device address and size of the current device's scratch.  The address is
// looked up (hipGetSymbolAddress) on the first call on each device and kept;
// later calls on that device return it.  Thread-safe.
hipError_t static_scratch(void** ptr, size_t* bytes);

}  // namespace pkv
