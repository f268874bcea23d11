// pkv_probe.h -- internal: the streaming-read probe behind pkv_read_probe.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pkv {

// Bytes one wave reads per slice (the probe reads whole slices only).
int64_t read_probe_slice_bytes();

// Read the first (bytes / slice) * slice bytes of buf once, workgroups x 256
// threads; sink: device uint32 [workgroups * 256], written (almost) never.
hipError_t launch_read_probe(const void* buf, int64_t bytes, int workgroups, bool nontemporal, uint32_t* sink,
                             hipStream_t stream);

}  // namespace pkv
