// pkv_probe.hip -- a plain streaming read of a device buffer: the rate HBM
// delivers to 16-byte vector loads on this GPU, the ceiling against which the
// decode kernels' K/V streaming is read.
//
// Every wave reads contiguous 16 KiB slices (64 lanes x 16 bytes x 16 loads in
// flight), slice i of the grid-wide list going to wave i mod waves.  Each lane
// folds what it loaded into one word and stores it only if it equals a value
// no buffer of random data produces in practice, so no load can be dropped and
// almost nothing is written.  Loads are plain or non-temporal (the decode
// kernels' K/V loads are non-temporal: every byte is read once).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "pkv_probe.h"

namespace pkv {
namespace {

constexpr int kProbeThreads = 256;
constexpr int kSliceLoads = 16;                       // 16-byte loads per lane per slice
constexpr int64_t kSliceBytes = 64 * 16 * kSliceLoads;   // 16 KiB per wave slice

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

template <bool NT>
__global__ void __launch_bounds__(kProbeThreads) read_probe_kernel(const u32x4* buf, int64_t slices,
                                                                   uint32_t* sink) {
    const int lane = threadIdx.x & 63;
    const int64_t wave = (int64_t)blockIdx.x * (kProbeThreads / 64) + (threadIdx.x >> 6);
    const int64_t waves = (int64_t)gridDim.x * (kProbeThreads / 64);
    uint32_t acc = 0;
    for (int64_t sl = wave; sl < slices; sl += waves) {
        const u32x4* p = buf + sl * (kSliceBytes / 16) + lane;
        u32x4 v[kSliceLoads];
#pragma unroll
        for (int i = 0; i < kSliceLoads; ++i) v[i] = NT ? __builtin_nontemporal_load(p + 64 * i) : p[64 * i];
#pragma unroll
        for (int i = 0; i < kSliceLoads; ++i) acc ^= v[i][0] ^ v[i][1] ^ v[i][2] ^ v[i][3];
    }
    if (acc == 0x9E3779B9u) sink[(int64_t)blockIdx.x * kProbeThreads + threadIdx.x] = acc;
}

}  // namespace

int64_t read_probe_slice_bytes() { return kSliceBytes; }

hipError_t launch_read_probe(const void* buf, int64_t bytes, int workgroups, bool nontemporal, uint32_t* sink,
                             hipStream_t stream) {
    const int64_t slices = bytes / kSliceBytes;
    if (slices <= 0 || workgroups <= 0) return hipErrorInvalidValue;
    const u32x4* b = reinterpret_cast<const u32x4*>(buf);
    if (nontemporal)
        hipLaunchKernelGGL(read_probe_kernel<true>, dim3((unsigned)workgroups), dim3(kProbeThreads), 0, stream, b,
                           slices, sink);
    else
        hipLaunchKernelGGL(read_probe_kernel<false>, dim3((unsigned)workgroups), dim3(kProbeThreads), 0, stream, b,
                           slices, sink);
    return hipGetLastError();
}

}  // namespace pkv
