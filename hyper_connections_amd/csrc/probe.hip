// Measurement probes: the launch floor and the HBM read ceiling that the decode kernels are
// measured against. They are not steps of the decode path.
//
//  k_probe_empty : does nothing; back to back it gives the per-launch floor of a call made of
//                  dependent kernels.
//  k_probe_read  : streams a buffer once with 16-byte nontemporal loads, U loads in flight per
//                  lane and a grid stride over the buffer; every block writes one word (the XOR
//                  of what its lanes read) so that no load can be dropped.
//  k_probe_barrier: n grid-wide barriers in a grid small enough to be resident at once: the cost
//                  of joining all blocks inside one launch, against the cost of a kernel boundary
//                  (k_probe_empty). Thread 0 of each block adds one to a device-scope arrival
//                  counter; the last arrival resets it and advances a generation word that the
//                  others poll (sleeping between polls). ORDERED: the arrival is a release and the
//                  wait ends with an acquire (what a barrier that hands data between blocks needs:
//                  the caches are written back and invalidated), else both are relaxed (the
//                  atomics alone). Every wait is bounded; a wait that runs out sets the third
//                  state word and ends the kernel.
#include "dhp_internal.hpp"

namespace {

__global__ void k_probe_empty() {}

template <int U>
__global__ __launch_bounds__(256) void k_probe_read(const u32x4* __restrict__ buf, long long n16,
                                                    uint32_t* __restrict__ sink) {
    const long long stride = (long long)gridDim.x * 256 * U;
    uint32_t acc = 0;
    for (long long base = (long long)blockIdx.x * 256 * U + threadIdx.x; base < n16; base += stride) {
        u32x4 v[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const long long i = base + (long long)u * 256;
            v[u] = __builtin_nontemporal_load(buf + (i < n16 ? i : n16 - 1));
        }
#pragma unroll
        for (int u = 0; u < U; ++u) acc ^= (v[u].x ^ v[u].y) ^ (v[u].z ^ v[u].w);
    }
    for (int o = 32; o > 0; o >>= 1) acc ^= __shfl_xor(acc, o);
    __shared__ uint32_t w[4];
    if ((threadIdx.x & 63) == 0) w[threadIdx.x >> 6] = acc;
    __syncthreads();
    if (threadIdx.x == 0) sink[blockIdx.x] = (w[0] ^ w[1]) ^ (w[2] ^ w[3]);
}

template <bool ORDERED>
__global__ __launch_bounds__(256) void k_probe_barrier(uint32_t* __restrict__ state, int n, uint32_t* __restrict__ sink) {
    __shared__ uint32_t ok_s;
    for (int i = 0; i < n; ++i) {
        __syncthreads();
        if (threadIdx.x == 0) {
            uint32_t ok = 1;
            const uint32_t gen = __hip_atomic_load(state + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            const uint32_t a = ORDERED
                ? __hip_atomic_fetch_add(state, 1u, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_AGENT)
                : __hip_atomic_fetch_add(state, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            if (a == gridDim.x - 1) {
                __hip_atomic_store(state, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                if (ORDERED) __hip_atomic_fetch_add(state + 1, 1u, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
                else __hip_atomic_fetch_add(state + 1, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            } else {
                uint32_t polls = 0;
                while (__hip_atomic_load(state + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == gen) {
                    if (++polls > (1u << 18)) {
                        ok = 0;
                        __hip_atomic_store(state + 2, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                        break;
                    }
                    __builtin_amdgcn_s_sleep(2);
                }
                if (ORDERED) __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
            }
            ok_s = ok;
        }
        __syncthreads();
        if (!ok_s) break;
    }
    if (threadIdx.x == 0) sink[blockIdx.x] = ok_s;
}

int launch_status(const char* what) {
    const hipError_t e = hipGetLastError();
    return e == hipSuccess ? DHP_OK : dhp_fail(DHP_ERR_LAUNCH, "%s launch: %s", what, hipGetErrorString(e));
}

}  // namespace

extern "C" {

int decodehp_probe_empty(int32_t count, void* stream) {
    if (count < 1 || count > 100000) return dhp_fail(DHP_ERR_UNSUPPORTED, "count=%d (1..100000)", count);
    DeviceFacts dev;
    if (!dhp_current_device(&dev)) return DHP_ERR_NO_DEVICE;
    for (int i = 0; i < count; ++i)
        hipLaunchKernelGGL(k_probe_empty, dim3(1), dim3(64), 0, static_cast<hipStream_t>(stream));
    return launch_status("empty probe");
}

int decodehp_probe_read(const void* buf, size_t bytes, int32_t blocks_per_cu, int32_t loads_in_flight,
                        uint32_t* sink, int32_t sink_words, void* stream) {
    if (!buf || !sink || bytes == 0) return dhp_fail(DHP_ERR_INVALID, "null buffer or sink, or zero bytes");
    if (bytes % 16 || reinterpret_cast<uintptr_t>(buf) % 16)
        return dhp_fail(DHP_ERR_MISALIGNED, "buffer and bytes must be 16-byte multiples");
    if (blocks_per_cu < 1 || blocks_per_cu > 16)
        return dhp_fail(DHP_ERR_UNSUPPORTED, "blocks_per_cu=%d (1..16)", blocks_per_cu);
    if (loads_in_flight != 1 && loads_in_flight != 2 && loads_in_flight != 4 && loads_in_flight != 8)
        return dhp_fail(DHP_ERR_UNSUPPORTED, "loads_in_flight=%d (1, 2, 4 or 8)", loads_in_flight);
    DeviceFacts dev;
    if (!dhp_current_device(&dev)) return DHP_ERR_NO_DEVICE;
    const int blocks = blocks_per_cu * dev.cus;
    if (sink_words < blocks) return dhp_fail(DHP_ERR_WORKSPACE, "sink holds %d words, %d needed", sink_words, blocks);
    const auto* p = static_cast<const u32x4*>(buf);
    const long long n16 = (long long)(bytes / 16);
    const hipStream_t s = static_cast<hipStream_t>(stream);
    switch (loads_in_flight) {
        case 1: hipLaunchKernelGGL(k_probe_read<1>, dim3(blocks), dim3(256), 0, s, p, n16, sink); break;
        case 2: hipLaunchKernelGGL(k_probe_read<2>, dim3(blocks), dim3(256), 0, s, p, n16, sink); break;
        case 4: hipLaunchKernelGGL(k_probe_read<4>, dim3(blocks), dim3(256), 0, s, p, n16, sink); break;
        default: hipLaunchKernelGGL(k_probe_read<8>, dim3(blocks), dim3(256), 0, s, p, n16, sink); break;
    }
    return launch_status("read probe");
}

// n barriers in one launch of `blocks` blocks of 256 threads (at most one per CU, so all are
// resident). state: 4 zeroed 32-bit words of device memory, left with a zero count (word 2 is
// set if a wait ran out); sink: `blocks` words.
int decodehp_probe_grid_barrier(int32_t blocks, int32_t n, int32_t ordered, uint32_t* state, uint32_t* sink,
                                void* stream) {
    if (!state || !sink) return dhp_fail(DHP_ERR_INVALID, "null state or sink");
    if (n < 0 || n > 10000) return dhp_fail(DHP_ERR_UNSUPPORTED, "n=%d (0..10000)", n);
    DeviceFacts dev;
    if (!dhp_current_device(&dev)) return DHP_ERR_NO_DEVICE;
    if (blocks < 1 || blocks > dev.cus) return dhp_fail(DHP_ERR_UNSUPPORTED, "blocks=%d (1..%d)", blocks, dev.cus);
    const hipStream_t s = static_cast<hipStream_t>(stream);
    if (ordered) hipLaunchKernelGGL(k_probe_barrier<true>, dim3(blocks), dim3(256), 0, s, state, n, sink);
    else hipLaunchKernelGGL(k_probe_barrier<false>, dim3(blocks), dim3(256), 0, s, state, n, sink);
    return launch_status("grid barrier probe");
}

}  // extern "C"
