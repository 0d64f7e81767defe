// Streaming-bandwidth probe for gfx950: what the HBM of one GPU delivers to plain access patterns,
// the ceiling the attention kernels' achieved bandwidth is read against. Not part of the attention
// library's interface: libstreamprobe.so is loaded by the benchmark only.
//
// Three patterns over buffers far larger than the 256 MB Infinity Cache, 16-byte accesses, every
// lane touching consecutive 16-byte chunks of its wave's 1 KB span (fully coalesced), and one of
// buffer-to-LDS staging from a buffer small enough to stay on chip:
//   read  : sum every chunk (one float per thread written at the end, so nothing is optimised away)
//   write : fill every chunk (plain stores, or non-temporal)
//   copy  : read a chunk, write it elsewhere
//   lds   : stage a buffer of a few tens of MB into LDS, over and over (see lds_read_kernel)
// One thread per kChunks chunks; the grid covers the buffer once (lds: a fixed grid).
#include <hip/hip_runtime.h>

#include <cstdint>

namespace {

constexpr int kThreads = 256;
constexpr int kChunks = 4;   // 16-byte chunks per thread, kThreads * 16 bytes apart

typedef uint32_t u4_t __attribute__((ext_vector_type(4)));

__global__ __launch_bounds__(kThreads) void read_kernel(const uint4* __restrict__ src, int64_t n, float* __restrict__ sink) {
    const int64_t base = static_cast<int64_t>(blockIdx.x) * kThreads * kChunks + threadIdx.x;
    uint32_t acc = 0;
#pragma unroll
    for (int c = 0; c < kChunks; ++c) {
        const int64_t e = base + static_cast<int64_t>(c) * kThreads;
        if (e < n) {
            const uint4 v = src[e];
            acc ^= v.x ^ v.y ^ v.z ^ v.w;
        }
    }
    if (acc == 0x9e3779b9u) sink[blockIdx.x] = static_cast<float>(acc);   // practically never
}

template <bool NT>
__global__ __launch_bounds__(kThreads) void write_kernel(uint4* __restrict__ dst, int64_t n) {
    const int64_t base = static_cast<int64_t>(blockIdx.x) * kThreads * kChunks + threadIdx.x;
#pragma unroll
    for (int c = 0; c < kChunks; ++c) {
        const int64_t e = base + static_cast<int64_t>(c) * kThreads;
        if (e < n) {
            const uint4 v = make_uint4(static_cast<uint32_t>(e), 1u, 2u, 3u);
            if constexpr (NT)
                __builtin_nontemporal_store(__builtin_bit_cast(u4_t, v), reinterpret_cast<u4_t*>(dst + e));
            else
                dst[e] = v;
        }
    }
}

__global__ __launch_bounds__(kThreads) void copy_kernel(const uint4* __restrict__ src, uint4* __restrict__ dst, int64_t n) {
    const int64_t base = static_cast<int64_t>(blockIdx.x) * kThreads * kChunks + threadIdx.x;
    uint4 v[kChunks];
#pragma unroll
    for (int c = 0; c < kChunks; ++c) {
        const int64_t e = base + static_cast<int64_t>(c) * kThreads;
        v[c] = (e < n) ? src[e] : make_uint4(0u, 0u, 0u, 0u);
    }
#pragma unroll
    for (int c = 0; c < kChunks; ++c) {
        const int64_t e = base + static_cast<int64_t>(c) * kThreads;
        if (e < n) dst[e] = v[c];
    }
}

// LDS staging from a buffer that stays on chip (sized like the attention kernels' staged rows:
// a few tens of MB, read over and over from the caches in front of HBM): each workgroup issues
// 1 KB contiguous buffer-to-LDS transfers, 16 bytes per lane, into its 16 KB of LDS, chunk after
// chunk with no compute, and waits for them at the end. The attention kernels stage their rows
// with the same instruction and grain.
typedef __attribute__((address_space(3))) void* lds_ptr_t;
// The LDS address of a __shared__ location (an address-space cast, kept in an SGPR: the same for
// the whole wave), as the buffer-to-LDS transfer takes it.
__device__ __forceinline__ lds_ptr_t lds_addr(char* p) {
    uint32_t a = static_cast<uint32_t>(reinterpret_cast<uintptr_t>((lds_ptr_t)p));
    asm volatile("" : "+s"(a));
    return (lds_ptr_t)static_cast<uintptr_t>(a);
}

constexpr int kLdsChunk = 16384;   // one workgroup's chunk: 16 transfers of 1 KB (4 per wave)
constexpr int kLdsGrid = 2048;     // 8 workgroups per CU
constexpr int kLdsPasses = 16;     // times the buffer is read

__global__ __launch_bounds__(kThreads) void lds_read_kernel(const uint4* __restrict__ src, int64_t chunks, int64_t per_wg) {
    __shared__ __attribute__((aligned(1024))) char buf[kLdsChunk];
    const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint4*>(src), 0, 0x7fffffff, 0x00020000);
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
    for (int64_t k = 0; k < per_wg; ++k) {
        const int64_t c = (static_cast<int64_t>(blockIdx.x) + k * gridDim.x) % chunks;
        const int base = static_cast<int>(c * kLdsChunk);
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int g = wave + 4 * u;
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, lds_addr(buf + g * 1024), 16, base + g * 1024 + lane * 16, 0, 0, 0);
        }
    }
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
}

unsigned blocks_for(int64_t n) {
    return static_cast<unsigned>((n + static_cast<int64_t>(kThreads) * kChunks - 1) / (static_cast<int64_t>(kThreads) * kChunks));
}

}  // namespace

extern "C" {

// pattern: 0 read, 1 write, 2 write (non-temporal), 3 copy, 4 LDS staging of a resident buffer.
// a, b: device buffers of `bytes` bytes (b unused by read, write and 4; sink: device
// float[blocks] for read). bytes: a multiple of 16 (of 16384 for 4). Pattern 4 moves `passes`
// times `bytes` into LDS (passes: the caller's; `b` is ignored there, and the byte count to time
// against is streamprobe_lds_bytes). Returns the hipError_t of the launch (0 on success). The
// caller times the launch on `stream`.
int streamprobe_launch(int pattern, void* a, void* b, float* sink, int64_t bytes, void* stream) {
    const int64_t n = bytes / 16;
    hipStream_t s = static_cast<hipStream_t>(stream);
    switch (pattern) {
        case 4: {
            const int64_t chunks = bytes / kLdsChunk;
            hipLaunchKernelGGL(lds_read_kernel, dim3(kLdsGrid), dim3(kThreads), 0, s, static_cast<const uint4*>(a), chunks,
                               chunks * kLdsPasses / kLdsGrid);
            break;
        }
        case 0: hipLaunchKernelGGL(read_kernel, dim3(blocks_for(n)), dim3(kThreads), 0, s, static_cast<const uint4*>(a), n, sink); break;
        case 1: hipLaunchKernelGGL((write_kernel<false>), dim3(blocks_for(n)), dim3(kThreads), 0, s, static_cast<uint4*>(a), n); break;
        case 2: hipLaunchKernelGGL((write_kernel<true>), dim3(blocks_for(n)), dim3(kThreads), 0, s, static_cast<uint4*>(a), n); break;
        case 3: hipLaunchKernelGGL(copy_kernel, dim3(blocks_for(n)), dim3(kThreads), 0, s, static_cast<const uint4*>(a), static_cast<uint4*>(b), n); break;
        default: return static_cast<int>(hipErrorInvalidValue);
    }
    return static_cast<int>(hipGetLastError());
}

// Blocks of the read pattern for `bytes` (the sink's length).
int64_t streamprobe_read_blocks(int64_t bytes) { return blocks_for(bytes / 16); }

// Bytes pattern 4 moves for a buffer of `bytes`.
int64_t streamprobe_lds_bytes(int64_t bytes) {
    const int64_t chunks = bytes / kLdsChunk;
    return chunks * kLdsPasses / kLdsGrid * kLdsGrid * kLdsChunk;
}

}  // extern "C"
