// HBM read-stream calibration (a measurement aid, built into its own library and
// used by the benchmark only; not part of the verify path or its C interface).
//
// It times what one GPU delivers to a kernel that reads a buffer once, so the
// benchmark can set a memory-bound kernel's bandwidth beside both the published
// peak and what a bare stream reaches on the same box.  Two ways of streaming,
// one 512-thread workgroup per CU over a contiguous share of the buffer each:
//   mode 0: 72 KiB tiles into LDS with global_load_lds_dwordx4, double
//           buffered, barriers that wait only for the tile being consumed (the
//           attention kernel's own way of streaming its cache, minus the math);
//   mode 1: plain 16-byte loads into registers, 8 in flight per lane.
// Each workgroup reads only whole units (72 KiB tiles, or 64 KiB steps in mode 1)
// of its share, so the bytes read are slightly below `bytes`; the count is
// returned.
//
//   int ddtv_calib_stream_read(const void* src, int64_t bytes, int mode,
//                              float* sink, int workgroups, hipStream_t stream,
//                              int64_t* bytes_read /* HOST */)
//     src        device buffer, 16-byte aligned, at least `bytes` long
//     sink       device float[workgroups * 512], overwritten (keeps the reads live)
//     workgroups 1 .. 65535 (the benchmark passes the CU count)
//   Returns 0, 1 for a bad argument (nothing launched) or 5 for a launch error.
//   Asynchronous on `stream`; the caller times it with events on that stream.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void;

constexpr int kThreads = 512;
constexpr int kLoads = 9;                          // 1 KiB loads per wave per tile
constexpr int kTileBytes = 8 * kLoads * 1024;      // 72 KiB
constexpr int kVgprUnroll = 8;
constexpr int kVgprStep = kThreads * 16 * kVgprUnroll;   // 64 KiB per workgroup step

__global__ __launch_bounds__(kThreads, 1) void stream_lds_kernel(const char* src, int64_t tiles, float* sink) {
    __shared__ f32x4 buf[2][kTileBytes / 16];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const char* base = src + (int64_t)blockIdx.x * tiles * kTileBytes;
    auto issue = [&](int64_t t) {
        char* lb = reinterpret_cast<char*>(buf[t & 1]);
#pragma unroll
        for (int k = 0; k < kLoads; ++k)
            __builtin_amdgcn_global_load_lds(base + t * kTileBytes + (wave * kLoads + k) * 1024 + lane * 16,
                                             (lds_void*)(lb + (wave * kLoads + k) * 1024), 16, 0, 0);
    };
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    if (tiles > 0) issue(0);
    for (int64_t i = 0; i < tiles; ++i) {
        // tile i has landed once at most the kLoads loads of tile i + 1 are pending
        if (i + 1 < tiles) {
            issue(i + 1);
            asm volatile("s_waitcnt vmcnt(%0)\n\ts_barrier" ::"n"(kLoads) : "memory");
        } else {
            asm volatile("s_waitcnt vmcnt(0)\n\ts_barrier" ::: "memory");
        }
        acc += buf[i & 1][threadIdx.x];
        // every wave's read of this buffer is done before it is refilled
        asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" : "+v"(acc)::"memory");
    }
    sink[(int64_t)blockIdx.x * kThreads + threadIdx.x] = (acc.x + acc.y) + (acc.z + acc.w);
}

__global__ __launch_bounds__(kThreads) void stream_vgpr_kernel(const char* src, int64_t steps, float* sink) {
    const char* base = src + (int64_t)blockIdx.x * steps * kVgprStep + threadIdx.x * 16;
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    for (int64_t i = 0; i < steps; ++i) {
        f32x4 v[kVgprUnroll];
#pragma unroll
        for (int u = 0; u < kVgprUnroll; ++u)
            v[u] = *reinterpret_cast<const f32x4*>(base + i * kVgprStep + u * (kThreads * 16));
#pragma unroll
        for (int u = 0; u < kVgprUnroll; ++u) acc += v[u];
    }
    sink[(int64_t)blockIdx.x * kThreads + threadIdx.x] = (acc.x + acc.y) + (acc.z + acc.w);
}

}  // namespace

extern "C" int ddtv_calib_stream_read(const void* src, int64_t bytes, int mode, float* sink, int workgroups,
                                      hipStream_t stream, int64_t* bytes_read) {
    if (!src || !sink || !bytes_read || bytes < 0 || workgroups < 1 || workgroups > 65535 ||
        (mode != 0 && mode != 1) || (reinterpret_cast<uintptr_t>(src) & 15) || (reinterpret_cast<uintptr_t>(sink) & 3))
        return 1;
    const int64_t unit = mode == 0 ? kTileBytes : kVgprStep;
    const int64_t per_wg = bytes / workgroups / unit;   // whole units per workgroup
    *bytes_read = per_wg * unit * workgroups;
    (void)hipGetLastError();
    if (mode == 0)
        hipLaunchKernelGGL(stream_lds_kernel, dim3(workgroups), dim3(kThreads), 0, stream,
                           static_cast<const char*>(src), per_wg, sink);
    else
        hipLaunchKernelGGL(stream_vgpr_kernel, dim3(workgroups), dim3(kThreads), 0, stream,
                           static_cast<const char*>(src), per_wg, sink);
    return hipGetLastError() == hipSuccess ? 0 : 5;
}
