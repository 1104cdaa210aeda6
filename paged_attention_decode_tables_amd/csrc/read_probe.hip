// read_probe.hip -- a plain HBM read stream with no math, the measuring
// stick for the decode kernels: the same bytes a decode step gathers (whole
// runs of a block per kv head, through the same page list) or a contiguous
// buffer, read with 16-byte nontemporal loads, all of an item's loads of
// several items in flight per wave. Every loaded dword is XORed into a
// per-thread sink, so nothing is dead code and a test can check that
// exactly the intended bytes were read.
#include "kernels.h"

namespace pa {

namespace {

constexpr int kProbeThreads = 256;
constexpr int kProbeItemsPerRound = 4;  // items whose loads are in flight together, per wave

// NI: 16-byte load instructions per item (pieces <= 64 * NI).
template <int NI>
__global__ __launch_bounds__(kProbeThreads) void k_read_probe(ProbeParams p)
{
    const int lane = threadIdx.x & 63;
    const int64_t wave = (int64_t)blockIdx.x * (kProbeThreads / 64) + (threadIdx.x >> 6);
    const int64_t nwaves = (int64_t)gridDim.x * (kProbeThreads / 64);
    const int nbase = p.base1 ? 2 : 1;
    const int64_t items = p.num_pages * p.runs_per_page * nbase;
    u32x4 acc = {0, 0, 0, 0};
    for (int64_t i0 = wave * kProbeItemsPerRound; i0 < items; i0 += nwaves * kProbeItemsPerRound) {
        u32x4 v[kProbeItemsPerRound][NI];
#pragma unroll
        for (int u = 0; u < kProbeItemsPerRound; ++u) {
            const int64_t i = i0 + u;
            // item i: base i % nbase, run (i / nbase) % runs_per_page of page (i / nbase) / runs_per_page
            const int64_t pr = i / nbase;
            const char* base = (i % nbase) ? p.base1 : p.base0;
            const int64_t page = i < items ? (int64_t)p.pages[pr / p.runs_per_page] : 0;
            const char* run = base + page * p.page_stride + (pr % p.runs_per_page) * p.run_stride;
#pragma unroll
            for (int k = 0; k < NI; ++k) {
                const int piece = k * 64 + lane;
                v[u][k] = (i < items && piece < p.pieces) ? load16_stream(run + 16 * piece) : u32x4{0, 0, 0, 0};
            }
        }
#pragma unroll
        for (int u = 0; u < kProbeItemsPerRound; ++u)
#pragma unroll
            for (int k = 0; k < NI; ++k) acc ^= v[u][k];
    }
    reinterpret_cast<u32x4*>(p.sink)[(int64_t)blockIdx.x * kProbeThreads + threadIdx.x] = acc;
}

}  // namespace

hipError_t launch_read_probe(const ProbeParams& p, int workgroups, hipStream_t st)
{
    const int ni = (p.pieces + 63) / 64;
    const dim3 grid(workgroups), block(kProbeThreads);
    if (ni <= 1)
        hipLaunchKernelGGL(k_read_probe<1>, grid, block, 0, st, p);
    else if (ni <= 2)
        hipLaunchKernelGGL(k_read_probe<2>, grid, block, 0, st, p);
    else if (ni <= 4)
        hipLaunchKernelGGL(k_read_probe<4>, grid, block, 0, st, p);
    else
        hipLaunchKernelGGL(k_read_probe<8>, grid, block, 0, st, p);
    return hipGetLastError();
}

}  // namespace pa
